"""CPU oracle for the MoE-layer forward (test infrastructure only).

Importable from the test suite, the smoke check and the benchmark's
CPU-baseline leg; the product package never imports it.
"""
