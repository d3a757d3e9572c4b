"""Seeded synthetic workloads shared by the oracle and the HIP path."""

from .configs import CONFIGS, LayerConfig  # noqa: F401
from .inputs import make_inputs  # noqa: F401
