"""Stored-form views of torch tensors for the oracle (test infrastructure).

The oracle decodes inputs itself, so it receives bit patterns for the 16-
and 8-bit formats and float32 values for float32; no torch conversion is
involved in what it computes.
"""

import numpy as np
import torch


def stored(t: torch.Tensor) -> np.ndarray:
    """CPU numpy array holding the tensor's stored form."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.float32, torch.int32, torch.int64):
        return t.numpy()
    raise TypeError(t.dtype)
