"""bf16 <-> float64 conversions for the oracle (test infrastructure only).

bf16 is the top half of an IEEE binary32, so widening is exact: shift the 16
bits into the high half of a 32-bit word and read it as float32.  Narrowing
rounds to nearest, ties to even.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits(x) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of a torch bf16 tensor or a uint16 array."""
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.bfloat16:
            raise TypeError(f"expected bf16 tensor, got {x.dtype}")
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.asarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {x.dtype}")
    return x


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(x) -> np.ndarray:
    """float64 copy of a bf16 tensor / uint16 bits / float array."""
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.bfloat16:
            return bits_to_f64(bf16_bits(x))
        return x.detach().cpu().to(torch.float64).numpy()
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bits_to_f64(x)
    return x.astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16, nearest-even.

    Goes through float32 first (numpy's RNE), then rounds the binary32 pattern
    to its top 16 bits with ties to even.  The double rounding can differ from a
    single fp64 -> bf16 rounding only when the float32 value lands exactly on a
    bf16 tie; that is used for reporting, never for a gate."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r

