"""Rounding rules and the activation used by the oracle (test infrastructure only).

The dataflow page fixes no precision; the workloads fix storage types
(fp32 payloads, bf16 activations and weights). The oracle computes in fp64
and rounds once where a buffer of the stated type is written.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc as _erfc


def to_f32(a) -> np.ndarray:
    """Round to the nearest fp32 (ties to even): numpy's float64 -> float32 cast."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def to_bf16(a32) -> np.ndarray:
    """Round fp32 values to bfloat16, ties to even; returned as float32 holding
    exactly representable bf16 values.

    bfloat16 keeps the top 16 bits of the fp32 encoding. Round-to-nearest-even
    on the dropped 16 bits: add 0x7FFF plus the lowest kept bit, then truncate.
    Inputs must be finite (the workloads never produce NaN or Inf).
    """
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if not np.all(np.isfinite(a32)):
        raise ValueError("to_bf16: non-finite input")
    bits = a32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


def gelu(z) -> np.ndarray:
    """Exact GELU in fp64: z * Phi(z), with Phi(z) = erfc(-z / sqrt(2)) / 2.

    The pages name no activation formula; the exact (erf) form is the plain
    definition (Hendrycks & Gimpel), not the tanh approximation. Phi is taken
    through erfc, which equals 1 + erf(z / sqrt(2)) over 2 but does not cancel
    for negative z: the erf form loses every digit below z ~ -8 in fp64
    (it returns 0 for GELU(-10) = -7.6e-23).
    """
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * _erfc(-z / np.sqrt(2.0))
