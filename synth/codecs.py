"""Storage encoders for the synthetic inputs: float32 -> bf16 bits and
float32 -> fp8 e4m3fn bits with a per-output-channel float32 scale.

Only encoders live here (turning random draws into the stored bytes of a
weight or activation).  Decoding those bytes into values is each consumer's
own business: the oracle and the GPU path decode them independently.

Formats:
  * bf16: the upper 16 bits of an IEEE binary32, produced by round-to-nearest-
    even on the discarded 16 bits.
  * fp8 e4m3fn (OCP 8-bit float, "fn" = finite only): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; no infinities, 0x7F/0xFF are NaN; the
    largest finite magnitude is 448 and the smallest subnormal 2^-9.
"""
from __future__ import annotations

import numpy as np

FP8_E4M3_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _e4m3_grid_round(a: np.ndarray) -> np.ndarray:
    """Round non-negative magnitudes (float64) to the nearest e4m3fn value, ties
    to even, saturating at 448."""
    a = np.minimum(a, FP8_E4M3_MAX)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                 # below 2^-6 the spacing stays 2^-9
    quantum = np.exp2(e - 3.0)              # 3 mantissa bits
    q = np.rint(a / quantum) * quantum      # np.rint rounds half to even
    return np.minimum(q, FP8_E4M3_MAX)


def e4m3_value_to_bits(q: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """Encode exact e4m3 magnitudes q (float64, already on the grid) with sign flags."""
    q = np.asarray(q, dtype=np.float64)
    with np.errstate(divide="ignore"):
        exp_unb = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    efield = np.where(normal, exp_unb + 7.0, 0.0)
    mant = np.where(normal, (q / np.exp2(exp_unb) - 1.0) * 8.0, q / 2.0 ** -9)
    bits = (efield.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    bits = np.where(q == 0, 0, bits)
    return (bits | (sign.astype(np.int64) << 7)).astype(np.uint8)


def f32_to_fp8_rowwise(w: np.ndarray):
    """Quantise a [N, K] float32 matrix to e4m3fn with one float32 scale per
    row (output channel): s_n = max_k |w[n,k]| / 448, code = RNE(w / s_n),
    saturating.  Returns (uint8 codes [N, K], float32 scales [N])."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1).astype(np.float64)
    scale = (amax / FP8_E4M3_MAX).astype(np.float32)
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    x = w.astype(np.float64) / scale.astype(np.float64)[:, None]
    q = _e4m3_grid_round(np.abs(x))
    return e4m3_value_to_bits(q, np.signbit(x)), scale
