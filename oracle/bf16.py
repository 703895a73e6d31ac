"""bfloat16 codec for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits, 7 stored significand bits. The pages store weights and the KV cache in
this type (MPK walk-through, section 3.3.1: every ``new_tensor`` is
``mi.bfloat16``). Rounding into it is round-to-nearest, ties-to-even, from the
exact value (float64 here), never via an intermediate float32.
"""
from __future__ import annotations

import numpy as np

_MAX_BF16 = float(np.uint32(0x7F7F0000).view(np.float32))     # (2 - 2^-7) * 2^127


def decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # signalling NaN patterns
        return u.view(np.float32).astype(np.float64)


def encode(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 bit pattern (uint16), ties to even.

    Finite values beyond the largest bf16 magnitude round to +-inf exactly when
    they are at or beyond the midpoint between that magnitude and 2^128.
    NaN maps to the canonical quiet NaN 0x7FC0 (with the input's sign).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    xf = np.where(fin, x, 0.0)
    ax = np.abs(xf)
    # quantum of the bf16 grid around |x|: 2^(e-8) for normal numbers, where
    # x = m * 2^e with m in [0.5, 1); 2^-133 below the smallest normal 2^-126.
    _, e = np.frexp(ax)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(ax / q) * q                # np.rint rounds half to even
    # the overflow threshold is the midpoint max + 2^(127-8); at it, ties-to-even
    # goes to 2^128, i.e. infinity (max's last significand bit is odd).
    r = np.where(ax >= _MAX_BF16 + 2.0 ** 119, np.inf, r)
    out[...] = np.copysign(r, xf)
    out = np.where(np.isinf(x), x, out)
    f32 = out.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = (np.signbit(x) & nan).astype(np.uint16) << np.uint16(15)
        bits = np.where(nan, np.uint16(0x7FC0) | sign, bits)
    return bits


def round_(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the bf16 grid, returned as float64."""
    return decode(encode(x))
