"""Pins for the oracle's bf16 codec (round to nearest, ties to even).

Checked against: the exhaustive decode/encode round trip over all 2^16 bit
patterns; torch's own float32 -> bfloat16 cast (an independent
implementation) on float32-representable inputs, including every exact
midpoint; and hand-derived cases for the float64-only behaviour (values just
off a midpoint that a float32 intermediate would collapse onto it).
"""
import numpy as np
import pytest
import torch

from oracle import bf16


def all_patterns():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16.decode(u)
    return u[~np.isnan(f)], f[~np.isnan(f)]


def test_roundtrip_exhaustive():
    u, f = all_patterns()
    assert np.array_equal(bf16.encode(f), u)


def torch_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_midpoints_and_neighbours_match_torch():
    u, f = all_patterns()
    fin = np.isfinite(f)
    u, f = u[fin], f[fin]
    order = np.argsort(f, kind="stable")
    f = f[order]
    f = np.unique(f)                                     # +0/-0 collapse
    mids = (f[:-1] + f[1:]) / 2.0                        # exact: 9 significant bits
    mids = mids[np.abs(mids) < 3.0e38]
    x32 = mids.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), mids)  # representable in f32
    nudged = np.concatenate([x32, np.nextafter(x32, np.float32(np.inf)),
                             np.nextafter(x32, np.float32(-np.inf))])
    assert np.array_equal(bf16.encode(nudged.astype(np.float64)), torch_bits(nudged))


def test_random_float32_match_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(10.0) ** rng.integers(-40, 38, 200_000).astype(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(bf16.encode(x.astype(np.float64)), torch_bits(x))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),            # tie between 0x3F80 and 0x3F81 -> even
    (1.0 + 3 * 2 ** -8, 0x3F82),        # tie between 0x3F81 and 0x3F82 -> even
    (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),  # just above a tie (float64 only)
    (1.0 + 3 * 2 ** -8 - 2 ** -40, 0x3F81),  # just below a tie (float64 only)
    (-2.0, 0xC000),
    (2.0 ** -133, 0x0001),              # smallest subnormal
    (2.0 ** -134, 0x0000),              # tie between 0 and it -> even (0)
    (1.5 * 2.0 ** -134, 0x0001),
    ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),   # largest finite
    ((2 - 2 ** -7) * 2.0 ** 127 + 2.0 ** 119, 0x7F80),   # midpoint to 2^128 -> inf
    ((2 - 2 ** -7) * 2.0 ** 127 + 2.0 ** 119 - 2.0 ** 90, 0x7F7F),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
])
def test_cases(x, bits):
    assert int(bf16.encode(np.array([x]))[0]) == bits


def test_nan():
    assert int(bf16.encode(np.array([np.nan]))[0]) & 0x7FFF == 0x7FC0
