"""Closed forms and invariants that pin the oracle's building blocks.

Each test checks a property fixed by mathematics (or a hand-derived value),
chosen so that a plausible slip -- eps outside the root, a missing gain, the
wrong RoPE pairing or sign, a softmax without the max shift, a transposed
attention operand -- fails at least one of them.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle.decoder import argmax_first, attend, rmsnorm, rope, rope_angles, silu, softmax

rng = np.random.default_rng(7)


# --- RMSNorm ------------------------------------------------------------------

@pytest.mark.parametrize("c,eps", [(3.0, 1e-5), (0.01, 1e-5), (-2.5, 0.5)])
def test_rmsnorm_constant_vector(c, eps):
    g = rng.standard_normal(16)
    y = rmsnorm(np.full(16, c), g, eps)
    assert np.allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)


def test_rmsnorm_mean_square():
    x = rng.standard_normal(64) * 3
    eps = 0.25
    y = rmsnorm(x, np.ones(64), eps)
    m = np.mean(x * x)
    assert math.isclose(np.mean(y * y), m / (m + eps), rel_tol=1e-13)


def test_rmsnorm_scale_invariant_without_eps():
    x = rng.standard_normal(32)
    g = rng.standard_normal(32)
    assert np.allclose(rmsnorm(7.5 * x, g, 0.0), rmsnorm(x, g, 0.0), rtol=1e-13)


def test_rmsnorm_gain_is_elementwise():
    x, g = rng.standard_normal(32), rng.standard_normal(32)
    assert np.allclose(rmsnorm(x, g, 1e-5), g * rmsnorm(x, np.ones(32), 1e-5), rtol=1e-14)


def test_rmsnorm_hand_value():
    # x = [3, 4]: mean square = 12.5; eps = 0.5 -> root 3.605551275463989
    y = rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.5)
    assert np.allclose(y, [3.0 / math.sqrt(13.0), 8.0 / math.sqrt(13.0)], rtol=1e-15)


# --- RoPE ---------------------------------------------------------------------

def test_rope_hand_value_pairs_half_split():
    # D = 4, theta = 1e4: w = [1, 1e-2]. u = e_0 rotates in the (0, 2) plane.
    out = rope(np.array([1.0, 0.0, 0.0, 0.0]), 1, 1e4)
    assert np.allclose(out, [math.cos(1.0), 0.0, math.sin(1.0), 0.0], rtol=0, atol=1e-15)
    out = rope(np.array([0.0, 1.0, 0.0, 0.0]), 3, 1e4)
    assert np.allclose(out, [0.0, math.cos(0.03), 0.0, math.sin(0.03)], rtol=0, atol=1e-15)
    assert np.allclose(rope_angles(2, 8, 100.0), [2.0, 2.0 / math.sqrt(10.0), 0.2, 0.2 / math.sqrt(10.0)])


def test_rope_position_zero_identity():
    u = rng.standard_normal((3, 64))
    assert np.array_equal(rope(u, 0, 5e5), u)


def test_rope_preserves_pair_norms():
    u = rng.standard_normal(128)
    r = rope(u, 12345, 5e5)
    n0 = u[:64] ** 2 + u[64:] ** 2
    n1 = r[:64] ** 2 + r[64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)


def test_rope_relative_position():
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p, pp in [(5, 9), (100, 37), (0, 1000)]:
        lhs = rope(q, p, 1e4) @ rope(k, pp, 1e4)
        rhs = q @ rope(k, pp - p, 1e4)
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-11)


def test_rope_composition():
    u = rng.standard_normal(64)
    assert np.allclose(rope(rope(u, 17, 1e4), 25, 1e4), rope(u, 42, 1e4), rtol=1e-12, atol=1e-13)


# --- softmax / attention ------------------------------------------------------

def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = rng.standard_normal((5, 40)) * 30
    p = softmax(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.allclose(softmax(s + 1000.0), p, rtol=1e-12)
    assert np.all(np.isfinite(softmax(np.array([1e4, 0.0]))))


def test_attention_equal_keys_gives_mean_value():
    k = np.tile(rng.standard_normal(16), (9, 1))
    v = rng.standard_normal((9, 16))
    assert np.allclose(attend(rng.standard_normal(16), k, v), v.mean(0), rtol=1e-13)


def test_attention_dominant_score_selects_row():
    k = rng.standard_normal((6, 8)) * 0.01
    q = np.zeros(8)
    q[0] = 1.0
    k[4, 0] = 1e4
    v = rng.standard_normal((6, 8))
    assert np.allclose(attend(q, k, v), v[4], rtol=1e-12)


def test_attention_brute_force():
    q, k, v = rng.standard_normal(4), rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    s = [sum(q[d] * k[i][d] for d in range(4)) / 2.0 for i in range(3)]
    w = [math.exp(x) for x in s]
    out = [sum(w[i] * v[i][d] for i in range(3)) / sum(w) for d in range(4)]
    assert np.allclose(attend(q, k, v), out, rtol=1e-13)


def test_attention_scale_is_inverse_sqrt_head_dim():
    # two keys whose scores differ by exactly sqrt(D) * ln 3 -> weights 3:1
    D = 16
    q = np.zeros(D)
    q[0] = 1.0
    k = np.zeros((2, D))
    k[0, 0] = math.sqrt(D) * math.log(3.0)
    v = np.array([[1.0] * D, [0.0] * D])
    assert np.allclose(attend(q, k, v), 0.75, rtol=1e-14)


# --- SiLU / argmax --------------------------------------------------------------

def test_silu_properties():
    z = np.linspace(-30, 30, 601)
    assert silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(silu(z) - silu(-z), z, rtol=1e-13, atol=1e-13)
    assert np.allclose(silu(z), z * expit(z), rtol=1e-13, atol=1e-300)


def test_argmax_first_on_ties():
    assert argmax_first(np.array([0.5, 2.0, 1.0, 2.0])) == 1
    assert argmax_first(np.array([-1.0, -1.0])) == 0
