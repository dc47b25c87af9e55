"""Pins for the oracle's RoPE: closed forms, invariants and a scalar brute force."""

import math

import numpy as np
import pytest

import oracle
from _brute import brute_rope_row


def test_inv_freq_closed_form():
    # D = 4, theta = 1e4: the second pair turns at 1e4 ** (-1/2) = 1/100 of the first.
    inv = oracle.rope_inv_freq(4, 1e4)
    assert inv[0] == 1.0
    assert abs(inv[1] - 0.01) < 1e-17
    # Geometric ladder from 1 down towards 1/theta: ratio theta**(-2/D) throughout.
    inv = oracle.rope_inv_freq(128, 1e6)
    ratio = inv[1:] / inv[:-1]
    assert np.allclose(ratio, 1e6 ** (-2.0 / 128), rtol=1e-13, atol=0)
    assert abs(inv[-1] * 1e6 ** (-2.0 / 128) - 1e-6) < 1e-18   # one more step reaches 1/theta


def test_unit_vector_closed_form_half_split_pairs():
    # D = 4, theta = 1e4, position 100: pair (1, 3) turns by exactly 1 rad,
    # pair (0, 2) by 100 rad. R e_1 = cos(1) e_1 + sin(1) e_3; R e_3 = -sin(1) e_1 + cos(1) e_3.
    table = oracle.rope_table(101, 4, 1e4)
    e = np.eye(4, dtype=np.float32)[:, None, :]          # [4 tokens, 1 head, 4]
    y = oracle.rope_rotate(e, np.full(4, 100), table)[:, 0, :]
    c1, s1 = math.cos(1.0), math.sin(1.0)
    c0, s0 = math.cos(100.0), math.sin(100.0)
    exp = np.array([[c0, 0, s0, 0], [0, c1, 0, s1], [-s0, 0, c0, 0], [0, -s1, 0, c1]])
    assert np.allclose(y, exp, atol=1e-7, rtol=0)


def test_position_zero_is_identity_bitwise():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 64)).astype(np.float32)
    table = oracle.rope_table(8, 64, 1e4)
    y = oracle.rope_rotate(x, np.zeros(5, dtype=np.int64), table)
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32))


def test_pair_norms_preserved():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 4, 128)).astype(np.float32)
    pos = rng.integers(0, 40000, size=50)
    table = oracle.rope_table(40000, 128, 1e6)
    y = oracle.rope_rotate(x, pos, table).astype(np.float64)
    xd = x.astype(np.float64)
    nx = xd[..., :64] ** 2 + xd[..., 64:] ** 2
    ny = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(ny, nx, rtol=2e-6, atol=1e-6)


def test_relative_position_property():
    # <R(p) q, R(p') k> depends only on p - p'.
    rng = np.random.default_rng(4)
    D = 64
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, D)).astype(np.float32)
    table = oracle.rope_table(5000, D, 1e4)
    def dot(p, pp):
        a = oracle.rope_rotate(q, [p], table).astype(np.float64)
        b = oracle.rope_rotate(k, [pp], table).astype(np.float64)
        return float((a * b).sum())
    base = dot(7, 3)
    for shift in (1, 100, 2500, 4990):
        assert abs(dot(7 + shift - 1, 3 + shift - 1) - base) < 2e-4 * (1 + abs(base))
    assert abs(dot(9, 3) - base) > 1e-3       # a different offset gives a different value


def test_table_identities():
    table = oracle.rope_table(3000, 32, 1e4).astype(np.float64)
    c, s = table[:, :16], table[:, 16:]
    assert np.allclose(c * c + s * s, 1.0, atol=3e-7, rtol=0)
    # angle addition: angle(p + 1) = angle(p) + angle(1)
    c1, s1 = c[1], s[1]
    assert np.allclose(c[1:], c[:-1] * c1 - s[:-1] * s1, atol=2e-5, rtol=0)
    assert np.allclose(s[1:], s[:-1] * c1 + c[:-1] * s1, atol=2e-5, rtol=0)


def test_rotation_matches_scalar_brute_force_bitwise():
    rng = np.random.default_rng(5)
    D, theta = 16, 1e6
    x = rng.standard_normal((6, 2, D)).astype(np.float32)
    pos = np.array([0, 1, 17, 255, 4096, 32767])
    table = oracle.rope_table(32768, D, theta)
    y = oracle.rope_rotate(x, pos, table)
    for t in range(6):
        for h in range(2):
            ref = np.array(brute_rope_row([float(v) for v in x[t, h]], int(pos[t]), theta),
                           dtype=np.float32)
            assert np.array_equal(y[t, h].view(np.uint32), ref.view(np.uint32)), (t, h)
