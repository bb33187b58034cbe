"""Pins of the oracle's QKNorm and 3D RoPE to closed forms, invariants and library routines.

Definitions follow the Sol Engine "H3 on device" page, fusion table row "fused
QKNorm + RoPE", read as an RMS norm over head_dim followed by RoFormer-style
adjacent-pair rotary embedding on (t, h, w) sections.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed=0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------- QKNorm

def test_qknorm_golden():
    for case in json.load(open(os.path.join(GOLD, "qknorm_exact.json")))["cases"]:
        got = oracle.qknorm(np.array(case["x"]), np.array(case["w"]), case["eps"])
        assert np.array_equal(got, np.array(case["expected"])), case["derivation"]


@pytest.mark.parametrize("eps", [1e-6, 3.0])
def test_qknorm_mean_square_closed_form(eps):
    # with w = 1: mean(x_hat^2) = ms / (ms + eps) per (token, head) row; eps outside the
    # root, a wrong reduction axis or a missing square would all break this.
    x = _rand((37, 3, 16), 1) * np.array([0.1, 1.0, 5.0])[None, :, None]
    xh = oracle.qknorm(x, np.ones(16), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(xh * xh, axis=-1), ms / (ms + eps), rtol=1e-13)


def test_qknorm_reduces_over_head_dim_only():
    x = _rand((5, 4, 8), 2)
    y = x.copy()
    y[:, 2, :] *= 1000.0                       # scale one head only
    a = oracle.qknorm(x, np.ones(8), 0.0)
    b = oracle.qknorm(y, np.ones(8), 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)   # scale-invariant per row, heads independent
    z = x.copy()
    z[3] *= 7.0                                # scale one token only
    np.testing.assert_allclose(oracle.qknorm(z, np.ones(8), 0.0), a, rtol=1e-13)


def test_qknorm_weight_is_per_channel():
    x = _rand((6, 2, 8), 3)
    w = np.array([0.5, 1.0, 2.0, 4.0, 0.25, 3.0, 1.5, 0.75])
    np.testing.assert_allclose(oracle.qknorm(x, w, 1e-6), oracle.qknorm(x, np.ones(8), 1e-6) * w, rtol=1e-15)


def test_qknorm_brute_force_scalar():
    x = _rand((3, 2, 8), 4)
    w = 0.9 + 0.2 * np.random.Generator(np.random.PCG64(5)).random(8)
    got = oracle.qknorm(x, w, 1e-6)
    for s in range(3):
        for h in range(2):
            row = [float(v) for v in x[s, h]]
            ms = math.fsum(v * v for v in row) / len(row)
            r = math.sqrt(ms + 1e-6)
            for d in range(8):
                assert abs(got[s, h, d] - row[d] / r * w[d]) <= 1e-15 * max(1.0, abs(got[s, h, d]))


# ---------------------------------------------------------------- RoPE

def test_rope_golden():
    for case in json.load(open(os.path.join(GOLD, "rope_width2.json")))["cases"]:
        x = np.array(case["x"], dtype=np.float64)[None, None, :]
        pos = np.array([case["pos"]])
        got = oracle.rope_3d(x, pos, tuple(case["sections"]), case["base"])[0, 0]
        np.testing.assert_allclose(got, case["expected"], rtol=0, atol=1e-15, err_msg=case["derivation"])


@pytest.mark.parametrize("sections,base", [((16, 24, 24), 10000.0), ((32, 48, 48), 10000.0), ((2, 4, 6), 7.0)])
def test_rope_equals_complex_multiplication(sections, base):
    # Textbook reduction: each adjacent pair (x0, x1) is the complex number x0 + i x1
    # multiplied by exp(i * pos_a * theta_i), theta_i = base^(-2i/d_a) -- here built with
    # numpy's logspace and complex exp, independent of the oracle's own arithmetic.
    D = sum(sections)
    S, H = 23, 3
    x = _rand((S, H, D), 6)
    pos = np.random.Generator(np.random.PCG64(7)).integers(0, 2100, size=(S, 3))
    got = oracle.rope_3d(x, pos, sections, base)
    off = 0
    for a, d_a in enumerate(sections):
        n = d_a // 2
        theta = np.logspace(0.0, -(d_a - 2) / d_a * math.log10(base), n) if n > 1 else np.ones(1)
        z = x[:, :, off:off + d_a:2] + 1j * x[:, :, off + 1:off + d_a:2]
        zr = z * np.exp(1j * pos[:, a][:, None, None] * theta[None, None, :])
        np.testing.assert_allclose(got[:, :, off:off + d_a:2], zr.real, atol=2e-12)
        np.testing.assert_allclose(got[:, :, off + 1:off + d_a:2], zr.imag, atol=2e-12)
        off += d_a


def test_rope_pair_isometry_and_identity():
    sections = (16, 24, 24)
    x = _rand((40, 2, 64), 8)
    pos = np.random.Generator(np.random.PCG64(9)).integers(0, 600, size=(40, 3))
    y = oracle.rope_3d(x, pos, sections, 10000.0)
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2, x[..., 0::2] ** 2 + x[..., 1::2] ** 2,
                               rtol=1e-13)
    zero = oracle.rope_3d(x, np.zeros((40, 3), dtype=np.int64), sections, 10000.0)
    assert np.array_equal(zero, x)


def test_rope_relative_position_and_composition():
    sections = (32, 48, 48)
    g = np.random.Generator(np.random.PCG64(10))
    q = _rand((1, 1, 128), 11)
    k = _rand((1, 1, 128), 12)
    for _ in range(5):
        p, pp, delta = g.integers(0, 1000, 3), g.integers(0, 1000, 3), g.integers(-300, 300, 3)
        a = np.dot(oracle.rope_3d(q, p[None], sections, 1e4).ravel(), oracle.rope_3d(k, pp[None], sections, 1e4).ravel())
        b = np.dot(oracle.rope_3d(q, (p + delta)[None], sections, 1e4).ravel(),
                   oracle.rope_3d(k, (pp + delta)[None], sections, 1e4).ravel())
        assert abs(a - b) <= 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)
        # R(a) R(b) = R(a + b)
        two = oracle.rope_3d(oracle.rope_3d(q, p[None], sections, 1e4), pp[None], sections, 1e4)
        one = oracle.rope_3d(q, (p + pp)[None], sections, 1e4)
        np.testing.assert_allclose(two, one, atol=1e-11)


def test_rope_section_order_and_adjacent_pairs():
    sections = (16, 24, 24)
    x = _rand((1, 1, 64), 13)
    for axis, (lo, hi) in enumerate([(0, 16), (16, 40), (40, 64)]):
        pos = np.zeros((1, 3), dtype=np.int64)
        pos[0, axis] = 5
        y = oracle.rope_3d(x, pos, sections, 10000.0)
        changed = np.nonzero(~np.isclose(y, x, rtol=0, atol=1e-14))[-1]
        assert changed.min() >= lo and changed.max() < hi, (axis, changed)
    for i in range(32):            # unit vector e_{2i} stays inside its pair (2i, 2i+1)
        e = np.zeros((1, 1, 64))
        e[0, 0, 2 * i] = 1.0
        y = oracle.rope_3d(e, np.array([[3, 4, 5]]), sections, 10000.0)
        nz = set(np.nonzero(np.abs(y[0, 0]) > 1e-15)[0].tolist())
        assert nz <= {2 * i, 2 * i + 1} and 2 * i in nz


def test_qknorm_rope_norm_preserved():
    x = _rand((9, 3, 64), 14)
    w = np.full(64, 1.0)
    pos = np.random.Generator(np.random.PCG64(15)).integers(0, 900, size=(9, 3))
    qh, kh = oracle.qknorm_rope(x, x, pos, w, w, (16, 24, 24), 10000.0, 1e-6)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(qh * qh, axis=-1), 64 * ms / (ms + 1e-6), rtol=1e-13)
    assert np.array_equal(qh, kh)
