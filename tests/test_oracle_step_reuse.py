"""Pins of the oracle's cross-step measurements: brute force and closed forms."""
import math

import numpy as np

import oracle


def test_mask_overlap_brute_force():
    g = np.random.Generator(np.random.PCG64(70))
    a = (g.random((2, 3, 9, 9)) < 0.4).astype(np.uint8) * g.integers(1, 4, (2, 3, 9, 9)).astype(np.uint8)
    b = (g.random((2, 3, 9, 9)) < 0.5).astype(np.uint8)
    c = oracle.mask_overlap(a, b)
    for bb in range(2):
        for h in range(3):
            both = sum(1 for i in range(9) for j in range(9) if a[bb, h, i, j] and b[bb, h, i, j])
            na = sum(1 for i in range(9) for j in range(9) if a[bb, h, i, j])
            assert c[bb, h].tolist() == [both, na]


def test_mask_overlap_special_cases():
    m = (np.random.Generator(np.random.PCG64(71)).random((1, 2, 8, 8)) < 0.3).astype(np.uint8)
    c = oracle.mask_overlap(m, m)
    assert (c[..., 0] == c[..., 1]).all()                      # identical masks overlap fully
    z = oracle.mask_overlap(m, 1 - m)
    assert (z[..., 0] == 0).all()                              # complements share nothing


def test_pooled_change_closed_forms():
    p = np.array([[3.0, 4.0], [0.0, 12.0]])                   # sum of squares 169
    assert oracle.pooled_change(p, p) == (0.0, 169.0)
    assert oracle.pooled_change(p, 2 * p) == (169.0, 169.0)    # cur - prev = prev
    assert oracle.relative_change(p, 2 * p) == 1.0
    assert oracle.relative_change(p, p + np.array([[0.0, 0.0], [5.0, 0.0]])) == math.sqrt(25.0 / 169.0)


def test_gate_closed_forms():
    p = np.array([[3.0, 4.0], [0.0, 12.0]])              # |p|^2 = 169
    q = p + np.array([[0.0, 0.0], [5.0, 0.0]])          # |q - p|^2 = 25: relative change 5/13
    assert oracle.keeps_mask(p, q, 5.0 / 13.0 + 1e-12, False)
    assert not oracle.keeps_mask(p, q, 5.0 / 13.0 - 1e-9, False)
    assert oracle.keeps_mask(p, p, 0.0, False)          # unchanged means keep the mask even at threshold 0
    assert not oracle.keeps_mask(p, p, 1.0, True)       # forced recompute
    z = np.zeros_like(p)
    assert oracle.keeps_mask(z, z, 0.0, False)
    assert not oracle.keeps_mask(z, p, 1e9, False)      # any change from all-zero means is infinite


def test_reuse_schedule_against_cumulative_drift():
    # steps drift along one direction by 1 per step from a base of norm 100: the change
    # against the reference is (s - ref)/100, so at threshold 0.025 the mask is selected
    # fresh every third step (changes 0.01, 0.02 keep it; 0.03 does not)
    base = np.zeros(4)
    base[0] = 100.0
    e = np.zeros(4)
    e[1] = 1.0
    steps = [base + s * e for s in range(8)]
    sched = oracle.reuse_schedule(steps, 0.025)
    assert [r for r, _ in sched] == [True, False, False, True, False, False, True, False]
    assert [ref for _, ref in sched] == [0, 0, 0, 3, 3, 3, 6, 6]
    assert all(r for r, _ in oracle.reuse_schedule(steps, 0.0))
    assert [r for r, _ in oracle.reuse_schedule(steps, 1.0)] == [True] + [False] * 7
