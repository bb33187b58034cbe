"""Pins of the oracle's block selection: closed forms, exact arithmetic and brute force.

The rule (mean-pooled q/k per block, dot-product scores, top-k per query block
with the diagonal kept, ties to the lower index) is the build's statement of
the selection that the Sol-Attn paragraph of the Sol Engine "H3 on device" page
names but whose text the page has lost.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_attention_qknorm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("keep,nB,k", [
    (0.5, 16, 8), (0.25, 64, 16), (1.0, 256, 256), (0.2, 256, 52), (0.15, 993, 149),
    (0.1, 993, 100), (0.3, 993, 298), (0.3, 10, 3), (1e-9, 5, 1), (1.0, 1, 1), (0.7, 10, 7),
])
def test_num_kept_closed_form(keep, nB, k):
    assert oracle.num_kept_blocks(keep, nB) == k


@pytest.mark.parametrize("keep", [0.0, -0.1, 1.5, float("nan")])
def test_num_kept_rejects_out_of_range(keep):
    with pytest.raises(ValueError):
        oracle.num_kept_blocks(keep, 10)


def test_num_kept_matches_config_table():
    expect = {("tiny", 0.5): 8, ("small", 0.25): 16, ("medium", 1.0): 256, ("medium", 0.2): 52,
              ("full", 0.15): 149, ("sweep", 0.1): 100, ("sweep", 0.15): 149, ("sweep", 0.3): 298}
    for (name, keep), k in expect.items():
        assert oracle.num_kept_blocks(keep, synth.get_config(name).nB) == k


def test_select_golden():
    g = json.load(open(os.path.join(GOLD, "select_exact.json")))
    qh = np.array(g["q_hat"], dtype=np.float64).reshape(1, g["S"], 1, g["D"])
    kh = np.array(g["k_hat"], dtype=np.float64).reshape(1, g["S"], 1, g["D"])
    pq = oracle.pool_blocks(qh[0], g["block"])[0]
    pk = oracle.pool_blocks(kh[0], g["block"])[0]
    assert np.array_equal(pq, np.array(g["pooled_q"], dtype=float))
    assert np.array_equal(pk, np.array(g["pooled_k"], dtype=float))
    assert np.array_equal(oracle.block_scores(pq, pk), np.array(g["scores"], dtype=float))
    assert np.array_equal(oracle.select_blocks(qh, kh, g["block"], 0.5)[0, 0], np.array(g["mask_keep_0_5"]))
    assert np.array_equal(oracle.select_blocks(qh, kh, g["block"], 0.3)[0, 0], np.array(g["mask_keep_0_3"]))


def _bf16_values(shape, seed):
    # bf16-representable values of q-hat's size (|x| < 16), as the pooled inputs are
    x = synth.bf16_from_f32(np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32) * 3)
    return x.float().numpy().astype(np.float64)


@pytest.mark.parametrize("S,block", [(1024, 64), (1000, 64), (130, 128)])
def test_pool_blocks_equals_fsum_mean(S, block):
    x = _bf16_values((S, 2, 8), 20)
    p = oracle.pool_blocks(x, block)
    nB = -(-S // block)
    assert p.shape == (2, nB, 8)
    for h in range(2):
        for i in range(nB):
            lo, hi = i * block, min(S, (i + 1) * block)
            for d in range(8):
                assert p[h, i, d] == math.fsum(x[lo:hi, h, d]) / (hi - lo)


def test_pool_sum_is_exact_in_any_order():
    # bf16 inputs with |x| in [2^-35, 16): every partial sum is exact in fp64.
    x = _bf16_values((128, 1, 4), 21)
    fwd = np.zeros(4)
    for t in range(128):
        fwd = fwd + x[t, 0]
    rev = np.zeros(4)
    for t in reversed(range(128)):
        rev = rev + x[t, 0]
    exact = [Fraction(0)] * 4
    for t in range(128):
        for d in range(4):
            exact[d] += Fraction(float(x[t, 0, d]))
    assert np.array_equal(fwd, rev)
    assert all(Fraction(float(fwd[d])) == exact[d] for d in range(4))


def test_block_scores_match_blas_and_scalar_order():
    g = np.random.Generator(np.random.PCG64(22))
    pq, pk = g.standard_normal((17, 32)), g.standard_normal((19, 32))
    s = oracle.block_scores(pq, pk)
    np.testing.assert_allclose(s, pq @ pk.T, rtol=0, atol=1e-12)
    for i in (0, 5, 16):
        for j in (0, 7, 18):
            acc = 0.0
            for d in range(32):
                acc = acc + float(pq[i, d]) * float(pk[j, d])     # scalar fp64, d ascending
            assert s[i, j] == acc


def _brute_topk(scores, k):
    n = scores.shape[0]
    m = np.zeros((n, n), dtype=np.uint8)
    for i in range(n):
        m[i, i] = 1
        for j in range(n):
            if j == i:
                continue
            rank = sum(1 for l in range(n) if l != i and (scores[i, l] > scores[i, j] or
                                                         (scores[i, l] == scores[i, j] and l < j)))
            if rank < k - 1:
                m[i, j] = 1
    return m


@pytest.mark.parametrize("seed,n,k", [(30, 12, 4), (31, 16, 8), (32, 9, 1), (33, 9, 9), (34, 20, 7)])
def test_select_topk_brute_force_with_ties(seed, n, k):
    g = np.random.Generator(np.random.PCG64(seed))
    scores = g.integers(-3, 4, size=(n, n)).astype(np.float64)   # many ties
    scores[g.random((n, n)) < 0.1] = -0.0
    assert np.array_equal(oracle.select_topk(scores, k), _brute_topk(scores, k))


def test_select_topk_signed_zero_ties():
    s = np.array([[5.0, -0.0, 0.0, 0.0], [0.0, 1.0, -0.0, 2.0], [0.0] * 4, [-0.0, 0.0, 0.0, 0.0]])
    m = oracle.select_topk(s, 2)
    assert m[0].tolist() == [1, 1, 0, 0]          # -0.0 at j=1 ties +0.0 at j=2: lower index
    assert m[1].tolist() == [0, 1, 0, 1]
    assert m[2].tolist() == [1, 0, 1, 0]
    assert m[3].tolist() == [1, 0, 0, 1]


def test_constant_inputs_keep_lowest_indices():
    qh = np.ones((1, 640, 2, 8))
    m = oracle.select_blocks(qh, qh, 64, 0.4)          # nB = 10, k = 4, all scores tie
    for i in range(10):
        want = {i} | set([j for j in range(10) if j != i][:3])
        assert set(np.nonzero(m[0, 0, i])[0].tolist()) == want


def test_mask_invariants_and_permutation_equivariance():
    g = np.random.Generator(np.random.PCG64(40))
    scores = g.standard_normal((15, 15))
    m = oracle.select_topk(scores, 5)
    assert (m.sum(axis=1) == 5).all() and (np.diag(m) == 1).all()
    perm = g.permutation(15)
    mp = oracle.select_topk(scores[np.ix_(perm, perm)], 5)
    assert np.array_equal(mp, m[np.ix_(perm, perm)])
    assert (oracle.select_topk(scores, 15) == 1).all()


def test_ranking_matches_exact_rationals_on_tiny():
    # Canonical fp64 scores give the same kept sets as exact rational scores on the tiny
    # config (its top-k boundaries are far wider than fp64 rounding).
    inp = synth.make_inputs("tiny")
    cfg = inp["cfg"]
    qh, kh = oracle.qknorm_rope(inp["q"].double().numpy(), inp["k"].double().numpy(), inp["pos_thw"].numpy(),
                                inp["w_q"].numpy(), inp["w_k"].numpy(), cfg.sections, cfg.rope_base, cfg.eps)
    qb = synth.bf16_from_f32(qh.astype(np.float32)).double().numpy()   # the bf16 tensors attention consumes
    kb = synth.bf16_from_f32(kh.astype(np.float32)).double().numpy()
    mask = oracle.select_blocks(qb, kb, cfg.block, cfg.keep_ratios[0])
    k = oracle.num_kept_blocks(cfg.keep_ratios[0], cfg.nB)
    for h in range(cfg.H):
        pq = [[sum(Fraction(float(v)) for v in qb[0, i * 64:(i + 1) * 64, h, d]) / 64 for d in range(cfg.D)]
              for i in range(cfg.nB)]
        pk = [[sum(Fraction(float(v)) for v in kb[0, i * 64:(i + 1) * 64, h, d]) / 64 for d in range(cfg.D)]
              for i in range(cfg.nB)]
        for i in range(cfg.nB):
            exact = [(sum(a * b for a, b in zip(pq[i], pk[j])), j) for j in range(cfg.nB) if j != i]
            exact.sort(key=lambda t: (-t[0], t[1]))
            want = {i} | {j for _, j in exact[:k - 1]}
            assert set(np.nonzero(mask[0, h, i])[0].tolist()) == want
