"""Pins of the oracle's block-sparse attention against a library routine, closed forms and brute force.

Reading: non-causal softmax attention of each query block over the tokens of
its kept key blocks (Sol-Attn paragraph, Sol Engine "H3 on device" page).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _qkv(S, H, D, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return [g.standard_normal((1, S, H, D)) for _ in range(3)]


def _sdpa(q, k, v, token_mask=None, scale=None):
    # torch's float64 CPU scaled_dot_product_attention; [B,S,H,D] -> [B,H,S,D] and back
    t = [torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v)]
    am = None if token_mask is None else torch.from_numpy(token_mask)
    o = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=am, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


def test_attention_golden():
    g = json.load(open(os.path.join(GOLD, "attention_exact.json")))
    q = np.array(g["q"], dtype=np.float64).reshape(1, 2, 1, g["D"])
    q[0, 0, 0, 0] = math.log(3.0)
    k = np.array(g["k"], dtype=np.float64).reshape(1, 2, 1, g["D"])
    v = np.array(g["v"], dtype=np.float64).reshape(1, 2, 1, g["D"])
    o = oracle.block_sparse_attention(q, k, v, np.ones((1, 1, 1, 1), np.uint8), g["block"], scale=g["scale"])
    np.testing.assert_allclose(o[0, :, 0], np.array(g["expected"], dtype=float), rtol=0, atol=1e-14)


@pytest.mark.parametrize("S,H,D,block", [(256, 2, 64, 64), (200, 1, 32, 64)])
def test_all_ones_mask_equals_library_dense_attention(S, H, D, block):
    q, k, v = _qkv(S, H, D, 50)
    nB = -(-S // block)
    o = oracle.block_sparse_attention(q, k, v, np.ones((1, H, nB, nB), np.uint8), block)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.dense_attention(q, k, v), o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,block,seed", [(256, 64, 51), (1000, 64, 52), (300, 128, 53)])
def test_block_mask_equals_library_token_mask(S, block, seed):
    H, D = 2, 16
    q, k, v = _qkv(S, H, D, seed)
    nB = -(-S // block)
    g = np.random.Generator(np.random.PCG64(seed + 100))
    mask = (g.random((1, H, nB, nB)) < 0.4).astype(np.uint8)
    mask[0, 0, 1, :] = 0                                            # one empty row
    mask[0, 1, :, nB - 1] = 1                                       # partial last block everywhere
    o = oracle.block_sparse_attention(q, k, v, mask, block)
    blk = np.minimum(np.arange(S) // block, nB - 1)
    tok = mask[0][:, blk][:, :, blk].astype(bool)                   # [H, S, S]
    ref = _sdpa(q, k, v, tok[None])
    for h in range(H):
        for i in range(nB):
            rows = slice(i * block, min(S, (i + 1) * block))
            if mask[0, h, i].any():
                np.testing.assert_allclose(o[0, rows, h], ref[0, rows, h], rtol=0, atol=1e-12)
            else:
                assert (o[0, rows, h] == 0).all()


def test_convex_combination_and_constant_v():
    S, H, D, block = 320, 1, 16, 64
    q, k, v = _qkv(S, H, D, 54)
    nB = 5
    mask = np.zeros((1, 1, nB, nB), np.uint8)
    mask[0, 0, :, 2] = 1
    mask[0, 0, 3, 4] = 1
    o = oracle.block_sparse_attention(q, k, v, mask, block)
    for i in range(nB):
        toks = np.concatenate([np.arange(j * 64, (j + 1) * 64) for j in np.nonzero(mask[0, 0, i])[0]])
        lo, hi = v[0, toks, 0].min(axis=0), v[0, toks, 0].max(axis=0)
        rows = o[0, i * 64:(i + 1) * 64, 0]
        assert (rows >= lo - 1e-12).all() and (rows <= hi + 1e-12).all()
    vc = np.full_like(v, 0.375)
    np.testing.assert_allclose(oracle.block_sparse_attention(q, k, vc, mask, block), 0.375, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_kept_values():
    S, H, D, block = 256, 1, 8, 64
    q, k, v = _qkv(S, H, D, 55)
    k[:] = k[:, :1]
    mask = np.zeros((1, 1, 4, 4), np.uint8)
    mask[0, 0, 0, [0, 3]] = 1
    mask[0, 0, 1:, 1] = 1
    o = oracle.block_sparse_attention(q, k, v, mask, block)
    mean03 = np.concatenate([v[0, 0:64, 0], v[0, 192:256, 0]]).mean(axis=0)
    np.testing.assert_allclose(o[0, 0:64, 0], np.broadcast_to(mean03, (64, D)), atol=1e-13)
    np.testing.assert_allclose(o[0, 64:, 0], np.broadcast_to(v[0, 64:128, 0].mean(axis=0), (192, D)), atol=1e-13)


def test_brute_force_scalar_loops():
    S, H, D, block = 20, 1, 4, 8
    q, k, v = _qkv(S, H, D, 56)
    mask = np.array([[[[1, 0, 1], [0, 1, 0], [1, 1, 1]]]], np.uint8)
    o = oracle.block_sparse_attention(q, k, v, mask, block, scale=0.7)
    for t in range(S):
        i = t // block
        keys = [u for u in range(S) if mask[0, 0, i, u // block]]
        logits = [0.7 * sum(q[0, t, 0, d] * k[0, u, 0, d] for d in range(D)) for u in keys]
        mx = max(logits)
        e = [math.exp(x - mx) for x in logits]
        z = math.fsum(e)
        for d in range(D):
            want = math.fsum(e[n] * v[0, u, 0, d] for n, u in enumerate(keys)) / z
            assert abs(o[0, t, 0, d] - want) < 1e-14


def test_rows_helper_matches_full_output():
    S, H, D, block = 300, 2, 16, 64
    q, k, v = _qkv(S, H, D, 57)
    nB = 5
    mask = (np.random.Generator(np.random.PCG64(58)).random((1, H, nB, nB)) < 0.5).astype(np.uint8)
    full = oracle.block_sparse_attention(q, k, v, mask, block)
    rows = oracle.block_sparse_attention_rows(q, k, v, mask, block, [(0, 1, 4), (0, 0, 2)])
    np.testing.assert_array_equal(rows[0, :44], full[0, 256:300, 1])
    assert (rows[0, 44:] == 0).all()
    np.testing.assert_array_equal(rows[1], full[0, 128:192, 0])
