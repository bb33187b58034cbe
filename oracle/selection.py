"""Block selection, in fp64 (oracle; test infrastructure only).

The pages describe Sol-Attn's selection only as dynamic, per step, training-
and calibration-free, and deciding which (query block, key block) tiles of the
attention are computed (Sol Engine "H3 on device" page, Sol-Attn paragraph;
KOCPC article on Sol-H3, "Specific outcomes of key optimizations"). The rule
itself is lost from the page text, so this oracle states the build's rule:

1. blocks: block i holds tokens [i*block, min((i+1)*block, S)); the last block
   may be partial and is pooled over its valid tokens only;
2. pooling: p_i = (sum of the block's rows) / n_i in fp64, per (batch, head),
   for q-hat and k-hat separately. The inputs are bf16 values, so the fp64
   sum is exact whenever every non-zero |x| >= 2^-35 and |x| < 16; then any
   summation order gives the same p_i;
3. scores: s_ij = sum_d p^q_i[d] * p^k_j[d] in fp64, d ascending, each product
   and each sum rounded on its own (no fused multiply-add), unscaled;
4. keep k = clamp(ceil(keep_ratio * nB - 1e-6), 1, nB) blocks per query row:
   the diagonal block i, plus the k-1 largest s_ij over j != i, ties going to
   the lower j (and -0.0 equal to +0.0).
"""
from __future__ import annotations

import math

import numpy as np


def num_kept_blocks(keep_ratio: float, nB: int) -> int:
    """k = clamp(ceil(keep_ratio * nB - 1e-6), 1, nB); the 1e-6 guard stops fp error raising k."""
    if not (keep_ratio > 0.0 and keep_ratio <= 1.0):
        raise ValueError("keep_ratio must lie in (0, 1]")
    k = math.ceil(keep_ratio * nB - 1e-6)
    return int(min(max(k, 1), nB))


def block_token_range(i: int, block: int, S: int):
    return i * block, min((i + 1) * block, S)


def pool_blocks(x, block: int) -> np.ndarray:
    """Mean of each block of tokens, per head. x: [S, H, D] -> [H, nB, D] fp64."""
    x = np.asarray(x, dtype=np.float64)
    S, H, D = x.shape
    nB = -(-S // block)
    p = np.empty((H, nB, D), dtype=np.float64)
    for i in range(nB):
        lo, hi = block_token_range(i, block, S)
        p[:, i, :] = np.sum(x[lo:hi], axis=0) / float(hi - lo)
    return p


def block_scores(pq, pk) -> np.ndarray:
    """s[i, j] = sum_d pq[i, d] * pk[j, d]: fp64, d ascending, no fused multiply-add."""
    pq = np.asarray(pq, dtype=np.float64)
    pk = np.asarray(pk, dtype=np.float64)
    s = np.zeros((pq.shape[0], pk.shape[0]), dtype=np.float64)
    for d in range(pq.shape[1]):
        prod = pq[:, None, d] * pk[None, :, d]
        s = s + prod
    return s


def select_topk(scores, k: int) -> np.ndarray:
    """uint8 mask [nB, nB]: row i keeps i plus the k-1 best j != i by (-s_ij, j)."""
    scores = np.asarray(scores, dtype=np.float64)
    nB = scores.shape[0]
    mask = np.zeros((nB, nB), dtype=np.uint8)
    cols = np.arange(nB)
    for i in range(nB):
        cand = cols[cols != i]
        key = -scores[i, cand] + 0.0          # -0.0 and +0.0 compare equal anyway
        order = np.lexsort((cand, key))       # primary: -score; secondary: lower j
        mask[i, cand[order[:k - 1]]] = 1
        mask[i, i] = 1
    return mask


def select_blocks(qh, kh, block: int, keep_ratio: float) -> np.ndarray:
    """uint8 block mask [B, H, nB, nB] from post-prologue q-hat, k-hat [B, S, H, D]."""
    qh = np.asarray(qh)
    kh = np.asarray(kh)
    B, S, H, D = qh.shape
    nB = -(-S // block)
    k = num_kept_blocks(keep_ratio, nB)
    mask = np.zeros((B, H, nB, nB), dtype=np.uint8)
    for b in range(B):
        pq = pool_blocks(qh[b], block)
        pk = pool_blocks(kh[b], block)
        for h in range(H):
            mask[b, h] = select_topk(block_scores(pq[h], pk[h]), k)
    return mask
