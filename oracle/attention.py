"""Block-sparse softmax attention, in fp64 (oracle; test infrastructure only).

Sol-Attn computes only the attention blocks that the per-step selection keeps
(Sol Engine "H3 on device" page, Sol-Attn paragraph; KOCPC article on Sol-H3,
"Technical Composition"). Reading: attention in a diffusion transformer is
non-causal; query block i attends to every valid token of each kept key block
and to nothing else, with scale 1/sqrt(D) unless given; a query block with no
kept key block outputs zeros. The result is the plain definition

    o_t = sum_{u in K(i)} softmax_u(q_t . k_u * scale) v_u,

K(i) = the tokens of the kept key blocks of t's block i.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np


def _kept_tokens(mask_row, block: int, S: int) -> np.ndarray:
    parts = [np.arange(j * block, min((j + 1) * block, S)) for j in np.nonzero(mask_row)[0]]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _attend(qrows, krows, vrows, scale: float) -> np.ndarray:
    if krows.shape[0] == 0:
        return np.zeros((qrows.shape[0], vrows.shape[1]), dtype=np.float64)
    logits = (qrows @ krows.T) * scale
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ vrows


def block_sparse_attention_rows(q, k, v, mask, block: int, rows: Iterable[Tuple[int, int, int]],
                                scale: Optional[float] = None) -> np.ndarray:
    """Output rows of selected (b, h, query block) triples: [len(rows), block, D].

    Rows past S in a partial last block are returned as zeros.
    """
    B, S, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = list(rows)
    out = np.zeros((len(rows), block, D), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        lo, hi = i * block, min((i + 1) * block, S)
        toks = _kept_tokens(mask[b, h, i], block, S)
        qr = np.asarray(q[b, lo:hi, h], dtype=np.float64)
        kr = np.asarray(k[b, toks, h], dtype=np.float64)
        vr = np.asarray(v[b, toks, h], dtype=np.float64)
        out[n, : hi - lo] = _attend(qr, kr, vr, scale)
    return out


def block_sparse_attention(q, k, v, mask, block: int, scale: Optional[float] = None) -> np.ndarray:
    """Full output [B, S, H, D] in fp64. q, k, v: [B, S, H, D]; mask: [B, H, nB, nB]."""
    B, S, H, D = q.shape
    nB = -(-S // block)
    o = np.zeros((B, S, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            blk = block_sparse_attention_rows(q, k, v, mask, block,
                                              [(b, h, i) for i in range(nB)], scale)
            o[b, :, h] = blk.reshape(nB * block, D)[:S]
    return o


def dense_attention(q, k, v, scale: Optional[float] = None) -> np.ndarray:
    """Dense non-causal softmax attention [B, S, H, D] in fp64 (the all-ones mask)."""
    B, S, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.zeros((B, S, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, :, h] = _attend(np.asarray(q[b, :, h], np.float64), np.asarray(k[b, :, h], np.float64),
                                 np.asarray(v[b, :, h], np.float64), scale)
    return o
