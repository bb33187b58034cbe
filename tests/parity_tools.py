"""Comparison helpers shared by the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import math
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

# Output tolerance of the attention (the band the layer's statement fixes for bf16 inputs).
ATTN_MAX_ABS = 2e-2
ATTN_REL_FRO = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), np.exp2(-133.0))


def check_prologue(got: np.ndarray, ref: np.ndarray, what: str) -> float:
    """|got - ref| <= ulp_bf16(ref) + 1e-6 rms(row); returns the fraction equal to RNE(ref)."""
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    err = np.abs(got - ref)
    bound = bf16_ulp(ref) + 1e-6 * rms
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements beyond 1 bf16 ulp; first at {tuple(idx)}: "
                             f"got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}")
    rne = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    # fp64 -> fp32 -> bf16 can double-round; count exact matches only as a report
    return float(np.mean(got == rne))


def check_attention(got: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got - ref))
    log(f"  {what}: max_abs={max_abs:.3e} rel_fro={rel:.3e}")
    assert max_abs <= ATTN_MAX_ABS, f"{what}: max-abs error {max_abs} > {ATTN_MAX_ABS}"
    assert rel <= ATTN_REL_FRO, f"{what}: relative Frobenius error {rel} > {ATTN_REL_FRO}"
    return max_abs, rel


def pooled_exactness_ok(x: np.ndarray) -> bool:
    """The precondition under which fp64 block sums of bf16 values are exact: 2^-35 <= |x| < 16 or x == 0."""
    ax = np.abs(x)
    nz = ax[ax > 0]
    return bool(ax.max() < 16.0 and (nz.size == 0 or nz.min() >= 2.0 ** -35))


def oracle_mask(qh: np.ndarray, kh: np.ndarray, block: int, keep: float, heads=None) -> np.ndarray:
    """Oracle mask for selected heads (all by default), per batch entry."""
    B, S, H, D = qh.shape
    heads = range(H) if heads is None else heads
    nB = -(-S // block)
    kk = oracle.num_kept_blocks(keep, nB)
    out = {}
    for b in range(B):
        for h in heads:
            pq = oracle.pool_blocks(qh[b, :, h:h + 1], block)[0]
            pk = oracle.pool_blocks(kh[b, :, h:h + 1], block)[0]
            out[(b, h)] = oracle.select_topk(oracle.block_scores(pq, pk), kk)
    return out


def oracle_head_masks(qh: torch.Tensor, kh: torch.Tensor, block: int, keeps, heads, b: int = 0, workers: int = 8):
    """Oracle masks of whole heads of a large layer: {keep: {h: uint8 [nB, nB]}}.

    qh, kh: the GPU's bf16 q-hat / k-hat copied to the host, [B, S, H, D]. Each head is pooled and scored
    once and selected at every keep ratio; heads run on a thread pool (NumPy releases the GIL in its array
    loops). The exactness precondition of the pooled sums is asserted on every head."""
    nB = -(-qh.shape[1] // block)

    def one(h):
        q64 = qh[b, :, h].double().numpy()[:, None, :]
        k64 = kh[b, :, h].double().numpy()[:, None, :]
        assert pooled_exactness_ok(q64) and pooled_exactness_ok(k64), f"head {h}: pooled sums not exact"
        s = oracle.block_scores(oracle.pool_blocks(q64, block)[0], oracle.pool_blocks(k64, block)[0])
        return {kp: oracle.select_topk(s, oracle.num_kept_blocks(kp, nB)) for kp in keeps}

    heads = list(heads)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(one, heads))
    return {kp: {h: r[kp] for h, r in zip(heads, res)} for kp in keeps}


def oracle_head_attention(qh: torch.Tensor, kh: torch.Tensor, v: torch.Tensor, mask_h: np.ndarray, block: int,
                          h: int, b: int = 0) -> np.ndarray:
    """The oracle's output for every query block of one head, [S, D] fp64 (BLAS does the threading)."""
    S = qh.shape[1]
    nB = -(-S // block)
    q64 = qh[b:b + 1, :, h:h + 1].double().numpy()
    k64 = kh[b:b + 1, :, h:h + 1].double().numpy()
    v64 = v[b:b + 1, :, h:h + 1].double().numpy()
    rows = oracle.block_sparse_attention_rows(q64, k64, v64, mask_h[None, None], block,
                                              [(0, 0, i) for i in range(nB)])
    return rows.reshape(nB * block, -1)[:S]
