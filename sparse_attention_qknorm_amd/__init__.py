"""Joint-sequence QKNorm + 3D RoPE, block selection and block-sparse attention on MI355X.

The per-layer self-attention of a video+audio diffusion transformer over one
joint token sequence, as the Sol Engine "H3 on device" page describes it
(fused QKNorm + RoPE in its fusion table; Sol-Attn's dynamic block sparsity).
Three calls, each a thin wrapper over the C ABI of libsaq.so (include/saq.h):

    qknorm_rope(q, k, pos_thw, (w_q, w_k), sections, base, eps)   # in place
    mask = select_blocks(q, k, keep_ratio, block)                 # uint8 [B,H,nB,nB]
    o = block_sparse_attn(q, k, v, mask, block)                   # bf16 [B,S,H,D]

Tensors live on a ROCm device; torch provides memory and the current stream
only. The library must be built (``python -m sparse_attention_qknorm_amd.build``);
without it every call raises.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from ._binding import SaqError, check, lib

__all__ = ["qknorm_rope", "qknorm_rope_out", "qknorm_rope_pool", "select_blocks", "select_blocks_pooled",
           "select_workspace_bytes", "block_sparse_attn", "kept_blocks", "SaqError", "lib"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_qkv(name: str, t: torch.Tensor, ref: Optional[torch.Tensor] = None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 [B,S,H,D] tensor")
    if ref is not None and (t.shape != ref.shape or t.device != ref.device):
        raise ValueError(f"{name} must match q's shape and device")


def qknorm_rope(q: torch.Tensor, k: torch.Tensor, pos_thw: torch.Tensor, weights: Tuple[torch.Tensor, torch.Tensor],
                sections: Sequence[int], base: float = 10000.0, eps: float = 1e-6) -> None:
    """Fused QKNorm + 3D RoPE, in place on q and k (saq_qknorm_rope)."""
    qknorm_rope_out(q, k, q, k, pos_thw, weights, sections, base, eps)


def qknorm_rope_out(q: torch.Tensor, k: torch.Tensor, q_out: torch.Tensor, k_out: torch.Tensor,
                    pos_thw: torch.Tensor, weights: Tuple[torch.Tensor, torch.Tensor], sections: Sequence[int],
                    base: float = 10000.0, eps: float = 1e-6) -> None:
    """Fused QKNorm + 3D RoPE from (q, k) into (q_out, k_out) (saq_qknorm_rope_out)."""
    _check_qkv("q", q)
    for n, t in (("k", k), ("q_out", q_out), ("k_out", k_out)):
        _check_qkv(n, t, q)
    w_q, w_k = weights
    B, S, H, D = q.shape
    if pos_thw.dtype != torch.int32 or tuple(pos_thw.shape) != (S, 3) or not pos_thw.is_contiguous() \
            or pos_thw.device != q.device:
        raise ValueError("pos_thw must be a contiguous int32 [S,3] tensor on q's device")
    for n, w in (("w_q", w_q), ("w_k", w_k)):
        if w.dtype != torch.float32 or tuple(w.shape) != (D,) or not w.is_contiguous() or w.device != q.device:
            raise ValueError(f"{n} must be a contiguous fp32 [D] tensor on q's device")
    dt, dh, dw = (int(x) for x in sections)
    st = lib().saq_qknorm_rope_out(q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(),
                                   pos_thw.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), B, S, H, D, dt, dh, dw,
                                   float(base), float(eps), _stream(q))
    check(st, "saq_qknorm_rope_out")


def _check_prologue_args(q, k, q_out, k_out, pos_thw, weights):
    _check_qkv("q", q)
    for n, t in (("k", k), ("q_out", q_out), ("k_out", k_out)):
        _check_qkv(n, t, q)
    B, S, H, D = q.shape
    if pos_thw.dtype != torch.int32 or tuple(pos_thw.shape) != (S, 3) or not pos_thw.is_contiguous() \
            or pos_thw.device != q.device:
        raise ValueError("pos_thw must be a contiguous int32 [S,3] tensor on q's device")
    for n, w in zip(("w_q", "w_k"), weights):
        if w.dtype != torch.float32 or tuple(w.shape) != (D,) or not w.is_contiguous() or w.device != q.device:
            raise ValueError(f"{n} must be a contiguous fp32 [D] tensor on q's device")


def qknorm_rope_pool(q: torch.Tensor, k: torch.Tensor, q_out: torch.Tensor, k_out: torch.Tensor,
                     pos_thw: torch.Tensor, weights: Tuple[torch.Tensor, torch.Tensor], sections: Sequence[int],
                     base: float = 10000.0, eps: float = 1e-6, block: int = 128,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """QKNorm + 3D RoPE into (q_out, k_out) plus the per-block pooled means, written into the returned
    selection workspace (saq_qknorm_rope_pool). Pass that workspace to select_blocks_pooled."""
    _check_prologue_args(q, k, q_out, k_out, pos_thw, weights)
    B, S, H, D = q.shape
    need = select_workspace_bytes(B, S, H, D, block)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dt, dh, dw = (int(x) for x in sections)
    w_q, w_k = weights
    st = lib().saq_qknorm_rope_pool(q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(),
                                    pos_thw.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), B, S, H, D, dt, dh, dw,
                                    float(base), float(eps), block, workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "saq_qknorm_rope_pool")
    return workspace


def select_blocks_pooled(shape: Sequence[int], keep_ratio: float, workspace: torch.Tensor, block: int = 128,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block mask from the pooled vectors qknorm_rope_pool left in `workspace` (saq_select_blocks_pooled).
    shape = (B, S, H, D) of q."""
    B, S, H, D = (int(x) for x in shape)
    nB = -(-S // block)
    if out is None:
        out = torch.empty((B, H, nB, nB), dtype=torch.uint8, device=workspace.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (B, H, nB, nB) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 [B,H,nB,nB] tensor")
    st = lib().saq_select_blocks_pooled(B, S, H, D, block, float(keep_ratio), out.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(workspace))
    check(st, "saq_select_blocks_pooled")
    return out


def kept_blocks(keep_ratio: float, nB: int) -> int:
    """k = clamp(ceil(keep_ratio * nB - 1e-6), 1, nB) (saq_kept_blocks)."""
    k = lib().saq_kept_blocks(float(keep_ratio), int(nB))
    check(min(k, 0), "saq_kept_blocks")
    return k


def select_workspace_bytes(B: int, S: int, H: int, D: int, block: int) -> int:
    n = lib().saq_select_blocks_workspace_bytes(B, S, H, D, block)
    if n == 0:
        raise ValueError("invalid sizes for select_blocks")
    return n


def select_blocks(q: torch.Tensor, k: torch.Tensor, keep_ratio: float, block: int = 128,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """uint8 block mask [B,H,nB,nB] with the diagonal and the top-k pooled-score blocks (saq_select_blocks)."""
    _check_qkv("q", q)
    _check_qkv("k", k, q)
    B, S, H, D = q.shape
    nB = -(-S // block)
    if out is None:
        out = torch.empty((B, H, nB, nB), dtype=torch.uint8, device=q.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (B, H, nB, nB) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 [B,H,nB,nB] tensor")
    need = select_workspace_bytes(B, S, H, D, block)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().saq_select_blocks(q.data_ptr(), k.data_ptr(), B, S, H, D, block, float(keep_ratio), out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "saq_select_blocks")
    return out


def block_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor, block: int = 128,
                      softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-sparse softmax attention over the kept blocks (saq_block_sparse_attn)."""
    _check_qkv("q", q)
    _check_qkv("k", k, q)
    _check_qkv("v", v, q)
    B, S, H, D = q.shape
    nB = -(-S // block)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (B, H, nB, nB) or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 [B,H,nB,nB] tensor")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_qkv("out", out, q)
    st = lib().saq_block_sparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), block_mask.data_ptr(), B, S, H, D,
                                     block, float(softmax_scale), out.data_ptr(), _stream(q))
    check(st, "saq_block_sparse_attn")
    return out
