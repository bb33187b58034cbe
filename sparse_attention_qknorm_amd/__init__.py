"""Joint-sequence QKNorm + 3D RoPE, block selection and block-sparse attention on MI355X.

The per-layer self-attention of a video+audio diffusion transformer over one
joint token sequence, as the Sol Engine "H3 on device" page describes it
(fused QKNorm + RoPE in its fusion table; Sol-Attn's dynamic block sparsity).
Three calls, each a thin wrapper over the C ABI of libsaq.so (include/saq.h):

    qknorm_rope(q, k, pos_thw, (w_q, w_k), sections, base, eps)   # in place
    mask = select_blocks(q, k, keep_ratio, block)                 # uint8 [B,H,nB,nB]
    o = block_sparse_attn(q, k, v, mask, block)                   # bf16 [B,S,H,D]

Also: ``attention_layer`` (the three steps with the pooling fused into the
prologue), ``qknorm_rope_pool`` + ``select_blocks_pooled`` (that fused form
call by call), ``block_sparse_attn_select`` (selection inside the attention
kernel), ``MaskReuse`` / ``mask_overlap`` / ``pooled_change`` (cross-step mask
reuse and its measurements), ``quantize`` / ``dequantize`` (INT8 / FP8 block
codecs).

Tensors live on a ROCm device; torch provides memory and the current stream
only. The library must be built (``python -m sparse_attention_qknorm_amd.build``);
without it every call raises.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from ._binding import SaqError, check, lib

__all__ = ["qknorm_rope", "qknorm_rope_out", "qknorm_rope_pool", "select_blocks", "select_blocks_pooled",
           "select_blocks_noalloc",
           "select_workspace_bytes", "block_sparse_attn", "kept_blocks", "mask_overlap", "pooled_change", "pooled_bytes",
           "MaskReuse", "quantize", "dequantize", "block_sparse_attn_select", "attention_layer",
           "SaqError", "lib"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_buf(name: str, t: torch.Tensor, device: Optional[torch.device] = None) -> None:
    """A buffer handed to the library: a contiguous device tensor (on `device` when given)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


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
    _check_buf("workspace", workspace, q.device)
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
    _check_buf("workspace", workspace)
    if out is None:
        out = torch.empty((B, H, nB, nB), dtype=torch.uint8, device=workspace.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (B, H, nB, nB) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 [B,H,nB,nB] tensor")
    _check_buf("out", out, workspace.device)
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
    _check_buf("out", out, q.device)
    _check_buf("workspace", workspace, q.device)
    st = lib().saq_select_blocks(q.data_ptr(), k.data_ptr(), B, S, H, D, block, float(keep_ratio), out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "saq_select_blocks")
    return out


def select_blocks_noalloc(q: torch.Tensor, k: torch.Tensor, keep_ratio: float, block: int = 128,
                          out: torch.Tensor = None) -> torch.Tensor:
    """select_blocks with the library's own device scratch instead of a workspace (saq_select_blocks_noalloc).
    With `out` given, nothing is allocated. Calls that overlap on one GPU race (one scratch per GPU)."""
    _check_qkv("q", q)
    _check_qkv("k", k, q)
    B, S, H, D = q.shape
    nB = -(-S // block)
    if out is None:
        out = torch.empty((B, H, nB, nB), dtype=torch.uint8, device=q.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (B, H, nB, nB) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 [B,H,nB,nB] tensor")
    _check_buf("out", out, q.device)
    st = lib().saq_select_blocks_noalloc(q.data_ptr(), k.data_ptr(), B, S, H, D, block, float(keep_ratio),
                                         out.data_ptr(), _stream(q))
    check(st, "saq_select_blocks_noalloc")
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
    _check_buf("block_mask", block_mask, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_qkv("out", out, q)
    st = lib().saq_block_sparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), block_mask.data_ptr(), B, S, H, D,
                                     block, float(softmax_scale), out.data_ptr(), _stream(q))
    check(st, "saq_block_sparse_attn")
    return out


def mask_overlap(mask_a: torch.Tensor, mask_b: torch.Tensor) -> torch.Tensor:
    """int64 [B, H, 2]: (#kept in both masks, #kept in mask_a) per head (saq_mask_overlap)."""
    for n, m in (("mask_a", mask_a), ("mask_b", mask_b)):
        if m.dtype != torch.uint8 or m.dim() != 4 or not m.is_contiguous() or not m.is_cuda:
            raise ValueError(f"{n} must be a contiguous uint8 [B,H,nB,nB] device tensor")
    if mask_a.shape != mask_b.shape or mask_a.device != mask_b.device:
        raise ValueError("masks must have the same shape and device")
    B, H, nB, _ = mask_a.shape
    counts = torch.empty((B, H, 2), dtype=torch.int64, device=mask_a.device)
    st = lib().saq_mask_overlap(mask_a.data_ptr(), mask_b.data_ptr(), B, H, nB, counts.data_ptr(), _stream(mask_a))
    check(st, "saq_mask_overlap")
    return counts


def pooled_change(ws_prev: torch.Tensor, ws_cur: torch.Tensor, shape: Sequence[int], block: int = 128,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp64 device tensor whose [0] = sum (P_cur - P_prev)^2 and [1] = sum P_prev^2 over the pooled block means
    in two selection workspaces (saq_pooled_change). The relative change is sqrt([0] / [1])."""
    B, S, H, D = (int(x) for x in shape)
    n = lib().saq_pooled_change_out_len()
    _check_buf("ws_cur", ws_cur)
    _check_buf("ws_prev", ws_prev, ws_cur.device)
    if out is None:
        out = torch.empty(n, dtype=torch.float64, device=ws_cur.device)
    if out.dtype != torch.float64:
        raise ValueError("out must be a float64 tensor")
    _check_buf("out", out, ws_cur.device)
    st = lib().saq_pooled_change(ws_prev.data_ptr(), ws_cur.data_ptr(), B, S, H, D, block, out.data_ptr(),
                                 out.numel(), _stream(ws_cur))
    check(st, "saq_pooled_change")
    return out


def pooled_bytes(B: int, S: int, H: int, D: int, block: int = 128) -> int:
    """Bytes of the pooled fp64 block means of q and k, [2][B][H][nB][D] (saq_pooled_bytes)."""
    n = lib().saq_pooled_bytes(B, S, H, D, block)
    if n == 0:
        raise ValueError(f"unsupported shape B={B} S={S} H={H} D={D} block={block}")
    return n


class MaskReuse:
    """Device buffers of one gated-selection loop (saq_select_blocks_reuse): the mask in use, the pooled means it
    was selected from, and the decision state. `step` keeps or recomputes the mask on the device, without a host
    round trip; `recomputed()` and `relative_change()` read the last decision back (they synchronise)."""

    def __init__(self, shape: Sequence[int], keep_ratio: float, threshold: float, block: int = 128,
                 device="cuda:0"):
        self.shape = tuple(int(x) for x in shape)
        B, S, H, D = self.shape
        nB = -(-S // block)
        self.keep_ratio, self.threshold, self.block = float(keep_ratio), float(threshold), int(block)
        self.mask = torch.zeros((B, H, nB, nB), dtype=torch.uint8, device=device)
        self.pooled_ref = torch.zeros(pooled_bytes(B, S, H, D, block), dtype=torch.uint8, device=device)
        self.state = torch.zeros(lib().saq_reuse_state_len(), dtype=torch.float64, device=device)
        self.started = False

    def step(self, workspace: torch.Tensor, force: bool = False) -> torch.Tensor:
        B, S, H, D = self.shape
        _check_buf("workspace", workspace, self.mask.device)
        f = 1 if (force or not self.started) else 0
        st = lib().saq_select_blocks_reuse(B, S, H, D, self.block, self.keep_ratio, self.threshold, f,
                                           self.mask.data_ptr(), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), self.pooled_ref.data_ptr(),
                                           self.pooled_ref.numel(), self.state.data_ptr(), self.state.numel(),
                                           _stream(workspace))
        check(st, "saq_select_blocks_reuse")
        self.started = True
        return self.mask

    def recomputed(self) -> bool:
        return bool(self.state[2].item() != 0.0)

    def relative_change(self) -> float:
        d2, p2 = self.state[:2].tolist()
        return (d2 / p2) ** 0.5 if p2 > 0 else (0.0 if d2 == 0 else float("inf"))


def quantize(x: torch.Tensor, fmt: str, block: int = 128, codes: Optional[torch.Tensor] = None,
             scales: Optional[torch.Tensor] = None):
    """Block-scaled INT8 (fmt="int8") or OCP E4M3 (fmt="fp8") codes of a bf16 [B,S,H,D] tensor: (codes [B,S,H,D]
    int8 / uint8, scales fp32 [B,H,nB]) (saq_quantize_int8 / saq_quantize_fp8)."""
    _check_qkv("x", x)
    B, S, H, D = x.shape
    nB = -(-S // block)
    cdt = {"int8": torch.int8, "fp8": torch.uint8}[fmt]
    if codes is None:
        codes = torch.empty((B, S, H, D), dtype=cdt, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nB), dtype=torch.float32, device=x.device)
    if codes.dtype != cdt or tuple(codes.shape) != (B, S, H, D) or not codes.is_contiguous():
        raise ValueError(f"codes must be a contiguous {cdt} [B,S,H,D] tensor")
    if scales.dtype != torch.float32 or tuple(scales.shape) != (B, H, nB) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous float32 [B,H,nB] tensor")
    _check_buf("codes", codes, x.device)
    _check_buf("scales", scales, x.device)
    fn = lib().saq_quantize_int8 if fmt == "int8" else lib().saq_quantize_fp8
    check(fn(x.data_ptr(), B, S, H, D, block, codes.data_ptr(), scales.data_ptr(), _stream(x)),
          f"saq_quantize_{fmt}")
    return codes, scales


def dequantize(codes: torch.Tensor, scales: torch.Tensor, fmt: str, block: int = 128,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [B,S,H,D] from block-scaled codes (saq_dequantize_int8 / saq_dequantize_fp8)."""
    cdt = {"int8": torch.int8, "fp8": torch.uint8}[fmt]
    if codes.dtype != cdt or codes.dim() != 4 or not codes.is_contiguous() or not codes.is_cuda:
        raise ValueError(f"codes must be a contiguous {cdt} [B,S,H,D] device tensor")
    B, S, H, D = codes.shape
    nB = -(-S // block)
    if scales.dtype != torch.float32 or tuple(scales.shape) != (B, H, nB) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous float32 [B,H,nB] tensor")
    _check_buf("scales", scales, codes.device)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=codes.device)
    _check_qkv("out", out)
    if out.shape != codes.shape or out.device != codes.device:
        raise ValueError("out must match codes' shape and device")
    fn = lib().saq_dequantize_int8 if fmt == "int8" else lib().saq_dequantize_fp8
    check(fn(codes.data_ptr(), scales.data_ptr(), B, S, H, D, block, out.data_ptr(), _stream(codes)),
          f"saq_dequantize_{fmt}")
    return out


def block_sparse_attn_select(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor,
                             keep_ratio: float, block: int = 128, scale: float = 0.0,
                             out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None):
    """Attention with the block selection folded in, from the pooled means qknorm_rope_pool left in `workspace`
    (saq_block_sparse_attn_select). Returns o; if `mask_out` (uint8 [B,H,nB,nB]) is given, the chosen rows are
    written into it."""
    _check_qkv("q", q)
    _check_qkv("k", k, q)
    _check_qkv("v", v, q)
    B, S, H, D = q.shape
    nB = -(-S // block)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv("out", out, q)
    _check_buf("workspace", workspace, q.device)
    mptr = None
    if mask_out is not None:
        if mask_out.dtype != torch.uint8 or tuple(mask_out.shape) != (B, H, nB, nB) or not mask_out.is_contiguous():
            raise ValueError("mask_out must be a contiguous uint8 [B,H,nB,nB] tensor")
        _check_buf("mask_out", mask_out, q.device)
        mptr = mask_out.data_ptr()
    st = lib().saq_block_sparse_attn_select(q.data_ptr(), k.data_ptr(), v.data_ptr(), workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(), B, S, H, D, block,
                                            float(keep_ratio), float(scale), out.data_ptr(), mptr, _stream(q))
    check(st, "saq_block_sparse_attn_select")
    return out


def attention_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos_thw: torch.Tensor,
                    weights: Tuple[torch.Tensor, torch.Tensor], sections: Sequence[int], keep_ratio: float,
                    block: int = 128, base: float = 10000.0, eps: float = 1e-6, scale: float = 0.0,
                    buffers: Optional[dict] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The whole layer in three library calls: fused QKNorm + 3D RoPE with block pooling, selection from the
    pooled means, block-sparse attention. q and k are not modified. Returns (o, block_mask).

    `buffers` (optional dict) keeps device buffers across calls of the same shape: keys "q_hat", "k_hat",
    "workspace", "mask", "o" are filled on first use and reused afterwards."""
    B, S, H, D = q.shape
    nB = -(-S // block)
    buf = {} if buffers is None else buffers
    if "q_hat" not in buf:
        buf["q_hat"], buf["k_hat"] = torch.empty_like(q), torch.empty_like(k)
        buf["workspace"] = torch.empty(select_workspace_bytes(B, S, H, D, block), dtype=torch.uint8, device=q.device)
        buf["mask"] = torch.empty((B, H, nB, nB), dtype=torch.uint8, device=q.device)
        buf["o"] = torch.empty_like(q)
    qknorm_rope_pool(q, k, buf["q_hat"], buf["k_hat"], pos_thw, weights, sections, base, eps, block,
                     workspace=buf["workspace"])
    select_blocks_pooled(q.shape, keep_ratio, buf["workspace"], block, out=buf["mask"])
    block_sparse_attn(buf["q_hat"], buf["k_hat"], v, buf["mask"], block, scale, out=buf["o"])
    return buf["o"], buf["mask"]
