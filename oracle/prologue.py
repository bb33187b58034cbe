"""QKNorm and 3D multimodal RoPE, in fp64 (oracle; test infrastructure only).

Source: Sol Engine "H3 on device" page, lossless-kernels fusion table, row
"fused QKNorm + RoPE" (it removes two read/write passes over Q and K plus the
3D MM-RoPE indexing). The page names both operations but defines neither; the
definitions below are the plainest reading:

* QKNorm is an RMS norm of each (token, head) row over head_dim, with epsilon
  inside the square root and a per-channel weight of shape [head_dim] shared by
  all heads (separate weights for q and k);
* the norm comes first, then RoPE (the order of the fused name);
* 3D MM-RoPE splits head_dim into contiguous sections of widths (d_t, d_h, d_w)
  in that order; in the section of axis a, the adjacent pair (2i, 2i+1) is
  rotated by the angle pos_a * base^(-2i/d_a) (the original RoFormer form).
"""
from __future__ import annotations

import numpy as np


def qknorm(x, w, eps: float) -> np.ndarray:
    """x / sqrt(mean_d(x^2) + eps) * w over the last axis (head_dim), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope_inv_freq(d_a: int, base: float) -> np.ndarray:
    """Frequencies base^(-2i/d_a), i = 0 .. d_a/2 - 1, in fp64."""
    i = np.arange(d_a // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / d_a)


def rope_3d(x, pos_thw, sections, base: float) -> np.ndarray:
    """Rotate adjacent pairs of each (t, h, w) section by pos_a * base^(-2i/d_a).

    x: [..., S, H, D] (any leading batch axes), pos_thw: int [S, 3],
    sections: (d_t, d_h, d_w) with sum D, each even.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos_thw, dtype=np.float64)
    D = x.shape[-1]
    assert sum(sections) == D and all(d % 2 == 0 for d in sections)
    out = np.empty_like(x)
    off = 0
    for axis, d_a in enumerate(sections):
        theta = pos[:, axis][:, None] * rope_inv_freq(d_a, base)[None, :]     # [S, d_a/2]
        c = np.cos(theta)[:, None, :]                                          # [S, 1, d_a/2]
        s = np.sin(theta)[:, None, :]
        x0 = x[..., off:off + d_a:2]
        x1 = x[..., off + 1:off + d_a:2]
        out[..., off:off + d_a:2] = x0 * c - x1 * s
        out[..., off + 1:off + d_a:2] = x0 * s + x1 * c
        off += d_a
    return out


def qknorm_rope(q, k, pos_thw, w_q, w_k, sections, base: float, eps: float):
    """The fused prologue: (RoPE(QKNorm(q)), RoPE(QKNorm(k))) in fp64, unrounded."""
    qh = rope_3d(qknorm(q, w_q, eps), pos_thw, sections, base)
    kh = rope_3d(qknorm(k, w_k, eps), pos_thw, sections, base)
    return qh, kh
