"""Seeded synthetic inputs for one joint video+audio self-attention layer.

This module holds none of the method's arithmetic. It only fixes shapes,
draws seeded random numbers, lays out token positions and rounds the draws to
bf16. Both the HIP path (through the tests and the bench) and the CPU oracle
are fed from here, so the two sides always see the same bytes.

Workload shapes follow the Sol Engine "H3 on device" page (intro: 1344x768,
24 fps, 124 frames; the attention runs over one joint video-plus-audio
sequence, Sol-Attn paragraph). The per-config sizes (heads, head_dim, latent
grid, audio token count, block size, keep ratios) are the build's stated
workloads; the pages give none of them.

Recipe (all generators are ``numpy.random.Generator(PCG64(1000*c + t))``):

* config index c: tiny 1, small 2, medium 3, full 4 (the sweep base reuses 4),
  sweep drift 5;
* stream t: 0/1/2 N(0,1) noise for q/k/v; 3/4 w_q/w_k ~ U(0.9, 1.1) fp32;
  5 locality-field frequencies and phases; 6 field directions shared by q and
  k; 7 field directions for v;
* every noise tensor is drawn once as fp32 in C order with shape (B,S,H,D);
* tiny: pure N(0,1); the others: X = N(0,1) + L_X with the smooth locality
  field L = 0.5 * sum_{r<4} phi_r(token) * u_r[h] / sqrt(2) (element RMS 0.5),
  phi_r(video t,h,w) = cos(2pi(a_r t/T + b_r h/Hg + c_r w/W) + psi_r),
  phi_r(audio j) = cos(2pi a_r j/A + psi_r), a_r,b_r,c_r ~ U{0..3} not all 0;
* the fp32 sum is rounded to bf16 with round-to-nearest-even (torch's cast);
* positions: video tokens in t-major raster order get (t, h, w); audio token
  j gets (T + j, 0, 0);
* sweep step s: X_s = bf16(X_base_fp32 + 0.05 * s * Delta), Delta ~ N(0,1)
  drawn once per tensor from config index 5.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "LayerConfig", "CONFIGS", "get_config", "positions_thw", "make_inputs",
    "make_sweep_inputs", "sweep_parts", "compose_sweep_step", "rng_for", "bf16_from_f32",
]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int                 # seed index c
    B: int
    H: int
    D: int
    T: int                     # latent frames
    Hg: int                    # latent grid height
    W: int                     # latent grid width
    A: int                     # audio tokens
    block: int
    keep_ratios: Tuple[float, ...]
    sections: Tuple[int, int, int]   # RoPE head_dim split (t, h, w)
    locality: bool
    rope_base: float = 10000.0
    eps: float = 1e-6
    steps: int = 1             # >1 only for the denoising-step sweep
    drift: float = 0.0

    @property
    def S_video(self) -> int:
        return self.T * self.Hg * self.W

    @property
    def S(self) -> int:
        return self.S_video + self.A

    @property
    def nB(self) -> int:
        return -(-self.S // self.block)


CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny", 1, 1, 2, 64, 4, 8, 16, 512, 64, (0.5,), (16, 24, 24), False),
    "small": LayerConfig("small", 2, 1, 8, 128, 8, 24, 42, 128, 128, (0.25,), (32, 48, 48), True),
    "medium": LayerConfig("medium", 3, 1, 24, 128, 8, 48, 84, 512, 128, (1.0, 0.2), (32, 48, 48), True),
    "full": LayerConfig("full", 4, 1, 40, 128, 31, 48, 84, 2048, 128, (0.15,), (32, 48, 48), True),
    "sweep": LayerConfig("sweep", 4, 1, 40, 128, 31, 48, 84, 2048, 128, (0.1, 0.15, 0.3), (32, 48, 48),
                         True, steps=8, drift=0.05),
}

SWEEP_DRIFT_INDEX = 5


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]


def rng_for(c: int, t: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * c + t))


def bf16_from_f32(x: np.ndarray) -> torch.Tensor:
    """Round an fp32 array to bf16 (round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def positions_thw(T: int, Hg: int, W: int, A: int) -> np.ndarray:
    """int32 [S, 3]: video (t, h, w) in t-major raster order, then audio j -> (T + j, 0, 0)."""
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    video = np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)
    audio = np.zeros((A, 3), dtype=np.int64)
    audio[:, 0] = T + np.arange(A)
    return np.ascontiguousarray(np.concatenate([video, audio], axis=0).astype(np.int32))


def _field_params(c: int):
    rng = rng_for(c, 5)
    freqs = np.zeros((4, 3), dtype=np.int64)
    for r in range(4):
        while True:
            f = rng.integers(0, 4, size=3)
            if f.any():
                break
        freqs[r] = f
    phases = rng.uniform(0.0, 2.0 * math.pi, size=4)
    return freqs, phases


def _field_basis(cfg: LayerConfig) -> np.ndarray:
    """phi[S, 4] (fp64) of the locality field."""
    freqs, phases = _field_params(cfg.index)
    pos = positions_thw(cfg.T, cfg.Hg, cfg.W, cfg.A)
    phi = np.empty((cfg.S, 4), dtype=np.float64)
    sv = cfg.S_video
    t = pos[:sv, 0].astype(np.float64)
    h = pos[:sv, 1].astype(np.float64)
    w = pos[:sv, 2].astype(np.float64)
    j = np.arange(cfg.A, dtype=np.float64)
    for r in range(4):
        a, b, cc = freqs[r]
        phi[:sv, r] = np.cos(2 * math.pi * (a * t / cfg.T + b * h / cfg.Hg + cc * w / cfg.W) + phases[r])
        if cfg.A:
            phi[sv:, r] = np.cos(2 * math.pi * a * j / cfg.A + phases[r])
    return phi


def _noise(c: int, t: int, shape) -> np.ndarray:
    return rng_for(c, t).standard_normal(size=shape, dtype=np.float32)


def _base_f32(cfg: LayerConfig, which: int, dirs: Optional[np.ndarray], phi: Optional[np.ndarray]) -> np.ndarray:
    """fp32 (B,S,H,D) noise + locality field for tensor `which` (0 q, 1 k, 2 v)."""
    x = _noise(cfg.index, which, (cfg.B, cfg.S, cfg.H, cfg.D))
    if cfg.locality:
        # L[s, h, :] = 0.5 / sqrt(2) * sum_r phi[s, r] * u[r, h, :], added in row chunks.
        u = (dirs * (0.5 / math.sqrt(2.0))).reshape(4, cfg.H * cfg.D)
        chunk = 8192
        for b in range(cfg.B):
            for s0 in range(0, cfg.S, chunk):
                s1 = min(cfg.S, s0 + chunk)
                add = (phi[s0:s1] @ u).astype(np.float32).reshape(s1 - s0, cfg.H, cfg.D)
                x[b, s0:s1] += add
    return x


def _dirs(cfg: LayerConfig):
    if not cfg.locality:
        return None, None, None
    u_qk = rng_for(cfg.index, 6).standard_normal(size=(4, cfg.H, cfg.D))
    u_v = rng_for(cfg.index, 7).standard_normal(size=(4, cfg.H, cfg.D))
    return u_qk, u_v, _field_basis(cfg)


def _weights(cfg: LayerConfig):
    w_q = rng_for(cfg.index, 3).uniform(0.9, 1.1, size=cfg.D).astype(np.float32)
    w_k = rng_for(cfg.index, 4).uniform(0.9, 1.1, size=cfg.D).astype(np.float32)
    return torch.from_numpy(w_q), torch.from_numpy(w_k)


def make_inputs(cfg: LayerConfig | str, tensors: Sequence[str] = ("q", "k", "v")) -> dict:
    """Seeded layer inputs on the host.

    Returns q, k, v as bf16 torch tensors [B, S, H, D], pos_thw int32 [S, 3],
    w_q and w_k fp32 [D], plus the config.
    """
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    u_qk, u_v, phi = _dirs(cfg)
    out = {"cfg": cfg}
    for which, name in enumerate(("q", "k", "v")):
        if name not in tensors:
            continue
        dirs = u_v if name == "v" else u_qk
        x = _base_f32(cfg, which, dirs, phi)
        out[name] = bf16_from_f32(x)
        del x
    out["pos_thw"] = torch.from_numpy(positions_thw(cfg.T, cfg.Hg, cfg.W, cfg.A))
    out["w_q"], out["w_k"] = _weights(cfg)
    return out


def make_sweep_inputs(cfg: LayerConfig | str, step: int, tensors: Sequence[str] = ("q", "k", "v")) -> dict:
    """Inputs of denoising step `step` of the sweep: bf16(X_base + drift*step*Delta)."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    u_qk, u_v, phi = _dirs(cfg)
    out = {"cfg": cfg}
    for which, name in enumerate(("q", "k", "v")):
        if name not in tensors:
            continue
        dirs = u_v if name == "v" else u_qk
        x = _base_f32(cfg, which, dirs, phi)
        if step:
            delta = _noise(SWEEP_DRIFT_INDEX, which, x.shape)
            x += np.float32(cfg.drift * step) * delta
            del delta
        out[name] = bf16_from_f32(x)
        del x
    out["pos_thw"] = torch.from_numpy(positions_thw(cfg.T, cfg.Hg, cfg.W, cfg.A))
    out["w_q"], out["w_k"] = _weights(cfg)
    return out


def sweep_parts(cfg: LayerConfig | str, name: str):
    """(X_base, Delta) of tensor `name` of the sweep as fp32 torch tensors [B, S, H, D] on the host, so that a
    step can be composed where the data lives (``compose_sweep_step``)."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    which = ("q", "k", "v").index(name)
    u_qk, u_v, phi = _dirs(cfg)
    x = _base_f32(cfg, which, u_v if name == "v" else u_qk, phi)
    delta = _noise(SWEEP_DRIFT_INDEX, which, x.shape)
    return torch.from_numpy(x), torch.from_numpy(delta)


def compose_sweep_step(base: torch.Tensor, delta: torch.Tensor, drift: float, step: int,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16(base + fp32(drift*step) * delta) with the product and the sum each rounded to fp32 (two separate
    elementwise ops, as make_sweep_inputs does on the host), on whatever device the tensors are on."""
    c = torch.tensor(np.float32(drift * step), dtype=torch.float32, device=base.device)
    x = base if step == 0 else base + delta * c
    if out is None:
        return x.to(torch.bfloat16)
    out.copy_(x)
    return out


def make_small_case(S: int, H: int, D: int, seed: int, sections: Tuple[int, int, int], T: int = 0,
                    Hg: int = 1, W: int = 1) -> dict:
    """Plain N(0,1) bf16 q/k/v of arbitrary shape (ragged sizes, edge cases).

    Positions: the first T*Hg*W tokens form a raster grid, the rest are audio.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    A = S - T * Hg * W
    assert A >= 0
    out = {}
    for name in ("q", "k", "v"):
        out[name] = bf16_from_f32(g.standard_normal(size=(1, S, H, D), dtype=np.float32))
    out["pos_thw"] = torch.from_numpy(positions_thw(T, Hg, W, A))
    out["w_q"] = torch.from_numpy(g.uniform(0.9, 1.1, size=D).astype(np.float32))
    out["w_k"] = torch.from_numpy(g.uniform(0.9, 1.1, size=D).astype(np.float32))
    out["sections"] = sections
    return out
