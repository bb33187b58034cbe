"""INT8 / FP8 block codecs for the attention exchange (oracle; test infrastructure only).

The pages send attention inputs between GPUs as INT8 and outputs as FP8 (KOCPC
article on Sol-H3, "Technical Composition": multi-GPU Sol-Attn with INT8 QKV and
FP8 output transfer). They give no scale granularity, rounding or format
variant. Readings taken here:

* one fp32 scale per (batch, token block, head) tile, the attention's own
  block of tokens over the full head_dim; scales are stored [B, H, nB];
* symmetric codes: INT8 in [-127, 127]; FP8 is OCP E4M3 ("FN": bias 7, no
  infinities, one NaN pattern per sign, largest finite 448);
* with amax the largest |x| of the tile (exact: x are bf16 values) and
  Q = 127 (INT8) or 448 (FP8): inv = fl32(Q / amax), the stored scale
  s = fl32(amax / Q), and each x encodes as round-to-nearest-even of
  fl32(x * inv) (an integer clamped to [-Q, Q] for INT8, the nearest E4M3
  value for FP8); a tile with amax < 2^-100 (all zero, or so small that inv
  would overflow fp32) has inv = s = 0, so every code is a zero (FP8 keeps
  the sign of x: x * 0 is a signed zero);
* decoding is fl32(value(code) * s), rounded to bf16 nearest-even.

The codes are integer decisions taken from floating point, so this oracle takes
them in the same fp32 steps the definition states (numpy float32 arithmetic is
IEEE single precision, correctly rounded); the E4M3 rounding is written out from
the format's definition and pinned against torch's float8_e4m3fn conversion.
"""
from __future__ import annotations

import numpy as np
import torch

INT8_MAX = 127
FP8_MAX = 448.0


# ------------------------------------------------------------------ E4M3 format

def e4m3_decode(code) -> np.ndarray:
    """Exact values (fp64) of E4M3 codes: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
    exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


_E4M3_MAGS = e4m3_decode(np.arange(127, dtype=np.uint8))     # codes 0..126: 0 .. 448, ascending


def e4m3_encode(v) -> np.ndarray:
    """Round fp32 values to the nearest E4M3 value, ties to the even code; magnitudes past 464 (the midpoint
    between 448 and the first unrepresentable step, 480) and NaN encode as NaN (no saturation)."""
    a32 = np.asarray(v, dtype=np.float32)
    a = np.abs(a32.astype(np.float64))
    neg = np.signbit(a32)
    idx = np.searchsorted(_E4M3_MAGS, a, side="left")          # mags[idx-1] < a <= mags[idx]
    idx_c = np.clip(idx, 1, 126)
    lo, hi = _E4M3_MAGS[idx_c - 1], _E4M3_MAGS[idx_c]
    d_lo, d_hi = a - lo, hi - a                                # exact in fp64
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((idx_c % 2) == 0))
    code = np.where(pick_hi, idx_c, idx_c - 1)
    code = np.where(a == 0.0, 0, code)
    code = np.where(a > 448.0, np.where(a > 464.0, 0x7F, 0x7E), code)   # 464 itself ties to 448 (even)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ------------------------------------------------------------------ block tiles

def _tiles(S: int, block: int):
    nB = -(-S // block)
    for i in range(nB):
        yield i, i * block, min(S, (i + 1) * block)


TINY_AMAX = 2.0 ** -100


def _scale_pair(amax: np.float32, qmax: float):
    if amax < TINY_AMAX:
        return np.float32(0.0), np.float32(0.0)
    q = np.float32(qmax)
    return np.float32(q / amax), np.float32(amax / q)


def quantize(x, block: int, fmt: str):
    """x: bf16 values as an array [B, S, H, D]. Returns (codes [B,S,H,D] int8 or uint8 E4M3, scales fp32 [B,H,nB])."""
    x32 = np.asarray(x, dtype=np.float32)
    B, S, H, D = x32.shape
    nB = -(-S // block)
    qmax = INT8_MAX if fmt == "int8" else FP8_MAX
    codes = np.zeros((B, S, H, D), dtype=np.int8 if fmt == "int8" else np.uint8)
    scales = np.zeros((B, H, nB), dtype=np.float32)
    for b in range(B):
        for i, t0, t1 in _tiles(S, block):
            for h in range(H):
                tile = x32[b, t0:t1, h, :]
                amax = np.float32(np.max(np.abs(tile)))
                inv, s = _scale_pair(amax, qmax)
                scales[b, h, i] = s
                v = (tile * inv).astype(np.float32)              # fl32(x * inv)
                if fmt == "int8":
                    codes[b, t0:t1, h, :] = np.clip(np.rint(v), -INT8_MAX, INT8_MAX).astype(np.int8)
                else:
                    codes[b, t0:t1, h, :] = e4m3_encode(v)
    return codes, scales


def dequantize(codes, scales, block: int, fmt: str) -> torch.Tensor:
    """bf16 tensor [B,S,H,D]: RNE_bf16(fl32(value(code) * s))."""
    c = np.asarray(codes)
    B, S, H, D = c.shape
    vals = c.astype(np.float32) if fmt == "int8" else e4m3_decode(c).astype(np.float32)
    out = np.zeros((B, S, H, D), dtype=np.float32)
    for b in range(B):
        for i, t0, t1 in _tiles(S, block):
            for h in range(H):
                out[b, t0:t1, h, :] = (vals[b, t0:t1, h, :] * np.float32(scales[b, h, i])).astype(np.float32)
    return torch.from_numpy(out).to(torch.bfloat16)
