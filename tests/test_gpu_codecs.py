"""GPU parity of the INT8 / FP8 block codecs: codes, scales and decoded bf16
values bit-exact against the oracle (the oracle takes the same fp32 steps the
definition states), exhaustively over every bf16 value at scale 1, on ragged
and multi-tile shapes, on degenerate tiles, and on sampled tiles of the full
layer's tensors with round-trip bounds checked on every element."""
import numpy as np
import pytest
import torch

import sparse_attention_qknorm_amd as saq
from oracle import codecs
from parity_tools import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
QMAX = {"int8": 127.0, "fp8": 448.0}


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _roundtrip(x_bf16: torch.Tensor, fmt: str, block: int):
    codes, scales = saq.quantize(x_bf16.to(DEV), fmt, block)
    y = saq.dequantize(codes, scales, fmt, block)
    torch.cuda.synchronize()
    return codes.cpu(), scales.cpu(), y.cpu()


def _compare(x_bf16: torch.Tensor, fmt: str, block: int, what: str):
    codes, scales, y = _roundtrip(x_bf16, fmt, block)
    rc, rs = codecs.quantize(x_bf16.float().numpy(), block, fmt)
    assert np.array_equal(scales.numpy().view(np.uint32), rs.view(np.uint32)), f"{what}: scales differ"
    got = codes.numpy().view(np.uint8)
    ref = rc.view(np.uint8)
    if not np.array_equal(got, ref):
        idx = np.argwhere(got != ref)[0]
        raise AssertionError(f"{what}: {int((got != ref).sum())} codes differ; first at {tuple(idx)}: "
                             f"x={float(x_bf16[tuple(idx)])!r} got {got[tuple(idx)]:#x} ref {ref[tuple(idx)]:#x}")
    ry = codecs.dequantize(rc, rs, block, fmt)
    assert torch.equal(y.view(torch.int16), ry.view(torch.int16)), f"{what}: decoded values differ"
    return codes, scales, y


def _all_bf16_upto(limit: float) -> np.ndarray:
    v = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    return v[np.isfinite(v) & (np.abs(v) <= limit)]


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_every_bf16_value_at_scale_one(fmt):
    # every tile holds +-Q, so inv = s = 1 and the codes are the format's own rounding of each value
    q = QMAX[fmt]
    v = _all_bf16_upto(q)
    D, block = 128, 128
    per_tile = block * D - 1
    tiles = -(-len(v) // per_tile)
    x = np.zeros((tiles, per_tile + 1), dtype=np.float32)
    flat = np.zeros(tiles * per_tile, dtype=np.float32)
    flat[:len(v)] = v
    x[:, 1:] = flat.reshape(tiles, per_tile)
    x[:, 0] = q
    x = x.reshape(1, tiles * block, 1, D)
    _compare(_bf16(x), fmt, block, f"{fmt} exhaustive")
    log(f"  {fmt}: all {len(v)} bf16 values with |x| <= {q:g} encode and decode as the oracle's")


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("B,S,H,D,block,seed", [
    (2, 1000, 3, 128, 128, 1),      # ragged last tile (104 tokens)
    (1, 333, 5, 64, 64, 2),         # ragged, D = 64
    (1, 1, 1, 64, 64, 3),           # one token
    (1, 640, 2, 128, 64, 4),        # block 64, D 128
    (1, 300, 4, 64, 128, 5),        # block 128, D 64
])
def test_random_shapes(fmt, B, S, H, D, block, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    # per-head magnitudes from 1e-3 to 1e3 and heavy tails, so scales and subnormal codes vary
    mag = np.exp(g.uniform(np.log(1e-3), np.log(1e3), size=(1, 1, H, 1)))
    x = g.standard_t(3, size=(B, S, H, D)) * mag
    _compare(_bf16(x), fmt, block, f"{fmt} {B}x{S}x{H}x{D} block {block}")


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_degenerate_tiles(fmt):
    x = np.zeros((1, 256, 2, 64), dtype=np.float32)
    x[0, :128, 0] = np.linspace(-1e-31, 1e-31, 128 * 64).reshape(128, 64)      # amax < 2^-100: a zero tile
    x[0, 128:, 0] = 0.0                                                          # all zero
    x[0, :128, 1] = 3.0                                                          # constant tile
    x[0, 128:, 1, :] = -2.0 ** -100                                              # at the tiny limit
    codes, scales, y = _compare(_bf16(x), fmt, 128, f"{fmt} degenerate")
    assert scales[0, 0].tolist() == [0.0, 0.0]
    assert not y[0, :, 0].float().any()
    assert torch.equal(y[0, :128, 1].float(), torch.full((128, 64), 3.0))


@pytest.mark.timeout(300)
def test_full_layer_tensors_sampled():
    # the full layer's v and a seeded q-like tensor: sampled tiles bit-exact, bounds on every element
    from sparse_attention_qknorm_amd import synth
    cfg = synth.get_config("full")
    log("[codecs] generating full v")
    v = synth.make_inputs(cfg, tensors=("v",))["v"]
    B, S, H, D = v.shape
    block = cfg.block
    g = np.random.Generator(np.random.PCG64(77))
    tiles = [(0, 0, 0), (0, cfg.nB - 1, H - 1), (0, S // block // 2, 7)] + \
        [(0, int(g.integers(0, cfg.nB)), int(g.integers(0, H))) for _ in range(40)]
    vd = v.to(DEV)
    for fmt in ("int8", "fp8"):
        codes, scales = saq.quantize(vd, fmt, block)
        y = saq.dequantize(codes, scales, fmt, block)
        torch.cuda.synchronize()
        c_h, s_h = codes.cpu().numpy().view(np.uint8), scales.cpu().numpy()
        y_h = y.cpu()
        for (b, i, h) in tiles:
            t0, t1 = i * block, min(S, (i + 1) * block)
            xt = v[b:b + 1, t0:t1, h:h + 1].float().numpy()
            rc, rs = codecs.quantize(xt, block, fmt)
            assert s_h[b, h, i] == rs[0, 0, 0]
            assert np.array_equal(c_h[b, t0:t1, h], rc.view(np.uint8)[0, :, 0])
            ry = codecs.dequantize(rc, rs, block, fmt)
            assert torch.equal(y_h[b, t0:t1, h].view(torch.int16), ry[0, :, 0].view(torch.int16))
        # every element: |y - x| within half a code step (INT8: s/2; FP8: |x|/16 + s*2^-10) plus bf16 rounding
        xf = vd.float()
        sf = scales.permute(0, 2, 1).repeat_interleave(block, dim=1)[:, :S].unsqueeze(-1)
        err = (y.float() - xf).abs()
        if fmt == "int8":
            bound = sf * 0.5 * (1 + 1e-6) + xf.abs() * 2.0 ** -8
        else:
            bound = xf.abs() * (2.0 ** -4 + 2.0 ** -8) * (1 + 1e-6) + sf * 2.0 ** -10
        assert bool((err <= bound).all())
        rel = float((y.float() - xf).norm() / xf.norm())
        log(f"  full v {fmt}: {len(tiles)} sampled tiles bit-exact; round-trip relative Frobenius error {rel:.2e}")
        del codes, scales, y, xf, sf, err, bound
