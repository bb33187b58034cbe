"""Pins of the oracle's INT8 / FP8 block codecs: the E4M3 format against torch's
float8_e4m3fn conversion (a library routine), closed forms at scale 1 and 2,
and rounding/error bounds against exact arithmetic."""
from fractions import Fraction

import numpy as np
import torch

from oracle import codecs


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_library_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_decode_closed_forms():
    d = codecs.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xB8, 0xFE], dtype=np.uint8))
    assert d.tolist() == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -1.0, -448.0]
    assert np.isnan(codecs.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_encode_closed_forms():
    v = np.array([1.0, 448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 464.0, 464.5, -1.0, -2.0 ** -11],
                 dtype=np.float32)
    # 2^-10 ties 0 / 2^-9 -> 0 (even); 3*2^-10 ties codes 1 / 2 -> 2; 1.0625 ties 1.0 / 1.125 -> 1.0 (0x38 even);
    # 1.1875 ties 1.125 / 1.25 -> 1.25 (0x3A); 464 ties 448 / (480) -> 448; 464.5 is NaN; -2^-11 -> -0
    assert codecs.e4m3_encode(v).tolist() == [0x38, 0x7E, 0x01, 0x00, 0x02, 0x38, 0x3A, 0x7E, 0x7F, 0xB8, 0x80]


def test_e4m3_encode_matches_library_exhaustively_on_bf16_and_random_fp32():
    # every bf16 value (as fp32), incl. all ties between E4M3 neighbours and the subnormal range
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 464.0)]
    assert np.array_equal(codecs.e4m3_encode(v), _torch_e4m3(v))
    g = np.random.Generator(np.random.PCG64(33))
    r = (g.random(1 << 20) * 470.0 - 235.0).astype(np.float32) * np.exp2(g.integers(-14, 2, 1 << 20)).astype(np.float32)
    r = r[np.abs(r) <= 464.0]
    assert np.array_equal(codecs.e4m3_encode(r), _torch_e4m3(r))


def test_e4m3_encode_is_nearest():
    g = np.random.Generator(np.random.PCG64(34))
    v = (g.random(20000) * 440.0).astype(np.float32) * np.exp2(g.integers(-12, 1, 20000)).astype(np.float32)
    c = codecs.e4m3_encode(v)
    got = codecs.e4m3_decode(c)
    mags = codecs.e4m3_decode(np.arange(127, dtype=np.uint8))
    best = np.min(np.abs(mags[None, :] - v.astype(np.float64)[:, None]), axis=1)
    assert np.array_equal(np.abs(got - v.astype(np.float64)), best)


def test_int8_closed_forms_at_scale_one_and_two():
    # amax = 127 gives inv = s = 1: codes are RNE of the values themselves
    vals = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -127.0, 3.25, -3.75]
    x = np.zeros((1, 1, 1, len(vals)), dtype=np.float32)
    x[0, 0, 0] = vals
    codes, scales = codecs.quantize(x, 64, "int8")
    assert codes[0, 0, 0].tolist() == [127, 0, 2, 2, 0, -2, 126, -127, 3, -4]
    assert scales.tolist() == [[[1.0]]]
    # amax = 254 gives inv = 0.5, s = 2
    codes, scales = codecs.quantize(x * 2, 64, "int8")
    assert codes[0, 0, 0].tolist() == [127, 0, 2, 2, 0, -2, 126, -127, 3, -4]
    assert scales.tolist() == [[[2.0]]]
    y = codecs.dequantize(codes, scales, 64, "int8").float().numpy()
    assert y[0, 0, 0].tolist() == [254.0, 0.0, 4.0, 4.0, 0.0, -4.0, 252.0, -254.0, 6.0, -8.0]


def test_quantize_tiles_and_bounds():
    g = np.random.Generator(np.random.PCG64(35))
    B, S, H, D, block = 2, 150, 3, 16, 64                     # partial last block of 22 tokens
    x = torch.from_numpy(g.standard_normal((B, S, H, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    x[0, 64:128, 1] = 0.0                                       # an all-zero tile
    for fmt, qmax in (("int8", 127), ("fp8", 448.0)):
        codes, scales = codecs.quantize(x, block, fmt)
        assert scales.shape == (B, H, 3)
        assert scales[0, 1, 1] == 0.0 and not codes[0, 64:128, 1].any()     # +0 inputs: +0 codes
        for b in range(B):
            for i, (t0, t1) in enumerate([(0, 64), (64, 128), (128, 150)]):
                for h in range(H):
                    amax = float(np.abs(x[b, t0:t1, h]).max())
                    assert scales[b, h, i] == np.float32(np.float32(amax) / np.float32(qmax))
                    if amax == 0:
                        continue
                    vals = codes[b, t0:t1, h].astype(np.float64) if fmt == "int8" else \
                        codecs.e4m3_decode(codes[b, t0:t1, h])
                    # the tile's largest element encodes to +-qmax; all codes within range
                    assert np.abs(vals).max() == qmax
                    # nearest code to x * inv, against exact rationals (up to the fp32 rounding of the product)
                    inv = np.float32(np.float32(qmax) / np.float32(amax))
                    xs = x[b, t0:t1, h].ravel()
                    for xv, cv in zip(xs[:64], vals.ravel()[:64]):
                        exact = Fraction(float(xv)) * Fraction(float(inv))
                        if fmt == "int8":
                            assert abs(Fraction(cv) - exact) <= Fraction(1, 2) + Fraction(1, 1 << 16)
                        else:
                            assert abs(Fraction(cv) - exact) <= abs(exact) / 16 + Fraction(1, 1 << 10)
        # round trip: |dequant - x| <= s/2 (int8) or half an E4M3 step, plus the bf16 rounding
        y = codecs.dequantize(codes, scales, block, fmt).double().numpy()
        s_full = np.repeat(np.transpose(scales, (0, 2, 1)), block, axis=1)[:, :S][..., None].astype(np.float64)
        if fmt == "int8":
            bound = s_full * 0.5 * (1 + 1e-6) + np.abs(x) * 2.0 ** -8 + 1e-30
        else:
            bound = np.abs(x) * (2.0 ** -4 + 2.0 ** -8) * (1 + 1e-6) + s_full * 2.0 ** -10 + 1e-30
        assert (np.abs(y - x) <= bound).all()


def test_fp8_full_range_tile_is_the_format_itself():
    # a tile whose amax is 448 has inv = s = 1: the codes are the E4M3 encoding of the values
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    n = (len(v) // 64) * 64
    x = v[:n].reshape(1, n // 64, 1, 64)
    x[0, 0, 0, 0] = 448.0
    codes, scales = codecs.quantize(x, 4096, "fp8")
    assert (scales == 1.0).all()
    assert np.array_equal(codes.ravel(), _torch_e4m3(x.ravel()))


def test_tiny_tiles_are_zero_tiles():
    x = np.zeros((1, 4, 1, 8), dtype=np.float32)
    x[0, :, 0, 0] = [2.0 ** -101, -2.0 ** -110, 0.0, 2.0 ** -120]   # amax < 2^-100
    x[0, :, 0, 1] = 0.0
    for fmt in ("int8", "fp8"):
        codes, scales = codecs.quantize(x, 64, fmt)
        vals = codes if fmt == "int8" else codecs.e4m3_decode(codes)
        assert scales.tolist() == [[[0.0]]] and not vals.any()            # zeros (FP8 keeps the sign of x)
        x2 = x.copy()
        x2[0, 0, 0, 0] = 2.0 ** -100                                  # at the limit: a real scale, finite inv
        codes, scales = codecs.quantize(x2, 64, fmt)
        q = 127 if fmt == "int8" else 448.0
        assert scales[0, 0, 0] == np.float32(np.float32(2.0 ** -100) / np.float32(q)) and np.isfinite(scales).all()
        v = codes[0, 0, 0, 0] if fmt == "int8" else codecs.e4m3_decode(codes[0, 0, 0, 0])
        assert v == q
