"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments with the documented status codes before
any HIP call (no compute runs here)."""
import ctypes
import os
import re

import pytest

import oracle
from sparse_attention_qknorm_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_binding.LIB_PATH),
                                reason="libsaq.so not built (python -m sparse_attention_qknorm_amd.build)")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t|const char\*)\s+(saq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("saq_qknorm_rope", "saq_select_blocks", "saq_block_sparse_attn", "saq_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(_binding.LIB_PATH)
    for name in _declared():
        assert hasattr(handle, name), name
    assert sorted(n for n, _, _ in _binding.SIGNATURES) == _declared()


def test_status_strings():
    lib = _binding.lib()
    for code in range(0, -10, -1):
        s = lib.saq_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.saq_status_string(-99).decode() == "unknown status"


@pytest.mark.parametrize("keep,nB", [(0.5, 16), (0.25, 64), (0.2, 256), (0.15, 993), (0.1, 993), (0.3, 993),
                                     (0.3, 10), (1e-9, 5), (1.0, 1), (1.0, 4096), (0.7, 10), (0.999999, 7)])
def test_kept_blocks_matches_oracle_rule(keep, nB):
    assert _binding.lib().saq_kept_blocks(keep, nB) == oracle.num_kept_blocks(keep, nB)


def test_kept_blocks_errors():
    lib = _binding.lib()
    assert lib.saq_kept_blocks(0.0, 10) == -5
    assert lib.saq_kept_blocks(1.01, 10) == -5
    assert lib.saq_kept_blocks(float("nan"), 10) == -5
    assert lib.saq_kept_blocks(0.5, 0) == -2


def test_workspace_bytes():
    lib = _binding.lib()
    # pooled means of q and k (padded to 256 bytes), then for nB <= 1024 four int8 limbs of every q and k
    # mean and an int32 exponent per k mean, nB padded to 256/512/1024; beyond that the uint64 score keys
    nB = 993
    pooled = (2 * 40 * nB * 128 * 8 + 255) // 256 * 256
    assert lib.saq_select_blocks_workspace_bytes(1, 127040, 40, 128, 128) == pooled + 40 * 1024 * (2 * 4 * 128 + 4)
    nB = 200
    pooled = (2 * 3 * nB * 64 * 8 + 255) // 256 * 256
    assert lib.saq_select_blocks_workspace_bytes(1, 200 * 64, 3, 64, 64) == pooled + 3 * 256 * (2 * 4 * 64 + 4)
    nB = 2000
    pooled = (2 * 2 * nB * 128 * 8 + 255) // 256 * 256
    assert lib.saq_select_blocks_workspace_bytes(1, 2000 * 128, 2, 128, 128) == pooled + 2 * nB * nB * 8
    assert lib.saq_select_blocks_workspace_bytes(1, 127040, 40, 96, 128) == 0     # unsupported D
    assert lib.saq_select_blocks_workspace_bytes(1, 127040, 40, 128, 32) == 0     # unsupported block
    assert lib.saq_select_blocks_workspace_bytes(1, 0, 40, 128, 128) == 0
    assert lib.saq_select_blocks_workspace_bytes(1, 64 * 4097, 1, 64, 64) == 0    # nB > 4096


FAKE = 0x10000          # a 16-byte aligned address that is never dereferenced: every call below
MISALIGNED = 0x10008    # fails validation on the host before any HIP call


def test_qknorm_rope_validation():
    lib = _binding.lib()
    args = dict(q=FAKE, k=FAKE * 2, pos=FAKE * 3, wq=FAKE * 4, wk=FAKE * 5)

    def call(q=args["q"], k=args["k"], pos=args["pos"], wq=args["wq"], wk=args["wk"], B=1, S=16, H=2, D=64,
             dt=16, dh=24, dw=24, base=1e4, eps=1e-6):
        return lib.saq_qknorm_rope(q, k, pos, wq, wk, B, S, H, D, dt, dh, dw, base, eps, None)

    assert call(q=None) == -1 and call(pos=None) == -1 and call(wk=None) == -1
    assert call(S=0) == -2 and call(H=-1) == -2
    assert call(D=96, dt=32, dh=32, dw=32) == -3
    assert call(dt=16, dh=24, dw=22) == -2            # sections do not sum to D
    assert call(dt=15, dh=25, dw=24) == -2            # odd section
    assert call(base=1.0) == -5 and call(eps=0.0) == -5 and call(eps=float("inf")) == -5
    assert call(q=MISALIGNED) == -4
    assert call(k=FAKE + 16) == -9                    # q and k overlap
    assert call(B=4096, S=4096, H=4, D=64) == -2      # > 2^31 elements


def test_qknorm_rope_out_aliasing():
    lib = _binding.lib()
    base = 1 << 20
    n = 16 * 2 * 64 * 2
    # q_out overlapping k_in is rejected; q_out == q_in (in place) passes validation
    st = lib.saq_qknorm_rope_out(base, base + 4 * n, base + 4 * n, base + 8 * n, FAKE, FAKE, FAKE,
                                 1, 16, 2, 64, 16, 24, 24, 1e4, 1e-6, None)
    assert st == -9
    st = lib.saq_qknorm_rope_out(base, base + 4 * n, base + 16, base + 8 * n, FAKE, FAKE, FAKE,
                                 1, 16, 2, 64, 16, 24, 24, 1e4, 1e-6, None)
    assert st == -9                                    # partial overlap of q_out with q_in


def test_select_blocks_validation():
    lib = _binding.lib()
    ws = 1 << 24

    def call(q=FAKE, k=FAKE * 2, B=1, S=1024, H=2, D=64, block=64, keep=0.5, mask=FAKE * 3, w=ws,
             wbytes=1 << 22):
        return lib.saq_select_blocks(q, k, B, S, H, D, block, keep, mask, w, wbytes, None)

    assert call(q=None) == -1 and call(mask=None) == -1
    assert call(block=32) == -3 and call(D=32) == -3
    assert call(keep=0.0) == -5 and call(keep=1.5) == -5
    assert call(w=None) == -6 and call(wbytes=16) == -6
    assert call(w=ws + 16) == -4                       # workspace must be 256-byte aligned
    assert call(q=MISALIGNED) == -4


def test_block_sparse_attn_validation():
    lib = _binding.lib()

    def call(q=FAKE, k=FAKE * 2, v=FAKE * 3, mask=FAKE * 4, B=1, S=1024, H=2, D=64, block=64, scale=0.0,
             o=1 << 24):
        return lib.saq_block_sparse_attn(q, k, v, mask, B, S, H, D, block, scale, o, None)

    assert call(o=None) == -1 and call(v=None) == -1
    assert call(block=256) == -3
    assert call(scale=float("nan")) == -5
    assert call(o=FAKE * 3) == -9                      # o aliases v
    assert call(o=(1 << 24) + 8) == -4


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="only meaningful on a host without a GPU")
def test_valid_call_without_device_reports_no_device():
    lib = _binding.lib()
    st = lib.saq_block_sparse_attn(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, 1024, 2, 64, 64, 0.0, 1 << 24, None)
    assert st == -8


def test_step_reuse_validation():
    lib = _binding.lib()
    # S=1024, H=2, D=64, block=64: nB=16, pooled 32 KiB, workspace 36 KiB
    assert lib.saq_pooled_bytes(1, 1024, 2, 64, 64) == 2 * 2 * 16 * 64 * 8
    assert lib.saq_pooled_bytes(1, 1024, 2, 96, 64) == 0
    n_state = lib.saq_reuse_state_len()
    assert n_state >= 3

    def call(mask=FAKE * 3, ws=1 << 24, wbytes=1 << 20, ref=1 << 25, rbytes=1 << 20, state=1 << 26, slen=n_state,
             keep=0.5, thr=0.05, S=1024, block=64):
        return lib.saq_select_blocks_reuse(1, S, 2, 64, block, keep, thr, 0, mask, ws, wbytes, ref, rbytes, state,
                                           slen, None)

    assert call(mask=None) == -1 and call(ref=None) == -1 and call(state=None) == -1
    assert call(block=32) == -3
    assert call(keep=0.0) == -5 and call(thr=-1e-3) == -5 and call(thr=float("nan")) == -5
    assert call(thr=float("inf")) == -5
    assert call(wbytes=100) == -6 and call(rbytes=32767) == -6 and call(slen=n_state - 1) == -6
    assert call(ws=(1 << 24) + 16) == -4 and call(ref=(1 << 25) + 8) == -4 and call(state=(1 << 26) + 4) == -4
    assert call(ref=(1 << 24) + 4096) == -9            # reference inside the workspace
    assert call(state=(1 << 25) + 256) == -9           # state inside the reference

    # pooled change / overlap
    out_len = lib.saq_pooled_change_out_len()
    assert lib.saq_pooled_change(None, 1 << 24, 1, 1024, 2, 64, 64, 1 << 26, out_len, None) == -1
    assert lib.saq_pooled_change(1 << 25, 1 << 24, 1, 1024, 2, 64, 64, 1 << 26, out_len - 1, None) == -6
    assert lib.saq_pooled_change(1 << 25, 1 << 24, 1, 1024, 2, 64, 64, (1 << 24) + 64, out_len, None) == -9
    assert lib.saq_mask_overlap(FAKE, None, 1, 2, 16, 1 << 24, None) == -1
    assert lib.saq_mask_overlap(FAKE, FAKE * 2, 1, 2, 0, 1 << 24, None) == -2
    assert lib.saq_mask_overlap(FAKE, FAKE * 2, 1, 2, 16, (1 << 24) + 4, None) == -4
    assert lib.saq_mask_overlap(FAKE + 8, FAKE * 2, 1, 2, 16, 1 << 24, None) == -4
    assert lib.saq_mask_overlap(FAKE, FAKE * 2, 1, 65536, 1, 1 << 24, None) == -2


def test_fused_prologue_pool_validation():
    lib = _binding.lib()

    def pool(q=FAKE, k=FAKE * 2, qo=FAKE * 3, ko=FAKE * 4, H=2, D=64, block=64, ws=1 << 24, wbytes=1 << 20):
        sec = (16, 24, 24) if D == 64 else (32, 48, 48)
        return lib.saq_qknorm_rope_pool(q, k, qo, ko, FAKE * 5, FAKE * 6, FAKE * 7, 1, 16, H, D, *sec, 1e4,
                                        1e-6, block, ws, wbytes, None)

    assert pool(q=None) == -1
    far = dict(q=1 << 27, k=2 << 27, qo=3 << 27, ko=4 << 27)
    assert pool(H=64, D=128, **far, wbytes=8) == -6                   # H*D = 8192 passes that check
    assert pool(H=65, D=128, **far, wbytes=8) == -3                   # H*D > 8192
    assert pool(block=96) == -3
    assert pool(wbytes=8) == -6
    assert pool(ws=(1 << 24) + 128) == -4

    def sel(mask=FAKE, ws=1 << 24, wbytes=1 << 20, keep=0.5):
        return lib.saq_select_blocks_pooled(1, 1024, 2, 64, 64, keep, mask, ws, wbytes, None)

    assert sel(mask=None) == -1 and sel(keep=2.0) == -5 and sel(wbytes=0) == -6
    assert sel(mask=(1 << 24) + 64) == -9


def test_codec_validation():
    lib = _binding.lib()
    # S=1024, H=2, D=64: x 256 KiB, codes 128 KiB, scales 2*16*4 = 128 B
    x, codes, scales = 1 << 24, 1 << 25, 1 << 26

    for q, d in ((lib.saq_quantize_int8, lib.saq_dequantize_int8), (lib.saq_quantize_fp8, lib.saq_dequantize_fp8)):
        def qc(x=x, codes=codes, scales=scales, S=1024, D=64, block=64):
            return q(x, 1, S, 2, D, block, codes, scales, None)

        def dc(x=x, codes=codes, scales=scales, S=1024, D=64, block=64):
            return d(codes, scales, 1, S, 2, D, block, x, None)

        for f in (qc, dc):
            assert f(x=None) == -1 and f(codes=None) == -1 and f(scales=None) == -1
            assert f(S=0) == -2 and f(D=96) == -3 and f(block=32) == -3
            assert f(x=x + 8) == -4 and f(codes=codes + 4) == -4 and f(scales=scales + 2) == -4
            assert f(codes=x + 1024) == -9                 # codes inside x
            assert f(scales=codes + 64) == -9              # scales inside codes


def test_attn_select_validation():
    lib = _binding.lib()
    # S=1024, H=2, D=128: tensors 512 KiB each; pooled 2*2*8*128*8 = 32 KiB
    q, k, v, o, ws = 1 << 24, 2 << 24, 3 << 24, 4 << 24, 5 << 24

    def call(q=q, ws=ws, wbytes=1 << 20, D=128, block=128, keep=0.5, scale=0.0, o=o, mask=None):
        return lib.saq_block_sparse_attn_select(q, k, v, ws, wbytes, 1, 1024, 2, D, block, keep, scale, o, mask, None)

    assert call(q=None) == -1 and call(ws=None) == -1 and call(o=None) == -1
    assert call(D=64, block=64) == -3 and call(block=64) == -3
    assert call(keep=0.0) == -5 and call(scale=float("inf")) == -5
    assert call(wbytes=32767) == -6
    assert call(ws=ws + 16) == -4 and call(o=o + 8) == -4
    assert call(o=q + 1024) == -9
    assert call(mask=ws + 1024) == -9                  # mask inside the pooled means
