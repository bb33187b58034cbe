"""The no-allocation selection entry point (saq_select_blocks_noalloc) against the workspace one.

Called through the C ABI on two calls in a row, the second on a smaller input, each compared byte for byte
with saq_select_blocks on the same tensors (and the smaller one with the oracle); oversized shapes are
refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import log, oracle_mask, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _prologue(cfg):
    inp = synth.make_inputs(cfg)
    g = {n: inp[n].to(DEV) for n in ("q", "k", "pos_thw", "w_q", "w_k")}
    saq.qknorm_rope(g["q"], g["k"], g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections, cfg.rope_base, cfg.eps)
    return g["q"], g["k"]


def _noalloc(q, k, keep, block):
    B, S, H, D = q.shape
    nB = -(-S // block)
    mask = torch.full((B, H, nB, nB), 0xAB, dtype=torch.uint8, device=DEV)
    st = saq.lib().saq_select_blocks_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), B, S, H,
                                             D, block, float(keep), ctypes.c_void_p(mask.data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, saq.lib().saq_status_string(st)
    return mask


@pytest.mark.timeout(300)
def test_noalloc_selection_matches_workspace_call_twice():
    for name in ("medium", "small"):                  # the second call is the smaller input
        cfg = synth.get_config(name)
        keep = cfg.keep_ratios[-1]
        q, k = _prologue(cfg)
        m_static = _noalloc(q, k, keep, cfg.block)
        m_ws = saq.select_blocks(q, k, keep, cfg.block)
        torch.cuda.synchronize()
        assert torch.equal(m_static, m_ws), f"{name}: masks differ between the two entry points"
        if name == "small":
            ref = oracle_mask(to64(q), to64(k), cfg.block, keep)
            m = m_static.cpu().numpy()
            for (b, h), r in ref.items():
                assert np.array_equal(m[b, h], r)
        log(f"  {name} (S={cfg.S}, H={cfg.H}, keep={keep}): no-allocation mask equals the workspace call's")


def test_noalloc_rejects_oversized_workspace():
    # nB = 4096 at H = 8 needs the 1 GB key matrix: refused before any launch
    q = torch.zeros((1, 64, 8, 128), dtype=torch.bfloat16, device=DEV)
    lib = saq.lib()
    st = lib.saq_select_blocks_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()), 1, 4096 * 128,
                                       8, 128, 128, 0.5, ctypes.c_void_p(q.data_ptr()), None)
    assert st == -6      # SAQ_ERR_WORKSPACE
