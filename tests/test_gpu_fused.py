"""GPU parity of the fused prologue + pooling path (QKNorm + 3D RoPE with the
selection's block pooling folded into the same pass).

The fused call must reproduce the separate calls bit for bit: the same q-hat and
k-hat bytes, the same pooled fp64 means (sums of bf16 values are exact in fp64),
hence the same mask; and the mask must equal the fp64 oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import log, oracle_mask, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both_paths(inp, sections, block, keep):
    g = {n: inp[n].to(DEV) for n in ("q", "k", "pos_thw", "w_q", "w_k")}
    B, S, H, D = g["q"].shape
    # separate calls
    qs, ks = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    saq.qknorm_rope_out(g["q"], g["k"], qs, ks, g["pos_thw"], (g["w_q"], g["w_k"]), sections)
    ws_s = torch.empty(saq.select_workspace_bytes(B, S, H, D, block), dtype=torch.uint8, device=DEV)
    m_s = saq.select_blocks(qs, ks, keep, block, workspace=ws_s)
    # fused
    qf, kf = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    ws_f = saq.qknorm_rope_pool(g["q"], g["k"], qf, kf, g["pos_thw"], (g["w_q"], g["w_k"]), sections, block=block)
    m_f = saq.select_blocks_pooled((B, S, H, D), keep, ws_f, block)
    torch.cuda.synchronize()
    nB = -(-S // block)
    npool = 2 * B * H * nB * D * 8
    return qs, ks, m_s, ws_s[:npool], qf, kf, m_f, ws_f[:npool]


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_fused_equals_separate_and_oracle(name):
    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    keep = cfg.keep_ratios[0]
    qs, ks, m_s, p_s, qf, kf, m_f, p_f = _both_paths(inp, cfg.sections, cfg.block, keep)
    assert torch.equal(qs, qf) and torch.equal(ks, kf)
    assert torch.equal(p_s, p_f), "pooled means differ between the fused and the separate pass"
    assert torch.equal(m_s, m_f)
    ref = oracle_mask(to64(qf), to64(kf), cfg.block, keep)
    m = m_f.cpu().numpy()
    for (b, h), r in ref.items():
        assert np.array_equal(m[b, h], r)
    log(f"  {name}: fused path bit-identical to the separate calls; mask equals the oracle's")


@pytest.mark.parametrize("S,H,D,block,keep,grid", [
    (1000, 3, 128, 128, 0.3, (2, 12, 16)),
    (1000, 2, 64, 64, 0.5, (4, 8, 16)),
    (1000, 2, 64, 128, 0.3, (4, 8, 16)),      # head_dim 64 with block 128 (last block 104 tokens)
    (1, 1, 128, 64, 1.0, (0, 1, 1)),
    (200, 64, 128, 64, 0.2, (2, 5, 10)),      # H*D = 8192, the fused path's limit
])
def test_fused_ragged_shapes(S, H, D, block, keep, grid):
    sections = (16, 24, 24) if D == 64 else (32, 48, 48)
    inp = synth.make_small_case(S, H, D, seed=11 + S, sections=sections, T=grid[0], Hg=grid[1], W=grid[2])
    qs, ks, m_s, p_s, qf, kf, m_f, p_f = _both_paths(inp, sections, block, keep)
    assert torch.equal(qs, qf) and torch.equal(ks, kf)
    assert torch.equal(p_s, p_f)
    assert torch.equal(m_s, m_f)
    # pooled means against the oracle's pooling of the same bf16 tensors
    B, S_, H_, D_ = qf.shape
    nB = -(-S // block)
    pooled = p_f.view(torch.float64).cpu().numpy().reshape(2, B, H_, nB, D_)
    assert np.array_equal(pooled[0, 0], oracle.pool_blocks(to64(qf)[0], block))
    assert np.array_equal(pooled[1, 0], oracle.pool_blocks(to64(kf)[0], block))


def test_fused_batch_of_two():
    a = synth.make_small_case(640, 2, 64, seed=7, sections=(16, 24, 24), T=2, Hg=8, W=32)
    b = synth.make_small_case(640, 2, 64, seed=8, sections=(16, 24, 24), T=2, Hg=8, W=32)
    inp = {n: torch.cat([a[n], b[n]], 0) for n in ("q", "k")}
    inp.update(pos_thw=a["pos_thw"], w_q=a["w_q"], w_k=a["w_k"])
    qs, ks, m_s, p_s, qf, kf, m_f, p_f = _both_paths(inp, (16, 24, 24), 64, 0.4)
    assert torch.equal(qs, qf) and torch.equal(ks, kf) and torch.equal(p_s, p_f) and torch.equal(m_s, m_f)


def test_fused_rejects_too_many_channels():
    q = torch.zeros((1, 8, 65, 128), dtype=torch.bfloat16, device=DEV)      # H*D = 8320 > 8192
    w = torch.ones(128, dtype=torch.float32, device=DEV)
    pos = torch.zeros((8, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(saq.SaqError):
        saq.qknorm_rope_pool(q, q.clone(), torch.empty_like(q), torch.empty_like(q), pos, (w, w), (32, 48, 48))


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_attention_layer_entry(name):
    # the one-call layer equals the step-by-step calls byte for byte, reuses its buffers, and leaves q, k alone
    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    g = {n: inp[n].to(DEV) for n in ("q", "k", "v", "pos_thw", "w_q", "w_k")}
    q0, k0 = g["q"].clone(), g["k"].clone()
    keep = cfg.keep_ratios[0]
    bufs = {}
    o1, m1 = saq.attention_layer(g["q"], g["k"], g["v"], g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections, keep,
                                 cfg.block, cfg.rope_base, cfg.eps, buffers=bufs)
    o1, m1 = o1.clone(), m1.clone()
    o2, m2 = saq.attention_layer(g["q"], g["k"], g["v"], g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections, keep,
                                 cfg.block, cfg.rope_base, cfg.eps, buffers=bufs)
    qs, ks = torch.empty_like(q0), torch.empty_like(k0)
    saq.qknorm_rope_out(g["q"], g["k"], qs, ks, g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections, cfg.rope_base,
                        cfg.eps)
    ms = saq.select_blocks(qs, ks, keep, cfg.block)
    os_ = saq.block_sparse_attn(qs, ks, g["v"], ms, cfg.block)
    torch.cuda.synchronize()
    assert torch.equal(g["q"], q0) and torch.equal(g["k"], k0)
    assert torch.equal(o1, o2) and torch.equal(m1, m2) and o2.data_ptr() == bufs["o"].data_ptr()
    assert torch.equal(m1, ms) and torch.equal(o1, os_)
