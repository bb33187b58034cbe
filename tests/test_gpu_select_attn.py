"""GPU parity of the attention with the block selection folded in
(block_sparse_attn_select): its mask and output must be the same bytes as the
two-call path (selection from the pooled means, then attention with that mask),
the mask must equal the oracle's selection and the output the oracle's
block-sparse attention, on ragged shapes, batches, ties and the keep extremes."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import check_attention, log, oracle_mask, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SECTIONS = (32, 48, 48)


def _both(inp, keep, sections=SECTIONS):
    g = {n: inp[n].to(DEV) for n in ("q", "k", "v", "pos_thw", "w_q", "w_k")}
    qh, kh = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    ws = saq.qknorm_rope_pool(g["q"], g["k"], qh, kh, g["pos_thw"], (g["w_q"], g["w_k"]), sections, block=128)
    m2 = saq.select_blocks_pooled(qh.shape, keep, ws, 128)
    o2 = saq.block_sparse_attn(qh, kh, g["v"], m2, 128)
    B, S, H, D = qh.shape
    nB = -(-S // 128)
    m1 = torch.full((B, H, nB, nB), 7, dtype=torch.uint8, device=DEV)
    o1 = saq.block_sparse_attn_select(qh, kh, g["v"], ws, keep, mask_out=m1)
    o0 = saq.block_sparse_attn_select(qh, kh, g["v"], ws, keep)           # without a mask to write
    torch.cuda.synchronize()
    assert torch.equal(m1, m2), "folded selection chose a different mask"
    assert torch.equal(o1, o2) and torch.equal(o0, o2), "folded path output differs from the two-call path"
    return qh, kh, g["v"], m1, o1


def _oracle_check(qh, kh, v, m, o, keep, heads, what):
    ref = oracle_mask(to64(qh), to64(kh), 128, keep, heads=heads)
    mh = m.cpu().numpy()
    for (b, h), r in ref.items():
        assert np.array_equal(mh[b, h], r), f"{what}: mask differs from the oracle on head {h}"
    for h in heads:
        sl = slice(h, h + 1)
        r = oracle.block_sparse_attention(to64(qh[:, :, sl]), to64(kh[:, :, sl]), to64(v[:, :, sl]), mh[:, sl], 128)
        check_attention(to64(o[:, :, sl]), r, f"{what} head {h}")


@pytest.mark.parametrize("keep", [0.25, 1.0])
def test_small_config(keep):
    cfg = synth.get_config("small")
    inp = synth.make_inputs(cfg)
    qh, kh, v, m, o = _both(inp, keep)
    _oracle_check(qh, kh, v, m, o, keep, [0, 5], f"small keep={keep}")
    log(f"  small keep={keep}: folded selection bit-identical to the two-call path; oracle mask and output match")


@pytest.mark.parametrize("S,H,keep,seed", [
    (1000, 3, 0.3, 1),      # ragged last block (104 tokens)
    (129, 2, 0.5, 2),       # a one-token last block
    (1, 1, 1.0, 3),         # a single token: nB = 1, only the diagonal
    (4000, 2, 0.01, 4),     # k = 1: only the diagonal
    (8192, 1, 0.9, 5),      # 64 blocks, nearly dense
])
def test_ragged_shapes(S, H, keep, seed):
    inp = synth.make_small_case(S, H, 128, seed=seed, sections=SECTIONS, T=0)
    qh, kh, v, m, o = _both(inp, keep)
    nB = -(-S // 128)
    assert (m.sum(dim=-1) == saq.kept_blocks(keep, nB)).all()
    _oracle_check(qh, kh, v, m, o, keep, [0], f"S={S} H={H} keep={keep}")


def test_batch_of_two_and_ties():
    a = synth.make_small_case(1280, 2, 128, seed=9, sections=SECTIONS, T=0)
    inp = {n: torch.cat([a[n], a[n] * 0 + 1], 0) for n in ("q", "k", "v")}       # batch 1: constant, all ties
    inp.update(pos_thw=torch.zeros_like(a["pos_thw"]), w_q=a["w_q"], w_k=a["w_k"])
    qh, kh, v, m, o = _both(inp, 0.3)
    mh = m.cpu().numpy()
    kk = saq.kept_blocks(0.3, 10)
    for h in range(2):                         # all scores tie: the diagonal plus the lowest other indices
        for i in range(10):
            want = sorted({i} | set([j for j in range(10) if j != i][:kk - 1]))
            assert np.nonzero(mh[1, h, i])[0].tolist() == want
    _oracle_check(qh, kh, v, m, o, 0.3, [1], "batch of two")
