"""GPU parity at the largest block count the selection and attention kernels take
(nB = 4096), for both block sizes, with a ragged last block: the prologue on
sampled tokens, the whole mask bit-exact against the oracle (separate and fused
pooling paths), attention outputs of sampled query blocks, and for block 128 /
head_dim 128 the attention with the selection folded in, bit-identical to the two
calls."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import check_attention, check_prologue, log, oracle_mask, pooled_exactness_ok, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # S, H, D, block, keep: nB = 4096 in both, last blocks of 47 and 28 tokens
    (4096 * 64 - 17, 1, 64, 64, 0.05),
    (4096 * 128 - 100, 1, 128, 128, 0.02),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("S,H,D,block,keep", CASES)
def test_largest_block_count(S, H, D, block, keep):
    nB = -(-S // block)
    assert nB == 4096
    sections = (16, 24, 24) if D == 64 else (32, 48, 48)
    log(f"[max nB] S={S} H={H} D={D} block={block} keep={keep}")
    inp = synth.make_small_case(S, H, D, seed=S % 1000 + D, sections=sections, T=0)
    g = {n: inp[n].to(DEV) for n in ("q", "k", "v", "pos_thw", "w_q", "w_k")}
    qh, kh = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    saq.qknorm_rope_out(g["q"], g["k"], qh, kh, g["pos_thw"], (g["w_q"], g["w_k"]), sections)
    mask = saq.select_blocks(qh, kh, keep, block)
    o = saq.block_sparse_attn(qh, kh, g["v"], mask, block)
    qf, kf = torch.empty_like(qh), torch.empty_like(kh)
    ws = saq.qknorm_rope_pool(g["q"], g["k"], qf, kf, g["pos_thw"], (g["w_q"], g["w_k"]), sections, block=block)
    mask_f = saq.select_blocks_pooled(qf.shape, keep, ws, block)
    torch.cuda.synchronize()
    assert torch.equal(qf, qh) and torch.equal(kf, kh) and torch.equal(mask_f, mask)

    # prologue: sampled tokens, the last (largest position) included
    rng = np.random.Generator(np.random.PCG64(S))
    toks = np.unique(np.concatenate([[0, 1, block - 1, block, S - 2, S - 1], rng.integers(0, S, 400)]))
    rq, rk = oracle.qknorm_rope(to64(inp["q"][:, toks]), to64(inp["k"][:, toks]), inp["pos_thw"].numpy()[toks],
                                inp["w_q"].numpy(), inp["w_k"].numpy(), sections, 10000.0, 1e-6)
    qh_c, kh_c = qh.cpu(), kh.cpu()
    check_prologue(to64(qh_c[:, toks]), rq, f"max nB q_hat ({len(toks)} tokens)")
    check_prologue(to64(kh_c[:, toks]), rk, f"max nB k_hat ({len(toks)} tokens)")

    # mask: the whole [nB, nB] of every head, from the GPU's own bf16 q_hat/k_hat
    m_gpu = mask.cpu().numpy()
    kk = saq.kept_blocks(keep, nB)
    assert (m_gpu.sum(axis=-1) == kk).all()
    q64, k64 = qh_c.double().numpy(), kh_c.double().numpy()
    assert pooled_exactness_ok(q64) and pooled_exactness_ok(k64)
    ref = oracle_mask(q64, k64, block, keep)
    for h in range(H):
        assert np.array_equal(m_gpu[0, h], ref[(0, h)]), f"mask differs on head {h}"
    log(f"  mask bit-exact over {nB}x{nB} (k={kk}), fused pooling path identical")

    # attention: first, last (ragged), middle and seeded random query blocks
    rows = sorted({(0, 0, i) for i in [0, 1, nB // 2, nB - 2, nB - 1, *rng.integers(0, nB, 5).tolist()]})
    v64 = inp["v"].double().numpy()
    refs = oracle.block_sparse_attention_rows(q64, k64, v64, m_gpu, block, rows)
    got = []
    for (b, h, i) in rows:
        blk = np.zeros((block, D))
        hi = min(S, (i + 1) * block)
        blk[:hi - i * block] = to64(o[b, i * block:hi, h])
        got.append(blk)
    check_attention(np.stack(got), refs, f"max nB attention ({len(rows)} query blocks)")
    assert torch.isfinite(o.float()).all()

    if block == 128 and D == 128:
        m1 = torch.empty_like(mask)
        o1 = saq.block_sparse_attn_select(qf, kf, g["v"], ws, keep, block, mask_out=m1)
        torch.cuda.synchronize()
        assert torch.equal(m1, mask) and torch.equal(o1, o)
        log("  folded selection at nB = 4096: mask and output bit-identical to the two calls")
