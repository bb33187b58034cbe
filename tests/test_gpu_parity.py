"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Tiny and small configs are compared element by element; ragged and degenerate
shapes are covered too. Bars: prologue within 1 bf16 ulp, masks bit-exact,
attention max-abs <= 2e-2 and relative Frobenius <= 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import (check_attention, check_prologue, log, oracle_mask, pooled_exactness_ok, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _upload(inp):
    return {n: inp[n].to(DEV) for n in ("q", "k", "v", "pos_thw", "w_q", "w_k")}


def _run_layer(inp, sections, base, eps, block, keep):
    g = _upload(inp)
    qh, kh = g["q"].clone(), g["k"].clone()
    saq.qknorm_rope(qh, kh, g["pos_thw"], (g["w_q"], g["w_k"]), sections, base, eps)
    mask = saq.select_blocks(qh, kh, keep, block)
    o = saq.block_sparse_attn(qh, kh, g["v"], mask, block)
    torch.cuda.synchronize()
    return qh, kh, mask, o


def _check_all(inp, sections, base, eps, block, keep, what, rows=None):
    log(f"[{what}] S={inp['q'].shape[1]} H={inp['q'].shape[2]} D={inp['q'].shape[3]} block={block} keep={keep}")
    qh, kh, mask, o = _run_layer(inp, sections, base, eps, block, keep)
    # a1-a2: fp64 oracle on the same bf16 inputs
    rq, rk = oracle.qknorm_rope(to64(inp["q"]), to64(inp["k"]), inp["pos_thw"].numpy(), inp["w_q"].numpy(),
                                inp["w_k"].numpy(), sections, base, eps)
    fq = check_prologue(to64(qh), rq, what + " q_hat")
    fk = check_prologue(to64(kh), rk, what + " k_hat")
    log(f"  prologue: fraction equal to RNE(ref): q {fq:.4f} k {fk:.4f}")
    # a3-a5: the oracle selects from the same bf16 q_hat/k_hat the GPU produced
    qh64, kh64 = to64(qh), to64(kh)
    assert pooled_exactness_ok(qh64) and pooled_exactness_ok(kh64)
    m_gpu = mask.cpu().numpy()
    ref = oracle_mask(qh64, kh64, block, keep)
    for (b, h), m in ref.items():
        assert np.array_equal(m_gpu[b, h], m), f"{what}: mask differs at b={b} h={h}"
    # a6: attention from the same bf16 q_hat/k_hat/v and mask
    v64 = to64(inp["v"])
    if rows is None:
        ro = oracle.block_sparse_attention(qh64, kh64, v64, m_gpu, block)
        check_attention(to64(o), ro, what + " o")
    else:
        got = to64(o)
        S = got.shape[1]
        ro = oracle.block_sparse_attention_rows(qh64, kh64, v64, m_gpu, block, rows)
        g = np.zeros_like(ro)
        for n, (b, h, i) in enumerate(rows):
            hi = min(S, (i + 1) * block)
            g[n, :hi - i * block] = got[b, i * block:hi, h]
        check_attention(g, ro, what + f" o ({len(rows)} sampled query blocks)")
    return qh, kh, mask, o


def test_tiny_config_end_to_end():
    cfg = synth.get_config("tiny")
    _check_all(synth.make_inputs(cfg), cfg.sections, cfg.rope_base, cfg.eps, cfg.block, cfg.keep_ratios[0], "tiny")


def test_small_config_end_to_end():
    cfg = synth.get_config("small")
    _check_all(synth.make_inputs(cfg), cfg.sections, cfg.rope_base, cfg.eps, cfg.block, cfg.keep_ratios[0], "small")


@pytest.mark.parametrize("S,H,D,block,keep,grid", [
    (1000, 2, 64, 64, 0.5, (4, 8, 16)),      # partial last block (40 tokens), audio tail
    (1000, 3, 128, 128, 0.3, (2, 12, 16)),   # partial last block (104 tokens), odd head count
    (127, 1, 64, 64, 1.0, (1, 8, 8)),        # two blocks, keep all
    (1, 1, 128, 128, 0.5, (0, 1, 1)),        # a single token: nB = 1
    (200, 2, 128, 64, 0.01, (2, 5, 10)),     # k = 1: the diagonal only
])
def test_ragged_and_degenerate_shapes(S, H, D, block, keep, grid):
    T, Hg, W = grid
    sections = (16, 24, 24) if D == 64 else (32, 48, 48)
    inp = synth.make_small_case(S, H, D, seed=S + H + D, sections=sections, T=T, Hg=Hg, W=W)
    _check_all(inp, sections, 10000.0, 1e-6, block, keep, f"ragged S={S}")


def test_batch_of_two():
    a = synth.make_small_case(640, 2, 64, seed=7, sections=(16, 24, 24), T=2, Hg=8, W=32)
    b = synth.make_small_case(640, 2, 64, seed=8, sections=(16, 24, 24), T=2, Hg=8, W=32)
    inp = {n: torch.cat([a[n], b[n]], 0) for n in ("q", "k", "v")}
    inp.update(pos_thw=a["pos_thw"], w_q=a["w_q"], w_k=a["w_k"])
    _check_all(inp, (16, 24, 24), 10000.0, 1e-6, 64, 0.4, "batch 2")


def test_constant_inputs_tie_break():
    # every pooled score ties: each row keeps i and the lowest k-1 other indices
    S, H, D, block = 640, 2, 64, 64
    q = torch.ones((1, S, H, D), dtype=torch.bfloat16, device=DEV)
    mask = saq.select_blocks(q, q.clone(), 0.4, block).cpu().numpy()
    for i in range(10):
        want = {i} | set([j for j in range(10) if j != i][:3])
        assert set(np.nonzero(mask[0, 0, i])[0].tolist()) == want


def test_user_mask_with_empty_rows_and_all_ones():
    inp = synth.make_small_case(700, 2, 128, seed=3, sections=(32, 48, 48), T=1, Hg=20, W=30)
    g = _upload(inp)
    nB = 6
    rng = np.random.Generator(np.random.PCG64(4))
    m = (rng.random((1, 2, nB, nB)) < 0.4).astype(np.uint8) * 7          # non-zero bytes count as kept
    m[0, 0, 2] = 0
    m[0, 1, 5] = 0
    mask = torch.from_numpy(m).to(DEV)
    o = saq.block_sparse_attn(g["q"], g["k"], g["v"], mask, 128)
    ref = oracle.block_sparse_attention(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), (m > 0).astype(np.uint8), 128)
    check_attention(to64(o), ref, "user mask")
    assert (to64(o)[0, 256:384, 0] == 0).all() and (to64(o)[0, 640:700, 1] == 0).all()
    ones = torch.ones((1, 2, nB, nB), dtype=torch.uint8, device=DEV)
    o1 = saq.block_sparse_attn(g["q"], g["k"], g["v"], ones, 128, softmax_scale=0.05)
    check_attention(to64(o1), oracle.dense_attention(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), scale=0.05),
                    "all-ones mask vs dense")


def test_constant_v_gives_constant_output():
    inp = synth.make_small_case(300, 1, 64, seed=5, sections=(16, 24, 24))
    g = _upload(inp)
    v = torch.full_like(g["v"], 0.375)
    mask = torch.ones((1, 1, 5, 5), dtype=torch.uint8, device=DEV)
    o = saq.block_sparse_attn(g["q"], g["k"], v, mask, 64)
    assert torch.all(o.float() == 0.375)


def test_outputs_are_deterministic():
    cfg = synth.get_config("small")
    inp = synth.make_inputs(cfg)
    a = _run_layer(inp, cfg.sections, cfg.rope_base, cfg.eps, cfg.block, 0.25)
    b = _run_layer(inp, cfg.sections, cfg.rope_base, cfg.eps, cfg.block, 0.25)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_out_of_place_prologue_matches_in_place():
    cfg = synth.get_config("tiny")
    inp = synth.make_inputs(cfg)
    g = _upload(inp)
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    saq.qknorm_rope_out(g["q"], g["k"], qo, ko, g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections)
    saq.qknorm_rope(g["q"], g["k"], g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections)
    assert torch.equal(qo, g["q"]) and torch.equal(ko, g["k"])


def test_host_or_strided_buffers_rejected_before_launch():
    # every buffer a wrapper hands to the library must be a contiguous tensor on the inputs' device: a host
    # tensor or a strided view is refused with ValueError before any call into the library
    inp = synth.make_small_case(256, 2, 64, seed=5, sections=(16, 24, 24), T=0)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    B, S, H, D = q.shape
    nB = S // 64
    mask = saq.select_blocks(q, k, 0.5, 64)
    ws = torch.empty(saq.select_workspace_bytes(B, S, H, D, 64), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    cases = {
        "block_sparse_attn mask on host": lambda: saq.block_sparse_attn(q, k, v, mask.cpu(), 64),
        "select_blocks out on host": lambda: saq.select_blocks(q, k, 0.5, 64, out=mask.cpu()),
        "select_blocks workspace on host": lambda: saq.select_blocks(q, k, 0.5, 64, workspace=ws.cpu()),
        "select_blocks workspace strided": lambda: saq.select_blocks(q, k, 0.5, 64, workspace=ws[::2]),
        "select_blocks_pooled workspace on host": lambda: saq.select_blocks_pooled(q.shape, 0.5, ws.cpu(), 64),
        "select_blocks_pooled out on host":
            lambda: saq.select_blocks_pooled(q.shape, 0.5, ws, 64, out=torch.empty((B, H, nB, nB), dtype=torch.uint8)),
        "pooled_change on host": lambda: saq.pooled_change(ws.cpu(), ws, q.shape, 64),
        "quantize scales on host":
            lambda: saq.quantize(q, "int8", 64, scales=torch.empty((B, H, nB), dtype=torch.float32)),
        "dequantize scales on host":
            lambda: saq.dequantize(torch.zeros((B, S, H, D), dtype=torch.int8, device=DEV),
                                   torch.ones((B, H, nB), dtype=torch.float32), "int8", 64),
        "mask_overlap across devices": lambda: saq.mask_overlap(mask, mask.cpu()),
    }
    for what, call in cases.items():
        with pytest.raises(ValueError):
            call()
    log(f"  {len(cases)} host or strided buffers refused before launch")
