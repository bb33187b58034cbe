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
    (1000, 2, 64, 128, 0.3, (4, 8, 16)),     # head_dim 64 with block 128
    (1280, 1, 64, 128, 0.5, (2, 8, 40)),     # head_dim 64 with block 128, whole blocks only
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


def test_zero_score_ties():
    # Scores that tie at exactly zero, next to positive and negative ones. Key blocks 2, 5 and 7 are all
    # zero (stored as -0.0 in head 0 and +0.0 in head 1), so every row scores them +0.0; query block 3 is
    # zero too (signed zeros again), so its row ties everywhere and keeps the lowest indices; key blocks 4
    # and 8 repeat block 1 exactly (equal non-zero scores); the rest are random, so some rows rank the zero
    # blocks above negative scores and below positive ones. The mask must be the oracle's, bit for bit.
    S, H, D, block, nB = 640, 2, 64, 64, 10
    rng = np.random.Generator(np.random.PCG64(21))
    q = torch.from_numpy(rng.standard_normal((1, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((1, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    for h, z in ((0, -0.0), (1, 0.0)):
        for j in (2, 5, 7):
            k[0, j * block:(j + 1) * block, h] = z
        q[0, 3 * block:4 * block, h] = z
        q[0, 3 * block:4 * block:2, h, ::3] = -z
    for j in (4, 8):
        k[0, j * block:(j + 1) * block] = k[0, block:2 * block]
    assert (k[0, 2 * block:3 * block, 0].view(torch.int16) == -32768).all()     # really -0.0
    for keep in (0.3, 0.5, 0.8):
        mask = saq.select_blocks(q.to(DEV), k.to(DEV), keep, block).cpu().numpy()
        ref = oracle_mask(to64(q), to64(k), block, keep)
        for (b, h), m in ref.items():
            assert np.array_equal(mask[b, h], m), f"keep={keep}: mask differs on head {h}"
        kk = saq.kept_blocks(keep, nB)
        for h in range(H):
            assert set(np.nonzero(mask[0, h, 3])[0].tolist()) == {3} | set([j for j in range(nB) if j != 3][:kk - 1])
    log("  zero-score ties (signed-zero inputs), repeated blocks: masks equal the oracle's at keep 0.3/0.5/0.8")


def _near_tie_keys(S, H, D, block, seed, scale_period=0):
    """k: every key block repeats one base block; in two blocks of three one element of one token is moved
    by one bf16 step, so pooled means differ by 2^-7 of an ulp in one coordinate and most scores of a row
    fall within a relative 2^-14 of each other. With scale_period p, block j is scaled by 2^(j mod p - 3)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nB = -(-S // block)
    base = rng.standard_normal((block, H, D)).astype(np.float32)
    kf = np.tile(base, (nB, 1, 1))[:S]
    if scale_period:
        for j in range(nB):
            kf[j * block:(j + 1) * block] *= 2.0 ** (j % scale_period - 3)
    kb = torch.from_numpy(kf).to(torch.bfloat16).view(torch.int16).numpy().copy()
    for j in range(nB):
        if j % 3 == 0:
            continue
        t = j * block + int(rng.integers(0, min(block, S - j * block)))
        d = int(rng.integers(0, D))
        kb[t, :, d] += 1 if j % 3 == 1 else -1                 # one step away from zero / towards zero
    k = torch.from_numpy(kb).view(torch.bfloat16)[None]
    q = torch.from_numpy(rng.standard_normal((1, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    return q, k


@pytest.mark.parametrize("S,H,D,block,keep,scale_period", [
    (50 * 128 - 37, 2, 128, 128, 0.3, 0),      # band of up to 49 near-tied keys
    (200 * 128 - 5, 2, 64, 128, 0.5, 0),       # band wider than a wavefront
    (120 * 128, 2, 128, 128, 0.2, 5),          # key blocks at five scales: ties within each scale
    (600 * 64 - 10, 1, 128, 64, 0.15, 3),      # 1024-column strips
])
def test_near_tie_scores(S, H, D, block, keep, scale_period):
    # Rows whose threshold falls among many exactly or nearly equal scores: the selection has to split
    # them by their exact fp64 scores, ties to the lower j. The mask must be the oracle's, bit for bit.
    q, k = _near_tie_keys(S, H, D, block, seed=S + D, scale_period=scale_period)
    mask = saq.select_blocks(q.to(DEV), k.to(DEV), keep, block).cpu().numpy()
    ref = oracle_mask(to64(q), to64(k), block, keep)
    for (b, h), m in ref.items():
        assert np.array_equal(mask[b, h], m), f"mask differs on head {h}"
    log(f"  near-tie scores S={S} D={D} block={block} keep={keep} scales={scale_period}: masks equal the oracle's")


@pytest.mark.parametrize("D,keep", [(64, 0.5), (128, 0.35), (128, 0.6)])
def test_mixed_scale_selection(D, keep):
    # Key blocks at very different scales: every fifth block scaled by 2^-28 (its scores sit within
    # about 2^-28 of zero next to ordinary ones), every seventh all zero, the rest at 2^-1..2^1.
    # Rows whose threshold falls among the near-zero scores must be split by exact fp64 scores.
    S, H, block = 300 * 64 - 17, 2, 64
    rng = np.random.Generator(np.random.PCG64(31 + D))
    kf = rng.standard_normal((1, S, H, D)).astype(np.float32)
    kf = np.sign(kf) * np.maximum(np.abs(kf), 2.0 ** -7)      # keeps every non-zero |x| >= 2^-35
    for j in range(-(-S // block)):
        sl = slice(j * block, (j + 1) * block)
        kf[0, sl] *= 0.0 if j % 7 == 0 else 2.0 ** -28 if j % 5 == 0 else 2.0 ** (j % 3 - 1)
    k = torch.from_numpy(kf).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((1, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    assert pooled_exactness_ok(to64(k)) and pooled_exactness_ok(to64(q))
    mask = saq.select_blocks(q.to(DEV), k.to(DEV), keep, block).cpu().numpy()
    ref = oracle_mask(to64(q), to64(k), block, keep)
    for (b, h), m in ref.items():
        assert np.array_equal(mask[b, h], m), f"mask differs on head {h}"
    log(f"  mixed-scale key blocks D={D} keep={keep}: masks equal the oracle's")


@pytest.mark.parametrize("case", range(12))
def test_selection_random_cases(case):
    # Seeded random shapes across the selection kernel's three strip layouts (nB padded to 256, 512,
    # 1024), both head sizes and block sizes, keep ratios from 0.03 to 0.97, per-block scales from
    # 2^-20 to 2, some all-zero blocks and some repeated blocks; masks must equal the oracle's.
    rng = np.random.Generator(np.random.PCG64(500 + case))
    D = (64, 128)[case % 2]
    block = (64, 128)[(case // 2) % 2]
    nB = int(rng.integers(2, 1025)) if case < 10 else (1024, 1000)[case - 10]
    S = nB * block - int(rng.integers(0, block))
    H = 1 if nB > 600 else 2
    keep = float(rng.uniform(0.03, 0.97))
    x = rng.standard_normal((2, 1, S, H, D)).astype(np.float32)
    x = np.sign(x) * np.clip(np.abs(x), 2.0 ** -14, 7.0)
    scale = 2.0 ** rng.integers(-20, 2, size=(2, nB))
    scale[:, rng.random(nB) < 0.05] = 0.0
    for t in range(2):
        for j in range(nB):
            x[t, 0, j * block:(j + 1) * block] *= scale[t, j]
    rep = rng.random(nB) < 0.05                                  # repeat block 0 of k
    for j in np.nonzero(rep)[0]:
        n = min(block, S - j * block)
        x[1, 0, j * block:j * block + n] = x[1, 0, :n]
    q = torch.from_numpy(x[0]).to(torch.bfloat16)
    k = torch.from_numpy(x[1]).to(torch.bfloat16)
    assert pooled_exactness_ok(to64(q)) and pooled_exactness_ok(to64(k))
    mask = saq.select_blocks(q.to(DEV), k.to(DEV), keep, block).cpu().numpy()
    ref = oracle_mask(to64(q), to64(k), block, keep)
    for (b, h), m in ref.items():
        assert np.array_equal(mask[b, h], m), f"case {case}: mask differs on head {h} (nB={nB} D={D} keep={keep:.3f})"
    log(f"  random selection case {case}: nB={nB} D={D} block={block} keep={keep:.3f}: masks equal the oracle's")


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


@pytest.mark.parametrize("order", ["ascending", "descending", "mixed"])
def test_large_score_jumps_between_tiles(order):
    # Key blocks at magnitudes 2^-6 .. 2^5, in ascending, descending or shuffled order along the key axis, so a
    # row's running maximum moves by tens of log2 units from one kept tile to the next (far beyond the lazy
    # rescale threshold) or stays far above every later tile. Head 0 attends densely, head 1 through a random
    # mask with the diagonal; the last block is partial. The online softmax must give the plain softmax.
    S, H, D, block = 12 * 128 + 40, 2, 128, 128
    nB = (S + block - 1) // block
    rng = np.random.Generator(np.random.PCG64({"ascending": 11, "descending": 12, "mixed": 13}[order]))
    f = 2.0 ** np.linspace(-6, 5, nB)
    if order == "descending":
        f = f[::-1]
    elif order == "mixed":
        f = rng.permutation(f)
    q = rng.standard_normal((1, S, H, D))
    k = rng.standard_normal((1, S, H, D))
    for j in range(nB):
        k[:, j * block:(j + 1) * block] *= f[j]
    v = rng.uniform(-1.0, 1.0, (1, S, H, D))
    qt, kt, vt = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (q, k, v))
    m = np.ones((1, H, nB, nB), dtype=np.uint8)
    m[0, 1] = rng.random((nB, nB)) < 0.5
    m[0, 1][np.arange(nB), np.arange(nB)] = 1
    o = saq.block_sparse_attn(qt.to(DEV), kt.to(DEV), vt.to(DEV), torch.from_numpy(m).to(DEV), block)
    ref = oracle.block_sparse_attention(to64(qt), to64(kt), to64(vt), m, block)
    check_attention(to64(o), ref, f"score jumps between tiles ({order})")


@pytest.mark.parametrize("D", [64, 128])
def test_prologue_rows_beyond_fp32_square_range(D):
    # Rows whose entries reach 2^61 .. 2^126, and one row of the largest finite bf16 throughout: their fp32
    # sum of squares overflows, so the norm takes its rescaled pass. Ordinary rows of the same tokens and
    # heads sit beside them. Both prologue kernels (in place, and fused with the pooling) against the oracle.
    sections = (D // 4, 3 * D // 8, 3 * D // 8)
    inp = synth.make_small_case(300, 2, D, seed=9 + D, sections=sections, T=2, Hg=6, W=10)
    q, k = inp["q"].double().clone(), inp["k"].double().clone()
    for n, e in enumerate((61, 75, 100, 126)):
        for x, t, h in ((q, 10 + n, 0), (k, 130 + n, 1)):
            x[0, t, h] = x[0, t, h] / x[0, t, h].abs().max() * 2.0 ** e
    q[0, 40, 1] = float(torch.finfo(torch.bfloat16).max)
    k[0, 299, 0] = -float(torch.finfo(torch.bfloat16).max)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    assert torch.isfinite(q.float()).all() and torch.isfinite(k.float()).all()
    rq, rk = oracle.qknorm_rope(to64(q), to64(k), inp["pos_thw"].numpy(), inp["w_q"].numpy(), inp["w_k"].numpy(),
                                sections, 10000.0, 1e-6)
    g = _upload(inp)
    qh, kh = q.to(DEV), k.to(DEV)
    saq.qknorm_rope(qh, kh, g["pos_thw"], (g["w_q"], g["w_k"]), sections)
    check_prologue(to64(qh), rq, f"D={D} huge rows q_hat")
    check_prologue(to64(kh), rk, f"D={D} huge rows k_hat")
    qf, kf = torch.empty_like(qh), torch.empty_like(kh)
    saq.qknorm_rope_pool(q.to(DEV), k.to(DEV), qf, kf, g["pos_thw"], (g["w_q"], g["w_k"]), sections, block=64)
    torch.cuda.synchronize()
    assert torch.equal(qf, qh) and torch.equal(kf, kh)
    assert abs(to64(qh)[0, 40, 1]).max() < 2 * np.sqrt(D)      # normalised, not zero
    assert abs(to64(qh)[0, 40, 1]).max() > 0.1


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
