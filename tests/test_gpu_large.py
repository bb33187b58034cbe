"""GPU parity at the medium, full (127,040-token) and sweep sizes, in the launch
configuration the bench times (block 128, head_dim 128).

Masks are compared bit for bit with the oracle's on every head (the oracle
pools, scores and selects from the GPU's own bf16 q_hat/k_hat, one head per
thread): at the medium size, at the full size, and at every keep ratio of the
sweep on one step. Attention is compared with the oracle on whole heads (every
query block of a head: two heads at the full size, one at each medium keep
ratio, one at the sweep's keep 0.1) and on sampled query blocks elsewhere
(first, last/partial, the block that mixes video and audio, audio blocks,
seeded random ones). Prologue rows are checked on sampled tokens. Properties
that hold at any size are checked on every output: finite, and inside the
per-(head, channel) range of V.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import (check_attention, check_prologue, log, oracle_head_attention, oracle_head_masks,
                          to64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class Layer:
    """One layer's inputs on host and device, and the GPU path's outputs."""

    def __init__(self, inp):
        self.inp = inp
        self.cfg = inp["cfg"]
        g = {n: inp[n].to(DEV) for n in ("q", "k", "v", "pos_thw", "w_q", "w_k")}
        self.v = g["v"]
        self.qh, self.kh = torch.empty_like(g["q"]), torch.empty_like(g["k"])
        c = self.cfg
        saq.qknorm_rope_out(g["q"], g["k"], self.qh, self.kh, g["pos_thw"], (g["w_q"], g["w_k"]), c.sections,
                            c.rope_base, c.eps)
        torch.cuda.synchronize()
        self.qh64_cache = None

    def run(self, keep):
        c = self.cfg
        mask = saq.select_blocks(self.qh, self.kh, keep, c.block)
        o = saq.block_sparse_attn(self.qh, self.kh, self.v, mask, c.block)
        torch.cuda.synchronize()
        return mask, o

    def host_qk(self):
        if self.qh64_cache is None:
            self.qh64_cache = (self.qh.cpu(), self.kh.cpu())
        return self.qh64_cache


def _sample_tokens(cfg, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, cfg.block - 1, cfg.block, cfg.S_video - 1, cfg.S_video, cfg.S - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, cfg.S, n)]))


def _check_prologue_sample(layer, seed):
    cfg, inp = layer.cfg, layer.inp
    toks = _sample_tokens(cfg, 1500, seed)
    qh, kh = layer.host_qk()
    rq, rk = oracle.qknorm_rope(to64(inp["q"][:, toks]), to64(inp["k"][:, toks]), inp["pos_thw"].numpy()[toks],
                                inp["w_q"].numpy(), inp["w_k"].numpy(), cfg.sections, cfg.rope_base, cfg.eps)
    fq = check_prologue(to64(qh[:, toks]), rq, f"{cfg.name} q_hat ({len(toks)} tokens)")
    fk = check_prologue(to64(kh[:, toks]), rk, f"{cfg.name} k_hat ({len(toks)} tokens)")
    log(f"  {cfg.name} prologue on {len(toks)} sampled tokens: RNE-exact fraction q {fq:.4f} k {fk:.4f}")


def _check_masks(layer, mask, keep, heads):
    cfg = layer.cfg
    qh, kh = layer.host_qk()
    m_gpu = mask.cpu().numpy()
    kk = saq.kept_blocks(keep, cfg.nB)
    assert (m_gpu.sum(axis=-1) == kk).all() and (np.diagonal(m_gpu, axis1=2, axis2=3) == 1).all()
    heads = list(heads)
    ref = oracle_head_masks(qh, kh, cfg.block, [keep], heads)[keep]
    for h in heads:
        assert np.array_equal(m_gpu[0, h], ref[h]), f"{cfg.name} keep={keep}: mask differs on head {h}"
    log(f"  {cfg.name} keep={keep}: masks bit-exact on {len(heads)} heads {_span(heads)}; k={kk} per row everywhere")
    return m_gpu


def _span(heads):
    return f"{heads[0]}..{heads[-1]}" if len(heads) > 3 else str(heads)


def _check_whole_head(layer, m_gpu, o, h, what):
    """Every query block of head h against the oracle."""
    qh, kh = layer.host_qk()
    ref = oracle_head_attention(qh, kh, layer.inp["v"], m_gpu[0, h], layer.cfg.block, h)
    check_attention(to64(o[0, :, h]), ref, f"{what} head {h} (all {layer.cfg.nB} query blocks)")


def _check_attention_sample(layer, m_gpu, o, rows, what):
    cfg = layer.cfg
    qh, kh = layer.host_qk()
    S, block = cfg.S, cfg.block
    heads = sorted({h for _, h, _ in rows})
    got = []
    refs = []
    for h in heads:
        hr = [(b, 0, i) for (b, hh, i) in rows if hh == h]
        q64 = qh[:, :, h:h + 1].double().numpy()
        k64 = kh[:, :, h:h + 1].double().numpy()
        v64 = layer.inp["v"][:, :, h:h + 1].double().numpy()
        refs.append(oracle.block_sparse_attention_rows(q64, k64, v64, m_gpu[:, h:h + 1], block, hr))
        for (b, _, i) in hr:
            blk = np.zeros((block, cfg.D))
            hi = min(S, (i + 1) * block)
            blk[:hi - i * block] = to64(o[b, i * block:hi, h])
            got.append(blk)
    check_attention(np.stack(got), np.concatenate(refs), f"{what} ({len(rows)} query blocks)")


def _check_properties(layer, o):
    # any size: finite, and each output channel inside [min, max] of that head's V channel
    assert torch.isfinite(o.float()).all()
    vmin = layer.v.float().amin(dim=1, keepdim=True)
    vmax = layer.v.float().amax(dim=1, keepdim=True)
    of = o.float()
    slack = 2e-2
    assert bool(((of >= vmin - slack) & (of <= vmax + slack)).all())


def _rows(cfg, n, seed, heads):
    rng = np.random.Generator(np.random.PCG64(seed))
    nB = cfg.nB
    audio0 = cfg.S_video // cfg.block
    fixed = [0, nB - 1, audio0, min(nB - 1, audio0 + 1), nB // 2]
    rows = []
    for h in heads:
        for i in fixed:
            rows.append((0, h, int(i)))
    for _ in range(n):
        rows.append((0, int(rng.choice(heads)), int(rng.integers(0, nB))))
    return sorted(set(rows))


@pytest.fixture(scope="module")
def medium():
    log("[medium] generating inputs")
    return Layer(synth.make_inputs("medium"))


@pytest.mark.timeout(300)
def test_medium_prologue_sampled(medium):
    _check_prologue_sample(medium, 1)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("keep", [0.2, 1.0])
def test_medium_select_and_attention(medium, keep):
    mask, o = medium.run(keep)
    if keep == 1.0:
        assert bool((mask == 1).all())
        m_gpu = mask.cpu().numpy()
    else:
        m_gpu = _check_masks(medium, mask, keep, range(medium.cfg.H))
    _check_properties(medium, o)
    _check_attention_sample(medium, m_gpu, o, _rows(medium.cfg, 16, 2, [0, 7, 23]), f"medium keep={keep} o")
    _check_whole_head(medium, m_gpu, o, 7, f"medium keep={keep} o")


@pytest.fixture(scope="module")
def full():
    log("[full] generating inputs (127040 tokens x 40 heads)")
    return Layer(synth.make_inputs("full"))


@pytest.mark.timeout(300)
def test_full_prologue_sampled(full):
    _check_prologue_sample(full, 3)


@pytest.mark.timeout(400)
def test_full_select_and_attention(full):
    keep = full.cfg.keep_ratios[0]
    mask, o = full.run(keep)
    m_gpu = _check_masks(full, mask, keep, range(full.cfg.H))
    _check_properties(full, o)
    _check_attention_sample(full, m_gpu, o, _rows(full.cfg, 12, 4, [3, 13, 26]), "full keep=0.15 o")
    for h in (0, 39):
        _check_whole_head(full, m_gpu, o, h, "full keep=0.15 o")
    # the same launch twice gives the same bytes
    mask2, o2 = full.run(keep)
    assert torch.equal(mask, mask2) and torch.equal(o, o2)


@pytest.mark.timeout(500)
@pytest.mark.parametrize("step", [1, 7])
def test_sweep_step(step):
    # every keep ratio of the sweep; on step 7 the masks of all heads and one whole head of attention at
    # keep 0.1, on step 1 sampled heads
    cfg = synth.get_config("sweep")
    log(f"[sweep] generating step {step}")
    layer = Layer(synth.make_sweep_inputs(cfg, step))
    heads = list(range(cfg.H)) if step == 7 else [5, 20, 33]
    for keep in cfg.keep_ratios:
        mask, o = layer.run(keep)
        m_gpu = _check_masks(layer, mask, keep, heads)
        _check_properties(layer, o)
        _check_attention_sample(layer, m_gpu, o, [(0, 5, 0), (0, 5, 976), (0, 5, 992), (0, 5, 500), (0, 31, 77)],
                                f"sweep step {step} keep={keep} o")
        if step == 7 and keep == min(cfg.keep_ratios):
            _check_whole_head(layer, m_gpu, o, 5, f"sweep step {step} keep={keep} o")


@pytest.mark.timeout(300)
def test_full_fused_prologue_pool_matches_separate(full):
    # the fused prologue + pooling pass gives the same q_hat/k_hat bytes and the same mask at full size
    c = full.cfg
    keep = c.keep_ratios[0]
    g = {n: full.inp[n].to(DEV) for n in ("q", "k", "pos_thw", "w_q", "w_k")}
    qf, kf = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    ws = saq.qknorm_rope_pool(g["q"], g["k"], qf, kf, g["pos_thw"], (g["w_q"], g["w_k"]), c.sections, c.rope_base,
                              c.eps, c.block)
    m_f = saq.select_blocks_pooled(qf.shape, keep, ws, c.block)
    m_s, _ = full.run(keep)
    torch.cuda.synchronize()
    assert torch.equal(qf, full.qh) and torch.equal(kf, full.kh)
    assert torch.equal(m_f, m_s)
    log("  full: fused prologue+pooling path bit-identical (q_hat, k_hat, all 40 heads' masks)")


@pytest.mark.timeout(400)
def test_full_sweep_reuse(full):
    # sweep step 1 against step 0 (the full inputs) at the full size: the pooled-change sums
    # against the oracle's exactly rounded sums of the same pooled means, the overlap counts
    # of the two fresh masks bit-exact, and the gate on either side of the measured change
    c = full.cfg
    keep = c.keep_ratios[0]
    cfg_s = synth.get_config("sweep")
    log("[full] generating sweep step 1 (q, k)")
    s1 = synth.make_sweep_inputs(cfg_s, 1, tensors=("q", "k"))
    pos, wq, wk = (full.inp[n].to(DEV) for n in ("pos_thw", "w_q", "w_k"))
    ws, masks = [], []
    for q, k in ((full.inp["q"], full.inp["k"]), (s1["q"], s1["k"])):
        q, k = q.to(DEV), k.to(DEV)
        qh, kh = torch.empty_like(q), torch.empty_like(k)
        ws.append(saq.qknorm_rope_pool(q, k, qh, kh, pos, (wq, wk), c.sections, c.rope_base, c.eps, c.block))
        masks.append(saq.select_blocks_pooled(q.shape, keep, ws[-1], c.block))
        del q, k, qh, kh
    shape = (c.B, c.S, c.H, c.D)
    out = saq.pooled_change(ws[0], ws[1], shape, c.block)
    counts = saq.mask_overlap(masks[1], masks[0])
    torch.cuda.synchronize()
    npool = saq.pooled_bytes(*shape, c.block)
    p0 = ws[0][:npool].view(torch.float64).cpu().numpy()
    p1 = ws[1][:npool].view(torch.float64).cpu().numpy()
    d2_ref, p2_ref = oracle.pooled_change(p0, p1)
    d2, p2 = out[:2].tolist()
    assert abs(d2 - d2_ref) <= 1e-12 * d2_ref and abs(p2 - p2_ref) <= 1e-12 * p2_ref
    m0, m1 = masks[0].cpu().numpy(), masks[1].cpu().numpy()
    assert np.array_equal(counts.cpu().numpy(), oracle.mask_overlap(m1, m0))
    r = (d2 / p2) ** 0.5
    ov = counts[..., 0].sum().item() / counts[..., 1].sum().item()
    log(f"  full sweep step 0 -> 1: relative pooled change {r:.5f}, mask overlap {ov:.4f} at keep={keep}")
    for thr, kept in ((2.0 * r, True), (0.5 * r, False)):
        reuse = saq.MaskReuse(shape, keep, thr, c.block, DEV)
        reuse.step(ws[0])
        m = reuse.step(ws[1])
        torch.cuda.synchronize()
        assert reuse.recomputed() != kept
        assert torch.equal(m, masks[0] if kept else masks[1])


@pytest.mark.timeout(300)
def test_full_folded_selection_matches_two_calls(full):
    # the attention with the selection folded in gives the same mask and output bytes at the full size
    c = full.cfg
    keep = c.keep_ratios[0]
    g = {n: full.inp[n].to(DEV) for n in ("q", "k", "pos_thw", "w_q", "w_k")}
    qf, kf = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    ws = saq.qknorm_rope_pool(g["q"], g["k"], qf, kf, g["pos_thw"], (g["w_q"], g["w_k"]), c.sections, c.rope_base,
                              c.eps, c.block)
    m2 = saq.select_blocks_pooled(qf.shape, keep, ws, c.block)
    o2 = saq.block_sparse_attn(qf, kf, full.v, m2, c.block)
    m1 = torch.empty_like(m2)
    o1 = saq.block_sparse_attn_select(qf, kf, full.v, ws, keep, c.block, mask_out=m1)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2) and torch.equal(o1, o2)
    log("  full: attention with the folded selection bit-identical to select + attention (mask and output)")
