"""GPU parity of the cross-step reuse kernels.

* mask overlap counts: bit-exact against the oracle's counts;
* pooled change (sum of squared differences of two steps' pooled block means,
  and the sum of squares of the first): within 1e-12 relative of the oracle's
  exactly rounded sums, and the same bits on every run;
* the gated selection: on a seeded denoising-step sequence, the keep/recompute
  decisions equal the oracle's gate run over the oracle's pooling of the same
  q-hat/k-hat, a recomputed mask equals a fresh selection (and the oracle's), a
  kept mask is the earlier one byte for byte, and the reference means are those
  of the step the mask in use was selected from.

Thresholds are placed between the oracle's relative changes, far from any of
them, so rounding cannot decide a gate.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import log, oracle_mask, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("B,H,nB,seed", [(2, 3, 37, 1), (1, 1, 1, 2), (1, 2, 1000, 3)])
def test_mask_overlap_counts(B, H, nB, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    a = (g.random((B, H, nB, nB)) < 0.3).astype(np.uint8) * g.choice(np.array([1, 2, 255], np.uint8), (B, H, nB, nB))
    b = (g.random((B, H, nB, nB)) < 0.6).astype(np.uint8)
    got = saq.mask_overlap(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)).cpu().numpy()
    assert np.array_equal(got, oracle.mask_overlap(a, b))


def _small_sweep_cfg():
    return dataclasses.replace(synth.get_config("small"), name="small_sweep", steps=8, drift=0.05)


class Steps:
    """Per-step fused prologue + pooling of a seeded sweep; keeps each step's workspace and q-hat/k-hat."""

    def __init__(self, cfg, steps):
        self.cfg = cfg
        parts = {n: synth.sweep_parts(cfg, n) for n in ("q", "k")}
        common = synth.make_inputs(cfg, tensors=())
        pos, wq, wk = common["pos_thw"].to(DEV), common["w_q"].to(DEV), common["w_k"].to(DEV)
        self.ws, self.qk = [], []
        for s in steps:
            q = synth.compose_sweep_step(*parts["q"], cfg.drift, s).to(DEV)
            k = synth.compose_sweep_step(*parts["k"], cfg.drift, s).to(DEV)
            qh, kh = torch.empty_like(q), torch.empty_like(k)
            self.ws.append(saq.qknorm_rope_pool(q, k, qh, kh, pos, (wq, wk), cfg.sections, cfg.rope_base, cfg.eps,
                                                cfg.block))
            self.qk.append((qh, kh))
        torch.cuda.synchronize()
        self.shape = tuple(self.qk[0][0].shape)
        B, S, H, D = self.shape
        self.npool = saq.pooled_bytes(B, S, H, D, cfg.block)

    def oracle_pooled(self, i):
        qh, kh = self.qk[i]
        q64, k64 = to64(qh), to64(kh)
        return np.stack([np.stack([oracle.pool_blocks(x[b], self.cfg.block) for b in range(x.shape[0])])
                         for x in (q64, k64)])


def test_pooled_change_against_oracle_and_deterministic():
    st = Steps(_small_sweep_cfg(), [0, 1, 1])
    p0, p1 = st.oracle_pooled(0), st.oracle_pooled(1)
    # the pooled block means in the workspace are the oracle's pooling of the same q-hat/k-hat
    assert np.array_equal(st.ws[0][:st.npool].view(torch.float64).cpu().numpy().reshape(p0.shape), p0)
    d2_ref, p2_ref = oracle.pooled_change(p0, p1)
    outs = [saq.pooled_change(st.ws[0], st.ws[1], st.shape, st.cfg.block) for _ in range(3)]
    torch.cuda.synchronize()
    d2, p2 = outs[0][:2].tolist()
    assert abs(d2 - d2_ref) <= 1e-12 * d2_ref and abs(p2 - p2_ref) <= 1e-12 * p2_ref
    for o in outs[1:]:
        assert torch.equal(o[:2], outs[0][:2])                 # same bits on every run
    same = saq.pooled_change(st.ws[1], st.ws[2], st.shape, st.cfg.block)
    assert same[0].item() == 0.0                               # the same step twice: no change at all
    log(f"  small sweep step 0 -> 1: relative pooled change {(d2 / p2) ** 0.5:.5f} "
        f"(oracle {(d2_ref / p2_ref) ** 0.5:.5f})")


def _threshold_between(changes, lo_rank):
    """A threshold between the lo_rank-th and the next distinct relative change, at their geometric mean."""
    vals = sorted(set(changes))
    a, b = vals[lo_rank], vals[lo_rank + 1]
    t = (a * b) ** 0.5
    assert min(abs(c - t) for c in changes) > 1e-6 * t
    return t


@pytest.mark.parametrize("keep", [0.25, 0.5])
def test_gated_selection_follows_oracle_schedule(keep):
    # steps 0..5 with step 3 repeated (an unchanged step must keep the mask even at threshold 0)
    seq = [0, 1, 2, 3, 3, 4, 5]
    st = Steps(_small_sweep_cfg(), seq)
    cfg = st.cfg
    pooled = [st.oracle_pooled(i) for i in range(len(seq))]
    # one-step relative change r1; the threshold sits between r1 and the two-step change, so
    # the oracle's gate keeps a mask for one step and recomputes on the next
    r1 = oracle.relative_change(pooled[0], pooled[1])
    r2 = oracle.relative_change(pooled[0], pooled[2])
    for thr in (0.0, (r1 * r2) ** 0.5):
        sched = oracle.reuse_schedule(pooled, thr)
        # keep every gate decision away from its boundary
        for i, (rec, ref) in enumerate(sched[1:], start=1):
            prev_ref = sched[i - 1][1]
            c = oracle.relative_change(pooled[prev_ref], pooled[i])
            assert c == 0.0 or abs(c - thr) > 1e-6 * max(thr, c)
        reuse = saq.MaskReuse(st.shape, keep, thr, cfg.block, DEV)
        used_from = {}
        for i in range(len(seq)):
            m = reuse.step(st.ws[i]).clone()
            torch.cuda.synchronize()
            rec, ref = sched[i]
            assert reuse.recomputed() == rec, f"threshold {thr}: step {i} decision differs from the oracle"
            fresh = saq.select_blocks_pooled(st.shape, keep, st.ws[i], cfg.block)
            if rec:
                assert torch.equal(m, fresh)
                used_from[i] = m
            else:
                assert torch.equal(m, used_from[ref])
            # the reference means are those of the step the mask came from
            got_ref = reuse.pooled_ref.view(torch.float64).cpu().numpy().reshape(pooled[ref].shape)
            assert np.array_equal(got_ref, pooled[ref])
            if i > 0:
                d2_ref, p2_ref = oracle.pooled_change(pooled[sched[i - 1][1]], pooled[i])
                d2, p2 = reuse.state[:2].tolist()
                assert abs(d2 - d2_ref) <= 1e-12 * d2_ref + 1e-300 and abs(p2 - p2_ref) <= 1e-12 * p2_ref
        log(f"  keep={keep} threshold={thr:.5f}: decisions {[int(r) for r, _ in sched]} match the oracle")
        if thr == 0.0:
            assert [r for r, _ in sched] == [True, True, True, True, False, True, True]
        else:
            assert any(not r for r, _ in sched[1:]) and any(r for r, _ in sched[1:])
    # the first recomputed mask against the oracle's selection
    qh, kh = st.qk[0]
    ref = oracle_mask(to64(qh), to64(kh), cfg.block, keep, heads=[0, 5])
    m0 = saq.select_blocks_pooled(st.shape, keep, st.ws[0], cfg.block).cpu().numpy()
    for (b, h), r in ref.items():
        assert np.array_equal(m0[b, h], r)


def test_gated_selection_force_and_reuse_state():
    st = Steps(_small_sweep_cfg(), [0, 4])
    reuse = saq.MaskReuse(st.shape, 0.25, 1e6, st.cfg.block, DEV)
    m0 = reuse.step(st.ws[0]).clone()
    m1 = reuse.step(st.ws[1]).clone()                        # huge threshold: kept
    torch.cuda.synchronize()
    assert not reuse.recomputed() and torch.equal(m0, m1)
    m2 = reuse.step(st.ws[1], force=True).clone()            # forced: recomputed
    torch.cuda.synchronize()
    assert reuse.recomputed()
    assert torch.equal(m2, saq.select_blocks_pooled(st.shape, 0.25, st.ws[1], st.cfg.block))
    assert not torch.equal(m2, m0)                           # four steps of drift move some blocks
