#!/usr/bin/env python3
"""Throughput of the joint-sequence attention layer on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload full] [--no-cpu-baseline]

One step is one pass of the whole layer over one batch of resident synthetic
input: fused QKNorm + 3D RoPE (out of place, from the pristine q/k into working
buffers, so every step sees the same input), block selection at the config's
keep ratio, and block-sparse attention. K steps are timed between two device
synchronisations. The kernels of each call are also bracketed by HIP events on
the stream they run on, which gives the per-call averages.

Printed (one JSON line): the metric (computed-tile attention TFLOP/s over the
whole layer time), ms per layer, the per-call times, dense-equivalent
TFLOP/s, the roofline of the dominant kernel (attention, MFMA-bound against the
bf16 dense peak) and the fp64 CPU oracle's throughput on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ATTN_SOURCE = os.path.join(ROOT, "sparse_attention_qknorm_amd", "csrc", "block_sparse_attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_sparse_attn_full_traffic.json")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def attn_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("block_sparse_attn.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "sparse_attention_qknorm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def computed_flops(mask, S: int, block: int, D: int) -> float:
    """4*D*sum over kept (i, j) of n_i*n_j, from the actual mask (torch uint8 [B,H,nB,nB] on device)."""
    import torch
    nB = mask.shape[-1]
    n = torch.full((nB,), float(block), dtype=torch.float64, device=mask.device)
    n[-1] = float(S - block * (nB - 1))
    m = (mask != 0).to(torch.float64)
    return float(4.0 * D * torch.einsum("bhij,i,j->", m, n, n).item())


def measured_traffic(kernel_hash: str, workload: str, keep: float, path: str):
    """HBM bytes per attention launch from the committed counter runs, if they were taken on this kernel source,
    this workload and keep ratio, and the attention kernel without the folded selection; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("kernel_hash") != kernel_hash or rec.get("config") != workload or rec.get("keep_ratio") != keep
            or path == "folded"):
        return None
    return rec.get("bytes_per_launch")


def config_for(name: str, seed=None):
    """The named workload's config, with its seed index replaced when `seed` is given: other draws of the
    same shapes, value distributions and structure."""
    from sparse_attention_qknorm_amd import synth
    cfg = synth.get_config(name)
    return cfg if seed is None else dataclasses.replace(cfg, index=int(seed))


def default_seed(cfg) -> bool:
    from sparse_attention_qknorm_amd import synth
    return cfg.index == synth.get_config(cfg.name).index


def cpu_baseline(inp, cfg, keep: float, budget_s: float) -> dict:
    """The fp64 oracle on a bounded sample of the same layer, scaled to computed TFLOP/s.

    Sample: four heads spread over the layer (prologue and selection of each over the whole sequence), then
    attention on seeded-random (head, query block) pairs of those heads for about budget_s seconds. The
    oracle's matrix products run on every host core through BLAS; that thread count is reported as cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:                                   # pragma: no cover - threadpoolctl missing
        threads = 1
    import torch
    S, H, D, block, nB = cfg.S, cfg.H, cfg.D, cfg.block, cfg.nB
    heads = sorted({0, H // 3, (2 * H) // 3, H - 1})
    last_n = S - block * (nB - 1)
    sizes = np.full(nB, block, dtype=np.float64)
    sizes[-1] = last_n
    t_pro = t_sel = 0.0
    per_head = {}
    for h in heads:
        t0 = time.perf_counter()
        q0 = inp["q"][:, :, h:h + 1].double().numpy()
        k0 = inp["k"][:, :, h:h + 1].double().numpy()
        qh, kh = oracle.qknorm_rope(q0, k0, inp["pos_thw"].numpy(), inp["w_q"].numpy(), inp["w_k"].numpy(),
                                    cfg.sections, cfg.rope_base, cfg.eps)
        t_pro += time.perf_counter() - t0
        qb = torch.from_numpy(qh.astype(np.float32)).to(torch.bfloat16).double().numpy()
        kb = torch.from_numpy(kh.astype(np.float32)).to(torch.bfloat16).double().numpy()
        t0 = time.perf_counter()
        mask = oracle.select_blocks(qb, kb, block, keep)
        t_sel += time.perf_counter() - t0
        per_head[h] = (qb, kb, inp["v"][:, :, h:h + 1].double().numpy(), mask)
    kk = oracle.num_kept_blocks(keep, nB)
    rng = np.random.Generator(np.random.PCG64(99))
    t0 = time.perf_counter()
    done = 0
    flops = 0.0
    while done < len(heads) * nB and (time.perf_counter() - t0) < budget_s:
        h = heads[int(rng.integers(0, len(heads)))]
        i = int(rng.integers(0, nB))
        qb, kb, v0, mask = per_head[h]
        oracle.block_sparse_attention_rows(qb, kb, v0, mask, block, [(0, 0, i)])
        flops += 4.0 * D * sizes[i] * float(sizes[mask[0, 0, i] != 0].sum())
        done += 1
    t_att = time.perf_counter() - t0
    # per-layer estimate: every head costs the sampled heads' mean prologue and selection; attention scales by FLOPs
    att_rate = flops / t_att
    layer_flops = 4.0 * D * float(sum((sizes[None, :] * sizes[:, None] * (per_head[h][3][0, 0] != 0)).sum()
                                      for h in heads)) * H / len(heads)
    layer_s = H * (t_pro + t_sel) / len(heads) + layer_flops / att_rate
    return {
        "value": float(layer_flops / layer_s / 1e12),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "ms_per_layer_est": float(layer_s * 1e3),
        "sample": (f"heads {heads} of the {cfg.name} layer: prologue over all {S} tokens and selection over all "
                   f"{nB} query blocks of each ({t_pro:.2f} s and {t_sel:.2f} s for the {len(heads)}), attention on {done} "
                   f"seeded-random (head, query block) pairs of those heads ({t_att:.2f} s, k={kk}); scaled to "
                   f"{H} heads. host: {platform.processor() or platform.machine()}, "
                   f"{len(os.sched_getaffinity(0))} cpus visible, BLAS threads {threads} (the oracle's matrix "
                   f"products use them all; everything else in it is single-threaded NumPy)"),
    }


def sweep(args) -> dict:
    """The denoising-step sweep with gated mask reuse.

    Eight steps of drifting inputs (step s = bf16(X_base + 0.05*s*Delta), composed on the device from resident
    fp32 parts), at each keep ratio of the sweep config. Every step runs the fused prologue + pooling, then per
    (keep, threshold) the gated selection and the attention with the mask it leaves. Measured per step: the
    relative change of the pooled means against the previous step, the overlap of the fresh mask with the
    previous step's fresh mask (kept blocks in both / kept blocks), the gate's decision, and when a mask is kept,
    its overlap with the fresh mask and the output error against attention with the fresh mask."""
    import torch

    import sparse_attention_qknorm_amd as saq
    from sparse_attention_qknorm_amd import synth

    cfg = config_for("sweep", args.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    saq.lib()
    keeps = [args.keep] if args.keep is not None else list(cfg.keep_ratios)
    thresholds = [float(x) for x in args.reuse_thresholds.split(",")]
    log(f"[sweep] generating base and drift tensors (S={cfg.S} H={cfg.H} D={cfg.D})")
    t0 = time.perf_counter()
    parts = {}
    for n in ("q", "k", "v"):
        b, d = synth.sweep_parts(cfg, n)
        parts[n] = (b.to(dev), d.to(dev))
        del b, d
        log(f"[sweep] {n} ready ({time.perf_counter() - t0:.0f} s)")
    common = synth.make_inputs(cfg, tensors=())
    pos, wq, wk = common["pos_thw"].to(dev), common["w_q"].to(dev), common["w_k"].to(dev)
    shape = (cfg.B, cfg.S, cfg.H, cfg.D)
    x = {n: torch.empty(shape, dtype=torch.bfloat16, device=dev) for n in ("q", "k", "v")}
    qh, kh = torch.empty_like(x["q"]), torch.empty_like(x["k"])
    wsb = saq.select_workspace_bytes(*shape, cfg.block)
    ws = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(2)]
    o_used, o_fresh = torch.empty_like(qh), torch.empty_like(qh)
    fresh = {kp: torch.empty((cfg.B, cfg.H, cfg.nB, cfg.nB), dtype=torch.uint8, device=dev) for kp in keeps}
    prev_fresh = {kp: torch.empty_like(fresh[kp]) for kp in keeps}
    reuse = {(kp, t): saq.MaskReuse(shape, kp, t, cfg.block, dev) for kp in keeps for t in thresholds}
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        return a, b

    rows = []
    for step in range(cfg.steps):
        for n in ("q", "k", "v"):
            synth.compose_sweep_step(*parts[n], cfg.drift, step, out=x[n])
        cur, prev = ws[step % 2], ws[(step + 1) % 2]
        ev_pro = timed(lambda: saq.qknorm_rope_pool(x["q"], x["k"], qh, kh, pos, (wq, wk), cfg.sections,
                                                     cfg.rope_base, cfg.eps, cfg.block, workspace=cur))
        change = saq.pooled_change(prev, cur, shape, cfg.block) if step else None
        row = {"step": step, "per_keep": {}}
        pending = []
        for kp in keeps:
            ev_fresh = timed(lambda: saq.select_blocks_pooled(shape, kp, cur, cfg.block, out=fresh[kp]))
            # attention on the fresh mask: the per-step select + attention time with the selection redone
            # every step
            ev_fresh_att = timed(lambda: saq.block_sparse_attn(qh, kh, x["v"], fresh[kp], cfg.block, out=o_fresh))
            ent = {"fresh_select": ev_fresh, "fresh_attn": ev_fresh_att, "thr": {}}
            if step:
                ent["overlap_prev"] = saq.mask_overlap(fresh[kp], prev_fresh[kp])
            for t in thresholds:
                r = reuse[(kp, t)]
                ev_sel = timed(lambda: r.step(cur))
                ev_att = timed(lambda: saq.block_sparse_attn(qh, kh, x["v"], r.mask, cfg.block, out=o_used))
                te = {"sel": ev_sel, "att": ev_att, "ov_fresh": saq.mask_overlap(r.mask, fresh[kp])}
                torch.cuda.synchronize()
                if not r.recomputed():
                    diff = (o_used.float() - o_fresh.float())
                    te["err"] = (float(diff.abs().max().item()),
                                 float(diff.norm().item() / max(o_fresh.float().norm().item(), 1e-30)))
                te["recomputed"] = r.recomputed()
                te["change_vs_ref"] = r.relative_change() if step else None
                ent["thr"][t] = te
            prev_fresh[kp].copy_(fresh[kp])
            row["per_keep"][kp] = ent
        torch.cuda.synchronize()
        row["pro_ms"] = ev_pro[0].elapsed_time(ev_pro[1])
        if change is not None:
            d2, p2 = change[:2].tolist()
            row["change_prev"] = (d2 / p2) ** 0.5
        line = [f"step {step}: prologue+pool {row['pro_ms']:.2f} ms"]
        if step:
            line.append(f"pooled change vs prev {row['change_prev']:.5f}")
        for kp, ent in row["per_keep"].items():
            ent["fresh_ms"] = ent.pop("fresh_select")
            ent["fresh_ms"] = ent["fresh_ms"][0].elapsed_time(ent["fresh_ms"][1])
            ent["fresh_attn_ms"] = ent.pop("fresh_attn")
            ent["fresh_attn_ms"] = ent["fresh_attn_ms"][0].elapsed_time(ent["fresh_attn_ms"][1])
            if "overlap_prev" in ent:
                c = ent["overlap_prev"].sum(dim=(0, 1)).tolist()
                ent["overlap_prev"] = c[0] / c[1]
            for t, te in ent["thr"].items():
                te["sel_ms"] = te.pop("sel")
                te["sel_ms"] = te["sel_ms"][0].elapsed_time(te["sel_ms"][1])
                te["att_ms"] = te.pop("att")
                te["att_ms"] = te["att_ms"][0].elapsed_time(te["att_ms"][1])
                c = te.pop("ov_fresh").sum(dim=(0, 1)).tolist()
                te["overlap_with_fresh"] = c[0] / c[1]
            line.append(f"keep {kp}: select {ent['fresh_ms']:.3f} + attention {ent['fresh_attn_ms']:.2f} ms, "
                        f"overlap vs prev {ent.get('overlap_prev', 1.0):.4f}, decisions " +
                        " ".join(f"{t}:{'R' if te['recomputed'] else 'K'}" for t, te in ent["thr"].items()))
        log("[sweep] " + "; ".join(line))
        rows.append(row)

    # summary per (keep, threshold): recompute count, worst output error of a kept mask, time saved
    summary = {}
    for kp in keeps:
        for t in thresholds:
            tes = [r["per_keep"][kp]["thr"][t] for r in rows]
            kept = [te for te in tes if not te["recomputed"]]
            fresh_ms = sum(r["per_keep"][kp]["fresh_ms"] for r in rows)
            gated_ms = sum(te["sel_ms"] for te in tes)
            summary[f"keep={kp},threshold={t}"] = {
                "recomputed_steps": [r["step"] for r, te in zip(rows, tes) if te["recomputed"]],
                "kept_mask_overlap_with_fresh_min": min([te["overlap_with_fresh"] for te in kept], default=1.0),
                "kept_mask_o_max_abs_vs_fresh": max([te["err"][0] for te in kept], default=0.0),
                "kept_mask_o_rel_fro_vs_fresh": max([te["err"][1] for te in kept], default=0.0),
                "select_ms_total_always": fresh_ms,
                "select_ms_total_gated": gated_ms,
                "attn_ms_total": sum(te["att_ms"] for te in tes),
            }
    per_step = [{"step": r["step"], "prologue_pool_ms": r["pro_ms"], "pooled_change_vs_prev": r.get("change_prev"),
                 "mask_overlap_vs_prev": {str(kp): r["per_keep"][kp].get("overlap_prev") for kp in keeps},
                 "fresh_select_ms": {str(kp): r["per_keep"][kp]["fresh_ms"] for kp in keeps},
                 "fresh_attn_ms": {str(kp): r["per_keep"][kp]["fresh_attn_ms"] for kp in keeps},
                 "fresh_select_plus_attn_ms": {str(kp): r["per_keep"][kp]["fresh_ms"] + r["per_keep"][kp]["fresh_attn_ms"]
                                               for kp in keeps}} for r in rows]
    return {"workload": f"sweep: {cfg.steps} denoising steps of the full layer (S={cfg.S}, H={cfg.H}, D={cfg.D}), "
                        f"step s = bf16(X_base + {cfg.drift}*s*Delta)",
            "seed": cfg.index, "keeps": keeps, "thresholds": thresholds, "per_step": per_step, "summary": summary}


def codec_bench(args) -> dict:
    """The INT8 / FP8 block codecs on the full layer's tensors: per-kernel time and HBM rate (algorithmic bytes:
    quantise reads 2 and writes 1 byte per element, dequantise the reverse, plus 4 bytes of scale per tile), and the
    end-to-end effect of the exchange formats: the layer recomputed from INT8-decoded q-hat/k-hat/v (selection
    included) against the bf16 layer, and the FP8 round trip of the output."""
    import torch

    import sparse_attention_qknorm_amd as saq
    from sparse_attention_qknorm_amd import synth

    cfg = config_for("full", args.seed)
    keep = args.keep if args.keep is not None else cfg.keep_ratios[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    saq.lib()
    log(f"[codecs] generating {cfg.name} inputs")
    inp = synth.make_inputs(cfg)
    q0, k0, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    pos, wq, wk = inp["pos_thw"].to(dev), inp["w_q"].to(dev), inp["w_k"].to(dev)
    qh, kh = torch.empty_like(q0), torch.empty_like(k0)
    ws = saq.qknorm_rope_pool(q0, k0, qh, kh, pos, (wq, wk), cfg.sections, cfg.rope_base, cfg.eps, cfg.block)
    mask = saq.select_blocks_pooled(qh.shape, keep, ws, cfg.block)
    o = saq.block_sparse_attn(qh, kh, v, mask, cfg.block)
    B, S, H, D = qh.shape
    n = B * S * H * D
    tiles = B * cfg.nB * H
    stream = torch.cuda.current_stream(dev)
    bufs = {f: (torch.empty(qh.shape, dtype=torch.int8 if f == "int8" else torch.uint8, device=dev),
                torch.empty((B, H, cfg.nB), dtype=torch.float32, device=dev)) for f in ("int8", "fp8")}
    y = torch.empty_like(qh)

    def time_call(fn, reps):
        for _ in range(args.warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {}
    for fmt, src in (("int8", qh), ("fp8", o)):
        c, sc = bufs[fmt]
        tq = time_call(lambda: saq.quantize(src, fmt, cfg.block, codes=c, scales=sc), args.steps)
        td = time_call(lambda: saq.dequantize(c, sc, fmt, cfg.block, out=y), args.steps)
        qbytes = 3.0 * n + 4.0 * tiles
        res[fmt] = {"quantize_ms": tq, "dequantize_ms": td,
                    "quantize_gbs": qbytes / (tq / 1e3) / 1e9, "dequantize_gbs": qbytes / (td / 1e3) / 1e9,
                    "quantize_frac_of_hbm_peak": qbytes / (tq / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "dequantize_frac_of_hbm_peak": qbytes / (td / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "algorithmic_bytes_per_launch": qbytes,
                    "tensor": "q_hat" if fmt == "int8" else "attention output o"}
        log(f"[codecs] {fmt}: quantize {tq:.3f} ms ({res[fmt]['quantize_gbs']:.0f} GB/s), "
            f"dequantize {td:.3f} ms ({res[fmt]['dequantize_gbs']:.0f} GB/s)")

    # end to end: the layer from INT8-decoded q-hat/k-hat/v, and the FP8 round trip of o
    dq = {}
    for name, t in (("q", qh), ("k", kh), ("v", v)):
        c, sc = saq.quantize(t, "int8", cfg.block)
        dq[name] = saq.dequantize(c, sc, "int8", cfg.block)
        del c, sc
    ws8 = torch.empty_like(ws)
    m8 = saq.select_blocks(dq["q"], dq["k"], keep, cfg.block, workspace=ws8)
    o8 = saq.block_sparse_attn(dq["q"], dq["k"], dq["v"], m8, cfg.block)
    counts = saq.mask_overlap(m8, mask)
    c, sc = saq.quantize(o, "fp8", cfg.block)
    of8 = saq.dequantize(c, sc, "fp8", cfg.block)
    torch.cuda.synchronize()

    def errs(a, b):
        d = a.float() - b.float()
        return {"max_abs": float(d.abs().max().item()), "rel_fro": float(d.norm().item() / b.float().norm().item())}

    cs = counts.sum(dim=(0, 1)).tolist()
    res["int8_qkv_layer"] = {"mask_overlap_with_bf16_mask": cs[0] / cs[1], "o_vs_bf16_layer": errs(o8, o)}
    res["fp8_o_roundtrip"] = errs(of8, o)
    log(f"[codecs] INT8 q/k/v layer: mask overlap {cs[0] / cs[1]:.4f}, o error {res['int8_qkv_layer']['o_vs_bf16_layer']}; "
        f"FP8 o round trip {res['fp8_o_roundtrip']}")
    return {"metric": "INT8 QKV / FP8 O block codecs: GB/s per kernel and error of the exchange formats",
            "n_gpus": 1, "data": "synthetic", "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": f"full layer tensors [1, {S}, {H}, {D}], tile = {cfg.block} tokens x {D} "
                                   f"channels of one head, keep_ratio={keep}", "seed": cfg.index},
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "achieved": res["int8"]["quantize_gbs"], "frac": res["int8"]["quantize_frac_of_hbm_peak"],
                         "kernel": "quantize_kernel<128,128,int8>", "traffic": None},
            **res}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="full", choices=["full", "medium", "small", "tiny", "sweep", "codecs"],
                    help="sweep: the 8-step drift sweep with gated mask reuse; codecs: the INT8/FP8 block "
                         "codecs on the full layer's tensors (each a separate measurement, printed as its own JSON "
                         "line)")
    ap.add_argument("--reuse-thresholds", default="0.005,0.01,0.02,0.04",
                    help="sweep only: relative pooled-change thresholds of the mask-reuse gate")
    ap.add_argument("--keep", type=float, default=None, help="keep ratio (default: the config's first)")
    ap.add_argument("--path", default="fused", choices=["fused", "split", "folded"],
                    help="fused: prologue with block pooling folded in, then selection from the pooled vectors; "
                         "split: the three separate calls qknorm_rope / select_blocks / block_sparse_attn; "
                         "folded: fused prologue, then attention with the selection inside the kernel "
                         "(block_sparse_attn_select)")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed index of the synthetic inputs (default: the workload's own); the committed traffic "
                         "record is reported only for the default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle attention in the CPU sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write elementwise copy (3 launches) after the timed "
                         "steps, as the reference kernel for scaling HBM byte counters")
    args = ap.parse_args(argv)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the layer would shard by "
              "heads across GPUs, with an all-to-all on either side of the attention). Run with --gpus 1.", file=sys.stderr)
        return 2

    if args.workload == "codecs":
        print(json.dumps(codec_bench(args)), flush=True)
        return 0
    if args.workload == "sweep":
        print(json.dumps({"metric": "mask reuse across denoising steps (gate decisions, overlap, output error)",
                          "n_gpus": 1, "data": "synthetic", **sweep(args)}), flush=True)
        return 0

    import torch

    import sparse_attention_qknorm_amd as saq
    from sparse_attention_qknorm_amd import synth

    cfg = config_for(args.workload, args.seed)
    keep = args.keep if args.keep is not None else cfg.keep_ratios[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    saq.lib()

    log(f"[bench] generating {cfg.name} inputs: B={cfg.B} S={cfg.S} H={cfg.H} D={cfg.D} block={cfg.block} keep={keep}")
    t0 = time.perf_counter()
    inp = synth.make_inputs(cfg)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    q0, k0, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    pos, wq, wk = inp["pos_thw"].to(dev), inp["w_q"].to(dev), inp["w_k"].to(dev)
    qh, kh = torch.empty_like(q0), torch.empty_like(k0)
    nB = cfg.nB
    mask = torch.empty((cfg.B, cfg.H, nB, nB), dtype=torch.uint8, device=dev)
    ws = torch.empty(saq.select_workspace_bytes(cfg.B, cfg.S, cfg.H, cfg.D, cfg.block), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q0)
    stream = torch.cuda.current_stream(dev)

    ev = {name: [] for name in ("pro", "sel", "att")}

    def step(record: bool):
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
        if args.path in ("fused", "folded"):
            saq.qknorm_rope_pool(q0, k0, qh, kh, pos, (wq, wk), cfg.sections, cfg.rope_base, cfg.eps, cfg.block,
                                 workspace=ws)
        else:
            saq.qknorm_rope_out(q0, k0, qh, kh, pos, (wq, wk), cfg.sections, cfg.rope_base, cfg.eps)
        if record:
            e[1].record(stream)
        if args.path == "fused":
            saq.select_blocks_pooled(qh.shape, keep, ws, cfg.block, out=mask)
        elif args.path == "split":
            saq.select_blocks(qh, kh, keep, cfg.block, out=mask, workspace=ws)
        if record:
            e[2].record(stream)
        if args.path == "folded":
            # the selection runs inside the attention kernel; no mask is written in the timed steps
            saq.block_sparse_attn_select(qh, kh, v, ws, keep, cfg.block, out=o, mask_out=None)
        else:
            saq.block_sparse_attn(qh, kh, v, mask, cfg.block, out=o)
        if record:
            e[3].record(stream)
            ev["pro"].append((e[0], e[1]))
            ev["sel"].append((e[1], e[2]))
            ev["att"].append((e[2], e[3]))

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    # FLOPs from the mask the timed steps used: the fused and split paths write it every step; the folded
    # path writes it only when asked, so one more (untimed) call fills it
    if args.path == "folded":
        saq.block_sparse_attn_select(qh, kh, v, ws, keep, cfg.block, out=o, mask_out=mask)
        torch.cuda.synchronize()
    flops = computed_flops(mask, cfg.S, cfg.block, cfg.D)
    dense_flops = 4.0 * cfg.D * cfg.H * cfg.B * float(cfg.S) ** 2

    def avg_ms(name):
        return float(np.mean([a.elapsed_time(b) for a, b in ev[name]]))

    ms = {n: avg_ms(n) for n in ev}
    att_s = ms["att"] / 1e3
    achieved = flops / att_s / 1e12
    khash = attn_source_hash()
    traffic = measured_traffic(khash, cfg.name, keep, args.path) if default_seed(cfg) else None
    pro_bytes = 8.0 * cfg.D * cfg.H * cfg.B * cfg.S + 12.0 * cfg.S

    result = {
        "metric": "joint-seq attention TFLOP/s + ms/layer (1 MI355X), % of bf16 MFMA peak",
        "value": flops / (ms_step / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one joint video+audio self-attention layer, B={cfg.B}, "
                               f"S={cfg.S} ({cfg.T}x{cfg.Hg}x{cfg.W} video + {cfg.A} audio tokens), H={cfg.H}, "
                               f"D={cfg.D}, block={cfg.block}, keep_ratio={keep}",
                   "global_batch": cfg.B, "seq_len": cfg.S, "heads": cfg.H, "head_dim": cfg.D,
                   "block": cfg.block, "keep_ratio": keep, "kept_blocks_per_row": saq.kept_blocks(keep, nB),
                   "seed": cfg.index,
                   "parallelism": "none (1 GPU)"},
        "ms_per_layer": ms_step,
        "path": args.path,
        "ms_per_call": ({"qknorm_rope_pool": ms["pro"], "select_blocks_pooled": ms["sel"],
                         "block_sparse_attn": ms["att"]} if args.path == "fused" else
                        {"qknorm_rope_pool": ms["pro"], "block_sparse_attn_select": ms["att"]}
                        if args.path == "folded" else
                        {"qknorm_rope": ms["pro"], "select_blocks": ms["sel"], "block_sparse_attn": ms["att"]}),
        "attention_tflops_computed": achieved,
        "attention_tflops_dense_equivalent": dense_flops / att_s / 1e12,
        "layer_tflops_dense_equivalent": dense_flops / (ms_step / 1e3) / 1e12,
        "attention_frac_of_bf16_peak": achieved / BF16_PEAK_TFLOPS,
        "computed_tflop_per_layer": flops / 1e12,
        "prologue_gbs": pro_bytes / (ms["pro"] / 1e3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic,
                     "kernel": ("d128::attn_kernel<false> (block 128, head_dim 128)" if args.path != "folded" else
                                "d128::attn_kernel<true> (block 128, head_dim 128, selection folded in)"),
                     "kernel_hash": khash,
                     "flop_per_launch": flops},
    }
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "launches": 3,
                                      "kernel": "torch elementwise mul by 1.0 (fp32)"}
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s of attention)")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, keep, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
