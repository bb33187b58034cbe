"""The C ABI driven from C++ with plain HIP memory and no torch
(tests/cabi/layer_client.cpp): the named calls and the fused-pooling calls give,
bit for bit, the outputs the Python binding gives on the same inputs, and the
block mask is the oracle's."""
import os
import subprocess

import numpy as np
import pytest
import torch

import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import log, oracle_mask

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cabi", "layer_client")


def _case(name):
    if name == "tiny":
        cfg = synth.get_config("tiny")
        inp = synth.make_inputs(cfg)
        return inp, cfg.sections, cfg.block, cfg.keep_ratios[0], cfg.rope_base, cfg.eps
    sections = (32, 48, 48)
    inp = synth.make_small_case(1000, 3, 128, seed=77, sections=sections, T=2, Hg=12, W=16)
    return inp, sections, 128, 0.3, 10000.0, 1e-6


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_c_client_matches_binding(name, tmp_path):
    if not os.path.exists(EXE):
        pytest.fail("tests/cabi/layer_client is not built (run the repository's build entry point)")
    inp, sections, block, keep, base, eps = _case(name)
    B, S, H, D = inp["q"].shape
    nB = -(-S // block)
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(fin, "wb") as f:
        np.array([B, S, H, D, *sections, block], dtype="<i4").tofile(f)
        np.array([keep, base, eps], dtype="<f8").tofile(f)
        for n in ("q", "k", "v"):
            _bits(inp[n]).astype("<i2").tofile(f)
        inp["pos_thw"].numpy().astype("<i4").tofile(f)
        inp["w_q"].numpy().astype("<f4").tofile(f)
        inp["w_k"].numpy().astype("<f4").tofile(f)
    log(f"[c client] {name}: B={B} S={S} H={H} D={D} block={block} keep={keep}")
    res = subprocess.run([EXE, fin, fout], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"layer_client exit {res.returncode}: {res.stdout}{res.stderr}"
    log("  " + res.stdout.strip())
    n, nm = B * S * H * D, B * H * nB * nB
    raw = np.fromfile(fout, dtype=np.uint8)
    assert raw.size == 2 * (3 * 2 * n + nm)
    parts, off = [], 0
    for size in (2 * n, 2 * n, nm, 2 * n) * 2:
        parts.append(raw[off:off + size])
        off += size

    g = {k: inp[k].to(DEV) for k in ("q", "k", "v", "pos_thw", "w_q", "w_k")}
    qh, kh = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    saq.qknorm_rope_out(g["q"], g["k"], qh, kh, g["pos_thw"], (g["w_q"], g["w_k"]), sections, base, eps)
    mask = saq.select_blocks(qh, kh, keep, block)
    o = saq.block_sparse_attn(qh, kh, g["v"], mask, block)
    qf, kf = torch.empty_like(qh), torch.empty_like(kh)
    ws = saq.qknorm_rope_pool(g["q"], g["k"], qf, kf, g["pos_thw"], (g["w_q"], g["w_k"]), sections, base, eps, block)
    mask_f = saq.select_blocks_pooled(qf.shape, keep, ws, block)
    o_f = saq.block_sparse_attn(qf, kf, g["v"], mask_f, block)
    torch.cuda.synchronize()
    mine = [_bits(qh), _bits(kh), mask.cpu().numpy(), _bits(o), _bits(qf), _bits(kf), mask_f.cpu().numpy(), _bits(o_f)]
    labels = ["q_hat", "k_hat", "mask", "o", "fused q_hat", "fused k_hat", "fused mask", "fused o"]
    for lab, got, ref in zip(labels, parts, mine):
        assert np.array_equal(got, ref.reshape(-1).view(np.uint8)), f"{name}: C client {lab} differs from the binding"
    ref_mask = oracle_mask(qh.cpu().double().numpy(), kh.cpu().double().numpy(), block, keep)
    m = mask.cpu().numpy()
    for (b, h), rm in ref_mask.items():
        assert np.array_equal(m[b, h], rm), f"{name}: mask differs from the oracle at (b={b}, h={h})"
    log(f"  {name}: C client outputs bit-identical to the binding (both paths); mask equals the oracle's")
