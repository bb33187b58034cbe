"""The layer's three calls captured in a HIP graph (through torch's graph API,
which captures the current stream the library launches on): every replay gives
the eager path's bytes, with eager work and synchronisations between replays.
None of the kernels on this path issues a memset, so nothing in the graph is a
memset node."""
import pytest
import torch

import sparse_attention_qknorm_amd as saq
from sparse_attention_qknorm_amd import synth
from parity_tools import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name", ["small"])
def test_graph_replays_match_eager(name):
    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    g = {n: inp[n].to(DEV) for n in ("q", "k", "v", "pos_thw", "w_q", "w_k")}
    keep = cfg.keep_ratios[0]
    args = (g["q"], g["k"], g["v"], g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections, keep, cfg.block,
            cfg.rope_base, cfg.eps)
    o_ref, m_ref = saq.attention_layer(*args)
    o_ref, m_ref = o_ref.clone(), m_ref.clone()
    torch.cuda.synchronize()

    bufs = {}
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        saq.attention_layer(*args, buffers=bufs)        # warm up on the capture stream, allocate the buffers
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        saq.attention_layer(*args, buffers=bufs)
    for rep in range(4):
        bufs["o"].zero_()
        bufs["mask"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["o"], o_ref), f"replay {rep}: output differs from the eager run"
        assert torch.equal(bufs["mask"], m_ref), f"replay {rep}: mask differs from the eager run"
        _ = (g["v"].float() * 2).sum().item()           # eager work between replays
    log(f"  {name}: 4 graph replays of the layer equal the eager run")


def test_graph_gated_selection_replays():
    # the gated selection decides on the device, so a step loop can be captured: replaying the capture with
    # new pooled means keeps or recomputes the mask exactly as the eager calls do
    cfg = synth.get_config("small")
    inp = synth.make_inputs(cfg)
    g = {n: inp[n].to(DEV) for n in ("q", "k", "pos_thw", "w_q", "w_k")}
    qh, kh = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    ws = saq.qknorm_rope_pool(g["q"], g["k"], qh, kh, g["pos_thw"], (g["w_q"], g["w_k"]), cfg.sections,
                              block=cfg.block)
    shape = tuple(qh.shape)
    eager = saq.MaskReuse(shape, 0.25, 0.5, cfg.block, DEV)
    m0 = eager.step(ws).clone()
    torch.cuda.synchronize()
    cap = saq.MaskReuse(shape, 0.25, 0.5, cfg.block, DEV)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        cap.step(ws)                                    # first call (forced recompute) outside the graph
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap.step(ws)
    for _ in range(3):
        cap.mask.zero_()                                # a kept mask must come back untouched: poison it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert not cap.recomputed()                     # same pooled means: the mask is kept
        assert not cap.mask.any()                       # ... so the poisoned bytes stay
    cap.mask.copy_(m0)
    torch.cuda.synchronize()
    assert torch.equal(cap.mask, m0)
