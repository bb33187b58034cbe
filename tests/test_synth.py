"""The seeded input generator: determinism, shapes and the stated position layout."""
import numpy as np
import torch

from sparse_attention_qknorm_amd import synth


def test_tiny_is_deterministic_and_shaped():
    a = synth.make_inputs("tiny")
    b = synth.make_inputs("tiny")
    cfg = a["cfg"]
    assert cfg.S == 1024 and cfg.nB == 16
    for name in ("q", "k", "v"):
        assert a[name].dtype == torch.bfloat16 and a[name].shape == (1, 1024, 2, 64)
        assert torch.equal(a[name], b[name])
    assert not torch.equal(a["q"], a["k"])
    assert a["w_q"].dtype == torch.float32 and ((a["w_q"] >= 0.9) & (a["w_q"] <= 1.1)).all()


def test_config_sizes():
    want = {"tiny": (1024, 16), "small": (8192, 64), "medium": (32768, 256), "full": (127040, 993)}
    for name, (S, nB) in want.items():
        cfg = synth.get_config(name)
        assert (cfg.S, cfg.nB) == (S, nB)
    full = synth.get_config("full")
    assert full.S_video == 124992 and full.S - full.block * (full.nB - 1) == 64


def test_positions_layout():
    pos = synth.positions_thw(2, 3, 4, 5)
    assert pos.dtype == np.int32 and pos.shape == (29, 3)
    assert pos[0].tolist() == [0, 0, 0] and pos[1].tolist() == [0, 0, 1] and pos[4].tolist() == [0, 1, 0]
    assert pos[12].tolist() == [1, 0, 0] and pos[23].tolist() == [1, 2, 3]
    assert pos[24:].tolist() == [[2, 0, 0], [3, 0, 0], [4, 0, 0], [5, 0, 0], [6, 0, 0]]


def test_locality_field_rms():
    inp = synth.make_inputs("small", tensors=("q",))
    x = inp["q"].float()
    var = x.var().item()
    assert 1.15 < var < 1.35                           # N(0,1) + field of element RMS 0.5


def test_sweep_step0_equals_base():
    # the drift recipe at step 0 is the base tensor; check on the small shape by reusing the
    # sweep path with the small config's seeds
    a = synth.make_sweep_inputs("small", 0, tensors=("k",))
    b = synth.make_inputs("small", tensors=("k",))
    assert torch.equal(a["k"], b["k"])
    c = synth.make_sweep_inputs(synth.CONFIGS["small"].__class__(**{**synth.CONFIGS["small"].__dict__,
                                                                   "drift": 0.05}), 3, tensors=("k",))
    d = (c["k"].float() - b["k"].float())
    assert 0.1 < d.std().item() < 0.2                  # 0.05 * 3 * N(0,1) plus bf16 rounding


def test_sweep_composition_matches_host_generator():
    import dataclasses
    cfg = dataclasses.replace(synth.get_config("small"), name="small_sweep", steps=8, drift=0.05)
    for name in ("q", "v"):
        base, delta = synth.sweep_parts(cfg, name)
        for step in (0, 1, 7):
            ref = synth.make_sweep_inputs(cfg, step, tensors=(name,))[name]
            got = synth.compose_sweep_step(base, delta, cfg.drift, step)
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (name, step)
