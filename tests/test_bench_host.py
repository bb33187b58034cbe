"""Host-side logic of bench.py (no GPU): the computed-FLOP count from a block
mask, the rule for reporting the committed HBM traffic record, the source hash
it is keyed on, the --seed option, and the refusal of more than one GPU."""
import json
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_computed_flops_counts_kept_tiles_with_partial_last_block():
    # S = 300, block 128: blocks of 128, 128 and 44 tokens; D = 64
    mask = torch.zeros((1, 2, 3, 3), dtype=torch.uint8)
    mask[0, 0] = torch.tensor([[1, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=torch.uint8)
    mask[0, 1, 2, 2] = 1
    n = [128, 128, 44]
    kept = [(0, 0), (1, 0), (1, 1), (2, 1), (2, 2), (2, 2)]
    expect = 4 * 64 * sum(n[i] * n[j] for i, j in kept)
    assert bench.computed_flops(mask, 300, 128, 64) == pytest.approx(expect, rel=0, abs=0)


def test_measured_traffic_only_for_the_record_it_was_taken_on(tmp_path, monkeypatch):
    rec = {"kernel_hash": "abc123", "config": "full", "keep_ratio": 0.15, "bytes_per_launch": 1.5e11}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("abc123", "full", 0.15, "fused") == 1.5e11
    assert bench.measured_traffic("abc123", "full", 0.15, "split") == 1.5e11
    assert bench.measured_traffic("abc123", "full", 0.15, "folded") is None     # another kernel
    assert bench.measured_traffic("def456", "full", 0.15, "fused") is None      # changed source
    assert bench.measured_traffic("abc123", "medium", 0.15, "fused") is None    # other workload
    assert bench.measured_traffic("abc123", "full", 0.3, "fused") is None       # other keep ratio
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("abc123", "full", 0.15, "fused") is None


def test_source_hash_is_stable_and_short():
    h = bench.attn_source_hash()
    assert h == bench.attn_source_hash() and len(h) == 16 and int(h, 16) >= 0


def test_committed_traffic_record_names_its_kernel():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    for key in ("kernel_hash", "config", "keep_ratio", "bytes_per_launch"):
        assert key in rec
    assert rec["bytes_per_launch"] > 0


def test_seed_option_replaces_only_the_seed_index():
    from sparse_attention_qknorm_amd import synth
    base = synth.get_config("tiny")
    assert bench.config_for("tiny") == base and bench.default_seed(base)
    other = bench.config_for("tiny", base.index + 17)
    assert other.index == base.index + 17 and not bench.default_seed(other)
    assert (other.S, other.H, other.D, other.block, other.keep_ratios) == (base.S, base.H, base.D, base.block,
                                                                            base.keep_ratios)
    a, b = synth.make_inputs(base), synth.make_inputs(other)
    assert a["q"].shape == b["q"].shape and not torch.equal(a["q"], b["q"])
    assert torch.equal(a["pos_thw"], b["pos_thw"])                 # positions are structure, not draws


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
