"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: a C++ driver (tests/sanitize/capi_driver.cpp)
calls every entry point with null, misaligned, overlapping, undersized and
overflow-prone arguments (INT32_MAX shapes) and with valid ones, on a host with
no GPU. The sanitizers instrument the host code only; device code is built as
usual and never runs."""
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_qknorm_amd", "csrc")
SOURCES = ["capi.hip", "select_blocks.hip", "qknorm_rope.hip", "block_sparse_attn.hip", "step_reuse.hip", "codecs.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = [
    pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available"),
    pytest.mark.skipif(torch.cuda.device_count() > 0, reason="expects a host without a GPU (valid calls report no device)"),
]


@pytest.mark.timeout(600)
def test_validation_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "capi_driver")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "sanitize", "capi_driver.cpp"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and "ok (0 failures)" in out, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
