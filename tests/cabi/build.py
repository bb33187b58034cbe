"""Build the C-ABI test client (tests/cabi/layer_client) against the in-tree
libsaq.so: hipcc, include/saq.h, an rpath relative to the binary so it finds
the library wherever the tree sits. Test infrastructure, called by the
repository's build entry point after the library is built."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "sparse_attention_qknorm_amd")
SRC = os.path.join(HERE, "layer_client.cpp")
EXE = os.path.join(HERE, "layer_client")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build() -> str:
    tmp = EXE + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", SRC,
           f"-L{PKG}", "-lsaq", "-Wl,-rpath,$ORIGIN/../../sparse_attention_qknorm_amd", "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("layer_client build failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
