"""Build the gfx950 HIP library ``libnvfp4_hip.so`` in-tree with hipcc.

Each source is compiled to an object on its own (in parallel), then the
objects are linked into the shared library.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4_hip.so")
SOURCES = ["nvfp4_api.hip", "nvfp4_stream.hip", "nvfp4_pack.hip", "nvfp4_dense.hip", "nvfp4_norm.hip", "nvfp4_mx.hip",
           "nvfp4_w8.hip", "nvfp4_bw.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # never let the compiler form packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(jobs: int | None = None) -> str:
    sources = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmpdir = tempfile.mkdtemp(prefix="nvfp4_build_")
    try:
        objs = [os.path.join(tmpdir, s + ".o") for s in sources]
        cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
        jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build())
