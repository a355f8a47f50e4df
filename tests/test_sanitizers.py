"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (oracle/nvfp4_oracle.c, gcc) driven through every entry point
  on exactly sized heap buffers, including the row-count guard of the
  projections (rows outside 1..NVO_MAX_ROWS compute nothing).
* The library's host side (argument validation, the sequence builder, the
  plan writer: every .hip source compiled for the host only, sanitizers on
  the host pass) driven with fake device addresses, including a 384-call
  decode step with norms written into an exactly sized plan.

Either run aborts on the first invalid access or undefined operation.
"""
import glob
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bit_weight_only_nvfp4_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only (no device code is built or run here)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return res.returncode, res.stdout + res.stderr


@pytest.fixture()
def tmp():
    d = tempfile.mkdtemp(prefix="nvfp4_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp):
    exe = os.path.join(tmp, "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-Wno-unknown-pragmas", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
                    "-o", exe, "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=120)
    assert rc == 0 and "oracle driver: ok" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_library_host_code_under_asan_ubsan(tmp):
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        o = os.path.join(tmp, os.path.basename(src) + ".o")
        objs.append(o)
        procs.append(subprocess.Popen(
            [HIPCC, "-fgpu-rdc", "--offload-host-only", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-fPIC", *HOST_SAN, "-Wno-undefined-internal", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-c", src, "-o", o], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, out
    exe = os.path.join(tmp, "host_driver")
    rc, out = _run([HIPCC, "-fgpu-rdc", "--hip-link", "--offload-arch=gfx950", "-O1", "-g", *HOST_SAN,
                    "-I", os.path.join(ROOT, "include"), *objs, "-x", "c++", os.path.join(SAN, "host_driver.cpp"),
                    "-o", exe])
    assert rc == 0, out
    env = dict(ENV)
    env.pop("NVFP4_SAN_HAS_DEVICE", None)
    if _has_gpu():
        env["NVFP4_SAN_HAS_DEVICE"] = "1"
    rc, out = _run([exe], env=env, timeout=120)
    assert rc == 0 and "host driver: ok" in out, out
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False
