"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code, on the CPU.

* The oracle (``oracle/oracle.c``) is compiled with gcc and both sanitizers and
  driven through every entry point on small fp32 and bf16 inputs
  (``tests/sanitize/oracle_driver.c``).
* The host side of the C ABI (``csrc/ffn_api.cpp`` and ``csrc/ffn_noalloc.hip``:
  argument checks, workspace layouts, the layout self-check) is compiled with
  hipcc, the sanitizers applied to the host pass only, linked with the library's
  kernel objects, and driven through the size queries and every entry point with
  arguments the host checks reject (``tests/sanitize/api_driver.cpp``) -- no
  call reaches a GPU.

A run passes when the driver exits 0 and neither sanitizer printed a report."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "transformer_ffn_fusion_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
REPORTS = ("AddressSanitizer", "runtime error", "LeakSanitizer")


def _run_clean(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    for word in REPORTS:
        assert word not in out, out
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer", *san,
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True)
    assert "ok" in _run_clean(exe, {"OMP_NUM_THREADS": "2"})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_c_abi_host_under_sanitizers(tmp_path):
    from transformer_ffn_fusion_amd import build as B
    objdir = os.path.join(ROOT, "transformer_ffn_fusion_amd", "_build")
    kernels = [o for o in glob.glob(os.path.join(objdir, "*.hip.o"))
               if not o.endswith("ffn_noalloc.hip.o")]
    if len(kernels) < 5:   # kernel objects come from the regular build
        B.build()
        kernels = [o for o in glob.glob(os.path.join(objdir, "*.hip.o"))
                   if not o.endswith("ffn_noalloc.hip.o")]
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        host_san += ["-Xarch_host", f]
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "ffn_api.cpp"), os.path.join(CSRC, "ffn_noalloc.hip"),
                os.path.join(SAN, "api_driver.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([HIPCC, *flags, "-c", src, "-o", o], check=True, capture_output=True)
        objs.append(o)
    exe = str(tmp_path / "api_san")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", *objs, *kernels, "-o", exe],
                   check=True, capture_output=True)
    # leak checking off: the HIP runtime keeps allocations of its own until exit
    assert "ok" in _run_clean(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
