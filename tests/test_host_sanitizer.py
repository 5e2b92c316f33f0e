"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer.  Every HIP source of the library is compiled with
the sanitizers on its host code only (each -fsanitize flag behind -Xarch_host;
the device code is the ordinary build), linked with tests/native/host_checks.cpp
and run here without a GPU: every call in that program is rejected by a host
check (NULL pointers, sizes outside the documented limits, misalignment, short
workspaces, inconsistent options) before anything touches a device, and
moe_workspace_bytes is swept over the size limits."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_expert_weight_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


def test_host_checks_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC) or shutil.which("g++") is None:
        pytest.skip("hipcc or g++ not available")
    objs = []
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *SAN, "-I", INCLUDE, "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    for s in srcs:
        objs.append(str(tmp_path / (os.path.basename(s)[:-4] + ".o")))
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    drv = str(tmp_path / "host_checks.o")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", INCLUDE, "-c", os.path.join(ROOT, "tests", "native", "host_checks.cpp"), "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--hip-link", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", *objs, drv, "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 0 and "host checks: 0 failed" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
