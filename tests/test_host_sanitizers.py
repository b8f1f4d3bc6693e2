"""The ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library sources together with ``tests/sanitize/abi_host_check.cpp``
with hipcc, the sanitizers on the host side only (device code is built as
usual), and runs the check program: sizing over many shapes, every
validation failure and calls that pass validation.  The program hands the
library stand-in device addresses, so it only runs where no GPU is visible.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunk_test_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


pytestmark = [
    pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed"),
    pytest.mark.skipif(_gpu_visible(), reason="stand-in device addresses: CPU-only check"),
]

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp"))]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *COMMON, *SAN, "-x", "hip", "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_host_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "abi host check: ok" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out
