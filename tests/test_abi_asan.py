"""The C-ABI layer's host code under AddressSanitizer (CPU only): api.hip is rebuilt with
the sanitizer on its host side only (the device code is unchanged and never launched here),
linked with the library's other objects, and every host-side ABI and binding check
(test_abi_host.py, test_binding_checks.py) runs against it in a process that preloads the
sanitizer runtime.  Argument validation, status strings and workspace-size arithmetic then
run with bounds and use-after-free checking."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from bit_quantized_grouped_amd import build as bqb  # noqa: E402


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_checks_under_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not shutil.which(bqb.hipcc()):
        pytest.skip("no clang AddressSanitizer runtime or hipcc in this image")
    objs = [os.path.join(bqb.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in bqb.SOURCES
            if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        bqb.build()
    api_o = str(tmp_path / "api_asan.o")
    so = str(tmp_path / "libmoe_q4_asan.so")
    cc = [bqb.hipcc(), *bqb.common_flags(), "-O1", "-g",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(bqb.CSRC, "api.hip"), "-o", api_o]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([bqb.hipcc(), f"--offload-arch={bqb.ARCH}", "-shared", "-fPIC", api_o, *objs,
                        "-o", so], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    nm = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_report" in nm            # the host code really is instrumented
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan_runner.py"), so],
                       capture_output=True, text=True, env=env, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
