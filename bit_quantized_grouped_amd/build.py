"""Build libmoe_q4.so (the C-ABI HIP library) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmoe_q4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
SOURCES = ["api.hip", "route.hip", "gemm_q4.hip", "combine.hip", "decode.hip", "dequant.hip", "router.hip",
           "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", os.path.join(ROOT, "include"),
        # packed fp32 VALU ops off: ordinary fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


# Kernels whose pipeline waits count their own vector loads (s_waitcnt vmcnt with
# a fixed count, then a barrier without a fence): the gate/up kernel on packed
# scale|bias words with 128-K chunks, whose x rows go straight into LDS.  A
# register spill would add scratch loads and stores to that count and turn the
# waits into races, so the build fails if any of them uses scratch.
# Template arguments: NMAT 2, MT, KC 128, NSUB, DEPTH, WAVES, BF false, SB true.
COUNTED_WAIT_KERNELS = re.compile(
    r"grouped_q4_kernelILi2ELi\d+ELi128ELi\d+ELi\d+ELi\d+ELb0ELb1EE")


def check_no_scratch(remarks: str) -> int:
    """Raise if a kernel matching COUNTED_WAIT_KERNELS reports scratch use; returns how
    many such kernels the remarks list."""
    name, seen = None, 0
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and COUNTED_WAIT_KERNELS.search(name):
            seen += 1
            if int(m.group(1)) != 0:
                raise RuntimeError(f"{name} uses {m.group(1)} bytes of scratch per lane: its "
                                   "counted load waits assume no spills")
    return seen


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src == "gemm_q4.hip" else []
    cmd = [hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if extra and check_no_scratch(r.stderr) == 0:
        raise RuntimeError("gemm_q4.hip: no counted-wait kernel in the resource remarks")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
