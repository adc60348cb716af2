"""Builds libattn_fwd.so (the HIP kernels and the C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libattn_fwd.so")
# the measured-ceilings kernels (microbench.py) are a library of their own
MB_SOURCE = os.path.join(CSRC, "microbench.hip")
MB_LIB_PATH = os.path.join(LIB_DIR, "libattn_microbench.so")
# (source, extra flags)
SOURCES = [
    (os.path.join(CSRC, "attn_fwd.hip"), ["-Rpass-analysis=kernel-resource-usage"]),
    (os.path.join(CSRC, "attn_fwd_d128.hip"), ["-Rpass-analysis=kernel-resource-usage"]),
    (os.path.join(CSRC, "attn_fwd_paged64.hip"), ["-Rpass-analysis=kernel-resource-usage"]),
    (os.path.join(CSRC, "attn_fwd_paged128.hip"), ["-Rpass-analysis=kernel-resource-usage"]),
    (os.path.join(CSRC, "attn_bwd.hip"), ["-Rpass-analysis=kernel-resource-usage"]),
]
# Kernels whose loads are tracked by explicit vmcnt waits must not touch
# scratch memory (a spill reload would count as an outstanding load).
NO_SCRATCH = ("attn_fwd_kernel", "attn_bwd_dkdv_kernel", "attn_bwd_dq_kernel")
HEADERS = [os.path.join(CSRC, f) for f in ("attn_fwd_common.hpp", "attn_fwd_kernel.hpp",
                                            "attn_fwd_launch.hpp",
                                            "attn_fwd_merge.hpp", "attn_fwd_lockstep.hpp")] + [
    os.path.join(INCLUDE, "attn_fwd.h"), os.path.join(INCLUDE, "attn_bwd.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
NOISE = ("is not a recognized feature for this target", "argument unused during compilation")


def _check_scratch(stderr: str) -> None:
    """Fail if a kernel listed in NO_SCRATCH uses scratch (from the
    kernel-resource-usage remarks)."""
    name = None
    for line in stderr.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line and name and any(k in name for k in NO_SCRATCH):
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size != 0:
                raise RuntimeError(f"{name} uses {size} bytes of scratch per lane")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if not any(n in l for n in NOISE) and "remark:" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    _check_scratch(res.stderr)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, out: str = LIB_PATH, extra: list[str] | None = None) -> str:
    """Compile every source (always, in parallel) and atomically replace the
    library; also builds the microbenchmark library next to it."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    objs, procs = [], []
    mb_tmp = MB_LIB_PATH + ".tmp"
    mb_cmd = [HIPCC, *FLAGS, "-shared", MB_SOURCE, "-o", mb_tmp]
    for src, flags in SOURCES:
        obj = os.path.join(os.path.dirname(out), os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *flags, *(extra or []), "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        objs.append(obj)
        procs.append(cmd)
    # the translation units are independent: compile them concurrently
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(procs) + 1) as ex:
        list(ex.map(lambda c: _run(c, verbose), procs + [mb_cmd]))
    os.replace(mb_tmp, MB_LIB_PATH)
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
