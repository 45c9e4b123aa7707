"""Build libmsq.so (gfx950) in-tree with hipcc.

    python -m block_wise_mixed_amd.build

Always recompiles.  The library is placed next to this file so that it travels
with the source tree; nothing is installed elsewhere.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsq.so")
# read-bandwidth probe used by bench.py for context (not part of the library's ABI)
PROBE_LIB = os.path.join(HERE, "libmsq_probe.so")
PROBE_SOURCES = ["msq_probe.hip"]
ARCH = "gfx950"

SOURCES = ["msq_host.cpp", "msq_pack.hip", "msq_gemv.hip", "msq_gemm.hip", "msq_alloc.hip",
           "msq_reorder.hip", "msq_tile16.hip"]

# Device code: O3, no fast-math (correctly rounded division, denormals kept),
# no packed-fp32 instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmsq.so)")


def _compile(cc: str, src: str, obj: str, extra=(), verbose: bool = False) -> None:
    cmd = [cc, *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _link(cc: str, objs, out: str, extra=()) -> None:
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


# Host-only build with AddressSanitizer and UndefinedBehaviorSanitizer on the
# host pass: no device code is generated, so the library serves only the
# host-side ABI (plan, argument checks, workspace sizes, status strings) on a
# machine without a GPU.  The sanitizer runtime is not linked in: the process
# that loads the library preloads clang's shared ASan runtime, which also
# carries the UBSan handlers.
SANITIZE_FLAGS = [
    "-O1", "-g", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]


def asan_runtime() -> Optional[str]:
    """Path of clang's shared ASan runtime next to hipcc's clang, or None."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """Build the host side of libmsq.so with ASan + UBSan into `out`."""
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    objdir = out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    jobs = max(1, min(len(SOURCES), (os.cpu_count() or 1) // 2))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(cc, so[0], so[1], extra=SANITIZE_FLAGS, verbose=verbose),
                    zip(SOURCES, objs)))
    _link(cc, objs, out)
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        _compile(cc, src, obj, verbose=verbose)
        objs.append(obj)
    _link(cc, objs, LIB)
    pobjs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        _compile(cc, src, obj, verbose=verbose)
        pobjs.append(obj)
    _link(cc, pobjs, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
