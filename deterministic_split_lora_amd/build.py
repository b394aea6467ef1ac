"""Builds liblora_det.so (the HIP kernels and the C entry points) for gfx950.

Run ``python -m deterministic_split_lora_amd.build`` or call ``build()``.  The
library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblora_det.so")
SOURCES = ["abi.hip", "shrink.hip", "expand.hip", "fused.hip", "streamed.hip", "sgmv_plan.hip"]
HEADERS = ["device.h", "kernels.h", "shrink_tile.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fp32 add / multiply in the kernels rounds on its own; fused
    # multiply-adds appear only where the source asks for one (fmaf)
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # only the C ABI (include/lora_det.h) is exported; the kernels' C++
    # launchers stay inside the library
    "-fvisibility=hidden",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _record_revision() -> None:
    """Writes the git revision of the sources next to the library (with
    "-dirty" when tracked files differ from it), so a copy of the tree without
    its history still says what the library was built from.  No git: no file."""
    import subprocess
    root = os.path.dirname(HERE)
    path = os.path.join(HERE, "build_revision.txt")
    try:
        rev = subprocess.run(["git", "-C", root, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip()
        dirty = subprocess.run(["git", "-C", root, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return
    if rev:
        with open(path, "w") as f:
            f.write(rev + ("-dirty" if dirty else "") + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source; always recompiles (a cross-compile, no GPU needed).
    Each source is compiled to an object in parallel, then the objects are
    linked into the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    inc = ["-I", os.path.join(os.path.dirname(HERE), "include")]
    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, os.path.splitext(s)[0] + ".o.tmp" + tag) for s in SOURCES]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    noise = "'-packed-fp32-ops' is not a recognized feature"

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 feature and says so;
        # that warning is harmless and filtered here
        return res.returncode, "\n".join(l for l in res.stderr.splitlines() if noise not in l)

    try:
        jobs = [[hipcc(), *compile_flags, *inc, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
            results = list(ex.map(run, jobs))
        errs = "\n".join(e for _, e in results if e.strip())
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("hipcc failed:\n" + errs)
        if verbose and errs:
            print(errs, file=sys.stderr)
        tmp = LIB + ".tmp" + tag
        rc, err = run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + err)
        os.replace(tmp, LIB)
        _record_revision()
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
