"""Build libpfs.so in-tree for gfx950 with hipcc.

    python -m paged_fp8_split_amd.build

Every HIP source is compiled with packed-FP32 instruction generation turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpfs.so")
SOURCES = [os.path.join(CSRC, "pfs_plan.cpp"), os.path.join(CSRC, "pfs_kernels.hip"),
           os.path.join(CSRC, "pfs_codec.hip"), os.path.join(CSRC, "pfs_noalloc.hip")]
ARCH = "gfx950"
# read-bandwidth probes for bench.py --ceiling (measurement only; libpfs does not use them)
PROBE_SOURCES = [os.path.join(CSRC, "pfs_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libpfs_probe.so")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpfs)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in VGPRs: the online-softmax rescale is VALU
        # work on them, and AGPR-resident accumulators would be copied around it
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", os.path.dirname(HERE),
    ]


def _digest(sources) -> str:
    """SHA-256 over the compile flags, the sources and every header they can
    include (csrc/*.h and include/*.h), so an edit anywhere shows up."""
    inc = os.path.join(os.path.dirname(HERE), "include")
    headers = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    headers += sorted(os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h"))
    # the include root is this tree's own path: hashed as a placeholder, so a
    # copy of the tree elsewhere keeps its build current
    root = os.path.dirname(HERE)
    h = hashlib.sha256(" ".join("<root>" if f == root else f for f in flags()).encode())
    for path in list(sources) + headers:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def _stamp(out) -> str:
    return out + ".srcsha"


def stale() -> bool:
    """True if either library is missing or was built from other sources than
    the tree holds now (content digest, not file times, so a copied tree whose
    build is current stays current)."""
    for sources, out in ((SOURCES, LIB), (PROBE_SOURCES, PROBE_LIB)):
        if not os.path.exists(out) or not os.path.exists(_stamp(out)):
            return True
        with open(_stamp(out)) as f:
            if f.read().strip() != _digest(sources):
                return True
    return False


def _compile(sources, out, verbose):
    digest = _digest(sources)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *flags(), "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    with open(_stamp(out), "w") as f:
        f.write(digest + "\n")
    return out


def build(verbose: bool = False) -> str:
    """Compile libpfs.so and the probe library libpfs_probe.so; returns the
    path of libpfs.so."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
