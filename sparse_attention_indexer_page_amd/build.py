"""Compile the gfx950 HIP sources of the indexer library into libidx.so.

Each source is compiled to an object under the package's ``_build/`` folder
(in parallel), then linked into ``libidx.so`` next to this file. Packed FP32
instructions are disabled for all device code, and MFMA results are placed in
VGPRs (the fused epilogue reads every accumulator).
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libidx.so")
# digest of the sources and flags the library at LIB was built from
DIGEST = LIB + ".digest"
SOURCES = ["idx_api.hip", "schedule.hip", "mqa_logits.hip", "prefill.hip", "topk.hip", "kv_write.hip",
           "q_quant.hip", "sparse_mla.hip", "validate.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the indexer library needs the ROCm toolchain")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the epilogue reads them with no AGPR moves
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-command-line-argument"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c"] + _flags() + ["-o", obj, os.path.join(CSRC, src)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s%s" % (src, res.stdout, res.stderr))
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    return obj


def source_digest() -> str:
    """SHA-256 over every file under csrc/ and include/, this script and the
    compiler flags: what the library's bits depend on."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    files += [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE))]
    files.append(os.path.abspath(__file__))
    for path in files:
        if os.path.isfile(path):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as fh:
                h.update(fh.read())
    h.update(" ".join(_flags()).encode())
    return h.hexdigest()


def up_to_date() -> bool:
    """True when libidx.so exists and was built from the current sources."""
    if not os.path.exists(LIB) or not os.path.exists(DIGEST):
        return False
    with open(DIGEST) as fh:
        return fh.read().strip() == source_digest()


def ensure_built(verbose: bool = False) -> str:
    """Builds libidx.so unless it was built from the current sources."""
    if not up_to_date():
        build(verbose)
    return LIB


def build(verbose: bool = False) -> str:
    """Compile every source and link libidx.so; returns the library path."""
    digest = source_digest()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "--offload-arch=" + ARCH, "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("linking libidx.so failed:\n%s%s" % (res.stdout, res.stderr))
    os.replace(tmp, LIB)
    with open(DIGEST + ".tmp%d" % os.getpid(), "w") as fh:
        fh.write(digest + "\n")
    os.replace(DIGEST + ".tmp%d" % os.getpid(), DIGEST)
    return LIB


CEILINGS_SRC = os.path.join(HERE, "ceilings", "ceilings.hip")
CEILINGS_LIB = os.path.join(HERE, "ceilings", "libidx_ceilings.so")


def build_ceilings(verbose: bool = False) -> str:
    """Compile the roofline-ceiling measurement kernels (bench.py --ceilings)
    into their own library; they are not part of libidx.so."""
    tmp = CEILINGS_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared"] + _flags() + ["-o", tmp, CEILINGS_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s%s" % (CEILINGS_SRC, res.stdout, res.stderr))
    os.replace(tmp, CEILINGS_LIB)
    return CEILINGS_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_ceilings(verbose="-v" in sys.argv))
