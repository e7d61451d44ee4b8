"""Build libkvq.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvq.so")
BUILD = os.path.join(PKG, "_build")

ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable", "-I", os.path.join(ROOT, "include"),
          # packed fp32 VALU instructions are disabled on purpose
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around
          # the rarely taken rescale branches)
          "-mllvm", "-amdgpu-mfma-vgpr-form"]
# per-source extra flags: the encoder must not contract (x - z) / s chains
EXTRA = {"encode.hip": ["-ffp-contract=off"]}
SOURCES = ["host.cpp", "encode.hip", "decode_generic.hip", "decode_mfma.hip", "decode_lut.hip",
           "combine.hip", "prefill_mfma.hip", "prefill_codes.hip", "scratch.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [hipcc(), *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libkvq.so into the package."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libkvq.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
