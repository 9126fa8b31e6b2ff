"""Build libkvq.so in-tree: every HIP source compiled for gfx950 with hipcc.

    python -m kv_cache_compression_kvq_amd.build

Floating-point flags are part of the library's contract:
  -ffp-contract=off                      no implicit fused multiply-adds; the
                                         kernels call fmaf where they mean it
  -fno-gpu-flush-denormals-to-zero       binary32 subnormals are honoured
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE division and square root
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         no packed fp32 instructions
No fast-math flag is ever used.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
PROBE_SRC = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noisy = [ln for ln in r.stderr.splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if any("warning" in ln for ln in noisy):
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libkvq.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # the bench's HBM stream reference (not part of libkvq)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PROBE_LIB} for {ARCH}")
    return LIB


if __name__ == "__main__":
    build()
