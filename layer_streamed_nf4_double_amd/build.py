"""Builds liblsn.so (all HIP sources for gfx950) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblsn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["gemm.hip", "gemm_nf4f.hip", "gemm_nf4t.hip", "gemm_bf16.hip", "attn.hip", "ops.hip", "lora.hip", "runtime.hip", "nf4_host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are switched off for device code on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-Wall", "-c",
               os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    # objects of sources no longer in SOURCES (an experiment's leftovers) go
    want = {os.path.basename(src) + ".o" for src in SOURCES}
    for name in os.listdir(BUILD):
        if name.endswith(".o") and name not in want:
            os.remove(os.path.join(BUILD, name))
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT, file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
