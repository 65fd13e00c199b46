"""Build libcsa.so (HIP, gfx950 only) in-tree, next to this file.

Usage: python -m long_context_attention_10_amd.build [-v]
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libcsa.so")
SOURCES = ["capi.hip", "compress.hip", "index_topk.hip", "attention.hip", "attention_bf16.hip",
           "layer.hip", "noalloc.hip", "backward.hip", "kvfp8.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from forming packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source additions: the indexer's scoring epilogue reads every matrix-core
# result with vector ALU ops, so its products are kept in VGPRs (no copies
# out of the accumulation registers).
EXTRA = {"index_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, verbose):
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose=False):
    """Compile every kernel source for gfx950 and link libcsa.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
