"""Build ``libcsa2.so`` (the CSA2 C-ABI library) for gfx950 with hipcc.

Each source is compiled to an object in ``_build/`` in parallel, then linked
in-tree next to this file, so the library travels with the source tree.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcsa2.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("CSA2_ARCH", "gfx950")

SOURCES = ["compress.hip", "index_scan.hip", "index_cand.hip", "select_topk.hip", "sparse_attn.hip",
           "dequant.hip", "csa2_api.cpp"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # no packed fp32 ops in generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-source extra flags
SOURCE_FLAGS = {
    # the attention's accumulators stay in vector registers (VGPR-form MFMA):
    # with them in the matrix-core registers the compiler copied all 128 of
    # them out on every tile for the rare softmax rescale
    "sparse_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
