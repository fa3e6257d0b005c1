"""ctypes loader for the in-tree ``libcsa2.so`` (the C ABI in include/csa2.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

# csa2_dtype
BF16, FP8_E4M3, NVFP4, F32, MXFP4 = 1, 2, 3, 4, 5
# csa2_status
OK, EINVAL, EUNSUPPORTED, ELAUNCH, EWORKSPACE = 0, -1, -2, -3, -4
SCORES_SCAN, SCORES_CAND = 0, 1
OP_SELECT, OP_SPARSE_ATTN = 1, 2

EXPORTS = (
    "csa2_status_string", "csa2_version", "csa2_compress", "csa2_index_scores",
    "csa2_select_topk", "csa2_sparse_attn", "csa2_dequant_fp8", "csa2_dequant_nvfp4",
    "csa2_workspace_bytes", "csa2_compress_nvfp4", "csa2_compress_step", "csa2_quant_nvfp4",
    "csa2_gather_scores", "csa2_gather_select", "csa2_sparse_attn_noalloc",
)
ATTN_SCRATCH_BYTES = 32 << 20

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().csa2_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")


def lib():
    """Load ``libcsa2.so`` once and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m "
            "compressed_sparse_attention_03_amd.build, or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "csa2_status_string": (ctypes.c_char_p, [I]),
        "csa2_version": (I, []),
        "csa2_compress": (I, [I, I, P, I64, P, I64, P, I64, P]),
        "csa2_index_scores": (I, [I, I, I, P, I, P, P, I, P, I64, I64, P, P, I, P, I64, P, P, I64, P]),
        "csa2_select_topk": (I, [I, I64, P, I64, P, I64, P, I, I, P, I64, P, SZ, P]),
        "csa2_sparse_attn": (I, [I, I, P, I64, P, I, P, I64, I64, P, I, I64, P, I, P, I, I, I64,
                                 P, P, F, P, I64, P, P, SZ, P]),
        "csa2_sparse_attn_noalloc": (I, [I, I, P, I64, P, I, P, I64, I64, P, I, I64, P, I, P, I,
                                         I, I64, P, P, F, P, I64, P, P]),
        "csa2_dequant_fp8": (I, [P, P, I64, I, P, I, P]),
        "csa2_dequant_nvfp4": (I, [P, P, I64, I, P, I, P]),
        "csa2_workspace_bytes": (SZ, [I, I64, I64, I64]),
        "csa2_compress_nvfp4": (I, [I, I, P, I64, P, I64, P, P, I64, P]),
        "csa2_compress_step": (I, [I, P, I64, P, I64, P, P, I, P, P, I64, I64, P]),
        "csa2_quant_nvfp4": (I, [P, I, I64, I, P, P, P]),
        "csa2_gather_scores": (I, [I, I, P, I64, I64, P, P, I, P, P, I64, P]),
        "csa2_gather_select": (I, [I, I, P, I64, I64, P, P, I, I, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != OK:
        raise Csa2Error(fn, status)
