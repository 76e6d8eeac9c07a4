"""ctypes loader for libwqmoe.so and the argument types of every export in
include/wqmoe.h.  No fallback: if the library is missing, importing the
binding's compute functions raises."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwqmoe.so")

WQ_OK, WQ_ERR_INVALID, WQ_ERR_UNSUPPORTED, WQ_ERR_DEVICE, WQ_ERR_HIP = 0, 1, 2, 3, 4
WQ_F16, WQ_BF16 = 0, 1
WQ_STAGE_GATE_UP, WQ_STAGE_DOWN, WQ_STAGE_RAW = 0, 1, 2
WQ_PACK_INTERLEAVE_GATE_UP = 1
WQ_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "wq_version", "wq_status_string", "wq_last_error",
    "moe_route", "moe_align_capacity", "moe_align", "moe_route_align", "moe_route_gate_up",
    "moe_gemm_workspace_bytes", "moe_w4a16_gemm", "moe_w8a16_gemm", "moe_w8a16_gemm_noalloc",
    "sparse24_w4a16_gemm", "sparse24_w8a16_gemm", "wq_quantize_w8",
    "dense_gemm_workspace_bytes", "dense_w4a16_gemm", "dense_w8a16_gemm",
    "wq_pack_w4_bytes", "wq_pack_w8_bytes", "wq_pack_w4", "wq_pack_w8",
    "wq_pack_sparse24_vals_bytes", "wq_pack_sparse24_meta_bytes", "wq_pack_sparse24",
    "moe_fp8_gemm_workspace_bytes", "moe_fp8_w8a8_gemm", "wq_pack_fp8_bytes", "wq_pack_fp8",
)


class WqMoeGemmDesc(C.Structure):
    _fields_ = [
        ("struct_size", C.c_size_t),
        ("stage", C.c_int),
        ("act_dtype", C.c_int),
        ("d_a", C.c_void_p),
        ("M", C.c_int), ("topk", C.c_int), ("E", C.c_int), ("n_out", C.c_int), ("k_in", C.c_int),
        ("d_w_packed", C.c_void_p),
        ("d_scales", C.c_void_p),
        ("group_size", C.c_int),
        ("d_k_perm", C.c_void_p),
        ("d_sorted_token_ids", C.c_void_p),
        ("d_expert_ids", C.c_void_p),
        ("d_num_tokens_post_padded", C.c_void_p),
        ("capacity", C.c_size_t),
        ("block_size", C.c_int),
        ("d_topk_weights", C.c_void_p),
        ("d_out", C.c_void_p),
        ("d_workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
    ]


class WqError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__("%s failed (%d): %s" % (where, status, msg))
        self.status = status


_lib = None


def load():
    """Load libwqmoe.so (built in-tree by weight_only_quantized_topk_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libwqmoe.so is not built (%s); run `python -m weight_only_quantized_topk_amd.build`"
                          % LIB_PATH)
    # torch first: the library and torch must share one HIP runtime.  Both need
    # libamdhip64.so.7, which torch bundles and ROCm installs; the loader maps
    # whichever comes first for both, and torch has to run on its own (loaded
    # the other way round, the library's hipGetDevice failed in a process where
    # torch then initialised the GPU)
    import torch  # noqa: F401
    L = C.CDLL(LIB_PATH)
    p, i, sz = C.c_void_p, C.c_int, C.c_size_t
    L.wq_version.restype = i
    L.wq_status_string.argtypes = [i]
    L.wq_status_string.restype = C.c_char_p
    L.wq_last_error.restype = C.c_char_p
    L.moe_route.argtypes = [p, i, i, i, i, p, p, p]
    L.moe_align_capacity.argtypes = [i, i, i, i]
    L.moe_align_capacity.restype = sz
    L.moe_align.argtypes = [p, i, i, i, i, p, p, p, sz, p]
    L.moe_route_align.argtypes = [p, i, i, i, i, i, p, p, p, p, p, sz, p]
    L.moe_gemm_workspace_bytes.argtypes = [i, i, i, i, i, i, sz, i]
    L.moe_gemm_workspace_bytes.restype = sz
    L.moe_w4a16_gemm.argtypes = [C.POINTER(WqMoeGemmDesc), p]
    L.moe_w8a16_gemm.argtypes = [C.POINTER(WqMoeGemmDesc), p]
    L.moe_w8a16_gemm_noalloc.argtypes = [C.POINTER(WqMoeGemmDesc), p]
    L.moe_route_gate_up.argtypes = [p, i, p, p, C.POINTER(WqMoeGemmDesc), i, p]
    L.sparse24_w4a16_gemm.argtypes = [p, i, i, i, p, p, p, i, p, i, p]
    L.sparse24_w8a16_gemm.argtypes = [p, i, i, i, p, p, p, i, p, i, p]
    L.wq_quantize_w8.argtypes = [p, C.c_int64, i, i, p, p, p]
    L.dense_gemm_workspace_bytes.argtypes = [i, i, i, i]
    L.dense_gemm_workspace_bytes.restype = sz
    L.dense_w4a16_gemm.argtypes = [p, i, i, i, p, p, i, p, p, i, p, sz, p]
    L.dense_w8a16_gemm.argtypes = [p, i, i, i, p, p, p, i, p, sz, p]
    L.wq_pack_w4_bytes.argtypes = [i, i, i]
    L.wq_pack_w4_bytes.restype = sz
    L.wq_pack_w8_bytes.argtypes = [i, i, i]
    L.wq_pack_w8_bytes.restype = sz
    L.wq_pack_w4.argtypes = [i, i, i, p, p, i, p, p, i, p, p, p]
    L.wq_pack_w8.argtypes = [i, i, i, p, p, p, i, p, p]
    L.wq_pack_sparse24_vals_bytes.argtypes = [i, i, i]
    L.wq_pack_sparse24_vals_bytes.restype = sz
    L.wq_pack_sparse24_meta_bytes.argtypes = [i, i]
    L.wq_pack_sparse24_meta_bytes.restype = sz
    L.wq_pack_sparse24.argtypes = [i, i, i, i, p, p, p, p, p, p]
    L.moe_fp8_gemm_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.moe_fp8_gemm_workspace_bytes.restype = sz
    L.moe_fp8_w8a8_gemm.argtypes = [C.POINTER(WqMoeGemmDesc), C.c_float, C.c_float, p]
    L.wq_pack_fp8_bytes.argtypes = [i, i, i]
    L.wq_pack_fp8_bytes.restype = sz
    L.wq_pack_fp8.argtypes = [i, i, i, p, p, p, i, p, p]
    for f in ("moe_route", "moe_align", "moe_route_align", "moe_route_gate_up", "moe_w4a16_gemm", "moe_w8a16_gemm",
              "moe_w8a16_gemm_noalloc", "sparse24_w4a16_gemm",
              "sparse24_w8a16_gemm",
              "wq_quantize_w8", "dense_w4a16_gemm", "dense_w8a16_gemm", "wq_pack_w4",
              "wq_pack_w8", "wq_pack_sparse24", "moe_fp8_w8a8_gemm", "wq_pack_fp8"):
        getattr(L, f).restype = i
    _lib = L
    return L


def check(status: int, where: str):
    if status != WQ_OK:
        raise WqError(status, where, load().wq_last_error().decode(errors="replace"))
