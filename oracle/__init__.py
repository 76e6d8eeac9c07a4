"""CPU oracle for the weight-only-quantized top-k MoE layer and the 2:4-sparse
W4A16 linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

The arithmetic lives in ``oracle.c`` (plain C, double accumulation); this module
only builds and loads it and marshals numpy arrays.  Inputs are the canonical
logical tensors of ``gen.synth`` (never a packed layout); 16-bit values are
passed as the float32 values that hold them exactly.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None
_lib_path = _LIB

# No fast-math and no FMA contraction: every sum is the plain sequence of
# double additions in ascending order, whatever the optimisation level, so
# results do not depend on the host CPU or on these flags.
_COMMON_FLAGS = ["-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-shared",
                 "-fPIC"]
# the build the tests load: portable code (it may run on another machine than the one that built it)
PORTABLE_FLAGS = ["-O2"] + _COMMON_FLAGS
# the build the CPU baseline times, compiled on the machine it runs on
NATIVE_FLAGS = ["-O3", "-march=native"] + _COMMON_FLAGS


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, PORTABLE_FLAGS)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc"] + PORTABLE_FLAGS + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def use_native_build(out_dir: str) -> str:
    """Compile oracle.c with NATIVE_FLAGS (-O3 -march=native) into out_dir and
    make this process's oracle calls use that build.  For timing the oracle
    as a CPU baseline on the host it runs on; the arithmetic is the same."""
    global _lib, _lib_path
    path = os.path.join(out_dir, "liboracle_native.so")
    subprocess.check_call(["gcc"] + NATIVE_FLAGS + [_SRC, "-o", path, "-lm"])
    _lib, _lib_path = None, path
    return path


def lib():
    global _lib
    if _lib is None:
        if _lib_path == _LIB and not os.path.exists(_LIB):
            build()
        L = C.CDLL(_lib_path)
        i64, i32, p = C.c_int64, C.c_int, C.c_void_p
        L.orc_route.argtypes = [p, i64, i32, i32, i32, p, p]
        L.orc_align_capacity.argtypes = [i64, i32, i32]
        L.orc_align_capacity.restype = i64
        L.orc_align.argtypes = [p, i64, i32, i32, p, p, p, i64]
        L.orc_moe_up.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, p, i32, p, i64, p, p]
        L.orc_moe_down.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, i32, p, i64, p, p]
        L.orc_moe_combine.argtypes = [i64, i32, i32, p, p, i64, p, p]
        L.orc_moe_layer.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, p, p, i32, p, p, p, i32, p, i64,
                                    p, p, p, p]
        L.orc_sparse24.argtypes = [i64, i32, i32, p, p, p, p, i32, p, i64, p]
        L.orc_quant_w8.argtypes = [i64, i32, p, i32, p, p]
        L.orc_fp8_decode.argtypes = [i64, p, p]
        L.orc_fp8_quant.argtypes = [i64, p, C.c_float, p]
        L.orc_fp8_moe_layer.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, p, p, p, C.c_float, C.c_float, p, i64,
                                        p, p, p, p]
        for f in ("orc_route", "orc_align", "orc_moe_up", "orc_moe_down", "orc_moe_combine", "orc_moe_layer",
                  "orc_sparse24", "orc_quant_w8", "orc_fp8_decode", "orc_fp8_quant", "orc_fp8_moe_layer"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


# ----------------------------------------------------------------------------
def route(logits: np.ndarray, topk: int, renormalize: bool = True):
    """-> (topk_weights [M, topk] float32, topk_ids [M, topk] int32)"""
    lg = _c(logits, np.float32)
    M, E = lg.shape
    w = np.empty((M, topk), np.float32)
    ids = np.empty((M, topk), np.int32)
    _check(lib().orc_route(_ptr(lg), M, E, topk, int(bool(renormalize)), _ptr(w), _ptr(ids)), "route")
    return w, ids


def align_capacity(T: int, E: int, block_size: int) -> int:
    return int(lib().orc_align_capacity(T, E, block_size))


def align(topk_ids: np.ndarray, E: int, block_size: int, capacity: Optional[int] = None):
    """-> (sorted_token_ids [cap] int32, expert_ids [cap/BS] int32, num_tokens_post_padded int)"""
    ids = _c(topk_ids, np.int32).reshape(-1)
    T = ids.size
    cap = align_capacity(T, E, block_size) if capacity is None else capacity
    st = np.empty(cap, np.int32)
    ex = np.empty(cap // block_size, np.int32)
    nt = np.zeros(1, np.int32)
    _check(lib().orc_align(_ptr(ids), T, E, block_size, _ptr(st), _ptr(ex), _ptr(nt), cap), "align")
    return st, ex, int(nt[0])


def _groups(s, n_out):
    return int(s.shape[1])


def moe_up(x, topk_ids, w1q, s1, g1=None, rows=None, want_gu=False):
    """-> (gu [R*topk, 2N] or None, h [R*topk, N]) in float64."""
    x = _c(x, np.float32)
    ids = _c(topk_ids, np.int32)
    M, K = x.shape
    topk = ids.shape[1]
    E, n_out, _ = w1q.shape
    N = n_out // 2
    rows_a = _c(rows, np.int64)
    R = M if rows_a is None else rows_a.size
    gu = np.empty((R * topk, n_out)) if want_gu else None
    h = np.empty((R * topk, N))
    _check(lib().orc_moe_up(M, K, N, E, topk, _ptr(x), _ptr(ids), _ptr(_c(w1q, np.int8)), _ptr(_c(s1, np.float32)),
                            _ptr(_c(g1, np.int32)), s1.shape[1], _ptr(rows_a), R, _ptr(gu), _ptr(h)), "moe_up")
    return gu, h


def moe_down(h, topk_ids, w2q, s2, g2=None, rows=None, M=None):
    """h [R*topk, N] -> y [R*topk, K] float64 (unweighted expert outputs)."""
    ids = _c(topk_ids, np.int32)
    topk = ids.shape[1]
    M = ids.shape[0] if M is None else M
    E, K, N = w2q.shape
    rows_a = _c(rows, np.int64)
    R = M if rows_a is None else rows_a.size
    h = _c(h, np.float64)
    assert h.shape == (R * topk, N)
    y = np.empty((R * topk, K))
    _check(lib().orc_moe_down(M, K, N, E, topk, _ptr(ids), _ptr(_c(w2q, np.int8)), _ptr(_c(s2, np.float32)),
                              _ptr(_c(g2, np.int32)), s2.shape[1], _ptr(rows_a), R, _ptr(h), _ptr(y)), "moe_down")
    return y


def moe_combine(y, topk_weights, rows=None):
    w = _c(topk_weights, np.float32)
    M, topk = w.shape
    rows_a = _c(rows, np.int64)
    R = M if rows_a is None else rows_a.size
    K = y.shape[1]
    out = np.empty((R, K))
    _check(lib().orc_moe_combine(M, K, topk, _ptr(w), _ptr(rows_a), R, _ptr(_c(y, np.float64)), _ptr(out)),
           "moe_combine")
    return out


def moe_layer(x, topk_weights, topk_ids, w1q, s1, g1, w2q, s2, g2, rows=None, want=("out",)):
    """Whole routed layer.  Returns a dict with 'out' [R, K] and, on request,
    'gu', 'h', 'y' (all float64)."""
    x = _c(x, np.float32)
    w = _c(topk_weights, np.float32)
    ids = _c(topk_ids, np.int32)
    M, K = x.shape
    topk = ids.shape[1]
    E, n_out, _ = w1q.shape
    N = n_out // 2
    rows_a = _c(rows, np.int64)
    R = M if rows_a is None else rows_a.size
    res = {"out": np.empty((R, K))}
    if "gu" in want:
        res["gu"] = np.empty((R * topk, n_out))
    if "h" in want:
        res["h"] = np.empty((R * topk, N))
    if "y" in want:
        res["y"] = np.empty((R * topk, K))
    rc = lib().orc_moe_layer(M, K, N, E, topk, _ptr(x), _ptr(w), _ptr(ids),
                             _ptr(_c(w1q, np.int8)), _ptr(_c(s1, np.float32)), _ptr(_c(g1, np.int32)), s1.shape[1],
                             _ptr(_c(w2q, np.int8)), _ptr(_c(s2, np.float32)), _ptr(_c(g2, np.int32)), s2.shape[1],
                             _ptr(rows_a), R, _ptr(res.get("gu")), _ptr(res.get("h")), _ptr(res.get("y")),
                             _ptr(res["out"]))
    _check(rc, "moe_layer")
    return res


def moe_layer_from_weights(wts, x_f32, topk_weights, topk_ids, rows=None, want=("out",)):
    """Convenience: the layer for a gen.synth.MoEWeights bundle."""
    return moe_layer(x_f32, topk_weights, topk_ids, wts.w1q, wts.s1_f32(), wts.g1, wts.w2q, wts.s2_f32(), wts.g2,
                     rows=rows, want=want)


def sparse24(x, vals, idx, s, group_size, rows=None):
    """y [R, N] float64 for the 2:4-sparse layer y = x W^T."""
    x = _c(x, np.float32)
    M, K = x.shape
    N = vals.shape[0]
    gs = K if group_size == -1 else group_size
    rows_a = _c(rows, np.int64)
    R = M if rows_a is None else rows_a.size
    y = np.empty((R, N))
    _check(lib().orc_sparse24(M, K, N, _ptr(x), _ptr(_c(vals, np.int8)), _ptr(_c(idx, np.uint8)),
                              _ptr(_c(s, np.float32)), gs, _ptr(rows_a), R, _ptr(y)), "sparse24")
    return y


def quant_w8(w, bf16: bool):
    """ExpertsInt8 load-time quantization of 16-bit weights w [..., k] (given as
    the float32 values that hold them): per row s = max|w| / 127 rounded to the
    16-bit type, q = w / s rounded half-to-even, clamped to +-127.  Returns
    (q int8 [..., k], s float32 [...]: the stored 16-bit scales' values)."""
    w = _c(w, np.float32)
    k = w.shape[-1]
    rows = w.size // k
    q = np.empty(w.shape, np.int8)
    s = np.empty(w.shape[:-1], np.float32)
    _check(lib().orc_quant_w8(rows, k, _ptr(w), int(bool(bf16)), _ptr(q), _ptr(s)), "quant_w8")
    return q, s


# ----------------------------------------------------------------------------
# FP8 (OCP E4M3) W8A8 MoE layer
# ----------------------------------------------------------------------------
def fp8_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8, any shape) -> their values (float64; NaN for 0x7F/0xFF)."""
    c = _c(codes, np.uint8)
    v = np.empty(c.shape, np.float64)
    _check(lib().orc_fp8_decode(c.size, _ptr(c), _ptr(v)), "fp8_decode")
    return v


def fp8_quant(v, scale: float) -> np.ndarray:
    """Codes of v / scale (float32 division), nearest E4M3 after saturating to
    +-448, ties to even; v float32 values (any shape)."""
    a = _c(v, np.float32)
    q = np.empty(a.shape, np.uint8)
    _check(lib().orc_fp8_quant(a.size, _ptr(a), float(scale), _ptr(q)), "fp8_quant")
    return q


def fp8_moe_layer(x, topk_weights, topk_ids, w1, sw1, w2, sw2, a1: float, a2: float, rows=None,
                  want=("out",)):
    """FP8 W8A8 layer: x [M, K] float32 values, w1 [E, 2N, K] / w2 [E, K, N]
    E4M3 codes, sw1 [E, 2N] / sw2 [E, K] float32 per-column weight scales, a1 /
    a2 static activation scales.  Returns a dict with 'out' [R, K] (float64)
    and on request 'gu' [R*topk, 2N], 'hq' [R*topk, N] (codes), 'y' [R*topk, K]."""
    x = _c(x, np.float32)
    w = _c(topk_weights, np.float32)
    ids = _c(topk_ids, np.int32)
    M, K = x.shape
    topk = ids.shape[1]
    E, n_out, _ = w1.shape
    N = n_out // 2
    rows_a = _c(rows, np.int64)
    R = M if rows_a is None else rows_a.size
    res = {"out": np.empty((R, K))}
    if "gu" in want:
        res["gu"] = np.empty((R * topk, n_out))
    if "hq" in want:
        res["hq"] = np.empty((R * topk, N), np.uint8)
    if "y" in want:
        res["y"] = np.empty((R * topk, K))
    rc = lib().orc_fp8_moe_layer(M, K, N, E, topk, _ptr(x), _ptr(w), _ptr(ids), _ptr(_c(w1, np.uint8)),
                                 _ptr(_c(sw1, np.float32)), _ptr(_c(w2, np.uint8)), _ptr(_c(sw2, np.float32)),
                                 float(a1), float(a2), _ptr(rows_a), R, _ptr(res.get("gu")), _ptr(res.get("hq")),
                                 _ptr(res.get("y")), _ptr(res["out"]))
    _check(rc, "fp8_moe_layer")
    return res
