"""Thin Python binding over libwqmoe.so.

Every function here only marshals arguments: torch tensors supply device
memory and the current HIP stream, numpy arrays supply host memory for the
offline packers.  All computation happens in the library's kernels (or, for
the packers, in its host code).  The names follow include/wqmoe.h.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Tuple

import numpy as np

from . import _lib
from ._lib import (WQ_BF16, WQ_F16, WQ_PACK_INTERLEAVE_GATE_UP, WQ_STAGE_DOWN, WQ_STAGE_GATE_UP, WQ_STAGE_RAW,
                   WqMoeGemmDesc, check, load)

__all__ = [
    "moe_route", "moe_align", "moe_route_align", "moe_align_capacity", "moe_gemm_workspace_bytes", "moe_w4a16_gemm", "moe_w8a16_gemm",
    "moe_route_gate_up",
    "moe_w8a16_gemm_noalloc", "sparse24_w4a16_gemm", "sparse24_w8a16_gemm", "quantize_w8", "dense_gemm_workspace_bytes", "dense_w4a16_gemm", "dense_w8a16_gemm",
    "pack_w4", "pack_w8", "pack_sparse24", "act_code", "moe_fp8_gemm_workspace_bytes", "moe_fp8_w8a8_gemm",
    "pack_fp8",
]


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream)
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def act_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float16:
        return WQ_F16
    if dtype == torch.bfloat16:
        return WQ_BF16
    raise ValueError("activation dtype must be float16 or bfloat16, got %s" % dtype)


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


# ----------------------------------------------------------------------------
# hot path
# ----------------------------------------------------------------------------
def moe_route(logits, topk: int, renormalize: bool = True, topk_weights=None, topk_ids=None, stream=None):
    """logits [M, E] float32 (device) -> (topk_weights [M, topk] f32, topk_ids [M, topk] i32)."""
    torch = _torch()
    M, E = logits.shape
    if topk_weights is None:
        topk_weights = torch.empty((M, topk), dtype=torch.float32, device=logits.device)
    if topk_ids is None:
        topk_ids = torch.empty((M, topk), dtype=torch.int32, device=logits.device)
    check(load().moe_route(_ptr(logits), M, E, topk, int(bool(renormalize)), _ptr(topk_weights), _ptr(topk_ids),
                           _stream(stream)), "moe_route")
    return topk_weights, topk_ids


def moe_route_align(logits, topk: int, renormalize: bool, block_size: int, topk_weights, topk_ids,
                    sorted_token_ids, expert_ids, num_tokens_post_padded, capacity: int, stream=None):
    """moe_route then moe_align in one call (one kernel for batches up to 16
    tokens); every output buffer is the caller's."""
    M, E = logits.shape
    check(load().moe_route_align(_ptr(logits), M, E, topk, int(bool(renormalize)), block_size, _ptr(topk_weights),
                                 _ptr(topk_ids), _ptr(sorted_token_ids), _ptr(expert_ids),
                                 _ptr(num_tokens_post_padded), capacity, _stream(stream)), "moe_route_align")
    return topk_weights, topk_ids, sorted_token_ids, expert_ids, num_tokens_post_padded


def moe_align_capacity(M: int, topk: int, E: int, block_size: int) -> int:
    return int(load().moe_align_capacity(M, topk, E, block_size))


def moe_align(topk_ids, E: int, block_size: int, capacity: Optional[int] = None, sorted_token_ids=None,
              expert_ids=None, num_tokens_post_padded=None, stream=None):
    """topk_ids [M, topk] i32 (device) -> (sorted_token_ids [cap], expert_ids [cap/BS], num_tokens_post_padded [1])."""
    torch = _torch()
    M, topk = topk_ids.shape
    cap = moe_align_capacity(M, topk, E, block_size) if capacity is None else capacity
    dev = topk_ids.device
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(max(cap // block_size, 1), dtype=torch.int32, device=dev)
    if num_tokens_post_padded is None:
        num_tokens_post_padded = torch.empty(4, dtype=torch.int32, device=dev)
    check(load().moe_align(_ptr(topk_ids), M, topk, E, block_size, _ptr(sorted_token_ids), _ptr(expert_ids),
                           _ptr(num_tokens_post_padded), cap, _stream(stream)), "moe_align")
    return sorted_token_ids, expert_ids, num_tokens_post_padded


def moe_gemm_workspace_bytes(stage: int, M: int, topk: int, E: int, n_out: int, k_in: int, capacity: int,
                             act_order: bool) -> int:
    return int(load().moe_gemm_workspace_bytes(stage, M, topk, E, n_out, k_in, capacity, int(bool(act_order))))


def _desc(stage: int, a, M: int, topk: int, E: int, n_out: int, k_in: int, w_packed, scales, group_size: int,
          k_perm, sorted_token_ids, expert_ids, num_tokens_post_padded, capacity: int, block_size: int, topk_weights,
          out, workspace, act_dtype: int):
    d = WqMoeGemmDesc()
    d.struct_size = C.sizeof(WqMoeGemmDesc)
    d.stage = stage
    d.act_dtype = act_dtype
    d.d_a = _ptr(a)
    d.M, d.topk, d.E, d.n_out, d.k_in = M, topk, E, n_out, k_in
    d.d_w_packed = _ptr(w_packed)
    d.d_scales = _ptr(scales)
    d.group_size = group_size
    d.d_k_perm = _ptr(k_perm)
    d.d_sorted_token_ids = _ptr(sorted_token_ids)
    d.d_expert_ids = _ptr(expert_ids)
    d.d_num_tokens_post_padded = _ptr(num_tokens_post_padded)
    d.capacity = capacity
    d.block_size = block_size
    d.d_topk_weights = _ptr(topk_weights)
    d.d_out = _ptr(out)
    d.d_workspace = _ptr(workspace)
    d.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return d


def _gemm(fn_name: str, stage: int, a, M: int, topk: int, E: int, n_out: int, k_in: int, w_packed, scales,
          group_size: int, k_perm, sorted_token_ids, expert_ids, num_tokens_post_padded, capacity: int,
          block_size: int, topk_weights, out, workspace, stream, act_dtype: int):
    d = _desc(stage, a, M, topk, E, n_out, k_in, w_packed, scales, group_size, k_perm, sorted_token_ids, expert_ids,
              num_tokens_post_padded, capacity, block_size, topk_weights, out, workspace, act_dtype)
    check(getattr(load(), fn_name)(C.byref(d), _stream(stream)), fn_name)
    return out


def moe_route_gate_up(wbits: int, logits, renormalize: bool, topk_weights, topk_ids, a, M, topk, E, n_out, k_in,
                      w_packed, scales, group_size, k_perm, sorted_token_ids, expert_ids, num_tokens_post_padded,
                      capacity, block_size, out, workspace=None, stream=None, act_dtype=WQ_BF16):
    """moe_route_align followed by the GATE_UP stage of moe_w{wbits}a16_gemm in
    one call (one kernel for the smallest batches); writes topk_weights,
    topk_ids, sorted_token_ids, expert_ids, num_tokens_post_padded and out."""
    d = _desc(WQ_STAGE_GATE_UP, a, M, topk, E, n_out, k_in, w_packed, scales, group_size, k_perm, sorted_token_ids,
              expert_ids, num_tokens_post_padded, capacity, block_size, None, out, workspace, act_dtype)
    check(load().moe_route_gate_up(_ptr(logits), int(bool(renormalize)), _ptr(topk_weights), _ptr(topk_ids),
                                   C.byref(d), wbits, _stream(stream)), "moe_route_gate_up")
    return out


def moe_w4a16_gemm(stage, a, M, topk, E, n_out, k_in, w_packed, scales, group_size, k_perm, sorted_token_ids,
                   expert_ids, num_tokens_post_padded, capacity, block_size, topk_weights, out, workspace=None,
                   stream=None, act_dtype=WQ_F16):
    return _gemm("moe_w4a16_gemm", stage, a, M, topk, E, n_out, k_in, w_packed, scales, group_size, k_perm,
                 sorted_token_ids, expert_ids, num_tokens_post_padded, capacity, block_size, topk_weights, out,
                 workspace, stream, act_dtype)


def moe_w8a16_gemm(stage, a, M, topk, E, n_out, k_in, w_packed, scales, sorted_token_ids, expert_ids,
                   num_tokens_post_padded, capacity, block_size, topk_weights, out, workspace=None, stream=None,
                   act_dtype=WQ_BF16):
    return _gemm("moe_w8a16_gemm", stage, a, M, topk, E, n_out, k_in, w_packed, scales, -1, None,
                 sorted_token_ids, expert_ids, num_tokens_post_padded, capacity, block_size, topk_weights, out,
                 workspace, stream, act_dtype)


def moe_w8a16_gemm_noalloc(stage, a, M, topk, E, n_out, k_in, w_packed, scales, sorted_token_ids, expert_ids,
                           num_tokens_post_padded, capacity, block_size, topk_weights, out, stream=None,
                           act_dtype=WQ_BF16):
    """moe_w8a16_gemm with the library's own scratch as the workspace (no
    workspace argument; nothing is allocated)."""
    return _gemm("moe_w8a16_gemm_noalloc", stage, a, M, topk, E, n_out, k_in, w_packed, scales, -1, None,
                 sorted_token_ids, expert_ids, num_tokens_post_padded, capacity, block_size, topk_weights, out,
                 None, stream, act_dtype)


def moe_fp8_gemm_workspace_bytes(stage: int, M: int, topk: int, E: int, n_out: int, k_in: int) -> int:
    return int(load().moe_fp8_gemm_workspace_bytes(stage, M, topk, E, n_out, k_in))


def moe_fp8_w8a8_gemm(stage, a, M, topk, E, n_out, k_in, w_packed, scales, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, capacity, block_size, topk_weights, out, workspace, in_scale: float,
                      out_scale: float = 1.0, stream=None, act_dtype=WQ_BF16):
    """FP8 (E4M3) W8A8 grouped GEMM: GATE_UP (x in act dtype -> H codes), DOWN
    (H codes -> out in act dtype) or RAW (x -> fp32); in_scale / out_scale are
    the static activation scales (a1, a2 for GATE_UP; a2 for DOWN)."""
    d = WqMoeGemmDesc()
    d.struct_size = C.sizeof(WqMoeGemmDesc)
    d.stage = stage
    d.act_dtype = act_dtype
    d.d_a = _ptr(a)
    d.M, d.topk, d.E, d.n_out, d.k_in = M, topk, E, n_out, k_in
    d.d_w_packed = _ptr(w_packed)
    d.d_scales = _ptr(scales)
    d.group_size = -1
    d.d_k_perm = None
    d.d_sorted_token_ids = _ptr(sorted_token_ids)
    d.d_expert_ids = _ptr(expert_ids)
    d.d_num_tokens_post_padded = _ptr(num_tokens_post_padded)
    d.capacity = capacity
    d.block_size = block_size
    d.d_topk_weights = _ptr(topk_weights)
    d.d_out = _ptr(out)
    d.d_workspace = _ptr(workspace)
    d.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().moe_fp8_w8a8_gemm(C.byref(d), float(in_scale), float(out_scale), _stream(stream)),
          "moe_fp8_w8a8_gemm")
    return out


def _sparse24(fn, x, vals, meta, scales, N, out, group_size, stream):
    torch = _torch()
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    check(fn(_ptr(x), M, K, N, _ptr(vals), _ptr(meta), _ptr(scales), group_size, _ptr(out), act_code(x.dtype),
             _stream(stream)), fn.__name__)
    return out


def sparse24_w4a16_gemm(x, vals, meta, scales, N: int, out=None, group_size: int = 128, stream=None):
    """x [M, K] fp16 (device) -> y [M, N] fp16, 4-bit kept codes."""
    return _sparse24(load().sparse24_w4a16_gemm, x, vals, meta, scales, N, out, group_size, stream)


def sparse24_w8a16_gemm(x, vals, meta, scales, N: int, out=None, group_size: int = 128, stream=None):
    """x [M, K] fp16 (device) -> y [M, N] fp16, 8-bit kept codes (packed with bits=8)."""
    return _sparse24(load().sparse24_w8a16_gemm, x, vals, meta, scales, N, out, group_size, stream)


def dense_gemm_workspace_bytes(M: int, K: int, N: int, act_order: bool = False) -> int:
    return int(load().dense_gemm_workspace_bytes(M, K, N, int(bool(act_order))))


def _dense(fn, x, N, w_packed, scales, extra, out, workspace, stream, act_order):
    torch = _torch()
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if workspace is None:
        nb = dense_gemm_workspace_bytes(M, K, N, act_order)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    check(fn(_ptr(x), M, K, N, _ptr(w_packed), _ptr(scales), *extra, _ptr(out), act_code(x.dtype), _ptr(workspace),
             workspace.numel(), _stream(stream)), fn.__name__)
    return out


def dense_w4a16_gemm(x, N: int, w_packed, scales, group_size: int = 128, k_perm=None, out=None, workspace=None,
                     stream=None):
    """Dense int4 linear: x [M, K] fp16 (device) -> y [M, N] fp16, weights
    packed by pack_w4 with E = 1."""
    return _dense(load().dense_w4a16_gemm, x, N, w_packed, scales, (group_size, _ptr(k_perm)), out, workspace,
                  stream, k_perm is not None)


def dense_w8a16_gemm(x, N: int, w_packed, scales, out=None, workspace=None, stream=None):
    """Dense int8 linear: x [M, K] bf16/fp16 (device) -> y [M, N], weights
    packed by pack_w8 with E = 1."""
    return _dense(load().dense_w8a16_gemm, x, N, w_packed, scales, (), out, workspace, stream, False)


def quantize_w8(w, q=None, scales=None, stream=None):
    """ExpertsInt8 load-time quantization on the device: w [..., k] bf16/fp16
    (the 16-bit checkpoint; leading dims = experts x output columns) ->
    (q int8 [..., k], scales [...] in w's dtype), one scale per row."""
    torch = _torch()
    if w.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("quantize_w8 takes bf16 or fp16 weights, got %s" % w.dtype)
    w = w.contiguous()
    k = w.shape[-1]
    rows = w.numel() // k if k else 0
    if q is None:
        q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    if scales is None:
        scales = torch.empty(w.shape[:-1], dtype=w.dtype, device=w.device)
    check(load().wq_quantize_w8(_ptr(w), rows, k, act_code(w.dtype), _ptr(q), _ptr(scales), _stream(stream)),
          "wq_quantize_w8")
    return q, scales


# ----------------------------------------------------------------------------
# offline packers (host numpy in / out)
# ----------------------------------------------------------------------------
def pack_w4(q: np.ndarray, scales_bits: np.ndarray, group_size: int, g_idx: Optional[np.ndarray] = None,
            row_perm: Optional[np.ndarray] = None, interleave_gate_up: bool = False
            ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """q int8 [E, n_out, k_in], scales uint16 [E, G, n_out] -> (packed uint8, scales uint16, k_perm or None)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    E, n_out, k_in = q.shape
    s = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    L = load()
    nbytes = int(L.wq_pack_w4_bytes(E, n_out, k_in))
    if nbytes == 0:
        raise ValueError("unsupported int4 shape %s" % (q.shape,))
    packed = np.empty(nbytes, np.uint8)
    sp = np.empty_like(s)
    gi = None if g_idx is None else np.ascontiguousarray(g_idx, dtype=np.int32)
    rp = None if row_perm is None else np.ascontiguousarray(row_perm, dtype=np.int32)
    kp = np.empty((E, k_in), np.int32) if gi is not None else None
    flags = WQ_PACK_INTERLEAVE_GATE_UP if interleave_gate_up else 0
    check(L.wq_pack_w4(E, n_out, k_in, _np_ptr(q), _np_ptr(s), group_size, _np_ptr(gi), _np_ptr(rp), flags,
                       _np_ptr(packed), _np_ptr(sp), _np_ptr(kp)), "wq_pack_w4")
    return packed, sp, kp


def pack_w8(q: np.ndarray, scales_bits: np.ndarray, row_perm: Optional[np.ndarray] = None,
            interleave_gate_up: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """q int8 [E, n_out, k_in], scales uint16 [E, 1, n_out] -> (packed uint8, scales uint16)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    E, n_out, k_in = q.shape
    s = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    L = load()
    nbytes = int(L.wq_pack_w8_bytes(E, n_out, k_in))
    if nbytes == 0:
        raise ValueError("unsupported int8 shape %s" % (q.shape,))
    packed = np.empty(nbytes, np.uint8)
    sp = np.empty_like(s)
    rp = None if row_perm is None else np.ascontiguousarray(row_perm, dtype=np.int32)
    flags = WQ_PACK_INTERLEAVE_GATE_UP if interleave_gate_up else 0
    check(L.wq_pack_w8(E, n_out, k_in, _np_ptr(q), _np_ptr(s), _np_ptr(rp), flags, _np_ptr(packed), _np_ptr(sp)),
          "wq_pack_w8")
    return packed, sp


def pack_fp8(codes: np.ndarray, scales: np.ndarray, row_perm: Optional[np.ndarray] = None,
             interleave_gate_up: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """E4M3 codes uint8 [E, n_out, k_in], scales float32 [E, n_out] -> (packed uint8, scales float32)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    E, n_out, k_in = c.shape
    s = np.ascontiguousarray(scales, dtype=np.float32).reshape(E, n_out)
    L = load()
    nbytes = int(L.wq_pack_fp8_bytes(E, n_out, k_in))
    if nbytes == 0:
        raise ValueError("unsupported FP8 shape %s" % (c.shape,))
    packed = np.empty(nbytes, np.uint8)
    sp = np.empty_like(s)
    rp = None if row_perm is None else np.ascontiguousarray(row_perm, dtype=np.int32)
    flags = WQ_PACK_INTERLEAVE_GATE_UP if interleave_gate_up else 0
    check(L.wq_pack_fp8(E, n_out, k_in, _np_ptr(c), _np_ptr(s), _np_ptr(rp), flags, _np_ptr(packed), _np_ptr(sp)),
          "wq_pack_fp8")
    return packed, sp


def pack_sparse24(vals: np.ndarray, idx: np.ndarray, scales_bits: np.ndarray, group_size: int = 128, bits: int = 4):
    """vals int8 [N, K/2], idx uint8 [N, K/2], scales uint16 [K/128, N] (group
    128) or [1, N] (group -1) -> (vals, meta, scales) packed for 4- or 8-bit
    kept codes."""
    vals = np.ascontiguousarray(vals, dtype=np.int8)
    idx = np.ascontiguousarray(idx, dtype=np.uint8)
    s = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    N, Kh = vals.shape
    K = 2 * Kh
    L = load()
    vb = int(L.wq_pack_sparse24_vals_bytes(N, K, bits))
    mb = int(L.wq_pack_sparse24_meta_bytes(N, K))
    if vb == 0 or mb == 0:
        raise ValueError("unsupported 2:4 shape N=%d K=%d" % (N, K))
    vp = np.empty(vb, np.uint8)
    mp = np.empty(mb, np.uint8)
    sp = np.empty_like(s)
    G = 1 if group_size == -1 else K // 128
    if s.shape != (G, N):
        raise ValueError("scales must be [%d, %d] for group_size %d, got %s" % (G, N, group_size, s.shape))
    check(L.wq_pack_sparse24(N, K, bits, group_size, _np_ptr(vals), _np_ptr(idx), _np_ptr(s), _np_ptr(vp),
                             _np_ptr(mp), _np_ptr(sp)), "wq_pack_sparse24")
    return vp, mp, sp


_ = (WQ_STAGE_GATE_UP, WQ_STAGE_DOWN, WQ_STAGE_RAW, WQ_F16, WQ_BF16, _lib)
