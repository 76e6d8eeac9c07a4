"""The fused MoE layer composed from the library's calls.

pack_moe() runs the offline packers once (host) and uploads the packed
weights; fused_moe() runs the hot path on the current stream:
    moe_route -> moe_align -> GATE_UP (int4/int8 GEMM + SiLU*up) -> DOWN (GEMM x
    routed weight + top-k combine)
Python only allocates buffers and passes pointers; every step runs in the
library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import ops
from ._lib import WQ_STAGE_DOWN, WQ_STAGE_GATE_UP

DECODE_BLOCK = 16    # token block of the small-batch kernel
PREFILL_BLOCK = 128  # token block of the large-batch kernel
PREFILL_BLOCK_THIN = 64


@dataclass
class PackedMoE:
    bits: int
    E: int
    K: int          # hidden size (w1 input, w2 output)
    N: int          # intermediate size
    group_size: int
    act: object     # torch dtype of activations and scales
    w1: object      # packed gate/up weights (device uint8)
    s1: object      # packed scales (device, act dtype bits)
    k_perm1: Optional[object]  # act-order input permutation of w1 (device int32) or None
    w2: object
    s2: object

    @property
    def act_code(self) -> int:
        return ops.act_code(self.act)


def pack_moe(bits: int, w1q: np.ndarray, s1_bits: np.ndarray, w2q: np.ndarray, s2_bits: np.ndarray, act,
             group_size: int = -1, g1: Optional[np.ndarray] = None, g2: Optional[np.ndarray] = None,
             device="cuda") -> PackedMoE:
    """Canonical weights (w1q [E,2N,K], s1 [E,G1,2N], w2q [E,K,N], s2 [E,G2,K], optional act-order g_idx) ->
    device-resident packed layout."""
    import torch
    E, n2, K = w1q.shape
    N = n2 // 2
    k_perm1 = None
    if bits == 4:
        row_perm = None
        if g2 is not None:
            w2p, s2p, kp2 = ops.pack_w4(w2q, s2_bits, group_size, g_idx=g2)
            row_perm = kp2
        else:
            w2p, s2p, _ = ops.pack_w4(w2q, s2_bits, group_size)
        w1p, s1p, kp1 = ops.pack_w4(w1q, s1_bits, group_size, g_idx=g1, row_perm=row_perm, interleave_gate_up=True)
        if kp1 is not None:
            k_perm1 = torch.from_numpy(kp1).to(device)
    elif bits == 8:
        w1p, s1p = ops.pack_w8(w1q, s1_bits, interleave_gate_up=True)
        w2p, s2p = ops.pack_w8(w2q, s2_bits)
    else:
        raise ValueError("bits must be 4 or 8")

    def dev(a):
        return torch.from_numpy(a).to(device)

    return PackedMoE(bits, E, K, N, group_size, act, dev(w1p), dev(s1p.view(np.int16)), k_perm1, dev(w2p),
                     dev(s2p.view(np.int16)))


def choose_block_size(M: int, topk: int, E: int, bits: int = 8) -> int:
    """Batch-size heuristic on the mean rows per touched expert, measured on
    MI355X: up to 16 the small-batch kernel (block 16: it rereads the token
    rows from L2 for every weight tile, cheap only while they are few), then
    the large-batch kernel with 64-row token tiles (less padding) up to 32 rows
    (int8) or 48 (int4: its weights cost less to reread), beyond that its
    128-row tiles (Mixtral shape: M=80 16->64 0.319 -> 0.297 ms; M=256 int4
    64->128 0.375 -> 0.352 ms).  With many experts (64 or more) routing is
    skewed and the head experts hold several times the mean: 64-row tiles
    from 6 mean rows, 128 above 48 (DeepSeek-V2 shape, top-6: M=256 0.472 ->
    0.353 ms, M=1024 128->64 0.797 -> 0.777 ms)."""
    T = M * topk
    if T == 0:
        return DECODE_BLOCK
    rows_per_expert = T / min(E, T)
    if E >= 64:
        small, thin = 6, 48
    else:
        small, thin = 16, (48 if bits == 4 else 32)
    if rows_per_expert <= small:
        return DECODE_BLOCK
    return PREFILL_BLOCK_THIN if rows_per_expert <= thin else PREFILL_BLOCK


class MoERunner:
    """The hot path for one batch shape with every buffer allocated up front, so
    a call allocates nothing.  marks: optional 3 events recorded on the stream
    after alignment, after GATE_UP and after DOWN (stage timing)."""

    def __init__(self, p: PackedMoE, M: int, topk: int, renormalize: bool = True, block_size: Optional[int] = None,
                 device="cuda"):
        import torch
        self.p, self.M, self.topk, self.renormalize = p, M, topk, renormalize
        self.bs = choose_block_size(M, topk, p.E, p.bits) if block_size is None else block_size
        self.cap = ops.moe_align_capacity(M, topk, p.E, self.bs)
        dev = torch.device(device)
        self.w = torch.empty((M, topk), dtype=torch.float32, device=dev)
        self.ids = torch.empty((M, topk), dtype=torch.int32, device=dev)
        self.st = torch.empty(max(self.cap, 1), dtype=torch.int32, device=dev)
        self.ex = torch.empty(max(self.cap // self.bs, 1), dtype=torch.int32, device=dev)
        self.nt = torch.empty(4, dtype=torch.int32, device=dev)
        act_order = p.k_perm1 is not None
        ws1 = ops.moe_gemm_workspace_bytes(WQ_STAGE_GATE_UP, M, topk, p.E, 2 * p.N, p.K, self.cap, act_order)
        ws2 = ops.moe_gemm_workspace_bytes(WQ_STAGE_DOWN, M, topk, p.E, p.K, p.N, self.cap, False)
        self.work1 = torch.empty(ws1, dtype=torch.uint8, device=dev) if ws1 else None
        self.work2 = torch.empty(ws2, dtype=torch.uint8, device=dev) if ws2 else None
        self.h = torch.empty((max(self.cap, 1), p.N), dtype=p.act, device=dev)
        self.out = torch.empty((M, p.K), dtype=p.act, device=dev)
        # the smallest batches route inside the GATE_UP call (moe_route_gate_up: without act-order one launch,
        # with it the routing launch also gathers the permuted rows)
        if act_order:
            self.route_in_gate_up = 1 <= M <= 16 and M * topk <= 64 and p.E <= 64 and self.cap <= 1024
        else:
            self.route_in_gate_up = (M * topk <= 16 and p.E <= 64 and self.bs in (16, 32) and self.cap <= 1024)

    def route_align(self, logits, stream=None):
        ops.moe_route_align(logits, self.topk, self.renormalize, self.bs, self.w, self.ids, self.st, self.ex,
                            self.nt, self.cap, stream=stream)

    def route_gate_up(self, x, logits, stream=None):
        q = self.p
        ops.moe_route_gate_up(q.bits, logits, self.renormalize, self.w, self.ids, x, self.M, self.topk, q.E, 2 * q.N,
                              q.K, q.w1, q.s1, q.group_size if q.bits == 4 else -1, q.k_perm1, self.st, self.ex,
                              self.nt, self.cap, self.bs, self.h, self.work1, stream, q.act_code)

    def gate_up(self, x, stream=None):
        p = self
        q = self.p
        if q.bits == 4:
            ops.moe_w4a16_gemm(WQ_STAGE_GATE_UP, x, p.M, p.topk, q.E, 2 * q.N, q.K, q.w1, q.s1, q.group_size,
                               q.k_perm1, p.st, p.ex, p.nt, p.cap, p.bs, None, p.h, p.work1, stream, q.act_code)
        else:
            ops.moe_w8a16_gemm(WQ_STAGE_GATE_UP, x, p.M, p.topk, q.E, 2 * q.N, q.K, q.w1, q.s1, p.st, p.ex, p.nt,
                               p.cap, p.bs, None, p.h, p.work1, stream, q.act_code)

    def down(self, stream=None):
        p = self
        q = self.p
        if q.bits == 4:
            ops.moe_w4a16_gemm(WQ_STAGE_DOWN, p.h, p.M, p.topk, q.E, q.K, q.N, q.w2, q.s2, q.group_size, None,
                               p.st, p.ex, p.nt, p.cap, p.bs, p.w, p.out, p.work2, stream, q.act_code)
        else:
            ops.moe_w8a16_gemm(WQ_STAGE_DOWN, p.h, p.M, p.topk, q.E, q.K, q.N, q.w2, q.s2, p.st, p.ex, p.nt, p.cap,
                               p.bs, p.w, p.out, p.work2, stream, q.act_code)

    def __call__(self, x, logits, marks=None, stream=None):
        if getattr(self, "route_in_gate_up", False):
            # one launch for route, sort and GATE_UP (timed as GATE_UP)
            if marks:
                marks[0].record()
            self.route_gate_up(x, logits, stream)
        else:
            self.route_align(logits, stream)
            if marks:
                marks[0].record()
            self.gate_up(x, stream)
        if marks:
            marks[1].record()
        self.down(stream)
        if marks:
            marks[2].record()
        return self.out

    def capture(self, x, logits):
        """Record one call (route -> align -> GATE_UP -> DOWN -> combine) into a
        HIP graph that reads x and logits from these tensors' memory and writes
        the runner's buffers; replay() reruns it after the caller updates the
        inputs in place.  The launches are validated once, here."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self(x, logits)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self(x, logits)
        self.graph, self._graph_inputs = g, (x, logits)
        return g

    def replay(self):
        self.graph.replay()
        return self.out

    def aux(self):
        return {"topk_weights": self.w, "topk_ids": self.ids, "sorted_token_ids": self.st, "expert_ids": self.ex,
                "num_tokens_post_padded": self.nt, "h": self.h, "y": self.work2, "block_size": self.bs,
                "capacity": self.cap}


def fused_moe(x, logits, p: PackedMoE, topk: int, renormalize: bool = True, block_size: Optional[int] = None,
              stream=None, keep=False):
    """x [M, K] act, logits [M, E] float32 -> out [M, K] act.  With keep=True also
    returns a dict of the intermediate device buffers."""
    r = MoERunner(p, x.shape[0], topk, renormalize, block_size, device=x.device)
    out = r(x, logits, stream=stream)
    return (out, r.aux()) if keep else out


# ----------------------------------------------------------------------------
# FP8 (E4M3) W8A8 layer
# ----------------------------------------------------------------------------
@dataclass
class PackedFp8MoE:
    E: int
    K: int
    N: int
    act: object     # torch dtype of the layer input and output
    a1: float       # static scale of the layer input
    a2: float       # static scale of H
    w1: object      # packed E4M3 gate/up weights (device uint8)
    s1: object      # float32 [E, 2N] packed row order
    w2: object
    s2: object

    @property
    def act_code(self) -> int:
        return ops.act_code(self.act)


def pack_moe_fp8(w1: np.ndarray, s1: np.ndarray, w2: np.ndarray, s2: np.ndarray, act, a1: float, a2: float,
                 device="cuda") -> PackedFp8MoE:
    """Canonical E4M3 codes (w1 [E,2N,K], w2 [E,K,N]) and float32 per-column
    scales (s1 [E,2N], s2 [E,K]) -> device-resident packed layout."""
    import torch
    E, n2, K = w1.shape
    w1p, s1p = ops.pack_fp8(w1, s1, interleave_gate_up=True)
    w2p, s2p = ops.pack_fp8(w2, s2)

    def dev(a):
        return torch.from_numpy(a).to(device)

    return PackedFp8MoE(E, K, n2 // 2, act, float(a1), float(a2), dev(w1p), dev(s1p), dev(w2p), dev(s2p))


class Fp8MoERunner:
    """The FP8 W8A8 hot path for one batch shape, buffers allocated up front:
    route -> align -> GATE_UP (x quantised with a1, H written as E4M3 codes of
    h / a2) -> DOWN (routed-weight sum, rounded once to the activation type)."""

    def __init__(self, p: PackedFp8MoE, M: int, topk: int, renormalize: bool = True,
                 block_size: Optional[int] = None, device="cuda"):
        import torch
        self.p, self.M, self.topk, self.renormalize = p, M, topk, renormalize
        self.bs = choose_block_size(M, topk, p.E, 8) if block_size is None else block_size
        self.cap = ops.moe_align_capacity(M, topk, p.E, self.bs)
        dev = torch.device(device)
        self.w = torch.empty((M, topk), dtype=torch.float32, device=dev)
        self.ids = torch.empty((M, topk), dtype=torch.int32, device=dev)
        self.st = torch.empty(max(self.cap, 1), dtype=torch.int32, device=dev)
        self.ex = torch.empty(max(self.cap // self.bs, 1), dtype=torch.int32, device=dev)
        self.nt = torch.empty(4, dtype=torch.int32, device=dev)
        ws1 = ops.moe_fp8_gemm_workspace_bytes(WQ_STAGE_GATE_UP, M, topk, p.E, 2 * p.N, p.K)
        ws2 = ops.moe_fp8_gemm_workspace_bytes(WQ_STAGE_DOWN, M, topk, p.E, p.K, p.N)
        self.work1 = torch.empty(max(ws1, 1), dtype=torch.uint8, device=dev)
        self.work2 = torch.empty(max(ws2, 1), dtype=torch.uint8, device=dev)
        self.h = torch.empty((max(self.cap, 1), p.N), dtype=torch.uint8, device=dev)
        self.out = torch.empty((M, p.K), dtype=p.act, device=dev)

    def route_align(self, logits, stream=None):
        ops.moe_route_align(logits, self.topk, self.renormalize, self.bs, self.w, self.ids, self.st, self.ex,
                            self.nt, self.cap, stream=stream)

    def gate_up(self, x, stream=None):
        q = self.p
        ops.moe_fp8_w8a8_gemm(WQ_STAGE_GATE_UP, x, self.M, self.topk, q.E, 2 * q.N, q.K, q.w1, q.s1, self.st,
                              self.ex, self.nt, self.cap, self.bs, None, self.h, self.work1, q.a1, q.a2, stream,
                              q.act_code)

    def down(self, stream=None):
        q = self.p
        ops.moe_fp8_w8a8_gemm(WQ_STAGE_DOWN, self.h, self.M, self.topk, q.E, q.K, q.N, q.w2, q.s2, self.st,
                              self.ex, self.nt, self.cap, self.bs, self.w, self.out, self.work2, q.a2, 1.0, stream,
                              q.act_code)

    __call__ = MoERunner.__call__
    capture = MoERunner.capture
    replay = MoERunner.replay

    def aux(self):
        return {"topk_weights": self.w, "topk_ids": self.ids, "sorted_token_ids": self.st, "expert_ids": self.ex,
                "num_tokens_post_padded": self.nt, "h": self.h, "block_size": self.bs, "capacity": self.cap}


def fused_moe_fp8(x, logits, p: PackedFp8MoE, topk: int, renormalize: bool = True,
                  block_size: Optional[int] = None, stream=None, keep=False):
    """x [M, K] act, logits [M, E] float32 -> out [M, K] act (FP8 W8A8 experts)."""
    r = Fp8MoERunner(p, x.shape[0], topk, renormalize, block_size, device=x.device)
    out = r(x, logits, stream=stream)
    return (out, r.aux()) if keep else out
