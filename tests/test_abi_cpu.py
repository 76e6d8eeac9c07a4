"""CPU-only checks of the C ABI: the library loads and exports every function
include/wqmoe.h declares, host-side validation rejects bad arguments with a
status code (no GPU call is reached), and the offline packers produce the
documented layouts."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import gen
import weight_only_quantized_topk_amd as wq
from weight_only_quantized_topk_amd import _lib
from tests.helpers import decode_sparse24, decode_w4, decode_w8, logical_rows

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, non-null: only ever seen by host-side validation below


def header_functions():
    txt = open(os.path.join(ROOT, "include", "wqmoe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_exports_match_header():
    L = wq.load()
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_status_strings_and_version():
    L = wq.load()
    assert L.wq_version() >= 1
    assert L.wq_status_string(0) == b"ok"
    assert L.wq_status_string(wq.WQ_ERR_UNSUPPORTED) == b"unsupported"


def test_align_capacity():
    L = wq.load()
    assert L.moe_align_capacity(3, 2, 4, 4) == 20
    assert L.moe_align_capacity(1, 2, 8, 16) == 32
    assert L.moe_align_capacity(4096, 6, 160, 128) == 24576 + 160 * 127 + 0 * 0 // 1 + (-(24576 + 160 * 127) % 128)
    assert L.moe_align_capacity(0, 2, 8, 16) == 0


def _status(fn, *args):
    L = wq.load()
    st = getattr(L, fn)(*args)
    return st, L.wq_last_error().decode()


def test_route_validation():
    p = C.c_void_p(FAKE)
    assert _status("moe_route", p, 4, 8, 9, 1, p, p, None)[0] == wq.WQ_ERR_INVALID      # topk > E
    assert _status("moe_route", p, -1, 8, 2, 1, p, p, None)[0] == wq.WQ_ERR_INVALID     # M < 0
    assert _status("moe_route", p, 4, 2048, 2, 1, p, p, None)[0] == wq.WQ_ERR_UNSUPPORTED
    assert _status("moe_route", p, 4, 64, 17, 1, p, p, None)[0] == wq.WQ_ERR_UNSUPPORTED
    st, msg = _status("moe_route", None, 4, 8, 2, 1, p, p, None)
    assert st == wq.WQ_ERR_INVALID and "logits" in msg
    assert _status("moe_route", C.c_void_p(FAKE + 4), 4, 8, 2, 1, p, p, None)[0] == wq.WQ_ERR_INVALID  # misaligned
    assert _status("moe_route", p, 0, 8, 2, 1, p, p, None)[0] == wq.WQ_OK  # nothing to do


def test_align_validation():
    p = C.c_void_p(FAKE)
    assert _status("moe_align", p, 4, 2, 8, 24, p, p, p, 1024, None)[0] == wq.WQ_ERR_UNSUPPORTED   # block size
    assert _status("moe_align", p, 4, 2, 8, 16, p, p, p, 16, None)[0] == wq.WQ_ERR_INVALID         # capacity
    assert _status("moe_align", p, 4, 2, 8, 16, p, p, p, 136, None)[0] == wq.WQ_ERR_INVALID        # not multiple
    assert _status("moe_align", p, 4, 2, 2000, 16, p, p, p, 1 << 20, None)[0] == wq.WQ_ERR_UNSUPPORTED
    assert _status("moe_align", p, 4, 2, 8, 16, None, p, p, 1024, None)[0] == wq.WQ_ERR_INVALID


def test_route_align_validation():
    """The fused call rejects what either of its two parts rejects, before any
    device work (the ids check against device memory is never reached)."""
    p = C.c_void_p(FAKE)
    args = lambda **k: [k.get("logits", p), k.get("M", 4), k.get("E", 8), k.get("topk", 2), 1, k.get("bs", 16),
                        p, p, k.get("st", p), p, p, k.get("cap", 1024), None]
    assert _status("moe_route_align", *args(topk=9))[0] == wq.WQ_ERR_INVALID            # topk > E
    assert _status("moe_route_align", *args(E=2000, topk=2))[0] == wq.WQ_ERR_UNSUPPORTED
    assert _status("moe_route_align", *args(topk=17, E=32))[0] == wq.WQ_ERR_UNSUPPORTED  # topk > 16
    assert _status("moe_route_align", *args(bs=24))[0] == wq.WQ_ERR_UNSUPPORTED         # block size
    assert _status("moe_route_align", *args(cap=16))[0] == wq.WQ_ERR_INVALID            # capacity
    assert _status("moe_route_align", *args(cap=136))[0] == wq.WQ_ERR_INVALID           # not a multiple
    assert _status("moe_route_align", *args(logits=None))[0] == wq.WQ_ERR_INVALID
    assert _status("moe_route_align", *args(st=None))[0] == wq.WQ_ERR_INVALID
    assert _status("moe_route_align", *args(M=-1))[0] == wq.WQ_ERR_INVALID


def test_quantize_w8_validation():
    """The load-time quantizer rejects bad sizes, dtypes and pointers before any
    device work; zero rows is a no-op."""
    p = C.c_void_p(FAKE)
    args = lambda **k: [k.get("w", p), k.get("rows", 16), k.get("k", 64), k.get("dt", wq.WQ_BF16), k.get("q", p),
                        k.get("s", p), None]
    assert _status("wq_quantize_w8", *args(k=0))[0] == wq.WQ_ERR_INVALID
    assert _status("wq_quantize_w8", *args(rows=-1))[0] == wq.WQ_ERR_INVALID
    assert _status("wq_quantize_w8", *args(dt=7))[0] == wq.WQ_ERR_INVALID
    assert _status("wq_quantize_w8", *args(k=60))[0] == wq.WQ_ERR_UNSUPPORTED        # k % 8
    assert _status("wq_quantize_w8", *args(w=None))[0] == wq.WQ_ERR_INVALID
    assert _status("wq_quantize_w8", *args(q=None))[0] == wq.WQ_ERR_INVALID
    assert _status("wq_quantize_w8", *args(s=None))[0] == wq.WQ_ERR_INVALID
    assert _status("wq_quantize_w8", *args(rows=0))[0] == wq.WQ_OK


def test_dense_validation_and_workspace():
    """The dense linear rejects bad sizes, formats and short workspaces before
    any device work; its workspace holds the routing arrays and, for a split
    long K, the fp32 slabs."""
    L = wq.load()
    p = C.c_void_p(FAKE)
    assert L.dense_gemm_workspace_bytes(1, 4096, 4096, 0) == 0   # 1..128 rows: one kernel, no workspace
    assert L.dense_gemm_workspace_bytes(2, 32768, 4096, 0) == 0  # rows too long for LDS: staged per chunk
    assert L.dense_gemm_workspace_bytes(16, 4096, 4096, 0) == 0
    assert L.dense_gemm_workspace_bytes(1, 4096, 4096, 1) > 0     # act-order gathers through the workspace
    assert L.dense_gemm_workspace_bytes(128, 4096, 4096, 0) == 0
    assert L.dense_gemm_workspace_bytes(129, 4096, 4096, 0) >= 129 * 4096 * 4
    assert L.dense_gemm_workspace_bytes(300, 4096, 256, 0) >= 4 * 300 * 256 * 4   # K split in 4
    assert L.dense_gemm_workspace_bytes(300, 4096, 256, 1) > L.dense_gemm_workspace_bytes(300, 4096, 256, 0)
    assert L.dense_gemm_workspace_bytes(0, 4096, 256, 0) == 0
    a4 = lambda **k: [k.get("x", p), k.get("M", 4), k.get("K", 512), k.get("N", 256), p, p, k.get("gs", 128), None,
                      k.get("y", p), k.get("dt", wq.WQ_F16), p, k.get("ws", 1 << 30), None]
    assert _status("dense_w4a16_gemm", *a4(K=500))[0] == wq.WQ_ERR_UNSUPPORTED      # K % 128
    assert _status("dense_w4a16_gemm", *a4(N=200))[0] == wq.WQ_ERR_UNSUPPORTED      # N % 16
    assert _status("dense_w4a16_gemm", *a4(gs=64))[0] == wq.WQ_ERR_UNSUPPORTED
    assert _status("dense_w4a16_gemm", *a4(dt=wq.WQ_BF16))[0] == wq.WQ_ERR_UNSUPPORTED
    assert _status("dense_w4a16_gemm", *a4(M=129, ws=16))[0] == wq.WQ_ERR_INVALID  # workspace too small
    assert _status("dense_w4a16_gemm", *a4(M=-1))[0] == wq.WQ_ERR_INVALID
    assert _status("dense_w4a16_gemm", *a4(x=None))[0] == wq.WQ_ERR_INVALID
    assert _status("dense_w4a16_gemm", *a4(M=0, ws=0))[0] == wq.WQ_OK
    # the act-order permutation is checked like every other pointer (the gather reads it 16 bytes at a time)
    a4p = lambda kp: [p, 40, 512, 256, p, p, 128, kp, p, wq.WQ_F16, p, 1 << 30, None]
    st, msg = _status("dense_w4a16_gemm", *a4p(C.c_void_p(FAKE + 4)))
    assert st == wq.WQ_ERR_INVALID and "k_perm" in msg
    a8 = lambda **k: [p, 4, k.get("K", 512), 256, p, p, p, wq.WQ_BF16, p, 1 << 30, None]
    assert _status("dense_w8a16_gemm", *a8(K=96))[0] == wq.WQ_ERR_UNSUPPORTED       # K % 64


def _desc(**kw):
    d = _lib.WqMoeGemmDesc()
    d.struct_size = C.sizeof(_lib.WqMoeGemmDesc)
    d.stage = wq.WQ_STAGE_GATE_UP
    d.act_dtype = wq.WQ_F16
    d.M, d.topk, d.E, d.n_out, d.k_in = 4, 2, 8, 1024, 256
    for f in ("d_a", "d_w_packed", "d_scales", "d_sorted_token_ids", "d_expert_ids", "d_num_tokens_post_padded",
              "d_out", "d_topk_weights"):
        setattr(d, f, FAKE)
    d.group_size = 128
    d.block_size = 16
    d.capacity = wq.moe_align_capacity(4, 2, 8, 16)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("fn,kw,expect", [
    ("moe_w4a16_gemm", dict(struct_size=8), wq.WQ_ERR_INVALID),
    ("moe_w4a16_gemm", dict(stage=7), wq.WQ_ERR_INVALID),
    ("moe_w4a16_gemm", dict(act_dtype=wq.WQ_BF16), wq.WQ_ERR_UNSUPPORTED),
    ("moe_w4a16_gemm", dict(topk=9), wq.WQ_ERR_INVALID),
    ("moe_w4a16_gemm", dict(k_in=200), wq.WQ_ERR_UNSUPPORTED),
    ("moe_w4a16_gemm", dict(n_out=1008), wq.WQ_ERR_UNSUPPORTED),       # gate/up needs n_out % 32
    ("moe_w4a16_gemm", dict(group_size=64), wq.WQ_ERR_UNSUPPORTED),
    ("moe_w4a16_gemm", dict(block_size=8), wq.WQ_ERR_UNSUPPORTED),
    ("moe_w4a16_gemm", dict(capacity=32), wq.WQ_ERR_INVALID),
    ("moe_w4a16_gemm", dict(d_a=None), wq.WQ_ERR_INVALID),
    ("moe_w4a16_gemm", dict(d_out=FAKE + 8), wq.WQ_ERR_INVALID),
    ("moe_w4a16_gemm", dict(stage=wq.WQ_STAGE_DOWN, n_out=256, k_in=512), wq.WQ_ERR_INVALID),  # no workspace
    ("moe_w4a16_gemm", dict(d_k_perm=FAKE), wq.WQ_ERR_INVALID),        # act-order needs the gather workspace
    ("moe_w8a16_gemm", dict(group_size=128), wq.WQ_ERR_UNSUPPORTED),   # int8 is per-column
    ("moe_w8a16_gemm", dict(group_size=-1, k_in=96), wq.WQ_ERR_UNSUPPORTED),
    ("moe_w8a16_gemm", dict(group_size=-1, d_k_perm=FAKE), wq.WQ_ERR_INVALID),
    ("moe_w8a16_gemm", dict(group_size=-1, M=1 << 24), wq.WQ_ERR_UNSUPPORTED),
    # the no-allocation variant takes no workspace and refuses one beyond its scratch
    ("moe_w8a16_gemm_noalloc", dict(group_size=-1, d_workspace=FAKE, workspace_bytes=1 << 20), wq.WQ_ERR_INVALID),
    ("moe_w8a16_gemm_noalloc", dict(group_size=-1, stage=wq.WQ_STAGE_DOWN, M=1 << 15, n_out=256, k_in=4096,
                                    capacity=wq.moe_align_capacity(1 << 15, 2, 8, 16)), wq.WQ_ERR_UNSUPPORTED),
    ("moe_w8a16_gemm_noalloc", dict(group_size=-1, k_in=96), wq.WQ_ERR_UNSUPPORTED),
])
def test_gemm_validation(fn, kw, expect):
    d = _desc(**kw)
    st, msg = _status(fn, C.byref(d), None)
    assert st == expect, msg
    assert msg


@pytest.mark.parametrize("wbits,kw,lp,expect,needle", [
    (8, dict(group_size=-1, stage=wq.WQ_STAGE_DOWN, n_out=256, k_in=512), FAKE, wq.WQ_ERR_INVALID, "GATE_UP"),
    (8, dict(group_size=-1, topk=17, E=32, capacity=wq.moe_align_capacity(4, 17, 32, 16)), FAKE,
     wq.WQ_ERR_UNSUPPORTED, "topk"),
    (5, dict(group_size=-1), FAKE, wq.WQ_ERR_INVALID, "wbits"),
    (8, dict(group_size=-1), None, wq.WQ_ERR_INVALID, "logits"),
    (8, dict(group_size=-1), FAKE + 4, wq.WQ_ERR_INVALID, "logits"),
    (4, dict(act_dtype=wq.WQ_BF16), FAKE, wq.WQ_ERR_UNSUPPORTED, "fp16"),
    (8, dict(group_size=-1, capacity=16), FAKE, wq.WQ_ERR_INVALID, "capacity"),
])
def test_route_gate_up_validation(wbits, kw, lp, expect, needle):
    """moe_route_gate_up rejects a stage other than GATE_UP, a top-k beyond
    the router's 16, a bad wbits, a NULL or misaligned logits pointer and the
    GEMM's own bad arguments, before any device work."""
    d = _desc(**kw)
    p = C.c_void_p(FAKE)
    st, msg = _status("moe_route_gate_up", C.c_void_p(lp) if lp else None, 1, p, p, C.byref(d), wbits, None)
    assert st == expect, msg
    assert needle in msg


def test_gemm_workspace_sizes():
    L = wq.load()
    assert L.moe_gemm_workspace_bytes(wq.WQ_STAGE_GATE_UP, 4, 2, 8, 1024, 256, 128, 0) == 0
    assert L.moe_gemm_workspace_bytes(wq.WQ_STAGE_GATE_UP, 4, 2, 8, 1024, 256, 128, 1) == 128 * 256 * 2
    assert L.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, 4, 2, 8, 256, 512, 128, 0) == 4 * 2 * 256 * 4
    # long k_in, few output tiles: the DOWN workspace holds 4 fp32 slabs (K split in 4)
    assert L.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, 300, 2, 8, 256, 4096, 1024, 0) == 4 * 600 * 256 * 4
    # a large grid is not split
    assert L.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, 4096, 6, 160, 5120, 1536, 1 << 16, 0) == 4096 * 6 * 5120 * 4


def test_sparse_validation():
    p = C.c_void_p(FAKE)
    L = wq.load()
    assert L.sparse24_w4a16_gemm(p, 4, 7168, 20480, p, p, p, 64, p, wq.WQ_F16, None) == wq.WQ_ERR_UNSUPPORTED
    assert L.sparse24_w4a16_gemm(p, 0, 7168, 20480, p, p, p, -1, p, wq.WQ_F16, None) == wq.WQ_OK   # channel-wise
    assert L.sparse24_w4a16_gemm(p, 4, 7000, 20480, p, p, p, 128, p, wq.WQ_F16, None) == wq.WQ_ERR_UNSUPPORTED
    assert L.sparse24_w4a16_gemm(p, 4, 7168, 20480, p, p, p, 128, p, wq.WQ_BF16, None) == wq.WQ_ERR_UNSUPPORTED
    assert L.sparse24_w4a16_gemm(None, 4, 7168, 20480, p, p, p, 128, p, wq.WQ_F16, None) == wq.WQ_ERR_INVALID
    assert L.sparse24_w4a16_gemm(p, 0, 7168, 20480, p, p, p, 128, p, wq.WQ_F16, None) == wq.WQ_OK


# ----------------------------------------------------------------------------
# packers
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("act_order,interleave,rowperm", [(False, False, False), (False, True, False),
                                                          (True, True, True), (True, False, False)])
def test_pack_w4_layout(act_order, interleave, rowperm):
    spec = gen.CFG3.with_(E=3, K=256, N=128, act_order=act_order)
    w = gen.make_moe_weights(spec, seed_config=401)
    q, s, g = w.w1q, w.s1, w.g1
    E, n_out, k_in = q.shape
    rp = None
    if rowperm:
        rng = np.random.default_rng(0)
        rp = np.stack([rng.permutation(n_out // 2 if interleave else n_out) for _ in range(E)]).astype(np.int32)
    packed, sp, kp = wq.pack_w4(q, s, 128, g_idx=g, row_perm=rp, interleave_gate_up=interleave)
    dec = decode_w4(packed, E, n_out, k_in)
    for e in range(E):
        rows = logical_rows(n_out, interleave, None if rp is None else rp[e])
        sig = kp[e] if act_order else np.arange(k_in)
        if act_order:
            assert (g[e][sig] == np.arange(k_in) // 128).all()          # groups become contiguous
            assert (np.diff(sig.reshape(-1, 128), axis=1) > 0).all()    # stable inside each group
        assert np.array_equal(dec[e], q[e][rows][:, sig])
        assert np.array_equal(sp[e], s[e][:, rows])


def test_pack_w8_layout():
    spec = gen.CFG2.with_(E=2, K=192, N=64)
    w = gen.make_moe_weights(spec, seed_config=402)
    for q, s, il in ((w.w1q, w.s1, True), (w.w2q, w.s2, False)):
        packed, sp = wq.pack_w8(q, s, interleave_gate_up=il)
        E, n_out, k_in = q.shape
        dec = decode_w8(packed, E, n_out, k_in)
        rows = logical_rows(n_out, il)
        assert np.array_equal(dec, q[:, rows, :])
        assert np.array_equal(sp, s[:, :, rows])


def test_pack_sparse24_layout():
    spec = gen.CFG4.with_(K=512, N=32)
    sw = gen.make_sparse_weights(spec, seed_config=403)
    vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s)
    v, i = decode_sparse24(vp, mp, spec.N, spec.K)
    assert np.array_equal(v, sw.vals) and np.array_equal(i, sw.idx)
    assert np.array_equal(sp, sw.s)
    assert vp.nbytes == spec.N * spec.K // 4 and mp.nbytes == spec.N * spec.K // 8


def test_pack_sparse24_per_column():
    """group_size -1: one scale row [1, N], copied as is; the values and
    metadata layout does not depend on the group size; other group sizes and
    wrongly shaped scales are rejected."""
    spec = gen.CFG4.with_(K=512, N=32, group_size=-1)
    sw = gen.make_sparse_weights(spec, seed_config=406)
    vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s, -1)
    assert sp.shape == (1, spec.N) and np.array_equal(sp, sw.s)
    vp2, mp2, _ = wq.pack_sparse24(sw.vals, sw.idx, np.ones((spec.K // 128, spec.N), np.uint16), 128)
    assert np.array_equal(vp, vp2) and np.array_equal(mp, mp2)
    with pytest.raises(ValueError):
        wq.pack_sparse24(sw.vals, sw.idx, sw.s, 128)
    L = wq.load()
    p = C.c_void_p(FAKE)
    assert L.wq_pack_sparse24(32, 512, 4, 64, p, p, p, p, p, p) == wq.WQ_ERR_UNSUPPORTED   # group size
    assert L.wq_pack_sparse24(32, 512, 6, 128, p, p, p, p, p, p) == wq.WQ_ERR_UNSUPPORTED  # bits
    assert L.wq_pack_sparse24_vals_bytes(32, 512, 8) == 2 * L.wq_pack_sparse24_vals_bytes(32, 512, 4)


def test_pack_sparse24_8bit_layout():
    """8-bit kept codes: lane l of 16-row tile t, chunk c holds 32 bytes, 8 per
    64-channel step, the step's 8 kept codes of row 16t + l%16 in natural order
    (two's complement); the metadata equals the 4-bit packing's."""
    spec = gen.CFG4.with_(K=512, N=32)
    sw = gen.make_sparse_weights(spec, seed_config=407)
    rng = np.random.default_rng(407)
    v8 = rng.integers(-128, 128, size=sw.vals.shape, dtype=np.int8)
    vp, mp, _ = wq.pack_sparse24(v8, sw.idx, sw.s, 128, bits=8)
    _, mp4, _ = wq.pack_sparse24(sw.vals, sw.idx, sw.s, 128, bits=4)
    assert np.array_equal(mp, mp4)
    assert vp.nbytes == spec.N * spec.K // 2
    C = spec.K // 256
    lanes = vp.view(np.int8).reshape(spec.N // 16, C, 64, 4, 8)      # [tile, chunk, lane, step, value]
    for t in range(spec.N // 16):
        for c in range(C):
            for l in range(64):
                n = 16 * t + (l & 15)
                for st in range(4):
                    first = (256 * c + 64 * st + 16 * (l >> 4)) // 2   # first kept index of the lane's 4 groups
                    assert np.array_equal(lanes[t, c, l, st], v8[n, first:first + 8])


def test_sparse24_metadata_roundtrip_all_patterns():
    """All 6 keep patterns x all 16 x 16 code pairs survive pack -> decode."""
    pairs = [(a, b) for a in range(4) for b in range(a + 1, 4)]
    combos = [(p, v0, v1) for p in pairs for v0 in range(-8, 8) for v1 in range(-8, 8)]   # 1536 groups
    K = 4 * 256
    N = 16 * ((len(combos) + K // 4 - 1) // (K // 4))
    vals = np.zeros((N, K // 2), np.int8)
    idx = np.tile(np.array([0, 1], np.uint8), (N, K // 4))
    flat_v = vals.reshape(-1, 2)
    flat_i = idx.reshape(-1, 2)
    for n, (p, v0, v1) in enumerate(combos):
        flat_v[n] = (v0, v1)
        flat_i[n] = p
    s = np.ones((K // 128, N), np.uint16)
    vp, mp, _ = wq.pack_sparse24(vals, idx, s)
    v2, i2 = decode_sparse24(vp, mp, N, K)
    assert np.array_equal(v2, vals) and np.array_equal(i2, idx)


def test_packer_rejects_bad_input():
    spec = gen.CFG3.with_(E=1, K=256, N=64, act_order=True)
    w = gen.make_moe_weights(spec, seed_config=404)
    bad = w.w1q.copy()
    bad[0, 0, 0] = 9
    with pytest.raises(wq.WqError):
        wq.pack_w4(bad, w.s1, 128)
    g = w.g1.copy()
    g[0, np.argmax(g[0] == 1)] = 0      # group 0 now has 129 members, group 1 has 127
    with pytest.raises(wq.WqError):
        wq.pack_w4(w.w1q, w.s1, 128, g_idx=g)
    idx = gen.make_sparse_weights(gen.CFG4.with_(K=256, N=16), seed_config=405).idx.copy()
    idx[0, 0], idx[0, 1] = 2, 1
    with pytest.raises(wq.WqError):
        wq.pack_sparse24(np.zeros((16, 128), np.int8), idx, np.ones((2, 16), np.uint16))


def test_pack_fp8_layout():
    """The FP8 packer: tiles of 16 rows x 128 channels (2 KiB); lane l's 32
    channels [32 (l / 16), +32) of row l % 16 in two halves, at 16 l and
    1024 + 16 l of the tile; gate/up interleave as for the int8 packer; float32
    scales in packed row order."""
    rng = np.random.default_rng(3)
    E, n_out, k_in = 2, 64, 256
    codes = rng.integers(0, 256, size=(E, n_out, k_in), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes
    scales = rng.uniform(0.5, 2.0, size=(E, n_out)).astype(np.float32)
    for il in (False, True):
        packed, sp = wq.pack_fp8(codes, scales, interleave_gate_up=il)
        C = k_in // 128
        t = packed.reshape(E, n_out // 16, C, 2, 64, 16)   # e, tile, chunk, half, lane, byte
        rows = logical_rows(n_out, il)
        for e in range(E):
            for p in range(n_out):
                lr = rows[p]
                assert sp[e, p] == scales[e, lr]
                got = np.empty(k_in, np.uint8)
                for l in range(64):
                    if l % 16 != p % 16:
                        continue
                    for c in range(C):
                        for h in range(2):
                            k0 = 128 * c + 32 * (l // 16) + 16 * h
                            got[k0:k0 + 16] = t[e, p // 16, c, h, l]
                assert np.array_equal(got, codes[e, lr]), (il, e, p)
    bad = codes.copy()
    bad[0, 0, 0] = 0x7F
    with pytest.raises(wq.WqError):
        wq.pack_fp8(bad, scales)


def test_fp8_gemm_validation():
    """moe_fp8_w8a8_gemm rejects bad scales, shapes and formats before any device work."""
    L = wq.load()
    assert L.moe_fp8_gemm_workspace_bytes(wq.WQ_STAGE_GATE_UP, 4, 2, 8, 1024, 256) == 1024  # x codes, 256-rounded
    assert L.moe_fp8_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, 4, 2, 8, 256, 512) == 4 * 2 * 256 * 4
    def st(**kw):
        scales = kw.pop("scales", (1 / 64, 1 / 16))
        kw.setdefault("group_size", -1)
        d = _desc(**kw)
        d.d_workspace, d.workspace_bytes = FAKE, 1 << 30
        return L.moe_fp8_w8a8_gemm(C.byref(d), scales[0], scales[1], None)
    assert st(k_in=192) == wq.WQ_ERR_UNSUPPORTED          # k_in % 128
    assert st(group_size=128) == wq.WQ_ERR_UNSUPPORTED
    assert st(d_k_perm=FAKE) == wq.WQ_ERR_INVALID
    assert st(scales=(0.0, 1.0)) == wq.WQ_ERR_INVALID      # in_scale must be > 0
    assert st(scales=(float("nan"), 1.0)) == wq.WQ_ERR_INVALID
    assert st(scales=(1.0, -1.0)) == wq.WQ_ERR_INVALID     # GATE_UP needs out_scale > 0
    assert st(n_out=1008) == wq.WQ_ERR_UNSUPPORTED         # gate/up n_out % 32
    assert st(d_a=None) == wq.WQ_ERR_INVALID
    assert st(M=0) == wq.WQ_OK
