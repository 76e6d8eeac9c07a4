"""GPU parity of the dense single-expert W4A16 / W8A16 linear layer
(dense_w4a16_gemm, dense_w8a16_gemm) against the oracle's projection with one
expert and top-1: every batch regime of the dispatch (the single-kernel paths
for 1..2 rows staged whole and for 3..128 rows staged per K chunk in token
groups of 16, 32 or 64 rows -- each size, its boundaries and a second group --
the grouped small-batch kernel with act-order, 64-row tiles up to 192, 128-row
tiles above, with a K split for a long K and few outputs), int8
per-column, int4 group-128, per-column and act-order weights, and output
counts that leave the last 8-tile workgroup partial.  Relative
Frobenius error <= 5e-3 and max abs error <= 3e-2 * max |ref|."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, host_f32, need_gpu, say, torch
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu

# one expert; the dense weight is the generator's w1 (n_out = 2N rows)
W8 = gen.CFG2.with_(name="w8-dense", E=1, topk=1, K=512, N=192)
W4 = gen.CFG3.with_(name="w4-dense", E=1, topk=1, K=512, N=192, act_order=False)
W4AO = W4.with_(name="w4ao-dense", act_order=True)
W4PC = W4.with_(name="w4pc-dense", group_size=-1)
W8LK = W8.with_(name="w8-dense-longk", K=4096, N=128)
# 400 outputs = 25 row tiles: the 8-tile workgroups of 5..16 rows end on a
# partial group
W8RAG = W8.with_(name="w8-dense-ragged", N=200)
W4RAG = W4.with_(name="w4-dense-ragged", N=200)
SPECS = {"w8": W8, "w4": W4, "w4ao": W4AO, "w4pc": W4PC, "w8lk": W8LK, "w8rag": W8RAG, "w4rag": W4RAG}
_cache = {}


def setup(key):
    if key not in _cache:
        spec = SPECS[key]
        wts = gen.make_moe_weights(spec, seed_config=640 + len(_cache))
        if spec.bits == 4:
            packed, sp, kp = wq.pack_w4(wts.w1q, wts.s1, spec.group_size, wts.g1)
        else:
            packed, sp = wq.pack_w8(wts.w1q, wts.s1)
            kp = None
        dev = (torch.from_numpy(packed).cuda(), torch.from_numpy(sp.view(np.int16)).cuda(),
               None if kp is None else torch.from_numpy(kp).cuda())
        _cache[key] = (spec, wts, dev)
    return _cache[key]


@pytest.mark.parametrize("key", ["w8", "w4", "w4ao", "w4pc", "w8rag", "w4rag"])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 13, 16, 17, 32, 33, 40, 64, 65, 128, 129, 150, 300])
def test_dense_matches_oracle(key, M):
    need_gpu()
    spec, wts, (wd, sd, kd) = setup(key)
    n_out, K = wts.w1q.shape[1], wts.w1q.shape[2]
    toks = gen.make_tokens(spec, M, seed_config=650 + M)
    x = dev_u16(toks.x, spec.act)
    say("dense", key, M)
    if spec.bits == 4:
        y = wq.dense_w4a16_gemm(x, n_out, wd, sd, spec.group_size, k_perm=kd)
    else:
        y = wq.dense_w8a16_gemm(x, n_out, wd, sd)
    torch.cuda.synchronize()
    ids = np.zeros((M, 1), np.int32)
    ref, _ = oracle.moe_up(toks.x_f32(), ids, wts.w1q, wts.s1_f32(), wts.g1, want_gu=True)
    assert_close_fp(host_f32(y), ref, "dense %s M=%d" % (key, M))


def test_dense_long_k_split():
    """K = 4096 with 256 outputs at M = 300: the large-batch DOWN kernel splits
    K into slices whose fp32 partial sums the combine adds."""
    need_gpu()
    spec, wts, (wd, sd, _) = setup("w8lk")
    n_out, K = wts.w1q.shape[1], wts.w1q.shape[2]
    M = 300
    assert wq.dense_gemm_workspace_bytes(M, K, n_out) >= 2 * M * n_out * 4
    toks = gen.make_tokens(spec, M, seed_config=660)
    say("dense long-k")
    y = wq.dense_w8a16_gemm(dev_u16(toks.x, spec.act), n_out, wd, sd)
    torch.cuda.synchronize()
    ref, _ = oracle.moe_up(toks.x_f32(), np.zeros((M, 1), np.int32), wts.w1q, wts.s1_f32(), None, want_gu=True)
    assert_close_fp(host_f32(y), ref, "dense long-k M=%d" % M)


@pytest.mark.parametrize("bits", [4, 8])
def test_dense_rows_too_long_for_lds(bits):
    """2 rows of K = 32768 do not fit the LDS whole, so the kernel that stages
    the tokens of one K chunk at a time runs (still one kernel, no workspace)."""
    need_gpu()
    base = W4 if bits == 4 else W8
    spec = base.with_(name="dense-longrow-%d" % bits, K=32768, N=64)
    wts = gen.make_moe_weights(spec, seed_config=680 + bits)
    if bits == 4:
        packed, sp, _ = wq.pack_w4(wts.w1q, wts.s1, spec.group_size)
    else:
        packed, sp = wq.pack_w8(wts.w1q, wts.s1)
    wd, sd = torch.from_numpy(packed).cuda(), torch.from_numpy(sp.view(np.int16)).cuda()
    n_out = wts.w1q.shape[1]
    M = 2
    assert wq.dense_gemm_workspace_bytes(M, spec.K, n_out) == 0
    toks = gen.make_tokens(spec, M, seed_config=681)
    x = dev_u16(toks.x, spec.act)
    y = wq.dense_w4a16_gemm(x, n_out, wd, sd, spec.group_size) if bits == 4 else wq.dense_w8a16_gemm(x, n_out, wd, sd)
    torch.cuda.synchronize()
    ref, _ = oracle.moe_up(toks.x_f32(), np.zeros((M, 1), np.int32), wts.w1q, wts.s1_f32(), None, want_gu=True)
    assert_close_fp(host_f32(y), ref, "dense long rows %d-bit" % bits)


def test_dense_equals_moe_raw_bits():
    """The dense call and the MoE RAW stage (one expert, top-1, the same block
    size) run the same multiply-adds in the same order: identical fp32 sums, so
    the dense result is the RAW result rounded once."""
    need_gpu()
    spec, wts, (wd, sd, _) = setup("w8")
    n_out, K = wts.w1q.shape[1], wts.w1q.shape[2]
    M = 150  # the grouped large-batch kernel, blocks of 64, one K slice (up to 128 rows a kernel of its own runs)
    toks = gen.make_tokens(spec, M, seed_config=670)
    x = dev_u16(toks.x, spec.act)
    y = wq.dense_w8a16_gemm(x, n_out, wd, sd)
    ids = torch.zeros((M, 1), dtype=torch.int32, device="cuda")
    cap = wq.moe_align_capacity(M, 1, 1, 64)
    st, ex, nt = wq.moe_align(ids, 1, 64, cap)
    raw = torch.empty((M, n_out), dtype=torch.float32, device="cuda")
    wq.moe_w8a16_gemm(wq.WQ_STAGE_RAW, x, M, 1, 1, n_out, K, wd, sd, st, ex, nt, cap, 64, None, raw,
                      act_dtype=wq.WQ_BF16)
    torch.cuda.synchronize()
    assert torch.equal(y, raw.to(torch.bfloat16))
