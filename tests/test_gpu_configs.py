"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (block size chosen by the batch-size heuristic).  Routing and
the padded sort are compared bit for bit over the whole batch (routing weights
exactly, with at most one weight in 10^4 allowed one ulp: the device and host
double exp may differ in their last bit).  The layer output is compared over
the whole tensor wherever the oracle takes about a minute or less (the tiny
layer, every Mixtral int8 batch up to 1024 tokens, the act-order int4 layer
up to 256 tokens, the DeepSeek-V2-shaped layer at 64 tokens); at 4096 tokens
over a contiguous run of 128 tokens plus every token that has a pair in some
expert's last, partly filled token tile (the ragged edge of each expert's
rows), plus the first and last token.  The benchmark's other rows at the 2:4
layer's shape -- 8-bit kept codes and the dense int4 linear layer -- likewise:
whole tensor up to 128 tokens, at 1024 tokens the first, last and one seeded
run of 128 rows."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, host_f32, need_gpu, say, torch, ulp_diff_f32
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu

# largest batch compared over the whole output tensor, per workload
FULL_MAX = {1: 16, 2: 1024, 3: 256, 5: 64}
RUN = 128  # contiguous run of tokens compared in the sampled cases

_cache = {}


def packed_config(cid):
    if cid not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        spec = gen.CONFIGS[cid]
        say("generating and packing config", cid, spec.name)
        wts = gen.make_moe_weights(spec)
        p = wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2,
                        torch.float16 if spec.act == "f16" else torch.bfloat16, spec.group_size, wts.g1, wts.g2)
        _cache[cid] = (spec, wts, p)
    return _cache[cid]


def run_rows(M, seed, run=RUN):
    """First and last row plus one contiguous run of `run` rows at a seeded offset."""
    if M <= run:
        return np.arange(M)
    r0 = int(np.random.default_rng(seed).integers(1, M - run))
    return np.unique(np.concatenate([[0, M - 1], np.arange(r0, r0 + run)]))


def ragged_tile_tokens(st, ex, nt, T, topk, bs):
    """Tokens with a pair in the last token tile of an expert when that tile is
    only partly filled.  Tiles are the kernels' row tiles: 16 rows for the
    small-batch kernel (block 16 / 32), else min(block, 128)."""
    tile = 16 if bs < 64 else min(bs, 128)
    toks = set()
    for b0 in range(0, nt, bs):
        e = ex[b0 // bs]
        if b0 + bs < nt and ex[(b0 + bs) // bs] == e:
            continue  # not the expert's last block
        valid = np.nonzero(st[b0:b0 + bs] < T)[0]
        if valid.size == 0:
            continue
        last = b0 + int(valid[-1])
        t0 = last - (last - b0) % tile
        if last - t0 + 1 < tile:
            toks.update((st[t0:last + 1] // topk).tolist())
    return toks


CASES = [(cid, M) for cid in (1, 2, 3, 5) for M in gen.CONFIGS[cid].m_sweep]


@pytest.mark.parametrize("cid,M", CASES)
@pytest.mark.timeout(900)
def test_config_layer(cid, M):
    need_gpu()
    spec, wts, p = packed_config(cid)
    toks = gen.make_tokens(spec, M)
    say("config", cid, "M", M)
    out, aux = wq.fused_moe(dev_u16(toks.x, spec.act), torch.from_numpy(toks.logits).cuda(), p, spec.topk,
                            spec.renormalize, keep=True)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.route(toks.logits, spec.topk, spec.renormalize)
    assert np.array_equal(aux["topk_ids"].cpu().numpy(), ids_ref)
    w_got = aux["topk_weights"].cpu().numpy()
    ud = ulp_diff_f32(w_got, w_ref)
    assert ud.max() <= 1
    assert int((ud > 0).sum()) <= max(1, w_ref.size // 10000), "%d routing weights differ" % int((ud > 0).sum())
    bs = aux["block_size"]
    st_ref, ex_ref, nt_ref = oracle.align(ids_ref, spec.E, bs)
    assert int(aux["num_tokens_post_padded"].cpu()[0]) == nt_ref
    assert np.array_equal(aux["sorted_token_ids"].cpu().numpy()[:st_ref.size], st_ref)
    assert np.array_equal(aux["expert_ids"].cpu().numpy()[:ex_ref.size], ex_ref)
    if M <= FULL_MAX[cid]:
        rows = np.arange(M)
    else:
        ragged = ragged_tile_tokens(st_ref, ex_ref, nt_ref, M * spec.topk, spec.topk, bs)
        rows = np.unique(np.concatenate([run_rows(M, seed=cid * 100 + M), np.array(sorted(ragged), np.int64)]))
    say("  oracle over %d of %d tokens" % (rows.size, M))
    ref = oracle.moe_layer_from_weights(wts, toks.x_f32(), w_got, ids_ref, rows=rows)["out"]
    what = "cfg%d M=%d (%s)" % (cid, M, "all tokens" if rows.size == M else "%d tokens" % rows.size)
    assert_close_fp(host_f32(out)[rows], ref, what)


_sparse = {}


@pytest.mark.parametrize("M", gen.CFG4.m_sweep)
def test_config_sparse24(M):
    need_gpu()
    spec = gen.CFG4
    if "w" not in _sparse:
        _cache.clear()
        torch.cuda.empty_cache()
        say("generating and packing config 4")
        sw = gen.make_sparse_weights(spec)
        vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s)
        _sparse["w"] = (sw, torch.from_numpy(vp).cuda(), torch.from_numpy(mp).cuda(),
                        torch.from_numpy(sp.view(np.int16)).cuda())
    sw, vd, md, sd = _sparse["w"]
    x = gen.make_sparse_x(spec, M)
    say("config 4 M", M)
    y = wq.sparse24_w4a16_gemm(dev_u16(x, "f16"), vd, md, sd, spec.N)
    torch.cuda.synchronize()
    rows = run_rows(M, seed=400 + M)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128, rows=rows)
    assert_close_fp(host_f32(y)[rows], ref, "cfg4 M=%d" % M)


@pytest.mark.parametrize("M", gen.CFG4.m_sweep)
def test_config_sparse24_8bit(M):
    """The 2:4 layer of the Yi-34B MLP shape with 8-bit kept codes (the 2:4
    support's 8-bit variant), at the benchmark's batch sizes."""
    need_gpu()
    spec = gen.CFG4.with_(bits=8)
    if "w8" not in _sparse:
        _sparse.clear()
        _cache.clear()
        torch.cuda.empty_cache()
        say("generating and packing config 4, 8-bit codes")
        sw = gen.make_sparse_weights(spec)
        vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s, bits=8)
        _sparse["w8"] = (sw, torch.from_numpy(vp).cuda(), torch.from_numpy(mp).cuda(),
                         torch.from_numpy(sp.view(np.int16)).cuda())
    sw, vd, md, sd = _sparse["w8"]
    x = gen.make_sparse_x(spec, M)
    say("config 4 8-bit M", M)
    y = wq.sparse24_w8a16_gemm(dev_u16(x, "f16"), vd, md, sd, spec.N)
    torch.cuda.synchronize()
    rows = run_rows(M, seed=450 + M)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128, rows=rows)
    assert_close_fp(host_f32(y)[rows], ref, "cfg4 8-bit M=%d" % M)


_dense = {}


@pytest.mark.parametrize("M", gen.CFG4.m_sweep)
def test_config_dense_w4(M):
    """The dense int4 linear layer of the same shape (K = 7168 -> 20480, group
    128), the 2:4 layer's dense counterpart, at the benchmark's batch sizes:
    every regime of its dispatch, against the oracle."""
    need_gpu()
    spec = gen.CFG3.with_(name="yi34b-dense-w4", E=1, topk=1, K=gen.CFG4.K, N=gen.CFG4.N // 2, act_order=False)
    if "w" not in _dense:
        _sparse.clear()
        _cache.clear()
        torch.cuda.empty_cache()
        say("generating and packing the dense int4 layer")
        wts = gen.make_moe_weights(spec, seed_config=460)
        packed, sp, _ = wq.pack_w4(wts.w1q, wts.s1, spec.group_size)
        _dense["w"] = (wts, torch.from_numpy(packed).cuda(), torch.from_numpy(sp.view(np.int16)).cuda())
    wts, wd, sd = _dense["w"]
    n_out = wts.w1q.shape[1]
    toks = gen.make_tokens(spec, M, seed_config=461)
    say("dense int4 M", M)
    y = wq.dense_w4a16_gemm(dev_u16(toks.x, spec.act), n_out, wd, sd, spec.group_size)
    torch.cuda.synchronize()
    rows = run_rows(M, seed=470 + M)
    ref, _ = oracle.moe_up(toks.x_f32()[rows], np.zeros((rows.size, 1), np.int32), wts.w1q, wts.s1_f32(), None,
                           want_gu=True)
    assert_close_fp(host_f32(y)[rows], ref, "dense int4 Yi-34B shape M=%d" % M)


_fp8 = {}


@pytest.mark.parametrize("M", gen.CFG_FP8.m_sweep)
@pytest.mark.timeout(900)
def test_config_fp8(M):
    """The FP8 W8A8 layer of the Mixtral-8x7B shape (the comparison method of
    the ExpertsInt8 latency table) at the benchmark's batch sizes: routing and
    sort bit for bit, the whole output tensor against the oracle."""
    need_gpu()
    spec = gen.CFG_FP8
    if "p" not in _fp8:
        _cache.clear()
        _sparse.clear()
        _dense.clear()
        torch.cuda.empty_cache()
        say("generating and packing the FP8 layer")
        wts = gen.make_fp8_weights(spec)
        _fp8["p"] = (wts, wq.pack_moe_fp8(wts.w1, wts.s1, wts.w2, wts.s2, torch.bfloat16, spec.a1, spec.a2))
    wts, p = _fp8["p"]
    toks = gen.make_tokens(spec, M)
    say("fp8 config M", M)
    out, aux = wq.fused_moe_fp8(dev_u16(toks.x, spec.act), torch.from_numpy(toks.logits).cuda(), p, spec.topk,
                                spec.renormalize, keep=True)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.route(toks.logits, spec.topk, spec.renormalize)
    assert np.array_equal(aux["topk_ids"].cpu().numpy(), ids_ref)
    w_got = aux["topk_weights"].cpu().numpy()
    ud = ulp_diff_f32(w_got, w_ref)
    assert ud.max() <= 1 and int((ud > 0).sum()) <= max(1, w_ref.size // 10000)
    bs = aux["block_size"]
    st_ref, ex_ref, nt_ref = oracle.align(ids_ref, spec.E, bs)
    assert int(aux["num_tokens_post_padded"].cpu()[0]) == nt_ref
    assert np.array_equal(aux["sorted_token_ids"].cpu().numpy()[:st_ref.size], st_ref)
    ref = oracle.fp8_moe_layer(toks.x_f32(), w_got, ids_ref, wts.w1, wts.s1, wts.w2, wts.s2, spec.a1, spec.a2)["out"]
    assert_close_fp(host_f32(out), ref, "fp8 Mixtral M=%d (all tokens)" % M)
