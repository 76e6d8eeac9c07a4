"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (block size chosen by the batch-size heuristic).  Routing and
the padded sort are compared bit for bit over the whole batch; the layer
output on sampled rows, which the oracle computes one by one."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, host_f32, need_gpu, say, torch, ulp_diff_f32
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu

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


def sample_rows(M, n=6, seed=0):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n - 2, replace=False)]))


CASES = [(cid, M) for cid in (1, 2, 3, 5) for M in gen.CONFIGS[cid].m_sweep]


@pytest.mark.parametrize("cid,M", CASES)
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
    assert ulp_diff_f32(aux["topk_weights"].cpu().numpy(), w_ref).max() <= 1
    bs = aux["block_size"]
    st_ref, ex_ref, nt_ref = oracle.align(ids_ref, spec.E, bs)
    assert int(aux["num_tokens_post_padded"].cpu()[0]) == nt_ref
    assert np.array_equal(aux["sorted_token_ids"].cpu().numpy()[:st_ref.size], st_ref)
    assert np.array_equal(aux["expert_ids"].cpu().numpy()[:ex_ref.size], ex_ref)
    rows = sample_rows(M, seed=cid * 100 + M)
    ref = oracle.moe_layer_from_weights(wts, toks.x_f32(), aux["topk_weights"].cpu().numpy(), ids_ref,
                                        rows=rows)["out"]
    assert_close_fp(host_f32(out)[rows], ref, "cfg%d M=%d (rows %s)" % (cid, M, rows.tolist()))


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
    rows = sample_rows(M, n=4, seed=400 + M)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128, rows=rows)
    assert_close_fp(host_f32(y)[rows], ref, "cfg4 M=%d" % M)
