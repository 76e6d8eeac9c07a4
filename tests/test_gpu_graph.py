"""The whole layer (route -> align -> gate/up -> down -> combine) captured as one
HIP graph: every replay equals the eager call bit for bit, with eager work and
synchronisations between the replays, and a replay after the inputs are
updated in place follows the new inputs.  Small-batch and large-batch kernels,
the one-launch routing paths, int8 per-column and int4 act-order weights, the
FP8 layer (one token: x quantised inside gate/up, the top-k sum inside DOWN),
the dense and 2:4 linear layers."""
import pytest

import gen
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, need_gpu, say, torch

pytestmark = pytest.mark.gpu

W8 = gen.CFG2.with_(name="w8-graph", E=8, topk=2, K=512, N=384)
W4AO = gen.CFG3.with_(name="w4ao-graph", E=8, topk=2, K=512, N=384)
F8 = gen.CFG_FP8.with_(name="fp8-graph", E=8, topk=2, K=512, N=384)
SPECS = {"w8": (W8, 520), "w4ao": (W4AO, 521), "fp8": (F8, 522)}
_packed = {}


def packed(key):
    if key not in _packed:
        spec, seed = SPECS[key]
        if key == "fp8":
            fw = gen.make_fp8_weights(spec, seed_config=seed)
            _packed[key] = (spec, wq.pack_moe_fp8(fw.w1, fw.s1, fw.w2, fw.s2, torch.bfloat16, spec.a1, spec.a2))
        else:
            wts = gen.make_moe_weights(spec, seed_config=seed)
            act = torch.float16 if spec.act == "f16" else torch.bfloat16
            _packed[key] = (spec, wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2, act, spec.group_size,
                                              wts.g1, wts.g2))
    return _packed[key]


def runner(key, p, M, spec):
    cls = wq.Fp8MoERunner if key == "fp8" else wq.MoERunner
    return cls(p, M, spec.topk, spec.renormalize)


def inputs(spec, M, seed):
    toks = gen.make_tokens(spec, M, seed_config=seed)
    return dev_u16(toks.x, spec.act), torch.from_numpy(toks.logits).cuda()


# one token (routing and sort inside the gate/up launch, the top-k sum inside DOWN), a few
# tokens, act-order with the routing launch gathering the rows (1 and 16 tokens), large batches
@pytest.mark.parametrize("key,M", [("w8", 1), ("w8", 5), ("w8", 300), ("w4ao", 1), ("w4ao", 16), ("w4ao", 40),
                                   ("w4ao", 600), ("fp8", 1), ("fp8", 300)])
def test_graph_replay_matches_eager(key, M):
    need_gpu()
    spec, p = packed(key)
    say("graph", key, M)
    x, lg = inputs(spec, M, 900 + M)
    eager = runner(key, p, M, spec)
    ref = eager(x, lg).clone()
    torch.cuda.synchronize()

    r = runner(key, p, M, spec)
    assert r.bs == eager.bs
    xs, ls = x.clone(), lg.clone()
    r.capture(xs, ls)
    for _ in range(3):
        out = r.replay().clone()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        eager(x, lg)  # eager work on the same stream between replays
        torch.cuda.synchronize()

    x2, lg2 = inputs(spec, M, 950 + M)
    ref2 = eager(x2, lg2).clone()
    xs.copy_(x2)
    ls.copy_(lg2)
    out2 = r.replay().clone()
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2)
    assert not torch.equal(ref2, ref)


def _graph_of(call):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    return g


def _check_replays(call, out, x, x2):
    """call() writes out from x; every replay of its graph equals the eager
    result bit for bit (eager work and synchronisations between the replays),
    and a replay after x is overwritten in place follows the new values."""
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _graph_of(call)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        call()  # eager work on the same buffers between replays
        torch.cuda.synchronize()
    x0 = x.clone()
    x.copy_(x2)
    call()
    torch.cuda.synchronize()
    ref2 = out.clone()
    x.copy_(x0)
    call()
    x.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    assert not torch.equal(ref2, ref)


@pytest.mark.parametrize("M", [1, 16, 64, 200])
def test_graph_replay_dense(M):
    """The dense int4 linear layer (one kernel up to 128 rows; identity
    routing, large-batch GEMM and combine above) as a graph."""
    need_gpu()
    import numpy as np
    spec = gen.CFG3.with_(name="w4-dense-graph", E=1, topk=1, K=512, N=192, act_order=False)
    wts = gen.make_moe_weights(spec, seed_config=530)
    packed_w, sp, _ = wq.pack_w4(wts.w1q, wts.s1, spec.group_size)
    wd, sd = torch.from_numpy(packed_w).cuda(), torch.from_numpy(sp.view(np.int16)).cuda()
    n_out, K = wts.w1q.shape[1], wts.w1q.shape[2]
    say("graph dense", M)
    x = dev_u16(gen.make_tokens(spec, M, seed_config=531).x, "f16")
    x2 = dev_u16(gen.make_tokens(spec, M, seed_config=532).x, "f16")
    y = torch.empty((M, n_out), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(1, wq.dense_gemm_workspace_bytes(M, K, n_out)), dtype=torch.uint8, device="cuda")
    _check_replays(lambda: wq.dense_w4a16_gemm(x, n_out, wd, sd, 128, out=y, workspace=ws), y, x, x2)


@pytest.mark.parametrize("M", [1, 16, 200])
def test_graph_replay_sparse24(M):
    """The 2:4-sparse int4 linear layer (decode, streaming and tile kernels) as a graph."""
    need_gpu()
    import numpy as np
    spec = gen.CFG4.with_(K=1024, N=256)
    sw = gen.make_sparse_weights(spec, seed_config=533)
    vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s)
    vd, md, sd = torch.from_numpy(vp).cuda(), torch.from_numpy(mp).cuda(), torch.from_numpy(sp.view(np.int16)).cuda()
    say("graph sparse", M)
    x = dev_u16(gen.make_sparse_x(spec, M, seed_config=534), "f16")
    x2 = dev_u16(gen.make_sparse_x(spec, M, seed_config=535), "f16")
    y = torch.empty((M, spec.N), dtype=torch.float16, device="cuda")
    _check_replays(lambda: wq.sparse24_w4a16_gemm(x, vd, md, sd, spec.N, out=y), y, x, x2)
