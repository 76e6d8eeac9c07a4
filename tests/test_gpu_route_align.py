"""GPU parity of moe_route and moe_align against the oracle: routing ids and
the whole padded sort are compared bit for bit; routing weights exactly, with
at most 1 ulp tolerated on a tiny fraction (the device and host exp in double
may differ in their last bit before the final rounding to float)."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import need_gpu, say, torch, ulp_diff_f32

pytestmark = pytest.mark.gpu


def route_check(logits: np.ndarray, topk: int, renorm: bool, what: str):
    say("route", what, logits.shape, topk, renorm)
    w_ref, ids_ref = oracle.route(logits, topk, renorm)
    w, ids = wq.moe_route(torch.from_numpy(logits).cuda(), topk, renorm)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    w = w.cpu().numpy()
    assert np.array_equal(ids, ids_ref), "%s: topk ids differ" % what
    ud = ulp_diff_f32(w, w_ref)
    n_bad = int((ud > 0).sum())
    if n_bad:
        say("  %s: %d of %d weights differ by 1 ulp" % (what, n_bad, w.size))
    assert ud.max() <= 1
    assert n_bad <= max(1, w.size // 10000)
    return ids


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_route_configs(cid):
    need_gpu()
    spec = gen.CONFIGS[cid]
    for M in spec.m_sweep:
        toks = gen.make_tokens(spec, M)
        route_check(toks.logits, spec.topk, spec.renormalize, "cfg%d M=%d" % (cid, M))


def test_route_edge_cases():
    need_gpu()
    rng = np.random.default_rng(7)
    route_check(np.zeros((5, 8), np.float32), 3, True, "all ties")
    route_check(np.ones((3, 1), np.float32), 1, True, "E=1")
    route_check(rng.standard_normal((33, 6)).astype(np.float32), 6, True, "topk=E")
    route_check(rng.standard_normal((70, 1024)).astype(np.float32), 16, True, "E=1024 topk=16")
    route_check(rng.standard_normal((70, 160)).astype(np.float32) * 4, 6, False, "no renorm")
    route_check(rng.integers(-2, 3, size=(200, 64)).astype(np.float32), 8, True, "many ties")
    route_check(rng.standard_normal((100003, 8)).astype(np.float32), 2, True, "large M")
    # the rank-counting top-k (E <= 64) at its edge and the arg-max rounds
    # above it, with ties
    for E, topk in ((64, 8), (65, 6), (100, 4), (128, 8), (129, 6), (192, 6), (193, 8), (256, 16), (257, 8)):
        for renorm in (True, False):
            lg = rng.standard_normal((37, E)).astype(np.float32)
            lg[:, ::7] = np.float32(0.25)  # tied logits across the lanes' slots
            route_check(lg, topk, renorm, "E=%d topk=%d" % (E, topk))
    # M = 0 launches nothing and succeeds
    wq.moe_route(torch.empty((0, 8), dtype=torch.float32, device="cuda"), 2)


def align_check(ids: np.ndarray, E: int, BS: int, what: str):
    say("align", what, ids.shape, E, BS)
    st_ref, ex_ref, nt_ref = oracle.align(ids, E, BS)
    st, ex, nt = wq.moe_align(torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(), E, BS)
    torch.cuda.synchronize()
    cap = st_ref.size
    assert int(nt.cpu()[0]) == nt_ref, what
    assert np.array_equal(st.cpu().numpy()[:cap], st_ref), "%s: sorted_token_ids differ" % what
    assert np.array_equal(ex.cpu().numpy()[:cap // BS], ex_ref), "%s: expert_ids differ" % what


@pytest.mark.parametrize("BS", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_align_configs(cid, BS):
    need_gpu()
    spec = gen.CONFIGS[cid]
    for M in spec.m_sweep:
        toks = gen.make_tokens(spec, M)
        _, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
        align_check(ids, spec.E, BS, "cfg%d M=%d" % (cid, M))


def test_align_edge_cases():
    need_gpu()
    rng = np.random.default_rng(11)
    align_check(np.zeros((4096, 6), np.int32), 160, 16, "all pairs to expert 0")
    align_check(np.full((777, 1), 159, np.int32), 160, 128, "all pairs to the last expert")
    align_check(np.arange(160, dtype=np.int32).reshape(80, 2), 160, 256, "one pair per expert")
    align_check(np.array([[3, 1]], np.int32), 8, 16, "M=1")
    align_check(rng.integers(0, 1024, size=(5000, 3)).astype(np.int32), 1024, 16, "E=1024")
    align_check(rng.integers(0, 7, size=(1031, 1)).astype(np.int32), 7, 32, "ragged chunk")
    align_check(rng.integers(0, 2, size=(100000, 2)).astype(np.int32), 2, 64, "E=2 many pairs")
    # M = 0: no pairs, all-sentinel output
    st, ex, nt = wq.moe_align(torch.empty((0, 2), dtype=torch.int32, device="cuda"), 8, 16, capacity=64)
    torch.cuda.synchronize()
    assert int(nt.cpu()[0]) == 0
    assert (st.cpu().numpy()[:64] == 0).all() and (ex.cpu().numpy()[:4] == -1).all()


def test_align_deterministic():
    need_gpu()
    rng = np.random.default_rng(12)
    ids = torch.from_numpy(rng.integers(0, 160, size=(4096, 6)).astype(np.int32)).cuda()
    a = [t.clone() for t in wq.moe_align(ids, 160, 16)]
    b = wq.moe_align(ids, 160, 16)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("M,E,topk", [(1, 8, 2), (7, 8, 2), (16, 160, 6), (17, 160, 6), (64, 8, 2), (300, 160, 6),
                                      (12, 1024, 8), (33, 1024, 8), (16, 2, 2),
                                      # single-wave sort: up to 64 pairs over up to 64 experts
                                      (1, 1, 1), (16, 64, 4), (11, 33, 5), (3, 4, 4), (16, 8, 2), (8, 65, 8),
                                      # more logits per lane, ties
                                      (64, 160, 6), (48, 256, 8), (40, 192, 6), (20, 129, 3)])
@pytest.mark.parametrize("bs", [16, 64, 128, 256])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_align_fused_equals_two_calls(M, E, topk, bs, renorm):
    """moe_route_align (one kernel up to 16 tokens -- one wave sorting the
    pairs when there are at most 64 of them over at most 64 experts -- two
    above) gives exactly the outputs of moe_route followed by moe_align."""
    need_gpu()
    rng = np.random.default_rng(1000 + M + E + bs)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    logits[:, : E // 2] += np.float32(0.5)  # skew: some experts get many tokens
    lg = torch.from_numpy(logits).cuda()
    say("route_align", M, E, topk, bs, renorm)
    w1, i1 = wq.moe_route(lg, topk, renorm)
    cap = wq.moe_align_capacity(M, topk, E, bs)
    st1, ex1, nt1 = wq.moe_align(i1, E, bs, cap)
    w2 = torch.full((M, topk), -1.0, dtype=torch.float32, device="cuda")
    i2 = torch.full((M, topk), -7, dtype=torch.int32, device="cuda")
    st2 = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    ex2 = torch.full((cap // bs,), -7, dtype=torch.int32, device="cuda")
    nt2 = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    wq.moe_route_align(lg, topk, renorm, bs, w2, i2, st2, ex2, nt2, cap)
    torch.cuda.synchronize()
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(i1, i2)
    assert int(nt1[0]) == int(nt2[0])
    assert torch.equal(st1[:cap], st2)
    assert torch.equal(ex1[: cap // bs], ex2)
