"""GPU parity of the grouped GEMM for batches of at most 4 tokens (the kernel
that stages a block's token rows in LDS): the DOWN stage with a long reduction
(64 or more 1 KiB chunks per weight tile) in 4, 2 or 1 K slices, int4 group-128,
int4 per-column and int8 weights; the int4 RAW stage of one token, with and
without act-order (the permutation applied while staging); the int4 GATE_UP
stage of one token (which runs the small-batch kernel after the gather); and
a token's top-k naming one expert more than once (more rows than the LDS
holds, and more than one block per expert); one token's DOWN with the top-k
sum folded in (top-k 1 to 4, block sizes 16 and 256, one expert named twice),
against the oracle.  Float comparisons:
relative Frobenius error <= 5e-3 and max abs error <= 3e-2 * max |ref|; the
RAW stage on exact-integer inputs bit for bit."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import act_round, dev_u16, host_f32, need_gpu, say, torch
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu

W4 = gen.CFG3.with_(name="w4-tiny", E=8, topk=2, K=256, N=8192, act_order=False)
W4AO = W4.with_(name="w4ao-tiny", act_order=True)
W4PC = W4.with_(name="w4pc-tiny", group_size=-1)
W8 = gen.CFG2.with_(name="w8-tiny", E=8, topk=2, K=256, N=4096)
W8_65 = W8.with_(name="w8-tiny-65", N=4160)    # 65 chunks: one K slice
W8_66 = W8.with_(name="w8-tiny-66", N=4224)    # 66 chunks: two K slices
W8T6 = W8.with_(name="w8-tiny-top6", topk=6)
# gate/up of one int4 token: a Mixtral-like hidden size
W4G = gen.CFG3.with_(name="w4-tiny-gu", E=8, topk=2, K=4096, N=256, act_order=False)
W4GAO = W4G.with_(name="w4ao-tiny-gu", act_order=True)
W4GPC = W4G.with_(name="w4pc-tiny-gu", group_size=-1)
SPECS = {"w4": W4, "w4ao": W4AO, "w4pc": W4PC, "w8": W8, "w8_65": W8_65, "w8_66": W8_66, "w8t6": W8T6,
         "w4g": W4G, "w4gao": W4GAO, "w4gpc": W4GPC}
_cache = {}


def setup(key):
    if key not in _cache:
        spec = SPECS[key]
        wts = gen.make_moe_weights(spec, seed_config=1100 + sorted(SPECS).index(key))
        p = wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2,
                        torch.float16 if spec.act == "f16" else torch.bfloat16, spec.group_size, wts.g1, wts.g2)
        _cache[key] = (spec, wts, p)
    return _cache[key]


def h_perm(spec, wts, e):
    if spec.bits == 4 and wts.g2 is not None:
        return np.argsort(wts.g2[e], kind="stable")
    return np.arange(spec.N)


def align_dev(ids, E, bs):
    cap = wq.moe_align_capacity(ids.shape[0], ids.shape[1], E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids).cuda(), E, bs, cap)
    return st, ex, nt, cap


def check_down(spec, wts, p, ids, w, bs, tag):
    M = ids.shape[0]
    T = M * spec.topk
    rng = np.random.default_rng(1200 + M)
    h_act = act_round(rng.standard_normal((T, spec.N)), spec.act)
    y_ref = oracle.moe_down(h_act, ids, wts.w2q, wts.s2_f32(), wts.g2)
    out_ref = oracle.moe_combine(y_ref, w)
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    stn, exn, ntn = st.cpu().numpy(), ex.cpu().numpy(), int(nt.cpu()[0])
    hs = np.zeros((cap, spec.N), np.float32)
    for pos in range(ntn):
        i = stn[pos]
        if i < T:
            hs[pos] = h_act[i][h_perm(spec, wts, exn[pos // bs])]
    hd = torch.from_numpy(hs).cuda().to(p.act)
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, M, spec.topk, spec.E, spec.K, spec.N, cap, False)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((M, spec.K), dtype=p.act, device="cuda")
    wd = torch.from_numpy(w).cuda()
    say("tiny down", tag)
    if spec.bits == 4:
        wq.moe_w4a16_gemm(wq.WQ_STAGE_DOWN, hd, M, spec.topk, spec.E, spec.K, spec.N, p.w2, p.s2, spec.group_size,
                          None, st, ex, nt, cap, bs, wd, out, work)
    else:
        wq.moe_w8a16_gemm(wq.WQ_STAGE_DOWN, hd, M, spec.topk, spec.E, spec.K, spec.N, p.w2, p.s2, st, ex, nt, cap,
                          bs, wd, out, work, act_dtype=p.act_code)
    torch.cuda.synchronize()
    assert_close_fp(host_f32(out), out_ref, "tiny DOWN %s" % tag)
    return ws


@pytest.mark.parametrize("key", ["w4", "w4ao", "w4pc", "w8", "w8_65", "w8_66"])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_down(key, M):
    need_gpu()
    spec, wts, p = setup(key)
    toks = gen.make_tokens(spec, M, seed_config=1150 + M)
    w, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
    ws = check_down(spec, wts, p, ids, w, 16, "%s M=%d" % (key, M))
    if key == "w8":
        # 64 chunks: four K slices of 16, so the workspace holds 4 fp32 slabs
        assert ws >= 4 * M * spec.topk * spec.K * 4


@pytest.mark.parametrize("bs", [16, 32, 128])
def test_down_repeated_expert(bs):
    """Top-6 of 4 tokens all naming expert 2 (24 rows: more than the 4 rows
    the LDS holds and, in blocks of 16, two blocks), plus expert 5 twice in one
    token."""
    need_gpu()
    spec, wts, p = setup("w8t6")
    ids = np.full((4, 6), 2, np.int32)
    ids[1, 3:5] = 5
    w = np.random.default_rng(1160).uniform(0.1, 1.0, ids.shape).astype(np.float32)
    check_down(spec, wts, p, ids, w, bs, "repeated expert bs=%d" % bs)


# one token with the top-k sum folded into DOWN: every compiled top-k (1-4),
# int8 and int4 group-128, block sizes up to 256
TOPK_SPECS = {"w8t1": W8.with_(name="w8-tiny-top1", topk=1), "w8t3": W8.with_(name="w8-tiny-top3", topk=3),
              "w8t4": W8.with_(name="w8-tiny-top4", topk=4), "w4t3": W4.with_(name="w4-tiny-top3", topk=3),
              "w4t4": W4PC.with_(name="w4pc-tiny-top4", topk=4)}


@pytest.mark.parametrize("key", sorted(TOPK_SPECS))
@pytest.mark.parametrize("bs", [16, 256])
def test_down_one_token_topk(key, bs):
    need_gpu()
    if key not in _cache:
        spec = TOPK_SPECS[key]
        wts = gen.make_moe_weights(spec, seed_config=1180 + sorted(TOPK_SPECS).index(key))
        _cache[key] = (spec, wts, wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2,
                                              torch.float16 if spec.act == "f16" else torch.bfloat16,
                                              spec.group_size, wts.g1, wts.g2))
    spec, wts, p = _cache[key]
    toks = gen.make_tokens(spec, 1, seed_config=1190 + bs)
    w, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
    check_down(spec, wts, p, ids, w, bs, "%s one token bs=%d" % (key, bs))


def test_down_one_token_same_expert_twice():
    """One token whose two slots name the same expert (two rows of one block)."""
    need_gpu()
    spec, wts, p = setup("w8")
    ids = np.array([[5, 5]], np.int32)
    w = np.array([[0.625, 0.375]], np.float32)
    check_down(spec, wts, p, ids, w, 16, "one token, expert 5 twice")


def run_gate_up(spec, p, xd, ids, bs):
    M = xd.shape[0]
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    act_order = p.k_perm1 is not None
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_GATE_UP, M, spec.topk, spec.E, 2 * spec.N, spec.K, cap, act_order)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    h = torch.full((cap, spec.N), float("nan"), dtype=p.act, device="cuda")
    wq.moe_w4a16_gemm(wq.WQ_STAGE_GATE_UP, xd, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1,
                      spec.group_size, p.k_perm1, st, ex, nt, cap, bs, None, h, work)
    torch.cuda.synchronize()
    return h, st, ex, nt


def check_gate_up(spec, wts, p, x, ids, bs, tag):
    h, st, ex, nt = run_gate_up(spec, p, dev_u16(gen.round_to(spec.act, x), spec.act), ids, bs)
    _, h_ref = oracle.moe_up(x, ids, wts.w1q, wts.s1_f32(), wts.g1)
    hg = host_f32(h)
    stn, exn, ntn = st.cpu().numpy(), ex.cpu().numpy(), int(nt.cpu()[0])
    T = ids.size
    got = np.empty((T, spec.N))
    for pos in range(ntn):
        i = stn[pos]
        if i < T:
            got[i, h_perm(spec, wts, exn[pos // bs])] = hg[pos]
        else:
            assert (hg[pos] == 0).all(), "pad row %d of H is not zero" % pos
    assert_close_fp(got, h_ref, "tiny H %s" % tag)


@pytest.mark.parametrize("key", ["w4g", "w4gao", "w4gpc"])
@pytest.mark.parametrize("bs", [16, 64])
def test_gate_up_one_token(key, bs):
    need_gpu()
    spec, wts, p = setup(key)
    toks = gen.make_tokens(spec, 1, seed_config=1170 + bs)
    _, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
    say("tiny gate_up", key, bs)
    check_gate_up(spec, wts, p, toks.x_f32(), ids, bs, "%s bs=%d" % (key, bs))


@pytest.mark.parametrize("key", ["w4g", "w4gao"])
def test_gate_up_one_token_repeated_expert(key):
    """One token whose top-2 names expert 3 twice: two rows of one expert."""
    need_gpu()
    spec, wts, p = setup(key)
    toks = gen.make_tokens(spec, 1, seed_config=1180)
    ids = np.array([[3, 3]], np.int32)
    say("tiny gate_up repeated", key)
    check_gate_up(spec, wts, p, toks.x_f32(), ids, 16, "%s repeated expert" % key)


@pytest.mark.parametrize("pair", [(6, 1), (3, 3)])
@pytest.mark.parametrize("act_order", [False, True])
def test_raw_exact_integer_one_token(act_order, pair):
    """Power-of-two group scales and x in {-1, 0, 1}: the RAW projection of
    one token is bit-exact (every partial sum is a dyadic number below 2^24);
    with expert 3 named twice, two rows for a one-row LDS, multiplied in two
    passes."""
    need_gpu()
    spec = W4GAO if act_order else W4G
    wts = gen.make_moe_weights(spec, seed_config=1190)
    E, n_out, K = wts.w1q.shape
    rng = np.random.default_rng(1191)
    G = wts.s1.shape[1]
    pow2 = np.array([0.25, 0.5, 1.0, 2.0], np.float32)[rng.integers(0, 4, size=(E, G, n_out))]
    s_bits = gen.round_to(spec.act, pow2)
    x = rng.integers(-1, 2, size=(1, K)).astype(np.float32)
    ids = np.array([pair], np.int32)
    ref, _ = oracle.moe_up(x, ids, wts.w1q, pow2, wts.g1, want_gu=True)
    packed, sp, kp = wq.pack_w4(wts.w1q, s_bits, spec.group_size, g_idx=wts.g1)
    st, ex, nt, cap = align_dev(ids, E, 16)
    out = torch.empty((2, n_out), dtype=torch.float32, device="cuda")
    kpd = torch.from_numpy(kp).cuda() if kp is not None else None
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_RAW, 1, 2, E, n_out, K, cap, kp is not None)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    say("tiny raw exact", act_order, pair)
    wq.moe_w4a16_gemm(wq.WQ_STAGE_RAW, dev_u16(gen.round_to(spec.act, x), spec.act), 1, 2, E, n_out, K,
                      torch.from_numpy(packed).cuda(), torch.from_numpy(sp.view(np.int16)).cuda(), spec.group_size,
                      kpd, st, ex, nt, cap, 16, None, out, work)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), "max diff %g" % np.abs(got - ref).max()
