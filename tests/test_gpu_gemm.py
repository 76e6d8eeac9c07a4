"""GPU parity of the grouped GEMMs, stage by stage and as a whole layer, on
shapes that span several tiles with ragged token counts, on both kernels
(small-batch blocks of 16 and 32, large-batch blocks of 64, 128 and 256 --
the last with batches small enough that the second 128-row half of a block is
padding only):
  - RAW stage, exact-integer case: the fp32 projection equals the oracle's bit
    for bit (all partial sums are dyadic numbers below 2^24);
  - GATE_UP: H against the oracle's silu(gate) * up;
  - DOWN: from the oracle's H (rounded to the activation type) to the combined
    output;
  - the whole layer (route -> align -> GATE_UP -> DOWN) against the oracle;
  - determinism and token-permutation equivariance, bit for bit.
Float comparisons use relative Frobenius error <= 5e-3 and max abs error <=
3e-2 * max |ref| per output tensor."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import act_round, dev_u16, host_f32, need_gpu, say, torch
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu

W4 = gen.CFG3.with_(name="w4-small", E=8, topk=2, K=512, N=384, act_order=False)
W4AO = W4.with_(name="w4ao-small", act_order=True)
W4PC = W4.with_(name="w4-percol-small", group_size=-1)
W8 = gen.CFG2.with_(name="w8-small", E=8, topk=2, K=512, N=384)
W8E = gen.CFG5.with_(name="w8-many-small", E=40, topk=6, K=256, N=256, zipf_s=1.1)
# 64 or more experts with skewed routing: the small-batch fused stage takes two
# token blocks per pass
W8E80 = gen.CFG5.with_(name="w8-many-80", E=80, topk=6, K=256, N=256, zipf_s=1.1)
# long k_in, narrow output: the large-batch DOWN splits K into 4 slices; their
# GATE_UP (8192 outputs) takes the 512-row shape
W4K = W4.with_(name="w4-longk", K=256, N=4096)
W8K = W8.with_(name="w8-longk", K=256, N=4096)
# an odd number of 64-channel K steps in DOWN (k_in = N = 320: 5 steps): the
# large-batch kernel's two-step loop ends on a single step
W8ODD = W8.with_(name="w8-odd-steps", K=512, N=320)
SPECS = {"w4": W4, "w4ao": W4AO, "w4pc": W4PC, "w8": W8, "w8e": W8E, "w4k": W4K, "w8k": W8K, "w8e80": W8E80,
         "w8odd": W8ODD}
SEED = {"w4": 501, "w4ao": 502, "w4pc": 503, "w8": 504, "w8e": 505, "w4k": 506, "w8k": 507, "w8e80": 508,
        "w8odd": 509}


def _pack(spec, wts):
    return wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2,
                       torch.float16 if spec.act == "f16" else torch.bfloat16, spec.group_size, wts.g1, wts.g2)


_cache = {}


def setup(key):
    if key not in _cache:
        spec = SPECS[key]
        wts = gen.make_moe_weights(spec, seed_config=SEED[key])
        _cache[key] = (spec, wts, _pack(spec, wts))
    return _cache[key]


def routed(spec, M, seed):
    toks = gen.make_tokens(spec, M, seed_config=seed)
    w, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
    return toks, w, ids


def align_dev(ids, E, bs):
    cap = wq.moe_align_capacity(ids.shape[0], ids.shape[1], E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids).cuda(), E, bs, cap)
    return st, ex, nt, cap


# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bs", [16, 64, 128])
@pytest.mark.parametrize("act_order", [False, True])
def test_raw_exact_integer(bits, bs, act_order):
    """Power-of-two group scales, x in {-1,0,1}: bit-exact fp32 projections."""
    need_gpu()
    if act_order and bits == 8:
        pytest.skip("act-order is an int4 (GPTQ) feature")
    spec = (W4AO if act_order else W4) if bits == 4 else W8
    wts = gen.make_moe_weights(spec, seed_config=510 + bits)
    E, n_out, K = wts.w1q.shape
    rng = np.random.default_rng(bits * 10 + bs)
    G = wts.s1.shape[1]
    pow2 = np.array([0.25, 0.5, 1.0, 2.0], np.float32)[rng.integers(0, 4, size=(E, G, n_out))]
    s_bits = gen.round_to(spec.act, pow2)
    M = 45
    x = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
    ids = np.stack([rng.choice(E, spec.topk, replace=False) for _ in range(M)]).astype(np.int32)
    gu_ref, _ = oracle.moe_up(x, ids, wts.w1q, pow2, wts.g1, want_gu=True)
    if bits == 4:
        packed, sp, kp = wq.pack_w4(wts.w1q, s_bits, spec.group_size, g_idx=wts.g1)
    else:
        packed, sp = wq.pack_w8(wts.w1q, s_bits)
        kp = None
    st, ex, nt, cap = align_dev(ids, E, bs)
    xd = dev_u16(gen.round_to(spec.act, x), spec.act)
    out = torch.empty((M * spec.topk, n_out), dtype=torch.float32, device="cuda")
    wd = torch.from_numpy(packed).cuda()
    sd = torch.from_numpy(sp.view(np.int16)).cuda()
    say("raw exact", bits, bs, act_order)
    if bits == 4:
        kpd = torch.from_numpy(kp).cuda() if kp is not None else None
        ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_RAW, M, spec.topk, spec.E, n_out, K, cap, kp is not None)
        work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
        wq.moe_w4a16_gemm(wq.WQ_STAGE_RAW, xd, M, spec.topk, E, n_out, K, wd, sd, spec.group_size, kpd, st, ex, nt,
                          cap, bs, None, out, work)
    else:
        wq.moe_w8a16_gemm(wq.WQ_STAGE_RAW, xd, M, spec.topk, E, n_out, K, wd, sd, st, ex, nt, cap, bs, None, out,
                          act_dtype=wq.WQ_BF16)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, gu_ref), "max diff %g" % np.abs(got - gu_ref).max()


def test_raw_over_65535_sub_blocks():
    """2^20 pairs in blocks of 16 rows: more 16-row sub-blocks than one grid
    dimension holds, so the small-batch kernel's grid continues in its third
    dimension.  Exact-integer inputs; sampled tokens bit for bit."""
    need_gpu()
    spec = W8.with_(name="w8-many-rows", N=64)
    wts = gen.make_moe_weights(spec, seed_config=515)
    E, n_out, K = wts.w1q.shape
    rng = np.random.default_rng(516)
    pow2 = np.array([0.25, 0.5, 1.0, 2.0], np.float32)[rng.integers(0, 4, size=(E, 1, n_out))]
    packed, sp = wq.pack_w8(wts.w1q, gen.round_to(spec.act, pow2))
    M, topk, bs = 1 << 19, 2, 16
    ids = np.argsort(rng.random((M, E)), axis=1)[:, :topk].astype(np.int32)
    cap = wq.moe_align_capacity(M, topk, E, bs)
    assert cap // 16 > 65535
    st, ex, nt = wq.moe_align(torch.from_numpy(ids).cuda(), E, bs, cap)
    g = torch.Generator(device="cuda").manual_seed(517)
    xd = torch.randint(-1, 2, (M, K), device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty((M * topk, n_out), dtype=torch.float32, device="cuda")
    say("raw over 65535 sub-blocks")
    wq.moe_w8a16_gemm(wq.WQ_STAGE_RAW, xd, M, topk, E, n_out, K, torch.from_numpy(packed).cuda(),
                      torch.from_numpy(sp.view(np.int16)).cuda(), st, ex, nt, cap, bs, None, out,
                      act_dtype=wq.WQ_BF16)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 77, 65535 * 8 // topk, M // 2, M - 2, M - 1])
    x_rows = xd[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref, _ = oracle.moe_up(x_rows, ids[rows], wts.w1q, pow2, None, want_gu=True)
    pairs = (rows[:, None] * topk + np.arange(topk)).ravel()
    got = out[torch.from_numpy(pairs).cuda()].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), "max diff %g" % np.abs(got - ref).max()


# ----------------------------------------------------------------------------
def run_gate_up(spec, p, xd, ids_np, bs):
    M = xd.shape[0]
    st, ex, nt, cap = align_dev(ids_np, spec.E, bs)
    act_order = p.k_perm1 is not None
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_GATE_UP, M, spec.topk, spec.E, 2 * spec.N, spec.K, cap, act_order)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    h = torch.full((cap, spec.N), float("nan"), dtype=p.act, device="cuda")
    if spec.bits == 4:
        wq.moe_w4a16_gemm(wq.WQ_STAGE_GATE_UP, xd, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1,
                          spec.group_size, p.k_perm1, st, ex, nt, cap, bs, None, h, work)
    else:
        wq.moe_w8a16_gemm(wq.WQ_STAGE_GATE_UP, xd, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1, st, ex, nt,
                          cap, bs, None, h, work, act_dtype=p.act_code)
    return h, st, ex, nt, cap


def h_perm(spec, wts, e):
    """Column order of H for expert e: canonical intermediate index of each H column."""
    if spec.bits == 4 and wts.g2 is not None:
        return np.argsort(wts.g2[e], kind="stable")
    return np.arange(spec.N)


@pytest.mark.parametrize("key", ["w4", "w4ao", "w4pc", "w8", "w8e", "w4k", "w8k"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [1, 37, 300])
def test_gate_up(key, bs, M):
    need_gpu()
    spec, wts, p = setup(key)
    toks, w, ids = routed(spec, M, seed=600 + M)
    say("gate_up", key, bs, M)
    h, st, ex, nt, cap = run_gate_up(spec, p, dev_u16(toks.x, spec.act), ids, bs)
    torch.cuda.synchronize()
    _, h_ref = oracle.moe_up(toks.x_f32(), ids, wts.w1q, wts.s1_f32(), wts.g1)
    hg = host_f32(h)
    stn = st.cpu().numpy()
    exn = ex.cpu().numpy()
    ntn = int(nt.cpu()[0])
    T = M * spec.topk
    got = np.empty((T, spec.N))
    for pos in range(ntn):
        i = stn[pos]
        if i < T:
            e = exn[pos // bs]
            got[i, h_perm(spec, wts, e)] = hg[pos]
        else:
            assert (hg[pos] == 0).all(), "pad row %d of H is not zero" % pos
    assert_close_fp(got, h_ref, "H %s bs=%d M=%d" % (key, bs, M))


@pytest.mark.parametrize("key", ["w4", "w4ao", "w8", "w8e", "w8odd"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [1, 37, 300])
def test_down(key, bs, M):
    """DOWN from the oracle's H rounded to the activation type."""
    _check_down(key, bs, M)


@pytest.mark.parametrize("key", ["w4k", "w8k"])
@pytest.mark.parametrize("bs", [64, 128])
@pytest.mark.parametrize("M", [37, 300])
def test_down_split_k(key, bs, M):
    """k_in = 4096 with 256 outputs: the large-batch DOWN (blocks of 64 or
    128 rows) writes 4 fp32 slabs of partial sums (its workspace says so)
    that the combine adds."""
    spec = SPECS[key]
    ws = _check_down(key, bs, M)
    assert ws >= 4 * M * spec.topk * spec.K * 4


@pytest.mark.parametrize("key", ["w4k", "w8k"])
@pytest.mark.parametrize("M", [1, 5, 64])
def test_down_decode_long_k(key, M):
    """k_in = 4096 with 256 outputs over few experts through the small-batch
    kernel (long reductions: 8 waves per workgroup; int8 takes 4 row tiles per
    workgroup, with one token block per pass at 5 tokens and two at 64)."""
    _check_down(key, 16, M)


@pytest.mark.parametrize("M", [5, 37, 90])
def test_gate_up_many_experts_two_blocks(M):
    """80 experts, top-6, Zipf-skewed routing, blocks of 16: the small-batch
    fused stage with two token blocks per pass (and its one-block tail)."""
    need_gpu()
    spec, wts, p = setup("w8e80")
    toks, w, ids = routed(spec, M, seed=780 + M)
    say("gate_up many experts", M)
    h, st, ex, nt, cap = run_gate_up(spec, p, dev_u16(toks.x, spec.act), ids, 16)
    _, h_ref = oracle.moe_up(toks.x_f32(), ids, wts.w1q, wts.s1_f32(), wts.g1)
    got = host_f32(h)
    stn, exn, ntn = st.cpu().numpy(), ex.cpu().numpy(), int(nt.cpu()[0])
    T = M * spec.topk
    rows = [pos for pos in range(ntn) if stn[pos] < T]
    assert_close_fp(got[rows], h_ref[stn[rows]], "H many experts M=%d" % M)
    pads = [pos for pos in range(ntn) if stn[pos] >= T]
    assert not np.any(got[pads])


@pytest.mark.parametrize("M", [5, 37, 90])
def test_down_many_experts_two_blocks(M):
    """80 experts, top-6, Zipf-skewed routing, blocks of 16: the small-batch
    DOWN with two token blocks per pass over 4 weight tiles (head experts
    spread over several workgroups)."""
    _check_down("w8e80", 16, M)


def test_down_split_wide_grid_w4():
    """int4, 4096 outputs, k_in 4096, M = 1024 (2048 pairs): the DOWN grid of
    512-row tiles is smaller than one round of resident workgroups, so K is
    split in 3 slices of unequal length (21, 21 and 22 K steps of 64 channels)
    on the 512 x 128 eight-wave shape (the workspace holds the most slabs any
    block size takes, 4); the output of sampled tokens against the oracle."""
    need_gpu()
    spec = W4.with_(name="w4-split-wide", K=4096, N=4096)
    wts = gen.make_moe_weights(spec, seed_config=508)
    p = _pack(spec, wts)
    M, bs = 1024, 128
    toks, w, ids = routed(spec, M, seed=760)
    T = M * spec.topk
    h_act = act_round(np.random.default_rng(761).standard_normal((T, spec.N)), spec.act)
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    stn, ntn = st.cpu().numpy(), int(nt.cpu()[0])
    hs = np.zeros((cap, spec.N), np.float32)
    live = stn[:ntn] < T
    hs[:ntn][live] = h_act[stn[:ntn][live]]
    hd = torch.from_numpy(hs).cuda().to(p.act)
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, M, spec.topk, spec.E, spec.K, spec.N, cap, False)
    assert ws >= 4 * T * spec.K * 4
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((M, spec.K), dtype=p.act, device="cuda")
    say("down split wide w4")
    wq.moe_w4a16_gemm(wq.WQ_STAGE_DOWN, hd, M, spec.topk, spec.E, spec.K, spec.N, p.w2, p.s2, spec.group_size,
                      None, st, ex, nt, cap, bs, torch.from_numpy(w).cuda(), out, work)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 100, 511, 777, M - 1])
    h_rows = h_act.reshape(M, spec.topk, spec.N)[rows].reshape(-1, spec.N)
    y_ref = oracle.moe_down(h_rows, ids, wts.w2q, wts.s2_f32(), wts.g2, rows=rows)
    out_ref = oracle.moe_combine(y_ref, w, rows=rows)
    assert_close_fp(host_f32(out)[rows], out_ref, "split-K DOWN, sampled tokens")


def _check_down(key, bs, M):
    need_gpu()
    spec, wts, p = setup(key)
    toks, w, ids = routed(spec, M, seed=700 + M)
    T = M * spec.topk
    _, h_ref = oracle.moe_up(toks.x_f32(), ids, wts.w1q, wts.s1_f32(), wts.g1)
    h_act = act_round(h_ref, spec.act)
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
    say("down", key, bs, M)
    if spec.bits == 4:
        wq.moe_w4a16_gemm(wq.WQ_STAGE_DOWN, hd, M, spec.topk, spec.E, spec.K, spec.N, p.w2, p.s2, spec.group_size,
                          None, st, ex, nt, cap, bs, wd, out, work)
    else:
        wq.moe_w8a16_gemm(wq.WQ_STAGE_DOWN, hd, M, spec.topk, spec.E, spec.K, spec.N, p.w2, p.s2, st, ex, nt, cap,
                          bs, wd, out, work, act_dtype=p.act_code)
    torch.cuda.synchronize()
    assert_close_fp(host_f32(out), out_ref, "out %s bs=%d M=%d" % (key, bs, M))
    return ws


# ----------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["w4", "w4ao", "w4pc", "w8", "w8e", "w8odd"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [1, 16, 53, 512])
def test_layer(key, bs, M):
    need_gpu()
    spec, wts, p = setup(key)
    toks = gen.make_tokens(spec, M, seed_config=800 + M)
    say("layer", key, bs, M)
    out, aux = wq.fused_moe(dev_u16(toks.x, spec.act), torch.from_numpy(toks.logits).cuda(), p, spec.topk,
                            spec.renormalize, block_size=bs, keep=True)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.route(toks.logits, spec.topk, spec.renormalize)
    assert np.array_equal(aux["topk_ids"].cpu().numpy(), ids_ref)
    ref = oracle.moe_layer_from_weights(wts, toks.x_f32(), aux["topk_weights"].cpu().numpy(), ids_ref)["out"]
    assert_close_fp(host_f32(out), ref, "layer %s bs=%d M=%d" % (key, bs, M))


@pytest.mark.parametrize("key", ["w4ao", "w8"])
@pytest.mark.parametrize("bs", [16, 64, 128])
def test_layer_deterministic_and_equivariant(key, bs):
    need_gpu()
    spec, wts, p = setup(key)
    M = 97
    toks = gen.make_tokens(spec, M, seed_config=900)
    x = dev_u16(toks.x, spec.act)
    lg = torch.from_numpy(toks.logits).cuda()
    say("determinism", key, bs)
    a = wq.fused_moe(x, lg, p, spec.topk, block_size=bs).clone()
    b = wq.fused_moe(x, lg, p, spec.topk, block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(M)).cuda()
    c = wq.fused_moe(x[perm].contiguous(), lg[perm].contiguous(), p, spec.topk, block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(c, a[perm])


def test_layer_empty_batch():
    need_gpu()
    spec, wts, p = setup("w8")
    out = wq.fused_moe(torch.empty((0, spec.K), dtype=torch.bfloat16, device="cuda"),
                       torch.empty((0, spec.E), dtype=torch.float32, device="cuda"), p, spec.topk)
    torch.cuda.synchronize()
    assert out.shape == (0, spec.K)


def test_large_batch_rejects_activations_over_4gib():
    """The large-batch kernel addresses activation rows with 32-bit byte
    offsets: a capacity whose rows x k_in x 2 bytes exceed 4 GiB is refused
    with WQ_ERR_UNSUPPORTED before anything is launched (the buffers are never
    touched, so small ones suffice)."""
    need_gpu()
    spec, wts, p = setup("w8")
    M, bs = 300, 128
    toks, w, ids = routed(spec, M, seed=990)
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    big = (1 << 28)  # rows; x 512 channels x 2 bytes = 2^38 bytes
    h = torch.empty((cap, spec.N), dtype=p.act, device="cuda")
    with pytest.raises(wq.WqError) as ei:
        wq.moe_w8a16_gemm(wq.WQ_STAGE_GATE_UP, dev_u16(toks.x, spec.act), M, spec.topk, spec.E, 2 * spec.N, spec.K,
                          p.w1, p.s1, st, ex, nt, big, bs, None, h, None, act_dtype=p.act_code)
    assert ei.value.status == 2
    torch.cuda.synchronize()
