"""GPU parity of the FP8 (OCP E4M3) W8A8 grouped GEMM against the oracle, on
shapes that span several tiles with ragged token counts, on both kernels
(small-batch blocks of 16 / 32, large-batch blocks of 64 / 128 / 256):
  - the activation codes equal the oracle's bit for bit for every finite
    bf16 and fp16 value, at several scales (the quantisation takes its
    rounding decision in float32 on both sides);
  - RAW stage, exact-integer case (integer codes, power-of-two scales, small
    integer activations): the fp32 projections equal the oracle's bit for bit,
    which pins the packed layout, the MFMA operand formats and the epilogue;
  - GATE_UP: the H codes equal the oracle's except where the two sides'
    sums round H to neighbouring codes: only the adjacent code, and on at most
    1 % of the values (gfx950's E4M3 MFMA drops the low bits of products far
    below the largest one it adds -- see test_mfma_accumulation_bound -- so its
    sums carry about 1e-4 relative error where the oracle's are exact, and an
    H value that close to an E4M3 rounding boundary may land on the other
    side: 0.1 % of the values here);
  - DOWN from the oracle's H codes (for one token also with the top-k sum
    folded into the GEMM: top-k 1 to 4, an expert named twice), and the whole
    layer, within the float tolerance (relative Frobenius error <= 5e-3, max abs error <= 3e-2 max |ref|);
  - determinism, bit for bit."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, host_f32, need_gpu, say, torch
from tests.helpers import assert_close_fp, logical_rows

pytestmark = pytest.mark.gpu

F8 = gen.CFG_FP8.with_(name="fp8-small", E=8, topk=2, K=512, N=384)
# many experts, Zipf-skewed routing
F8E = gen.CFG_FP8.with_(name="fp8-many", E=40, topk=6, K=256, N=256, zipf_s=1.1)
# DOWN with k_in = 4096 and 256 outputs: the large-batch kernel splits K
F8K = gen.CFG_FP8.with_(name="fp8-longk", K=256, N=4096)
SPECS = {"f8": F8, "f8e": F8E, "f8k": F8K}
SEED = {"f8": 1301, "f8e": 1302, "f8k": 1303}
_cache = {}


def setup(key):
    if key not in _cache:
        spec = SPECS[key]
        wts = gen.make_fp8_weights(spec, seed_config=SEED[key])
        p = wq.pack_moe_fp8(wts.w1, wts.s1, wts.w2, wts.s2, torch.bfloat16, spec.a1, spec.a2)
        _cache[key] = (spec, wts, p)
    return _cache[key]


def align_dev(ids, E, bs):
    cap = wq.moe_align_capacity(ids.shape[0], ids.shape[1], E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids).cuda(), E, bs, cap)
    return st, ex, nt, cap


def run_stage(stage, p, spec, a, M, ids, bs, w=None, act=torch.bfloat16):
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    if stage == wq.WQ_STAGE_DOWN:
        n_out, k_in, wp, sp = spec.K, spec.N, p.w2, p.s2
        out = torch.empty((M, spec.K), dtype=act, device="cuda")
        in_scale = spec.a2
    else:
        n_out, k_in, wp, sp = 2 * spec.N, spec.K, p.w1, p.s1
        in_scale = spec.a1
        if stage == wq.WQ_STAGE_GATE_UP:
            out = torch.full((cap, spec.N), 0x7F, dtype=torch.uint8, device="cuda")  # NaN codes: unwritten
        else:
            out = torch.empty((M * spec.topk, n_out), dtype=torch.float32, device="cuda")
    ws = wq.moe_fp8_gemm_workspace_bytes(stage, M, spec.topk, spec.E, n_out, k_in)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    tw = None if w is None else torch.from_numpy(w).cuda()
    wq.moe_fp8_w8a8_gemm(stage, a, M, spec.topk, spec.E, n_out, k_in, wp, sp, st, ex, nt, cap, bs, tw, out, work,
                         in_scale, spec.a2, act_dtype=wq.act_code(act))
    return out, work, st, ex, nt, cap


def finite_patterns(act):
    """Every finite bit pattern of the 16-bit type, as uint16, padded to a multiple of 128."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if act == "bf16":
        finite = (u & 0x7F80) != 0x7F80
    else:
        finite = (u & 0x7C00) != 0x7C00
    v = u[finite]
    pad = (-v.size) % 128
    return np.concatenate([v, np.zeros(pad, np.uint16)])


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("a1", [1.0, 3.0, 2.0 ** -6, 0.37])
def test_activation_codes_bit_exact(act, a1):
    """All finite 16-bit values through the RAW stage's quantisation: the codes
    it leaves in the workspace equal the oracle's."""
    need_gpu()
    bits = finite_patterns(act)
    K = 128
    M = bits.size // K
    spec = F8.with_(name="fp8-quant", E=1, topk=1, K=K, N=128, a1=a1)
    wts = gen.make_fp8_weights(spec, seed_config=1310)
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    p = wq.pack_moe_fp8(wts.w1, wts.s1, wts.w2, wts.s2, tdt, a1, spec.a2)
    x = dev_u16(bits.reshape(M, K), act)
    ids = np.zeros((M, 1), np.int32)
    say("fp8 quant", act, a1)
    _, work, *_ = run_stage(wq.WQ_STAGE_RAW, p, spec, x, M, ids, 16, act=tdt)
    torch.cuda.synchronize()
    got = work[:M * K].cpu().numpy().reshape(M, K)
    ref = oracle.fp8_quant(gen.bits_to_f32(act, bits).reshape(M, K), a1)
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, "%d codes differ, e.g. x=%r code %#x (oracle %#x)" % (
        bad[0].size, float(gen.bits_to_f32(act, bits.reshape(M, K)[bad][:1])[0]), got[bad][0], ref[bad][0])


def _int_codes(rng, shape, lim):
    """E4M3 codes of random integers in [-lim, lim] (E4M3 holds every integer up to 16)."""
    vals = np.arange(-lim, lim + 1)
    codes = np.array([oracle.fp8_quant(np.array([float(v)], np.float32), 1.0)[0] for v in vals], np.uint8)
    idx = rng.integers(0, vals.size, size=shape)
    return codes[idx]


@pytest.mark.parametrize("bs", [16, 64, 128])
def test_raw_exact_integer(bs):
    need_gpu()
    spec = F8
    rng = np.random.default_rng(1320 + bs)
    E, K, n_out = spec.E, spec.K, 2 * spec.N
    w1 = _int_codes(rng, (E, n_out, K), 16)
    s1 = np.exp2(rng.integers(-2, 3, size=(E, n_out))).astype(np.float32)
    w2 = _int_codes(rng, (E, K, spec.N), 16)
    s2 = np.ones((E, K), np.float32)
    p = wq.pack_moe_fp8(w1, s1, w2, s2, torch.bfloat16, 1.0, 1.0)
    M = 45
    x = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    ids = np.stack([rng.choice(E, spec.topk, replace=False) for _ in range(M)]).astype(np.int32)
    ref = oracle.fp8_moe_layer(x, np.ones((M, spec.topk), np.float32), ids, w1, s1, w2, s2, 1.0, 1.0,
                               want=("out", "gu"))["gu"]
    say("fp8 raw exact", bs)
    out, *_ = run_stage(wq.WQ_STAGE_RAW, p, spec.with_(a1=1.0), dev_u16(gen.round_to("bf16", x), "bf16"), M, ids,
                        bs)
    torch.cuda.synchronize()
    got = np.empty((M * spec.topk, n_out))
    got[:, logical_rows(n_out, True)] = out.cpu().numpy()  # RAW columns are in packed (gate/up interleaved) order
    assert np.array_equal(got, ref), "max diff %g" % np.abs(got - ref).max()


def test_mfma_accumulation_bound():
    """The E4M3 MFMA's sum over 128 channels, through the RAW stage with one
    large product and 127 small ones (all weights 1.0): products within 2^-11
    of the largest are added exactly; far smaller ones may lose their low bits
    (gfx950 measured: 256 + 127 * 2^-9 gives 256.234375, 7 units short).  The
    error stays below 2^-11 of the largest product times the 4 groups of 32
    channels -- the bound the H-code comparison above relies on."""
    need_gpu()
    K, N, E = 128, 128, 1
    w1 = np.full((E, 2 * N, K), 0x38, np.uint8)  # 1.0
    w2 = np.full((E, K, N), 0x38, np.uint8)
    p = wq.pack_moe_fp8(w1, np.ones((E, 2 * N), np.float32), w2, np.ones((E, K), np.float32), torch.bfloat16,
                        1.0, 1.0)
    rows = []
    for small in (2.0 ** -9, 2.0 ** -6, 2.0 ** -3, 1.0):
        for big in (16.0, 256.0, 448.0):
            v = np.full(K, small, np.float32)
            v[0] = big
            rows.append(v)
    x = np.stack(rows)
    M = x.shape[0]
    spec = F8.with_(name="fp8-acc", E=E, topk=1, K=K, N=N, a1=1.0)
    say("fp8 accumulation bound")
    out, *_ = run_stage(wq.WQ_STAGE_RAW, p, spec, dev_u16(gen.round_to("bf16", x), "bf16"), M,
                        np.zeros((M, 1), np.int32), 16)
    torch.cuda.synchronize()
    got = out[:, 0].cpu().numpy().astype(np.float64)
    exact = x.astype(np.float64).sum(axis=1)
    big = x[:, 0].astype(np.float64)
    for g_, e_, b_, v in zip(got, exact, big, x):
        say("  %g + 127 x %g: exact %.9g, MFMA %.9g" % (b_, v[1], e_, g_))
    assert np.all(np.abs(got - exact) <= 4 * 2.0 ** -11 * big)
    near = x[:, 1] >= big * 2.0 ** -11
    assert np.array_equal(got[near], exact[near])


def value_rank(codes):
    """Position of each code's value among the sorted distinct finite E4M3 values."""
    vals = oracle.fp8_decode(np.arange(256, dtype=np.uint8))
    table = np.unique(vals[np.isfinite(vals)])  # -448 .. 448, one zero
    return np.searchsorted(table, oracle.fp8_decode(codes))


def routed(spec, M, seed):
    toks = gen.make_tokens(spec, M, seed_config=seed)
    w, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
    return toks, w, ids


@pytest.mark.parametrize("key", ["f8", "f8e", "f8k"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [1, 37, 300])
def test_gate_up(key, bs, M):
    need_gpu()
    spec, wts, p = setup(key)
    toks, w, ids = routed(spec, M, seed=1330 + M)
    say("fp8 gate_up", key, bs, M)
    h, _, st, ex, nt, cap = run_stage(wq.WQ_STAGE_GATE_UP, p, spec, dev_u16(toks.x, "bf16"), M, ids, bs)
    torch.cuda.synchronize()
    ref = oracle.fp8_moe_layer(toks.x_f32(), w, ids, wts.w1, wts.s1, wts.w2, wts.s2, spec.a1, spec.a2,
                               want=("out", "hq"))["hq"]
    hg = h.cpu().numpy()
    stn, ntn = st.cpu().numpy(), int(nt.cpu()[0])
    T = M * spec.topk
    live = np.nonzero(stn[:ntn] < T)[0]
    pads = np.nonzero(stn[:ntn] >= T)[0]
    assert not hg[pads].any(), "pad rows of H are not code 0"
    got = np.empty_like(ref)
    got[stn[live]] = hg[live]
    diff = got != ref
    n_diff = int(diff.sum())
    say("  %d of %d H codes differ from the oracle's" % (n_diff, ref.size))
    assert n_diff <= max(2, ref.size // 100), "%d of %d H codes differ" % (n_diff, ref.size)
    # a differing code holds a neighbour of the oracle's value (+0 and -0 count as one point)
    if n_diff:
        assert np.all(np.abs(value_rank(got[diff]) - value_rank(ref[diff])) <= 1)
    # one neighbouring code differs by at most 1/8 of its value (3 mantissa bits), so the max-abs
    # bound on H is 1/8 of max |H|; the Frobenius bound is the usual one
    assert_close_fp(oracle.fp8_decode(got), oracle.fp8_decode(ref), "H %s bs=%d M=%d" % (key, bs, M),
                    max_abs=0.125)


@pytest.mark.parametrize("key", ["f8", "f8e", "f8k"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [1, 37, 300])
def test_down(key, bs, M):
    """DOWN from the oracle's H codes to the combined output."""
    need_gpu()
    spec, wts, p = setup(key)
    toks, w, ids = routed(spec, M, seed=1340 + M)
    res = oracle.fp8_moe_layer(toks.x_f32(), w, ids, wts.w1, wts.s1, wts.w2, wts.s2, spec.a1, spec.a2,
                               want=("out", "hq"))
    T = M * spec.topk
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    stn, ntn = st.cpu().numpy(), int(nt.cpu()[0])
    hs = np.zeros((cap, spec.N), np.uint8)
    live = stn[:ntn] < T
    hs[:ntn][live] = res["hq"][stn[:ntn][live]]
    say("fp8 down", key, bs, M)
    out, *_ = run_stage(wq.WQ_STAGE_DOWN, p, spec, torch.from_numpy(hs).cuda(), M, ids, bs, w=w)
    torch.cuda.synchronize()
    assert_close_fp(host_f32(out), res["out"], "fp8 out %s bs=%d M=%d" % (key, bs, M))


@pytest.mark.parametrize("key", ["f8", "f8e"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [1, 16, 53, 512])
def test_layer(key, bs, M):
    need_gpu()
    spec, wts, p = setup(key)
    toks = gen.make_tokens(spec, M, seed_config=1350 + M)
    say("fp8 layer", key, bs, M)
    out, aux = wq.fused_moe_fp8(dev_u16(toks.x, "bf16"), torch.from_numpy(toks.logits).cuda(), p, spec.topk,
                                spec.renormalize, block_size=bs, keep=True)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.route(toks.logits, spec.topk, spec.renormalize)
    assert np.array_equal(aux["topk_ids"].cpu().numpy(), ids_ref)
    ref = oracle.fp8_moe_layer(toks.x_f32(), aux["topk_weights"].cpu().numpy(), ids_ref, wts.w1, wts.s1, wts.w2,
                               wts.s2, spec.a1, spec.a2)["out"]
    assert_close_fp(host_f32(out), ref, "fp8 layer %s bs=%d M=%d" % (key, bs, M))


@pytest.mark.parametrize("bs", [16, 128])
def test_layer_deterministic_and_equivariant(bs):
    need_gpu()
    spec, wts, p = setup("f8")
    M = 97
    toks = gen.make_tokens(spec, M, seed_config=1360)
    x = dev_u16(toks.x, "bf16")
    lg = torch.from_numpy(toks.logits).cuda()
    say("fp8 determinism", bs)
    a = wq.fused_moe_fp8(x, lg, p, spec.topk, block_size=bs).clone()
    b = wq.fused_moe_fp8(x, lg, p, spec.topk, block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    perm = torch.from_numpy(np.random.default_rng(2).permutation(M)).cuda()
    c = wq.fused_moe_fp8(x[perm].contiguous(), lg[perm].contiguous(), p, spec.topk, block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(c, a[perm])


# one token with the top-k sum folded into DOWN (32 or more 2 KiB chunks per
# tile): every compiled top-k (1-4), small and large blocks, an expert named twice
@pytest.mark.parametrize("topk", [1, 2, 3, 4])
@pytest.mark.parametrize("bs", [16, 256])
@pytest.mark.parametrize("twice", [False, True])
def test_down_one_token(topk, bs, twice):
    need_gpu()
    if twice and topk == 1:
        pytest.skip("one slot cannot name an expert twice")
    spec0, wts, p = setup("f8k")
    spec = spec0.with_(topk=topk)
    toks = gen.make_tokens(spec, 1, seed_config=1370 + topk)
    rng = np.random.default_rng(1380 + topk + 10 * twice)
    ids = rng.permutation(spec.E)[:topk].astype(np.int32).reshape(1, topk)
    if twice:
        ids[0, -1] = ids[0, 0]
    w = rng.uniform(0.1, 1.0, size=(1, topk)).astype(np.float32)
    res = oracle.fp8_moe_layer(toks.x_f32(), w, ids, wts.w1, wts.s1, wts.w2, wts.s2, spec.a1, spec.a2,
                               want=("out", "hq"))
    st, ex, nt, cap = align_dev(ids, spec.E, bs)
    stn, ntn = st.cpu().numpy(), int(nt.cpu()[0])
    hs = np.zeros((cap, spec.N), np.uint8)
    live = stn[:ntn] < topk
    hs[:ntn][live] = res["hq"][stn[:ntn][live]]
    say("fp8 one-token down", topk, bs, twice)
    out, *_ = run_stage(wq.WQ_STAGE_DOWN, p, spec, torch.from_numpy(hs).cuda(), 1, ids, bs, w=w)
    torch.cuda.synchronize()
    assert_close_fp(host_f32(out), res["out"], "fp8 one token topk=%d bs=%d twice=%s" % (topk, bs, twice))


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("bs", [16, 32])
def test_gate_up_one_token_quantised_in_kernel(act, bs):
    """One token's GATE_UP quantises x inside the GEMM: its H codes are the
    oracle's (up to the neighbouring-code rule above), in both 16-bit types."""
    need_gpu()
    spec, wts, _ = setup("f8")
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    p = wq.pack_moe_fp8(wts.w1, wts.s1, wts.w2, wts.s2, tdt, spec.a1, spec.a2)
    toks, w, ids = routed(spec.with_(act=act), 1, seed=1390 + bs)
    say("fp8 one-token gate_up", act, bs)
    h, _, st, ex, nt, cap = run_stage(wq.WQ_STAGE_GATE_UP, p, spec, dev_u16(toks.x, act), 1, ids, bs, act=tdt)
    torch.cuda.synchronize()
    ref = oracle.fp8_moe_layer(toks.x_f32(), w, ids, wts.w1, wts.s1, wts.w2, wts.s2, spec.a1, spec.a2, want=("out", "hq"))["hq"]
    hg = h.cpu().numpy()
    stn, ntn = st.cpu().numpy(), int(nt.cpu()[0])
    live = np.nonzero(stn[:ntn] < spec.topk)[0]
    got = np.empty_like(ref)
    got[stn[live]] = hg[live]
    diff = got != ref
    assert int(diff.sum()) <= max(2, ref.size // 100)
    if diff.any():
        assert np.all(np.abs(value_rank(got[diff]) - value_rank(ref[diff])) <= 1)
