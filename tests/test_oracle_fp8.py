"""Pins of the oracle's FP8 (OCP E4M3) W8A8 layer, each against something
other than the oracle itself:
  - decoding: all 256 codes against torch's float8_e4m3fn conversion (a
    library routine) and hand-derived values;
  - encoding: a brute-force nearest search over the table of finite E4M3
    values (ties to the even mantissa, saturation at 448), and torch's
    float8_e4m3fn cast on in-range values;
  - the gate/up projections of a quantised input reduce, for integer codes
    and power-of-two scales, to the int8 layer's projections (a function of
    the oracle pinned by its own tests) bit for bit;
  - the whole layer on tiny shapes equals a numpy float64 re-computation
    that quantises with the brute-force nearest search;
  - the layer is linear in a1 where quantisation is the identity, and
    saturating: H values beyond 448 a2 are clamped."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def table():
    """(codes, values) of the 254 finite E4M3 codes."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    return codes, vals


def brute_encode(t: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code to each t after clamping to [-448, 448]; on a
    tie the code with an even mantissa (bit 0) wins; zero keeps the sign."""
    codes, vals = table()
    out = np.empty(t.shape, np.uint8)
    for i, v in enumerate(np.asarray(t, np.float64).ravel()):
        a = min(abs(v), 448.0)
        pos = vals >= 0
        cand_c, cand_v = codes[pos & (codes < 0x80)], vals[pos & (codes < 0x80)]
        d = np.abs(cand_v - a)
        best = np.nonzero(d == d.min())[0]
        if best.size > 1:
            best = [b for b in best if (cand_c[b] & 1) == 0]
        c = int(cand_c[best[0]])
        if np.signbit(v):
            c |= 0x80
        out.ravel()[i] = c
    return out


def test_decode_all_codes_match_torch():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.fp8_decode(c)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    ok = ~np.isnan(v)
    assert np.array_equal(v[ok], t[ok])
    # hand-derived: 0x38 = 2^0 (exponent field 7), 0x7E = 1.75 * 2^8, 0x08 the smallest
    # normal 2^-6, 0x01 the smallest subnormal 2^-9, 0xC5 = -(1 + 5/8) * 2
    assert (v[0x38], v[0x7E], v[0x08], v[0x01], v[0xC5], v[0x00], v[0x80]) == (1.0, 448.0, 2 ** -6, 2 ** -9, -3.25,
                                                                               0.0, 0.0)
    assert np.signbit(v[0x80]) and not np.signbit(v[0x00])


def test_encode_matches_brute_force_nearest():
    codes, vals = table()
    pos = np.sort(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2                      # exact ties
    eps = np.concatenate([mids * (1 - 2 ** -20), mids * (1 + 2 ** -20)])
    rng = np.random.default_rng(5)
    rand = rng.standard_normal(2000) * np.exp2(rng.integers(-12, 10, 2000))
    t = np.concatenate([pos, mids, eps, rand, [0.0, 2 ** -10, 3 * 2 ** -10, 447.9, 448.0, 449.0, 464.0, 500.0, 1e6]])
    t = np.concatenate([t, -t]).astype(np.float32)
    got = oracle.fp8_quant(t, 1.0)
    assert np.array_equal(got, brute_encode(t.astype(np.float64)))
    # torch's cast on in-range values (it does not saturate)
    inr = np.abs(t) <= 448
    tt = torch.from_numpy(t[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inr], tt)


def test_encode_hand_cases():
    # 1/3 in float32 is 0.3333333432674408 = 1.333.. * 2^-2 (exponent field 5); its neighbours
    # 0.3125 (0x2A: mantissa 2) and 0.34375 (0x2B: mantissa 3) -> the nearer 0x2B.  A tie between
    # 2^-9 and 2 * 2^-9 (1.5 * 2^-9) goes to the even mantissa 2 (0x02); 2.5 * 2^-9 to 0x02 as
    # well; 3.5 * 2^-9 to 0x04.  1000 saturates to 0x7E; -0.0 keeps its sign.
    q = oracle.fp8_quant(np.array([1.0, 1.5 * 2 ** -9, 2.5 * 2 ** -9, 3.5 * 2 ** -9, 1000.0, -0.0], np.float32),
                         1.0)
    assert q.tolist()[1:] == [0x02, 0x02, 0x04, 0x7E, 0x80]
    q3 = oracle.fp8_quant(np.array([1.0], np.float32), 3.0)
    assert q3.tolist() == [0x2B]


def _int_codes(rng, shape, lim=16):
    """E4M3 codes of random integers in [-lim, lim] (E4M3 holds every integer up to 16)."""
    codes, vals = table()
    lut = {int(v): int(c) for c, v in zip(codes, vals) if v == int(v) and abs(v) <= lim and not (v == 0 and c)}
    ints = rng.integers(-lim, lim + 1, size=shape)
    return np.vectorize(lut.get)(ints).astype(np.uint8), ints


def test_gate_up_reduces_to_int8_layer():
    """Integer weight codes, power-of-two column scales, an input already on the
    E4M3 grid of a power-of-two a1 (so quantising it is the identity): the
    projections equal the int8 layer's (orc_moe_up) bit for bit."""
    rng = np.random.default_rng(11)
    E, topk, K, N, M = 3, 2, 64, 24, 7
    c1, q1 = _int_codes(rng, (E, 2 * N, K))
    sw1 = np.exp2(rng.integers(-3, 3, size=(E, 2 * N))).astype(np.float32)
    a1 = 2.0 ** -4
    xc, _ = _int_codes(rng, (M, K), lim=12)
    x = (oracle.fp8_decode(xc) * a1).astype(np.float32)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(M)]).astype(np.int32)
    w = np.full((M, topk), 0.5, np.float32)
    c2, _ = _int_codes(rng, (E, K, N))
    sw2 = np.ones((E, K), np.float32)
    got = oracle.fp8_moe_layer(x, w, ids, c1, sw1, c2, sw2, a1, 1.0, want=("out", "gu"))["gu"]
    ref, _ = oracle.moe_up(x, ids, q1.astype(np.int8), sw1[:, None, :], None, want_gu=True)
    assert np.array_equal(got, ref)
    # every gate/up value is an exact dyadic number here; a1 = 1/16 times an integer
    assert np.all(np.abs(got * 16 / np.repeat(sw1[ids.ravel()], 1, axis=0) - np.round(
        got * 16 / np.repeat(sw1[ids.ravel()], 1, axis=0))) == 0)


def _numpy_layer(x, w, ids, c1, sw1, c2, sw2, a1, a2):
    """The reading re-computed with numpy: brute-force quantisation, float64 matmuls."""
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    a1, a2 = np.float32(a1), np.float32(a2)  # the layer takes float32 scales
    tx = (x.astype(np.float32) / a1).astype(np.float32)
    xd = dec(brute_encode(tx.astype(np.float64))) * np.float64(a1)
    M, topk = ids.shape
    N = c1.shape[1] // 2
    out = np.zeros((M, c2.shape[1]))
    hq = np.empty((M * topk, N), np.uint8)
    for m in range(M):
        for j in range(topk):
            e = ids[m, j]
            W1 = dec(c1[e]) * sw1[e][:, None].astype(np.float64)
            gu = W1 @ xd[m]
            g, u = gu[:N], gu[N:]
            h = g / (1 + np.exp(-g)) * u
            th = (h.astype(np.float32) / a2).astype(np.float32)
            hq[m * topk + j] = brute_encode(th.astype(np.float64))
            hd = dec(hq[m * topk + j]) * np.float64(a2)
            W2 = dec(c2[e]) * sw2[e][:, None].astype(np.float64)
            out[m] += np.float64(w[m, j]) * (W2 @ hd)
    return out, hq


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_layer_matches_numpy_recomputation(seed):
    rng = np.random.default_rng(100 + seed)
    E, topk, K, N, M = 4, 2, 48, 16, 5
    codes, vals = table()
    finite = codes[np.abs(vals) <= 16]
    c1 = rng.choice(finite, size=(E, 2 * N, K)).astype(np.uint8)
    c2 = rng.choice(finite, size=(E, K, N)).astype(np.uint8)
    sw1 = rng.uniform(1e-3, 4e-3, size=(E, 2 * N)).astype(np.float32)
    sw2 = rng.uniform(1e-3, 4e-3, size=(E, K)).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    a1, a2 = 1 / 64, 1 / 3000.0
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(M)]).astype(np.int32)
    w = rng.uniform(0, 1, size=(M, topk)).astype(np.float32)
    res = oracle.fp8_moe_layer(x, w, ids, c1, sw1, c2, sw2, a1, a2, want=("out", "hq"))
    ref, hq_ref = _numpy_layer(x, w, ids, c1, sw1, c2, sw2, a1, a2)
    assert np.array_equal(res["hq"], hq_ref)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-15)


def test_layer_row_subset_and_saturation():
    """Evaluating a subset of tokens gives those tokens' rows; a tiny a2 saturates
    every nonzero H code at +-448."""
    rng = np.random.default_rng(7)
    E, topk, K, N, M = 3, 1, 32, 8, 6
    codes, vals = table()
    finite = codes[np.abs(vals) <= 8]
    c1 = rng.choice(finite, size=(E, 2 * N, K)).astype(np.uint8)
    c2 = rng.choice(finite, size=(E, K, N)).astype(np.uint8)
    sw1 = np.full((E, 2 * N), 0.01, np.float32)
    sw2 = np.full((E, K), 0.01, np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    ids = rng.integers(0, E, size=(M, topk)).astype(np.int32)
    w = np.ones((M, topk), np.float32)
    full = oracle.fp8_moe_layer(x, w, ids, c1, sw1, c2, sw2, 1 / 64, 1e-3, want=("out", "hq"))
    rows = np.array([4, 1])
    sub = oracle.fp8_moe_layer(x, w, ids, c1, sw1, c2, sw2, 1 / 64, 1e-3, rows=rows, want=("out", "hq"))
    assert np.array_equal(sub["out"], full["out"][rows])
    sat = oracle.fp8_moe_layer(x, w, ids, c1, sw1, c2, sw2, 1 / 64, 1e-12, want=("out", "hq"))["hq"]
    assert set(np.unique(sat & 0x7F).tolist()) <= {0x00, 0x7E}
