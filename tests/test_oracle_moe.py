"""Pins for the oracle's MoE layer (dequantisation, both projections, SiLU-and-mul,
weighted combine): hand-worked examples, the exact-integer special case against
numpy's int64 matmul, textbook mat-vecs, closed forms and invariants.

Each pin is chosen so that a plausible slip in the oracle fails at least one:
a wrong group index (act-order example, permutation invariance), a transposed
operand (non-square exact-integer case), a swapped gate/up half (worked
example), a dropped routing weight or slot (worked example, topk=1 identity),
a wrong sign in SiLU (closed form)."""
import json
import math
import os

import numpy as np
import pytest

import gen
import oracle


def _load(golden_dir, name):
    return json.load(open(os.path.join(golden_dir, name)))


def test_layer_worked_example(golden_dir):
    g = _load(golden_dir, "layer_example.json")
    x = np.array(g["x"], np.float32)
    w, ids = oracle.route(np.array(g["logits"], np.float32), g["topk"])
    assert ids.tolist() == g["ids"]
    np.testing.assert_allclose(w, g["weights"], rtol=2 ** -22)
    res = oracle.moe_layer(x, np.array(g["weights"], np.float32), ids,
                           np.array(g["w1q"], np.int8), np.array(g["s1"], np.float32), None,
                           np.array(g["w2q"], np.int8), np.array(g["s2"], np.float32), None,
                           want=("out", "gu", "h", "y"))
    np.testing.assert_allclose(res["gu"], g["gu"], rtol=0, atol=0)
    np.testing.assert_allclose(res["h"], g["h"], rtol=1e-15)
    np.testing.assert_allclose(res["y"], g["y"], rtol=1e-15)
    np.testing.assert_allclose(res["out"], g["out"], rtol=1e-15)


def test_actorder_group_lookup(golden_dir):
    g = _load(golden_dir, "actorder_example.json")
    gu, _ = oracle.moe_up(np.array(g["x"], np.float32), np.zeros((1, 1), np.int32),
                          np.array(g["w1q"], np.int8), np.array(g["s1"], np.float32),
                          np.array(g["g_idx"], np.int32), want_gu=True)
    assert gu.tolist() == g["gu"]


def _int_problem(rng, E, K, N, M, topk, bits):
    qmax = 7 if bits == 4 else 127
    w1q = rng.integers(-qmax - (bits == 4), qmax + 1, size=(E, 2 * N, K), dtype=np.int8)
    w2q = rng.integers(-qmax - (bits == 4), qmax + 1, size=(E, K, N), dtype=np.int8)
    x = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(M)]).astype(np.int32)
    return w1q, w2q, x, ids


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_integer_projections(bits):
    """All-ones / power-of-two scales with x in {-1,0,1}: every partial sum is an
    integer (times a power of two) below 2^24, so the projections equal numpy's
    int64 matmul exactly.  K != N != 2N catches a transposed operand."""
    rng = np.random.default_rng(bits)
    E, K, N, M, topk = 3, 256, 384, 7, 2
    w1q, w2q, x, ids = _int_problem(rng, E, K, N, M, topk, bits)
    G1 = K // 128
    s1 = np.ones((E, G1, 2 * N), np.float32)
    s1[:, 1, :] = 0.5                                                  # second group scaled by 2^-1
    gu, h = oracle.moe_up(x, ids, w1q, s1, None, want_gu=True)
    W1 = w1q.astype(np.int64).astype(np.float64)
    W1[:, :, 128:] *= 0.5
    for m in range(M):
        for j in range(topk):
            e = ids[m, j]
            ref = W1[e] @ x[m].astype(np.float64)
            assert np.array_equal(gu[m * topk + j], ref)
    # down projection with an integer hidden vector: pass integer h
    hint = rng.integers(-2, 3, size=(M * topk, N)).astype(np.float64)
    s2 = np.full((E, 1, K), 2.0, np.float32)
    y = oracle.moe_down(hint, ids, w2q, s2)
    for m in range(M):
        for j in range(topk):
            e = ids[m, j]
            ref = 2 * (w2q[e].astype(np.int64) @ hint[m * topk + j].astype(np.int64))
            assert np.array_equal(y[m * topk + j], ref.astype(np.float64))


def test_single_token_single_expert_is_matvec():
    """E=1, topk=1, one token: the layer is the textbook
    out = W2 (silu(W1g x) * W1u x), computed here with numpy's matmul."""
    spec = gen.CFG1.with_(E=1, topk=1, K=256, N=256)
    wts = gen.make_moe_weights(spec, seed_config=101)
    x = gen.make_tokens(spec, 1, seed_config=101).x_f32()
    res = oracle.moe_layer_from_weights(wts, x, np.ones((1, 1), np.float32), np.zeros((1, 1), np.int32),
                                        want=("out", "h"))
    s1 = wts.s1_f32()[0]                         # [G, 2N]
    W1 = wts.w1q[0].astype(np.float64) * np.repeat(s1, 128, axis=0).T.astype(np.float64)
    s2 = wts.s2_f32()[0]
    W2 = wts.w2q[0].astype(np.float64) * np.repeat(s2, 128, axis=0).T.astype(np.float64)
    a = W1 @ x[0].astype(np.float64)
    gate, up = a[:256], a[256:]
    h = gate / (1 + np.exp(-gate)) * up
    np.testing.assert_allclose(res["h"][0], h, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["out"][0], W2 @ h, rtol=1e-11, atol=1e-11)


def test_silu_closed_forms():
    """silu(0) = 0 so a zero token gives a zero output; silu(a) -> a for large a,
    silu(a) -> 0 for very negative a."""
    E, K, N = 2, 128, 16
    w1q = np.ones((E, 2 * N, K), np.int8)
    w2q = np.ones((E, K, N), np.int8)
    s1 = np.ones((E, 1, 2 * N), np.float32)
    s2 = np.ones((E, 1, K), np.float32)
    ids = np.array([[0, 1]], np.int32)
    wts = np.array([[0.5, 0.5]], np.float32)
    zero = oracle.moe_layer(np.zeros((1, K), np.float32), wts, ids, w1q, s1, None, w2q, s2, None)["out"]
    assert (zero == 0).all()
    big = oracle.moe_layer(np.full((1, K), 0.5, np.float32), wts, ids, w1q, s1, None, w2q, s2, None,
                           want=("out", "h"))
    # gate = up = 64 -> h = 64 * 64 * sigma(64), sigma(64) = 1 - 1.6e-28
    np.testing.assert_allclose(big["h"], 64.0 * 64.0, rtol=1e-15)
    neg = oracle.moe_layer(np.full((1, K), -0.5, np.float32), wts, ids, w1q, s1, None, w2q, s2, None,
                           want=("h",))
    # gate = up = -64 -> h = (-64) * sigma(-64) * (-64) = 4096 * e^-64 / (1 + e^-64)
    np.testing.assert_allclose(neg["h"], 4096.0 * math.exp(-64) / (1 + math.exp(-64)), rtol=1e-13)


def _small_w4(seed, act_order):
    spec = gen.CFG1.with_(E=4, topk=2, K=384, N=256, act_order=act_order)
    return spec, gen.make_moe_weights(spec, seed_config=seed), gen.make_tokens(spec, 9, seed_config=seed)


def test_actorder_permutation_invariance():
    """With sigma = stable argsort(g), the problem (x[:, sigma], q[:, :, sigma],
    g[sigma]) has sorted groups and the same result; a wrong group lookup breaks
    this because the unsorted problem then uses the wrong scales."""
    spec, wts, toks = _small_w4(201, act_order=True)
    x = toks.x_f32()
    w, ids = oracle.route(toks.logits, spec.topk)
    ref = oracle.moe_layer_from_weights(wts, x, w, ids, want=("out", "h"))
    # gate/up problem: permute K of w1 per expert (the same sigma for all experts
    # needs one shared g1; use expert-wise sorted problems one expert at a time)
    for e in range(spec.E):
        sig = np.argsort(wts.g1[e], kind="stable")
        sel = (ids == e)
        if not sel.any():
            continue
        ids_e = np.zeros((x.shape[0], 1), np.int32)
        gu_ref, _ = oracle.moe_up(x, ids_e, wts.w1q[e:e + 1], wts.s1_f32()[e:e + 1], wts.g1[e:e + 1],
                                  want_gu=True)
        gu_perm, _ = oracle.moe_up(x[:, sig], ids_e, wts.w1q[e:e + 1][:, :, sig], wts.s1_f32()[e:e + 1],
                                   wts.g1[e:e + 1][:, sig], want_gu=True)
        np.testing.assert_allclose(gu_perm, gu_ref, rtol=1e-12, atol=1e-12)
        # the sorted problem's groups are contiguous blocks of 128
        assert (wts.g1[e][sig] == np.arange(spec.K) // 128).all()
    # down projection: permuting N of w2 together with h
    for e in range(spec.E):
        sig2 = np.argsort(wts.g2[e], kind="stable")
        ids_e = np.zeros((x.shape[0], 1), np.int32)
        h = np.random.default_rng(e).standard_normal((x.shape[0], spec.N))
        y_ref = oracle.moe_down(h, ids_e, wts.w2q[e:e + 1], wts.s2_f32()[e:e + 1], wts.g2[e:e + 1])
        y_perm = oracle.moe_down(h[:, sig2], ids_e, wts.w2q[e:e + 1][:, :, sig2], wts.s2_f32()[e:e + 1],
                                 wts.g2[e:e + 1][:, sig2])
        np.testing.assert_allclose(y_perm, y_ref, rtol=1e-12, atol=1e-12)
    assert np.isfinite(ref["out"]).all()


def test_actorder_matters():
    """Canary for the pin above: ignoring g_idx changes the result."""
    spec, wts, toks = _small_w4(202, act_order=True)
    x = toks.x_f32()
    w, ids = oracle.route(toks.logits, spec.topk)
    a = oracle.moe_layer_from_weights(wts, x, w, ids)["out"]
    b = oracle.moe_layer(x, w, ids, wts.w1q, wts.s1_f32(), None, wts.w2q, wts.s2_f32(), None)["out"]
    assert np.abs(a - b).max() > 1e-3 * np.abs(a).max()


def test_token_permutation_equivariance():
    spec, wts, toks = _small_w4(203, act_order=False)
    x = toks.x_f32()
    w, ids = oracle.route(toks.logits, spec.topk)
    out = oracle.moe_layer_from_weights(wts, x, w, ids)["out"]
    perm = np.random.default_rng(0).permutation(x.shape[0])
    out_p = oracle.moe_layer_from_weights(wts, x[perm], w[perm], ids[perm])["out"]
    assert np.array_equal(out_p, out[perm])
    # the row subset option evaluates exactly those tokens
    sub = oracle.moe_layer_from_weights(wts, x, w, ids, rows=np.array([5, 0, 3]))["out"]
    assert np.array_equal(sub, out[[5, 0, 3]])


def test_expert_relabelling_invariance():
    spec, wts, toks = _small_w4(204, act_order=True)
    x = toks.x_f32()
    w, ids = oracle.route(toks.logits, spec.topk)
    out = oracle.moe_layer_from_weights(wts, x, w, ids)["out"]
    pe = np.array([2, 0, 3, 1])                          # new expert j is old expert pe[j]
    lg2 = toks.logits[:, pe]
    w2, ids2 = oracle.route(lg2, spec.topk)
    assert (pe[ids2] == ids).all()
    out2 = oracle.moe_layer(x, w2, ids2, wts.w1q[pe], wts.s1_f32()[pe], wts.g1[pe],
                            wts.w2q[pe], wts.s2_f32()[pe], wts.g2[pe])["out"]
    assert np.array_equal(out2, out)


def test_identical_experts_make_routing_irrelevant():
    """All experts equal and weights renormalised: out = the single expert's
    output, whatever the routing."""
    spec = gen.CFG1.with_(E=4, topk=2, K=256, N=128)
    wts = gen.make_moe_weights(spec, seed_config=205)
    for a in ("w1q", "s1", "w2q", "s2"):
        arr = getattr(wts, a)
        setattr(wts, a, np.ascontiguousarray(np.broadcast_to(arr[:1], arr.shape)))
    toks = gen.make_tokens(spec, 6, seed_config=205)
    x = toks.x_f32()
    w, ids = oracle.route(toks.logits, 2)
    out = oracle.moe_layer_from_weights(wts, x, w, ids)["out"]
    one = oracle.moe_layer_from_weights(wts, x, np.ones((6, 1), np.float32), np.zeros((6, 1), np.int32))["out"]
    np.testing.assert_allclose(out, one, rtol=1e-6 * 4, atol=1e-9)   # sum of w is 1 within float32 rounding


def test_topk1_unit_weight_combine_is_identity():
    spec, wts, toks = _small_w4(206, act_order=False)
    x = toks.x_f32()
    ids = np.random.default_rng(1).integers(0, spec.E, size=(x.shape[0], 1)).astype(np.int32)
    res = oracle.moe_layer_from_weights(wts, x, np.ones((x.shape[0], 1), np.float32), ids, want=("out", "y"))
    assert np.array_equal(res["out"], res["y"])


def test_projection_is_linear_in_x():
    spec, wts, toks = _small_w4(207, act_order=True)
    x = toks.x_f32()
    _, ids = oracle.route(toks.logits, spec.topk)
    gu1, _ = oracle.moe_up(x, ids, wts.w1q, wts.s1_f32(), wts.g1, want_gu=True)
    gu2, _ = oracle.moe_up(2 * x, ids, wts.w1q, wts.s1_f32(), wts.g1, want_gu=True)
    assert np.array_equal(gu2, 2 * gu1)


def test_per_column_scales_equal_single_group():
    """W8 per-column scales are the one-group case: s[e, 0, r] scales row r."""
    spec = gen.CFG2.with_(E=2, K=256, N=128)
    wts = gen.make_moe_weights(spec, seed_config=208)
    toks = gen.make_tokens(spec, 3, seed_config=208)
    x = toks.x_f32()
    _, ids = oracle.route(toks.logits, 2)
    gu, _ = oracle.moe_up(x, ids, wts.w1q, wts.s1_f32(), None, want_gu=True)
    for m in range(3):
        for j in range(2):
            e = ids[m, j]
            W = wts.w1q[e].astype(np.float64) * wts.s1_f32()[e, 0][:, None].astype(np.float64)
            np.testing.assert_allclose(gu[m * 2 + j], W @ x[m].astype(np.float64), rtol=1e-12, atol=1e-12)
