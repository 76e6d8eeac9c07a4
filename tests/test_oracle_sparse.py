"""Pins for the oracle's 2:4-sparse W4A16 layer: a hand-worked example, the
exact-integer case against numpy's int64 matmul of the dense-with-zeros matrix,
and the dense-with-zeros identity in floating point."""
import json
import os

import numpy as np

import gen
import oracle


def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "sparse_example.json")))
    y = oracle.sparse24(np.array(g["x"], np.float32), np.array(g["vals"], np.int8), np.array(g["idx"], np.uint8),
                        np.array(g["s"], np.float32), g["group_size"])
    assert y.tolist() == g["y"]


def dense_codes(vals, idx):
    """Scatter the kept codes into a dense [N, K] matrix with zeros elsewhere."""
    N, Kh = vals.shape
    K = 2 * Kh
    D = np.zeros((N, K), np.int64)
    grp = np.repeat(np.arange(Kh // 2), 2)[None, :] * 4
    cols = grp + idx.astype(np.int64)
    np.put_along_axis(D, cols, vals.astype(np.int64), axis=1)
    return D


def test_exact_integer_equals_dense_with_zeros():
    spec = gen.CFG4.with_(K=512, N=96)
    sw = gen.make_sparse_weights(spec, seed_config=301)
    rng = np.random.default_rng(0)
    x = rng.integers(-1, 2, size=(5, spec.K)).astype(np.float32)
    ones = np.ones_like(sw.s_f32())
    y = oracle.sparse24(x, sw.vals, sw.idx, ones, 128)
    D = dense_codes(sw.vals, sw.idx)
    assert np.array_equal(y, (x.astype(np.int64) @ D.T).astype(np.float64))
    # exactly two kept per group of four
    assert ((D.reshape(spec.N, -1, 4) != 0).sum(-1) <= 2).all()


def test_exact_integer_8bit_and_per_column():
    """8-bit kept codes and channel-wise scales (group -1): exact integers vs
    the int64 matmul of the dense-with-zeros matrix, and per-column scales
    equal one group spanning all of K."""
    spec = gen.CFG4.with_(K=512, N=48, bits=8, group_size=-1)
    sw = gen.make_sparse_weights(spec, seed_config=305)
    assert sw.vals.min() < -8 and sw.s.shape == (1, spec.N)
    rng = np.random.default_rng(1)
    x = rng.integers(-1, 2, size=(4, spec.K)).astype(np.float32)
    y = oracle.sparse24(x, sw.vals, sw.idx, np.ones((1, spec.N), np.float32), -1)
    D = dense_codes(sw.vals, sw.idx)
    assert np.array_equal(y, (x.astype(np.int64) @ D.T).astype(np.float64))
    s = sw.s_f32()
    y1 = oracle.sparse24(x, sw.vals, sw.idx, s, -1)
    y2 = oracle.sparse24(x, sw.vals, sw.idx, np.repeat(s, spec.K // 128, axis=0), 128)
    assert np.array_equal(y1, y2)


def test_float_equals_dense_with_zeros():
    spec = gen.CFG4.with_(K=1024, N=64)
    sw = gen.make_sparse_weights(spec, seed_config=302)
    x = gen.make_sparse_x(spec, 3, seed_config=302)
    xf = gen.bits_to_f32("f16", x)
    y = oracle.sparse24(xf, sw.vals, sw.idx, sw.s_f32(), 128)
    D = dense_codes(sw.vals, sw.idx).astype(np.float64)
    W = D * np.repeat(sw.s_f32(), 128, axis=0).T.astype(np.float64)
    np.testing.assert_allclose(y, xf.astype(np.float64) @ W.T, rtol=1e-12, atol=1e-12)


def test_group_scales_follow_dense_position():
    """A kept code's scale group is that of its dense position k // 128: moving
    every scale group changes the result."""
    spec = gen.CFG4.with_(K=512, N=32)
    sw = gen.make_sparse_weights(spec, seed_config=303)
    xf = gen.bits_to_f32("f16", gen.make_sparse_x(spec, 2, seed_config=303))
    a = oracle.sparse24(xf, sw.vals, sw.idx, sw.s_f32(), 128)
    b = oracle.sparse24(xf, sw.vals, sw.idx, np.roll(sw.s_f32(), 1, axis=0), 128)
    assert np.abs(a - b).max() > 1e-3


def test_row_subset():
    spec = gen.CFG4.with_(K=256, N=48)
    sw = gen.make_sparse_weights(spec, seed_config=304)
    xf = gen.bits_to_f32("f16", gen.make_sparse_x(spec, 7, seed_config=304))
    full = oracle.sparse24(xf, sw.vals, sw.idx, sw.s_f32(), 128)
    sub = oracle.sparse24(xf, sw.vals, sw.idx, sw.s_f32(), 128, rows=np.array([6, 2]))
    assert np.array_equal(sub, full[[6, 2]])
