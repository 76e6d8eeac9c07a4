"""The seeded generator produces the distributions and structure the configs
describe (no method arithmetic is checked here)."""
import numpy as np

import gen


def test_determinism_and_ranges():
    a = gen.make_moe_weights(gen.CFG1)
    b = gen.make_moe_weights(gen.CFG1)
    assert np.array_equal(a.w1q, b.w1q) and np.array_equal(a.s2, b.s2)
    assert a.w1q.min() >= -8 and a.w1q.max() <= 7
    s = a.s1_f32()
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    t = gen.make_tokens(gen.CFG1, 16)
    assert t.x.shape == (16, 256) and t.logits.shape == (16, 4)


def test_actorder_groups_have_exactly_group_size_members():
    spec = gen.CFG3.with_(E=2, K=512, N=256)
    w = gen.make_moe_weights(spec, seed_config=91)
    for g in (w.g1, w.g2):
        for e in range(spec.E):
            assert (np.bincount(g[e]) == 128).all()
            assert not (g[e] == np.arange(g.shape[1]) // 128).all()


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -3.1], np.float32)
    bits = gen.f32_to_bf16_bits(v)
    back = gen.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[3] == np.float32(1.0078125)
    assert abs(back[4] + 3.1) < 3.1 * 2 ** -8


def test_sparse_keep_positions():
    spec = gen.CFG4.with_(K=256, N=64)
    sw = gen.make_sparse_weights(spec, seed_config=92)
    pairs = sw.idx.reshape(spec.N, -1, 2)
    assert (pairs[..., 0] < pairs[..., 1]).all() and pairs.max() <= 3
    assert len({tuple(p) for p in pairs.reshape(-1, 2).tolist()}) == 6


def test_zipf_bias_skews_routing():
    t = gen.make_tokens(gen.CFG5, 512)
    top1 = t.logits.argmax(1)
    counts = np.bincount(top1, minlength=160)
    assert counts[0] > 5 * counts.mean()
