"""GPU parity of the 2:4-sparse W4A16 linear layer against the oracle: an
exact-integer case (fp16 output holds the integer results exactly), and float
cases spanning several tiles with ragged token counts."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, host_f32, need_gpu, say, torch
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu


def run_sparse(sw, x_bits, N, group_size=128, bits=4):
    vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s, group_size, bits=bits)
    fn = wq.sparse24_w4a16_gemm if bits == 4 else wq.sparse24_w8a16_gemm
    y = fn(dev_u16(x_bits, "f16"), torch.from_numpy(vp).cuda(), torch.from_numpy(mp).cuda(),
           torch.from_numpy(sp.view(np.int16)).cuda(), N, group_size=group_size)
    torch.cuda.synchronize()
    return host_f32(y)


def test_sparse_exact_integer():
    need_gpu()
    spec = gen.CFG4.with_(K=512, N=96)
    sw = gen.make_sparse_weights(spec, seed_config=310)
    rng = np.random.default_rng(0)
    x = rng.integers(-1, 2, size=(37, spec.K)).astype(np.float32)
    ones = np.ones((spec.K // 128, spec.N), np.float32)
    sw.s = gen.round_to("f16", ones)
    say("sparse exact")
    y = run_sparse(sw, gen.round_to("f16", x), spec.N)
    ref = oracle.sparse24(x, sw.vals, sw.idx, ones, 128)
    assert np.abs(ref).max() < 2048
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("M", [1, 16, 45, 72, 96, 130])
def test_sparse_float(M):
    need_gpu()
    spec = gen.CFG4.with_(K=1024, N=256)
    sw = gen.make_sparse_weights(spec, seed_config=311)
    x = gen.make_sparse_x(spec, M, seed_config=311)
    say("sparse float", M)
    y = run_sparse(sw, x, spec.N)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128)
    assert_close_fp(y, ref, "sparse M=%d" % M)


@pytest.mark.parametrize("M", [1, 16, 40, 100, 200])
def test_sparse_float_long_k(M):
    """K = 2304 (9 chunks of 256: two full blocks of 4 in flight plus a tail)
    and N = 512, through each batch-size kernel (16/32/64-token streaming on 8
    or 16 waves, 256 x 64 tiles)."""
    need_gpu()
    spec = gen.CFG4.with_(K=2304, N=512)
    sw = gen.make_sparse_weights(spec, seed_config=313)
    x = gen.make_sparse_x(spec, M, seed_config=313)
    say("sparse long-k", M)
    y = run_sparse(sw, x, spec.N)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128)
    assert_close_fp(y, ref, "sparse K=2304 M=%d" % M)


@pytest.mark.parametrize("N", [512, 112])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_sparse_decode_kernel(M, N):
    """M <= 4: the decode kernel (token rows staged in LDS, waves splitting the
    9 chunks of K = 2304 with a tail, two row tiles per workgroup; N = 112 has
    an odd tile count, so the last workgroup holds one valid tile)."""
    need_gpu()
    spec = gen.CFG4.with_(K=2304, N=N)
    sw = gen.make_sparse_weights(spec, seed_config=315)
    x = gen.make_sparse_x(spec, M, seed_config=316 + M)
    say("sparse decode", M, N)
    y = run_sparse(sw, x, spec.N)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128)
    assert_close_fp(y, ref, "sparse decode M=%d N=%d" % (M, N))


@pytest.mark.parametrize("M", [1, 3])
def test_sparse_exact_integer_decode(M):
    """Exact-integer case through the decode kernel: unit scales, x in
    {-1, 0, 1}, so every output is an integer the fp16 result holds exactly."""
    need_gpu()
    spec = gen.CFG4.with_(K=512, N=96)
    sw = gen.make_sparse_weights(spec, seed_config=317)
    x = np.random.default_rng(M).integers(-1, 2, size=(M, spec.K)).astype(np.float32)
    ones = np.ones((spec.K // 128, spec.N), np.float32)
    sw.s = gen.round_to("f16", ones)
    say("sparse exact decode", M)
    y = run_sparse(sw, gen.round_to("f16", x), spec.N)
    ref = oracle.sparse24(x, sw.vals, sw.idx, ones, 128)
    assert np.abs(ref).max() < 2048
    assert np.array_equal(y.astype(np.float64), ref)


def test_sparse_decode_too_long_for_lds():
    """M = 4 with K = 16384: the token rows (128 KiB) do not fit the decode
    kernel's LDS, so the streaming kernel runs; same result contract."""
    need_gpu()
    spec = gen.CFG4.with_(K=16384, N=64)
    sw = gen.make_sparse_weights(spec, seed_config=318)
    x = gen.make_sparse_x(spec, 4, seed_config=318)
    say("sparse long row")
    y = run_sparse(sw, x, spec.N)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128)
    assert_close_fp(y, ref, "sparse K=16384 M=4")


@pytest.mark.parametrize("M", [1, 3, 16, 100, 200])
def test_sparse_per_column_scales(M):
    """group_size -1 (one scale per output column, the pages' channel-wise
    variant) through each batch-size kernel: decode (M <= 4), streaming,
    256 x 64 tiles."""
    need_gpu()
    spec = gen.CFG4.with_(K=2304, N=512, group_size=-1)
    sw = gen.make_sparse_weights(spec, seed_config=319)
    assert sw.s.shape == (1, spec.N)
    x = gen.make_sparse_x(spec, M, seed_config=319)
    say("sparse per-column", M)
    y = run_sparse(sw, x, spec.N, group_size=-1)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), -1)
    assert_close_fp(y, ref, "sparse per-column M=%d" % M)


@pytest.mark.parametrize("gs", [128, -1])
@pytest.mark.parametrize("M", [1, 3, 16, 100, 200])
def test_sparse_8bit(M, gs):
    """8-bit kept codes (the pages' 8-bit variant of the 2:4 support), group
    128 and channel-wise, through each batch-size kernel."""
    need_gpu()
    spec = gen.CFG4.with_(K=2304, N=512, bits=8, group_size=gs)
    sw = gen.make_sparse_weights(spec, seed_config=320)
    assert sw.vals.min() < -8 and sw.vals.max() > 7
    x = gen.make_sparse_x(spec, M, seed_config=320)
    say("sparse 8-bit", M, gs)
    y = run_sparse(sw, x, spec.N, group_size=gs, bits=8)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), gs)
    assert_close_fp(y, ref, "sparse 8-bit M=%d gs=%d" % (M, gs))


@pytest.mark.parametrize("M", [2, 37])
def test_sparse_8bit_exact_integer(M):
    """Exact-integer case for 8-bit codes: unit scales, x in {-1, 0, 1} with
    one nonzero channel in 16, codes in [-128, 127]: every output is an integer
    below 2048 in magnitude, held exactly by fp16."""
    need_gpu()
    spec = gen.CFG4.with_(K=512, N=96, bits=8)
    sw = gen.make_sparse_weights(spec, seed_config=321)
    rng = np.random.default_rng(M)
    x = rng.integers(-1, 2, size=(M, spec.K)).astype(np.float32) * (rng.random((M, spec.K)) < 1 / 16)
    ones = np.ones((spec.K // 128, spec.N), np.float32)
    sw.s = gen.round_to("f16", ones)
    say("sparse 8-bit exact", M)
    y = run_sparse(sw, gen.round_to("f16", x), spec.N, bits=8)
    ref = oracle.sparse24(x, sw.vals, sw.idx, ones, 128)
    assert np.abs(ref).max() < 2048
    assert np.array_equal(y.astype(np.float64), ref)


def test_sparse_large_batch_narrow_n():
    """M > 128 with N not a multiple of 256: the streaming kernel, with a
    partial last workgroup of row tiles."""
    need_gpu()
    spec = gen.CFG4.with_(K=512, N=112)
    sw = gen.make_sparse_weights(spec, seed_config=314)
    x = gen.make_sparse_x(spec, 150, seed_config=314)
    say("sparse narrow-n")
    y = run_sparse(sw, x, spec.N)
    ref = oracle.sparse24(gen.bits_to_f32("f16", x), sw.vals, sw.idx, sw.s_f32(), 128)
    assert_close_fp(y, ref, "sparse N=112 M=150")


def test_sparse_matches_dense_with_zeros_on_gpu():
    """The 2:4 kernel and the dense int4 kernel (RAW stage, one expert, top-1)
    agree on the same weights with zeros at the pruned positions."""
    need_gpu()
    spec = gen.CFG4.with_(K=512, N=128)
    sw = gen.make_sparse_weights(spec, seed_config=312)
    x = gen.make_sparse_x(spec, 20, seed_config=312)
    y_sp = run_sparse(sw, x, spec.N)
    dense = np.zeros((1, spec.N, spec.K), np.int8)
    grp = np.repeat(np.arange(spec.K // 4), 2)[None, :] * 4
    np.put_along_axis(dense[0], grp + sw.idx.astype(np.int64), sw.vals, axis=1)
    s_dense = np.ascontiguousarray(sw.s[None, :, :])                 # [1, G, N]
    packed, sp, _ = wq.pack_w4(dense, s_dense, 128)
    M = x.shape[0]
    ids = np.zeros((M, 1), np.int32)
    cap = wq.moe_align_capacity(M, 1, 1, 16)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids).cuda(), 1, 16, cap)
    out = torch.empty((M, spec.N), dtype=torch.float32, device="cuda")
    wq.moe_w4a16_gemm(wq.WQ_STAGE_RAW, dev_u16(x, "f16"), M, 1, 1, spec.N, spec.K, torch.from_numpy(packed).cuda(),
                      torch.from_numpy(sp.view(np.int16)).cuda(), 128, None, st, ex, nt, cap, 16, None, out)
    torch.cuda.synchronize()
    dense_y = out.cpu().numpy().astype(np.float64)
    assert_close_fp(y_sp, dense_y, "2:4 vs dense-with-zeros")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [256, 768])
def test_sparse_exact_integer_large_batch(bits, K):
    """The large-batch kernel (M > 128, N a multiple of 256) bit for bit on an
    exact-integer case: one 256-channel chunk, and three (an odd count, so the
    chunk loop ends on its first register slot), with a ragged last token tile."""
    need_gpu()
    spec = gen.CFG4.with_(K=K, N=256, bits=bits)
    sw = gen.make_sparse_weights(spec, seed_config=330 + bits)
    rng = np.random.default_rng(K + bits)
    M = 150
    density = 1 / 4 if bits == 4 else 1 / 16  # every sum stays an integer below 2048 (exact in fp16)
    x = rng.integers(-1, 2, size=(M, spec.K)).astype(np.float32) * (rng.random((M, spec.K)) < density)
    ones = np.ones((spec.K // 128, spec.N), np.float32)
    sw.s = gen.round_to("f16", ones)
    say("sparse large-batch exact", bits, K)
    y = run_sparse(sw, gen.round_to("f16", x), spec.N, bits=bits)
    ref = oracle.sparse24(x, sw.vals, sw.idx, ones, 128)
    assert np.abs(ref).max() < 2048
    assert np.array_equal(y.astype(np.float64), ref)
