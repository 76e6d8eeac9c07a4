"""GPU parity of the ExpertsInt8 load-time quantizer (wq_quantize_w8) against
the oracle: codes and scales bit for bit (the rounding decisions are taken in
float32 on both sides), on ragged shapes (row counts not a multiple of the 4
rows per workgroup, k not a multiple of a wave's 512 channels), zero rows and
a Mixtral-sized expert (rows held in registers up to 16384 weights, longer
rows in two passes); then the quantized weights through the packer and the
int8 GEMM against the oracle on the same codes."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import need_gpu, say, torch
from tests.helpers import assert_close_fp

pytestmark = pytest.mark.gpu

TD = {"bf16": "bfloat16", "f16": "float16"}


def _weights(act, shape, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    bits = gen.round_to(act, (rng.standard_normal(shape) * scale).astype(np.float32))
    return bits, gen.bits_to_f32(act, bits)


def _run(act, bits):
    w = torch.from_numpy(bits.view(np.int16)).cuda().view(getattr(torch, TD[act]))
    q, s = wq.quantize_w8(w)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.float().cpu().numpy()


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1, 8), (3, 33, 1000), (2, 48, 4096), (1, 7, 14336), (1, 5, 16392)])
def test_quant_matches_oracle(act, shape):
    need_gpu()
    bits, w = _weights(act, shape, 600 + shape[-1] + shape[1])
    if shape[1] > 2:
        bits[0, 2] = 0                                # an all-zero row
        w[0, 2] = 0.0
    say("quant", act, shape)
    q, s = _run(act, bits)
    q_ref, s_ref = oracle.quant_w8(w, bf16=(act == "bf16"))
    assert np.array_equal(s, s_ref), "scales differ at %s" % (np.argwhere(s != s_ref)[:5],)
    assert np.array_equal(q, q_ref), "codes differ at %s" % (np.argwhere(q != q_ref)[:5],)


def test_quant_mixtral_expert_bf16():
    """One Mixtral expert's w1 (2 x 14336 rows of 4096 bf16 weights)."""
    need_gpu()
    bits, w = _weights("bf16", (1, 2 * 14336, 4096), 610)
    say("quant mixtral expert")
    q, s = _run("bf16", bits)
    q_ref, s_ref = oracle.quant_w8(w, bf16=True)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(q, q_ref)


def test_quantize_pack_gemm():
    """bf16 checkpoint -> GPU quantizer -> wq_pack_w8 -> RAW int8 GEMM, against
    the oracle's projection with the oracle's own codes and scales."""
    need_gpu()
    E, n_out, K, M, topk = 4, 256, 512, 37, 2
    bits, w = _weights("bf16", (E, n_out, K), 620)
    q, s = _run("bf16", bits)
    q_ref, s_ref = oracle.quant_w8(w, bf16=True)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    s_bits = gen.round_to("bf16", s_ref)[:, None, :]          # [E, 1, n_out], exact (already bf16 values)
    packed, sp = wq.pack_w8(q, s_bits)
    rng = np.random.default_rng(621)
    x = gen.bits_to_f32("bf16", gen.round_to("bf16", rng.standard_normal((M, K)).astype(np.float32)))
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(M)]).astype(np.int32)
    bs = 16
    cap = wq.moe_align_capacity(M, topk, E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids).cuda(), E, bs, cap)
    out = torch.empty((M * topk, n_out), dtype=torch.float32, device="cuda")
    xd = torch.from_numpy(gen.round_to("bf16", x).view(np.int16)).cuda().view(torch.bfloat16)
    wq.moe_w8a16_gemm(wq.WQ_STAGE_RAW, xd, M, topk, E, n_out, K, torch.from_numpy(packed).cuda(),
                      torch.from_numpy(sp.view(np.int16)).cuda(), st, ex, nt, cap, bs, None, out,
                      act_dtype=wq.WQ_BF16)
    torch.cuda.synchronize()
    ref, _ = oracle.moe_up(x, ids, q_ref, s_ref[:, None, :], want_gu=True)
    assert_close_fp(out.cpu().numpy(), ref, "quantized RAW projection")
