"""GPU parity of moe_route_gate_up, the call that routes, sorts and runs the
GATE_UP stage: for up to 16 pairs over up to 64 experts (blocks of 16 or 32,
no act-order) one kernel whose every workgroup routes and sorts the batch
itself; with act-order one token in the same kernel, each workgroup gathering
the permuted row into LDS, and up to 16 tokens (64 pairs, 64 experts) a
routing launch that also gathers the permuted rows; otherwise the separate
launches.  Its outputs -- routing weights and
ids, sorted_token_ids, expert_ids, num_tokens_post_padded and every H row up
to the padded total -- equal those of moe_route_align followed by the GEMM's
GATE_UP call bit for bit (int8 bf16 and fp16, int4 group-128 and per-column,
both softmax modes, ties, both block sizes), including past the one-kernel
limits and for an empty batch."""
import numpy as np
import pytest

import gen
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, need_gpu, say, torch

pytestmark = pytest.mark.gpu

SPECS = {
    "w8bf": gen.CFG2.with_(name="rgu-w8bf", E=8, topk=2, K=256, N=512),
    "w8f16": gen.CFG2.with_(name="rgu-w8f16", E=8, topk=2, K=256, N=512, act="f16"),
    "w4g": gen.CFG3.with_(name="rgu-w4g", E=8, topk=2, K=256, N=512, act_order=False),
    "w4pc": gen.CFG3.with_(name="rgu-w4pc", E=8, topk=2, K=256, N=512, act_order=False, group_size=-1),
    "w8e64": gen.CFG2.with_(name="rgu-w8e64", E=64, topk=4, K=256, N=256),
    "w8e5": gen.CFG2.with_(name="rgu-w8e5", E=5, topk=3, K=256, N=256),
    # act-order int4: the routing launch also gathers the permuted rows
    "w4ao": gen.CFG3.with_(name="rgu-w4ao", E=8, topk=2, K=256, N=512, act_order=True),
    "w4aoe64": gen.CFG3.with_(name="rgu-w4aoe64", E=64, topk=4, K=384, N=256, act_order=True),
    "w4ao6": gen.CFG3.with_(name="rgu-w4ao6", E=8, topk=6, K=1024, N=256, act_order=True),
}
_cache = {}


def setup(key):
    if key not in _cache:
        spec = SPECS[key]
        wts = gen.make_moe_weights(spec, seed_config=1300 + sorted(SPECS).index(key))
        act = torch.float16 if spec.act == "f16" else torch.bfloat16
        p = wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2, act, spec.group_size, wts.g1, wts.g2)
        _cache[key] = (spec, p)
    return _cache[key]


def buffers(M, topk, E, cap, bs, N, act):
    dev = "cuda"
    return dict(w=torch.full((M, topk), -1.0, device=dev), ids=torch.full((M, topk), -7, dtype=torch.int32, device=dev),
                st=torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev),
                ex=torch.full((max(cap // bs, 1),), -7, dtype=torch.int32, device=dev),
                nt=torch.full((4,), -7, dtype=torch.int32, device=dev),
                h=torch.full((max(cap, 1), N), float("nan"), dtype=act, device=dev))


def run_pair(key, M, bs, renorm, ties=False):
    spec, p = setup(key)
    rng = np.random.default_rng(1400 + M + bs + 7 * renorm)
    logits = rng.standard_normal((M, spec.E)).astype(np.float32)
    if ties:
        logits[:, ::3] = np.float32(0.5)
    x_bits = gen.f32_to_bf16_bits(rng.standard_normal((M, spec.K))) if spec.act == "bf16" else \
        gen.f32_to_f16_bits(rng.standard_normal((M, spec.K)))
    x = dev_u16(x_bits, spec.act)
    lg = torch.from_numpy(logits).cuda()
    cap = wq.moe_align_capacity(M, spec.topk, spec.E, bs)
    gs = spec.group_size if spec.bits == 4 else -1
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_GATE_UP, M, spec.topk, spec.E, 2 * spec.N, spec.K, cap,
                                     p.k_perm1 is not None)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
    a = buffers(M, spec.topk, spec.E, cap, bs, spec.N, p.act)
    b = buffers(M, spec.topk, spec.E, cap, bs, spec.N, p.act)
    say("route_gate_up", key, M, bs, renorm, ties)
    # the two separate calls
    wq.moe_route_align(lg, spec.topk, renorm, bs, a["w"], a["ids"], a["st"], a["ex"], a["nt"], cap)
    if spec.bits == 4:
        wq.moe_w4a16_gemm(wq.WQ_STAGE_GATE_UP, x, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1, gs,
                          p.k_perm1, a["st"], a["ex"], a["nt"], cap, bs, None, a["h"], work, None, p.act_code)
    else:
        wq.moe_w8a16_gemm(wq.WQ_STAGE_GATE_UP, x, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1, a["st"],
                          a["ex"], a["nt"], cap, bs, None, a["h"], work, None, p.act_code)
    # the one call
    wq.moe_route_gate_up(spec.bits, lg, renorm, b["w"], b["ids"], x, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1,
                         p.s1, gs, p.k_perm1, b["st"], b["ex"], b["nt"], cap, bs, b["h"], work, None, p.act_code)
    torch.cuda.synchronize()
    nt = int(a["nt"][0])
    assert int(b["nt"][0]) == nt
    for k in ("w", "ids"):
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k
    assert torch.equal(a["st"][:cap], b["st"][:cap])
    assert torch.equal(a["ex"][: cap // bs], b["ex"][: cap // bs])
    assert torch.equal(a["h"][:nt].view(torch.int16), b["h"][:nt].view(torch.int16)), "H rows differ"
    return nt


@pytest.mark.parametrize("key", ["w8bf", "w8f16", "w4g", "w4pc", "w4ao"])
@pytest.mark.parametrize("M", [1, 2, 3, 8])
@pytest.mark.parametrize("bs", [16, 32])
def test_route_gate_up_equals_two_calls(key, M, bs):
    need_gpu()
    run_pair(key, M, bs, renorm=True)


@pytest.mark.parametrize("key", ["w4ao", "w4aoe64", "w4ao6"])
@pytest.mark.parametrize("bs", [16, 32])
def test_route_gate_up_act_order_one_token(key, bs):
    """One token of an act-order int4 layer: one kernel that routes, sorts and
    gathers the token's row in each expert's channel order into LDS (top-2,
    top-4 and top-6: both of its launch shapes) -- the same outputs as the two
    calls with the gathered rows in the workspace."""
    need_gpu()
    run_pair(key, 1, bs, renorm=True)


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("key,M", [("w8e64", 4), ("w8e64", 1), ("w8e5", 5), ("w8bf", 1)])
def test_route_gate_up_softmax_modes_and_ties(key, M, renorm):
    need_gpu()
    run_pair(key, M, 16, renorm=renorm, ties=True)


@pytest.mark.parametrize("key,M,bs", [("w8bf", 9, 16), ("w8bf", 32, 16), ("w4g", 2, 64), ("w8e64", 5, 16),
                                      ("w4ao", 16, 16), ("w4ao", 2, 128), ("w4ao", 17, 16), ("w4aoe64", 16, 16),
                                      ("w4aoe64", 3, 32)])
def test_route_gate_up_past_the_one_kernel_limits(key, M, bs):
    """More than 16 pairs, blocks of 64, or 20 pairs over 64 experts: the
    separate launches, with the same outputs; act-order int4 at the limits of
    the routing-and-gather launch (16 tokens, 64 pairs, a capacity of 1024
    rows, blocks of 128 feeding the large-batch kernel) and past them."""
    need_gpu()
    run_pair(key, M, bs, renorm=True)


def test_route_gate_up_empty_batch():
    need_gpu()
    spec, p = setup("w8bf")
    cap = wq.moe_align_capacity(0, spec.topk, spec.E, 16)
    b = buffers(1, spec.topk, spec.E, cap, 16, spec.N, p.act)
    lg = torch.empty((0, spec.E), dtype=torch.float32, device="cuda")
    x = torch.empty((0, spec.K), dtype=p.act, device="cuda")
    wq.moe_route_gate_up(8, lg, True, b["w"], b["ids"], x, 0, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1, -1,
                         None, b["st"], b["ex"], b["nt"], cap, 16, b["h"], None, None, p.act_code)
    torch.cuda.synchronize()
    assert int(b["nt"][0]) == 0
