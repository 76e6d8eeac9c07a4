"""moe_w8a16_gemm_noalloc against moe_w8a16_gemm, through the C ABI.

The no-allocation variant runs the same kernels with the library's own
file-scope scratch array as the workspace, so its outputs must equal those of
the entry point that takes the caller's workspace bit for bit.  Two DOWN calls
in a row -- a large-batch one whose K is split over 4 fp32 slabs, then a
smaller small-batch one -- check that the second call sees none of the first
call's scratch contents; a GATE_UP call (no workspace needed) and the
rejection of a call whose workspace would exceed the scratch complete it."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, need_gpu, say, torch

pytestmark = pytest.mark.gpu

# DOWN with n_out = 256 outputs and k_in = 4096: the large-batch kernel splits K in 4
SPEC = gen.CFG2.with_(name="w8-noalloc", E=8, topk=2, K=256, N=4096)


def _setup():
    wts = gen.make_moe_weights(SPEC, seed_config=1201)
    p = wq.pack_moe(8, wts.w1q, wts.s1, wts.w2q, wts.s2, torch.bfloat16, -1)
    return wts, p


def _down_pair(p, M, bs, seed):
    """One DOWN call through each entry point on the same inputs."""
    rng = np.random.default_rng(seed)
    toks = gen.make_tokens(SPEC, M, seed_config=seed)
    w_np, ids_np = oracle.route(toks.logits, SPEC.topk, True)
    cap = wq.moe_align_capacity(M, SPEC.topk, SPEC.E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids_np).cuda(), SPEC.E, bs, cap)
    h = torch.from_numpy(rng.standard_normal((cap, SPEC.N)).astype(np.float32)).cuda().to(torch.bfloat16)
    tw = torch.from_numpy(w_np).cuda()
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, M, SPEC.topk, SPEC.E, SPEC.K, SPEC.N, cap, False)
    assert 0 < ws <= wq._lib.WQ_NOALLOC_SCRATCH_BYTES
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    ref = torch.empty((M, SPEC.K), dtype=torch.bfloat16, device="cuda")
    got = torch.full((M, SPEC.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    say("no-alloc DOWN M=%d block %d (workspace %d bytes)" % (M, bs, ws))
    wq.moe_w8a16_gemm(wq.WQ_STAGE_DOWN, h, M, SPEC.topk, SPEC.E, SPEC.K, SPEC.N, p.w2, p.s2, st, ex, nt, cap, bs,
                      tw, ref, work)
    wq.moe_w8a16_gemm_noalloc(wq.WQ_STAGE_DOWN, h, M, SPEC.topk, SPEC.E, SPEC.K, SPEC.N, p.w2, p.s2, st, ex, nt,
                              cap, bs, tw, got)
    torch.cuda.synchronize()
    return ws, ref, got


def test_noalloc_down_matches_workspace_entry_point():
    need_gpu()
    wts, p = _setup()
    ws1, ref1, got1 = _down_pair(p, 300, 128, 1202)
    assert ws1 >= 4 * 300 * SPEC.topk * SPEC.K * 4  # K split in 4 slabs
    assert torch.equal(got1, ref1)
    ws2, ref2, got2 = _down_pair(p, 3, 16, 1203)  # smaller: stale scratch from the first call must not show
    assert ws2 < ws1
    assert torch.equal(got2, ref2)


def test_noalloc_gate_up_matches_workspace_entry_point():
    need_gpu()
    wts, p = _setup()
    M, bs = 37, 16
    toks = gen.make_tokens(SPEC, M, seed_config=1204)
    _, ids_np = oracle.route(toks.logits, SPEC.topk, True)
    cap = wq.moe_align_capacity(M, SPEC.topk, SPEC.E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids_np).cuda(), SPEC.E, bs, cap)
    x = dev_u16(toks.x, "bf16")
    ref = torch.empty((cap, SPEC.N), dtype=torch.bfloat16, device="cuda")
    got = torch.full((cap, SPEC.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    say("no-alloc GATE_UP M=%d" % M)
    wq.moe_w8a16_gemm(wq.WQ_STAGE_GATE_UP, x, M, SPEC.topk, SPEC.E, 2 * SPEC.N, SPEC.K, p.w1, p.s1, st, ex, nt,
                      cap, bs, None, ref)
    wq.moe_w8a16_gemm_noalloc(wq.WQ_STAGE_GATE_UP, x, M, SPEC.topk, SPEC.E, 2 * SPEC.N, SPEC.K, p.w1, p.s1, st, ex,
                              nt, cap, bs, None, got)
    torch.cuda.synchronize()
    ntp = int(nt.cpu()[0])
    assert torch.equal(got[:ntp], ref[:ntp])


def test_noalloc_refuses_workspace_beyond_scratch():
    """A DOWN call whose workspace would exceed the scratch is refused before
    anything is launched (the buffers are never touched)."""
    need_gpu()
    wts, p = _setup()
    M, bs = 1 << 15, 128
    cap = wq.moe_align_capacity(M, SPEC.topk, SPEC.E, bs)
    ws = wq.moe_gemm_workspace_bytes(wq.WQ_STAGE_DOWN, M, SPEC.topk, SPEC.E, SPEC.K, SPEC.N, cap, False)
    assert ws > wq._lib.WQ_NOALLOC_SCRATCH_BYTES
    small = torch.empty(16, dtype=torch.int32, device="cuda")
    h = torch.empty((16, SPEC.N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((16, SPEC.K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(wq.WqError) as ei:
        wq.moe_w8a16_gemm_noalloc(wq.WQ_STAGE_DOWN, h, M, SPEC.topk, SPEC.E, SPEC.K, SPEC.N, p.w2, p.s2, small,
                                  small, small, cap, bs, small, out)
    assert ei.value.status == wq.WQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()
