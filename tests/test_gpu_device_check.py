"""Foreign pointers are refused before anything is launched.

The second-device illegal access in moe_align_block_size_kernel ("Marlin moe
integration", nm-vllm PR 266, review thread) is what the library's device check
guards against: every hot-path call takes device memory of the current device
only and answers anything else with WQ_ERR_DEVICE.  One GPU shows it with host
memory: the buffers handed over here are pinned host tensors, which the GPU
could read without faulting even if the check were missing, so a broken check
shows up as a wrong status or a written output, never as a fault.  Every
output buffer is filled with a sentinel first and must still hold it."""
import numpy as np
import pytest

import gen
import oracle
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, need_gpu, say, torch

pytestmark = pytest.mark.gpu

W8 = gen.CFG2.with_(name="w8-devcheck", E=8, topk=2, K=512, N=384)
W4 = gen.CFG3.with_(name="w4-devcheck", E=8, topk=2, K=512, N=384, act_order=False)


def pinned(t):
    """A pinned host copy of a tensor (mapped for the GPU, so never a fault)."""
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t.cpu())
    assert h.is_pinned() and not h.is_cuda
    return h


def expect_device_error(call, what):
    say("device check:", what)
    with pytest.raises(wq.WqError) as ei:
        call()
    torch.cuda.synchronize()
    assert ei.value.status == wq.WQ_ERR_DEVICE, "%s: status %d (%s)" % (what, ei.value.status, ei.value)


def test_route_and_align_refuse_host_memory():
    need_gpu()
    M, E, topk, bs = 37, 8, 2, 16
    rng = np.random.default_rng(31)
    logits = torch.from_numpy(rng.standard_normal((M, E)).astype(np.float32)).cuda()
    w = torch.full((M, topk), -7.0, device="cuda")
    ids = torch.full((M, topk), -7, dtype=torch.int32, device="cuda")
    expect_device_error(lambda: wq.moe_route(pinned(logits), topk, True, w, ids), "moe_route, host logits")
    assert bool((w == -7.0).all()) and bool((ids == -7).all())
    # a host output buffer is refused the same way
    w_host = pinned(w)
    expect_device_error(lambda: wq.moe_route(logits, topk, True, w_host, ids), "moe_route, host topk_weights")
    assert bool((w_host == -7.0).all()) and bool((ids == -7).all())

    _, ids_ref = oracle.route(logits.cpu().numpy(), topk, True)
    cap = wq.moe_align_capacity(M, topk, E, bs)
    st = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    ex = torch.full((cap // bs,), -7, dtype=torch.int32, device="cuda")
    nt = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    host_ids = pinned(torch.from_numpy(ids_ref))
    expect_device_error(lambda: wq.moe_align(host_ids, E, bs, cap, st, ex, nt), "moe_align, host topk_ids")
    for t in (st, ex, nt):
        assert bool((t == -7).all())
    st_host = pinned(st)
    expect_device_error(lambda: wq.moe_align(torch.from_numpy(ids_ref).cuda(), E, bs, cap, st_host, ex, nt),
                        "moe_align, host sorted_token_ids")
    assert bool((st_host == -7).all()) and bool((ex == -7).all())


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("stage", [wq.WQ_STAGE_GATE_UP, wq.WQ_STAGE_DOWN])
def test_moe_gemm_refuses_host_memory(bits, stage):
    need_gpu()
    spec = W8 if bits == 8 else W4
    wts = gen.make_moe_weights(spec, seed_config=40 + bits)
    p = wq.pack_moe(bits, wts.w1q, wts.s1, wts.w2q, wts.s2, torch.bfloat16 if bits == 8 else torch.float16,
                    spec.group_size)
    M, bs = 37, 16
    toks = gen.make_tokens(spec, M, seed_config=41)
    w_np, ids_np = oracle.route(toks.logits, spec.topk, True)
    cap = wq.moe_align_capacity(M, spec.topk, spec.E, bs)
    st, ex, nt = wq.moe_align(torch.from_numpy(ids_np).cuda(), spec.E, bs, cap)
    x = dev_u16(toks.x, spec.act)
    if stage == wq.WQ_STAGE_GATE_UP:
        a, n_out, k_in, w_pk, s_pk, tw = x, 2 * spec.N, spec.K, p.w1, p.s1, None
        out = torch.full((cap, spec.N), 3.0, dtype=p.act, device="cuda")
    else:
        a = torch.zeros((cap, spec.N), dtype=p.act, device="cuda")
        n_out, k_in, w_pk, s_pk = spec.K, spec.N, p.w2, p.s2
        tw = torch.from_numpy(w_np).cuda()
        out = torch.full((M, spec.K), 3.0, dtype=p.act, device="cuda")
    ws = wq.moe_gemm_workspace_bytes(stage, M, spec.topk, spec.E, n_out, k_in, cap, False)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None

    def call(a_=a, w_=w_pk, st_=st, out_=out):
        if bits == 8:
            wq.moe_w8a16_gemm(stage, a_, M, spec.topk, spec.E, n_out, k_in, w_, s_pk, st_, ex, nt, cap, bs, tw, out_,
                              work, act_dtype=p.act_code)
        else:
            wq.moe_w4a16_gemm(stage, a_, M, spec.topk, spec.E, n_out, k_in, w_, s_pk, spec.group_size, None, st_,
                              ex, nt, cap, bs, tw, out_, work)

    name = "moe_w%da16_gemm stage %d" % (bits, stage)
    expect_device_error(lambda: call(a_=pinned(a)), name + ", host activations")
    expect_device_error(lambda: call(w_=pinned(w_pk)), name + ", host weights")
    expect_device_error(lambda: call(st_=pinned(st)), name + ", host sorted_token_ids")
    assert bool((out == 3.0).all())
    out_host = pinned(out)
    expect_device_error(lambda: call(out_=out_host), name + ", host output")
    assert bool((out_host == 3.0).all())
    # the same call on device memory runs
    call()
    torch.cuda.synchronize()
    assert not bool((out == 3.0).all())


@pytest.mark.parametrize("bits", [8, 4])
def test_route_gate_up_refuses_host_memory(bits):
    """moe_route_gate_up (one kernel at this size) refuses host logits, host
    routing outputs and a host H buffer, and writes nothing."""
    need_gpu()
    spec = W8 if bits == 8 else W4
    wts = gen.make_moe_weights(spec, seed_config=50 + bits)
    p = wq.pack_moe(bits, wts.w1q, wts.s1, wts.w2q, wts.s2, torch.bfloat16 if bits == 8 else torch.float16,
                    spec.group_size)
    M, bs = 2, 16
    toks = gen.make_tokens(spec, M, seed_config=51)
    cap = wq.moe_align_capacity(M, spec.topk, spec.E, bs)
    x = dev_u16(toks.x, spec.act)
    lg = torch.from_numpy(toks.logits).cuda()
    w = torch.full((M, spec.topk), -7.0, device="cuda")
    ids = torch.full((M, spec.topk), -7, dtype=torch.int32, device="cuda")
    st = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    ex = torch.full((cap // bs,), -7, dtype=torch.int32, device="cuda")
    nt = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    h = torch.full((cap, spec.N), 3.0, dtype=p.act, device="cuda")
    gs = spec.group_size if bits == 4 else -1

    def call(lg_=lg, w_=w, st_=st, h_=h):
        wq.moe_route_gate_up(bits, lg_, True, w_, ids, x, M, spec.topk, spec.E, 2 * spec.N, spec.K, p.w1, p.s1, gs,
                             None, st_, ex, nt, cap, bs, h_, None, None, p.act_code)

    name = "moe_route_gate_up w%d" % bits
    expect_device_error(lambda: call(lg_=pinned(lg)), name + ", host logits")
    expect_device_error(lambda: call(w_=pinned(w)), name + ", host topk_weights")
    expect_device_error(lambda: call(st_=pinned(st)), name + ", host sorted_token_ids")
    h_host = pinned(h)
    expect_device_error(lambda: call(h_=h_host), name + ", host H")
    assert bool((h_host == 3.0).all())
    for t in (w, ids, st, ex, nt):
        assert bool((t == -7).all())
    assert bool((h == 3.0).all())
    call()
    torch.cuda.synchronize()
    assert int(nt[0]) > 0 and not bool((h == 3.0).all())


def test_sparse24_and_dense_refuse_host_memory():
    need_gpu()
    spec = gen.CFG4.with_(name="sparse-devcheck", K=512, N=256)
    sw = gen.make_sparse_weights(spec, seed_config=42)
    vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s)
    vd, md = torch.from_numpy(vp).cuda(), torch.from_numpy(mp).cuda()
    sd = torch.from_numpy(sp.view(np.int16)).cuda()
    M = 5
    x = torch.from_numpy(gen.make_sparse_x(spec, M).view(np.int16)).cuda().view(torch.float16)
    y = torch.full((M, spec.N), 3.0, dtype=torch.float16, device="cuda")
    for fn in (wq.sparse24_w4a16_gemm,):
        expect_device_error(lambda: fn(pinned(x), vd, md, sd, spec.N, out=y), "sparse24, host x")
        expect_device_error(lambda: fn(x, pinned(vd), md, sd, spec.N, out=y), "sparse24, host values")
        expect_device_error(lambda: fn(x, vd, pinned(md), sd, spec.N, out=y), "sparse24, host metadata")
    assert bool((y == 3.0).all())

    rng = np.random.default_rng(43)
    q = rng.integers(-8, 8, size=(1, spec.N, spec.K), dtype=np.int8)
    s = gen.round_to("f16", rng.uniform(0.005, 0.02, size=(1, spec.K // 128, spec.N)).astype(np.float32))
    packed, spk, _ = wq.pack_w4(q, s, 128)
    wd, sdd = torch.from_numpy(packed).cuda(), torch.from_numpy(spk.view(np.int16)).cuda()
    for m in (2, 40):  # the one-kernel small-batch path and the grouped path with a workspace
        xm = torch.from_numpy(gen.make_sparse_x(spec, m).view(np.int16)).cuda().view(torch.float16)
        ym = torch.full((m, spec.N), 3.0, dtype=torch.float16, device="cuda")
        nb = wq.dense_gemm_workspace_bytes(m, spec.K, spec.N)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        expect_device_error(lambda: wq.dense_w4a16_gemm(pinned(xm), spec.N, wd, sdd, 128, out=ym, workspace=ws),
                            "dense_w4a16_gemm M=%d, host x" % m)
        expect_device_error(lambda: wq.dense_w4a16_gemm(xm, spec.N, pinned(wd), sdd, 128, out=ym, workspace=ws),
                            "dense_w4a16_gemm M=%d, host weights" % m)
        if nb:
            expect_device_error(lambda: wq.dense_w4a16_gemm(xm, spec.N, wd, sdd, 128, out=ym,
                                                            workspace=pinned(ws)),
                                "dense_w4a16_gemm M=%d, host workspace" % m)
        assert bool((ym == 3.0).all())
