"""Benchmark of the fused weight-only-quantized MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--m 1024]

A step is one pass of the hot path -- moe_route, moe_align, the fused gate/up
GEMM (SiLU*up epilogue) and the down GEMM with the routed weight and top-k
combine -- over one batch of M synthetic tokens whose inputs are already in
HBM.  The default workload is the Mixtral-8x7B-shaped W8A16 layer (E=8, top-2,
K=4096, N=14336, int8 per-column weights, bf16 activations) at M=1024, the
prompt length of the end-to-end latency workload in "[Kernel] W8A16 Int8
inside FusedMoE" (vLLM PR 7415, latency table).  The other batch sizes of that
layer's sweep are timed too and reported under "sweep"; the other workloads
(int4 act-order Mixtral, the 2:4-sparse int4 linear layer, the DeepSeek-V2
shaped int8 layer, the 2:4 layer with 8-bit codes, and the dense int4 linear
layer of the 2:4 layer's shape)
under "rows", with the ExpertsInt8 load-time quantizer on Mixtral's w1 (HBM
GB/s).

Timing: before every step (warm-up and timed) 1 GiB of scratch memory is
read (or, with --flush write, written), outside the timed span, so the
weights come from HBM and not from the 256 MB last-level cache -- a read
leaves the cache full of clean lines, as the other layers' weight reads of a
decode step do, where a write leaves dirty lines whose write-back then
competes with the first kernels' reads; each step is bracketed by stream events, and the
time per step is the mean over the K timed steps of its event span (route ->
combine).  Each batch is timed twice: launched call by call (which also gives
the per-stage split), and as one captured HIP graph replayed K times (the
same kernels without per-launch host work); the reported time per step is the
faster of the two, named in "launch" (the 2:4 and dense linear rows are timed
the same way).  The wall time of the K steps, flushes
included, is reported as well.

Printed: one JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (the gate/up GEMM, timed with stream events), and the CPU
oracle timed on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}   # dense
FLUSH_BYTES = 1 << 30
PackedFp8MoE = ()  # the FP8 layer's packed type, bound in main() once the package is imported
# rocprofv3 counter summary of the large-batch gate/up kernel at the default
# workload; its traffic figure is used only while the kernel sources hash the same
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_prefill_gate_up_mixtral_w8a16_m1024.md")
KERNEL_SOURCES = ("gemm_prefill.hip", "common.hpp")  # plus the kernel-argument part of launch.hpp


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 over the large-batch kernel's sources: gemm_prefill.hip,
    common.hpp, from launch.hpp the kernel-argument struct and the stage
    constants (the rest of that header declares other kernels), and the
    compiler flags of gemm_prefill.hip (the include path left out)."""
    csrc = os.path.join(ROOT, "weight_only_quantized_topk_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "launch.hpp")) as fh:
        text = fh.read()
    for part in re.findall(r"constexpr int STAGE_\w+ = \d+;", text) + re.findall(r"struct GemmArgs \{.*?\n\};", text, re.S):
        h.update(part.encode())
    from weight_only_quantized_topk_amd import build as _build
    h.update(" ".join(_build.FLAGS[:-2] + _build.SOURCE_FLAGS.get("gemm_prefill.hip", [])).encode())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary, or None when absent or taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    mh = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    mt = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not mh or not mt or mh.group(1) != kernel_source_hash():
        return None
    return int(mt.group(1))


def moe_alg_counts(spec, M, ids_np, packed):
    """Algorithmic bytes / flops of the gate/up GEMM launch and of the layer.
    Bytes: packed weights and scales of the experts the batch touches (plus the
    act-order permutation), the activations read and the outputs written (no
    padding rows, no re-reads, no H / Y round trips)."""
    touched = int(np.unique(ids_np).size)
    T = M * spec.topk
    E = spec.E
    act = 2
    fp8 = isinstance(packed, PackedFp8MoE)
    w1_bytes = packed.w1.numel() // E * touched
    s1_bytes = packed.s1.numel() * packed.s1.element_size() // E * touched
    w2_bytes = packed.w2.numel() // E * touched
    s2_bytes = packed.s2.numel() * packed.s2.element_size() // E * touched
    perm_bytes = touched * spec.K * 4 if getattr(spec, "act_order", False) else 0
    h_bytes = 1 if fp8 else act  # FP8 writes H as 1-byte codes
    g1 = {
        "bytes": w1_bytes + s1_bytes + M * spec.K * act + T * spec.N * h_bytes,
        "flops": 2 * T * (2 * spec.N) * spec.K,
    }
    layer = {
        "bytes": w1_bytes + s1_bytes + w2_bytes + s2_bytes + perm_bytes + 2 * M * spec.K * act,
        "flops": 6 * T * spec.N * spec.K,
    }
    return touched, g1, layer


def rates(nbytes, flops, ms, peak_tf=2500.0):
    """GB/s and TFLOP/s of a launch, with fractions of the HBM peak and of the
    dense MFMA peak of its data type (2.5 PFLOP/s bf16/fp16, 5.0 fp8)."""
    gbps = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    return {"GBps": gbps, "TFLOPs": tf, "frac_hbm": gbps / HBM_PEAK_GBPS, "frac_mfma": tf / peak_tf}


def rounded(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


class Timer:
    """Per-step stream events with a cache flush (1 GiB read, or write) before every step."""

    def __init__(self, torch, mode="read"):
        self.torch = torch
        self.mode = mode
        self.scratch = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        # a float32 sum reads the buffer once (an integer sum would first copy
        # it to int64, a 2 GiB write)
        self.words = self.scratch.view(torch.float32)
        self.n = 0

    def flush(self):
        self.n += 1
        if self.mode == "write":
            self.scratch.fill_(self.n & 0xFF)
        else:
            self.sink = self.words.sum()

    def run(self, step, steps, warmup, nmarks):
        """step(marks) runs one step, recording marks (a list of nmarks events) or
        nothing.  Returns (per-step span ms from the step start to each mark
        [steps, nmarks], wall ms of the timed loop per step)."""
        torch = self.torch
        for _ in range(warmup):
            self.flush()
            step(None)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nmarks + 1)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.flush()
            ev[i][0].record()
            step(ev[i][1:])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        spans = np.array([[e[0].elapsed_time(e[k]) for k in range(1, nmarks + 1)] for e in ev])
        return spans, wall


def host_cpu():
    """(CPU model name, physical cores, logical CPUs) of this host, from
    /proc/cpuinfo (physical cores = distinct (physical id, core id) pairs)."""
    model, cores, logical = "unknown", set(), 0
    try:
        phys = core = None
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "processor":
                    logical += 1
                elif k == "model name" and model == "unknown":
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return model, (len(cores) or None), (logical or os.cpu_count())


def cpu_baseline(spec, wts, toks, seconds):
    """The oracle, as it stands, on the first n tokens of the same batch (route +
    layer for those tokens), n chosen so the run takes about `seconds`.  It is
    compiled here with -O3 -march=native (same arithmetic as the test build) and
    runs OpenMP on OMP_NUM_THREADS threads (else one per logical CPU)."""
    import tempfile

    import oracle
    build_dir = tempfile.mkdtemp(prefix="wq_oracle_")
    oracle.use_native_build(build_dir)
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    model, phys_cores, logical = host_cpu()
    x = toks.x_f32()
    s1, s2 = wts.s1_f32(), wts.s2_f32()

    def run(n):
        t0 = time.perf_counter()
        w, ids = oracle.route(toks.logits[:n], spec.topk, spec.renormalize)
        oracle.moe_layer(x[:n], w, ids, wts.w1q, s1, wts.g1, wts.w2q, s2, wts.g2)
        return time.perf_counter() - t0

    n0 = int(min(toks.M, max(1, threads // spec.topk)))   # enough tokens to occupy every thread
    per = run(n0) / n0
    n = int(max(1, min(toks.M, seconds / max(per, 1e-6))))
    dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "route + layer for the first %d of the %d tokens of the timed batch, %.1f s, fp64 "
                      "accumulation, OpenMP over (token, slot, output row)" % (n, toks.M, dt),
            "cpu_model": model, "physical_cores": phys_cores, "logical_cpus": logical,
            "build": "gcc " + " ".join(oracle.NATIVE_FLAGS[:2] + ["-ffp-contract=off", "-fopenmp"])}


def cpu_table(seconds):
    """The oracle timed on this host for each configuration and batch size
    (cpu_baseline's sample rule: the first n tokens, n chosen for about
    `seconds`); the 2:4 layer by its oracle on the first n rows."""
    import gen
    out = []
    for cid in (1, 2, 3, 5):
        spec = gen.CONFIGS[cid]
        log("bench: cpu table: generating %s" % spec.name)
        wts = gen.make_moe_weights(spec)
        for m in spec.m_sweep:
            r = cpu_baseline(spec, wts, gen.make_tokens(spec, m), seconds)
            r.update(config=cid, workload=spec.name, M=m)
            log("bench: cpu table: %s M=%d %.2f tokens/s" % (spec.name, m, r["value"]))
            out.append(r)
        del wts
    import tempfile
    import oracle
    oracle.use_native_build(tempfile.mkdtemp(prefix="wq_oracle_"))
    spec = gen.CFG4
    log("bench: cpu table: generating %s" % spec.name)
    sw = gen.make_sparse_weights(spec)
    s_f32 = sw.s_f32()
    model, phys_cores, logical = host_cpu()
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    for m in spec.m_sweep:
        xf = gen.bits_to_f32("f16", gen.make_sparse_x(spec, m))

        def run(n):
            t0 = time.perf_counter()
            oracle.sparse24(xf[:n], sw.vals, sw.idx, s_f32, spec.group_size)
            return time.perf_counter() - t0

        per = run(1)
        n = int(max(1, min(m, seconds / max(per, 1e-6))))
        dt = run(n)
        out.append({"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                    "sample": "the first %d of the %d rows, %.1f s" % (n, m, dt), "cpu_model": model,
                    "physical_cores": phys_cores, "logical_cpus": logical, "config": 4, "workload": spec.name, "M": m})
        log("bench: cpu table: %s M=%d %.2f rows/s" % (spec.name, m, n / dt))
    return out


def measure_moe(torch, wq, gen, timer, spec, packed, m, steps, warmup):
    act = torch.float16 if spec.act == "f16" else torch.bfloat16
    toks = gen.make_tokens(spec, m)
    x = torch.from_numpy(toks.x.view(np.int16)).cuda().view(act)
    lg = torch.from_numpy(toks.logits).cuda()
    fp8 = isinstance(packed, PackedFp8MoE)
    runner = (wq.Fp8MoERunner if fp8 else wq.MoERunner)(packed, m, spec.topk, spec.renormalize)
    # the stage times: events recorded between route+align, GATE_UP and DOWN
    spans, wall = timer.run(lambda marks: runner(x, lg, marks=marks), steps, warmup, 3)
    ra, g1e = spans[:, 0], spans[:, 1] - spans[:, 0]
    down = spans[:, 2] - spans[:, 1]

    # the layer time launched eagerly: the same step with no event between its
    # stages (each recorded event is a packet the stream waits on)
    def plain(marks):
        runner(x, lg)
        if marks:
            marks[0].record()

    pspans, wall = timer.run(plain, steps, warmup, 1)
    lay = pspans[:, 0]
    # the same step replayed as one captured HIP graph (no per-launch host work)
    runner.capture(x, lg)

    def replay(marks):
        runner.replay()
        if marks:
            marks[0].record()

    gspans, gwall = timer.run(replay, steps, warmup, 1)
    graph_ms = float(gspans[:, 0].mean())
    ids_np = runner.ids.cpu().numpy()
    touched, g1, layer = moe_alg_counts(spec, m, ids_np, packed)
    eager_ms = float(lay.mean())
    ms = min(eager_ms, graph_ms)
    r = dict(M=m, ms_per_step=ms, launch="graph" if graph_ms <= eager_ms else "eager", eager_ms_per_step=eager_ms,
             graph_ms_per_step=graph_ms, ms_per_step_median=float(np.median(lay)), wall_ms_per_step=wall,
             graph_wall_ms_per_step=gwall,
             tokens_per_s=m / (ms * 1e-3), route_align_ms=float(ra.mean()), gate_up_ms=float(g1e.mean()),
             down_ms=float(down.mean()), touched_experts=touched, block_size=runner.bs,
             gate_up_alg_bytes=g1["bytes"], gate_up_alg_flops=g1["flops"],
             layer_alg_bytes=layer["bytes"], layer_alg_flops=layer["flops"])
    peak = MFMA_PEAK_TFLOPS["fp8" if fp8 else spec.act]
    r.update({"gate_up_" + k: v for k, v in rates(g1["bytes"], g1["flops"], r["gate_up_ms"], peak).items()})
    r.update({"layer_" + k: v for k, v in rates(layer["bytes"], layer["flops"], ms, peak).items()})
    return toks, r


def graph_run(torch, timer, call, steps, warmup):
    """call() (its tensors fixed) recorded once as a HIP graph and replayed:
    the per-replay event spans and wall time, as Timer.run returns them."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()

    def replay(marks):
        g.replay()
        if marks:
            marks[0].record()

    return timer.run(replay, steps, warmup, 1)


def eager_and_graph(torch, timer, call, steps, warmup):
    """Times call() launched eagerly and replayed as a graph; the faster one is
    the step time (named in "launch"), both are reported."""
    def step(marks):
        call()
        if marks:
            marks[0].record()

    spans, wall = timer.run(step, steps, warmup, 1)
    gspans, gwall = graph_run(torch, timer, call, steps, warmup)
    eager_ms, graph_ms = float(spans[:, 0].mean()), float(gspans[:, 0].mean())
    use_graph = graph_ms <= eager_ms
    sp = gspans if use_graph else spans
    return dict(ms_per_step=min(eager_ms, graph_ms), launch="graph" if use_graph else "eager",
                eager_ms_per_step=eager_ms, graph_ms_per_step=graph_ms,
                ms_per_step_median=float(np.median(sp[:, 0])), wall_ms_per_step=gwall if use_graph else wall)


def measure_sparse(torch, wq, gen, timer, spec, dev, m, steps, warmup):
    vd, md, sd = dev
    x = torch.from_numpy(gen.make_sparse_x(spec, m).view(np.int16)).cuda().view(torch.float16)
    y = torch.empty((m, spec.N), dtype=torch.float16, device="cuda")
    fn = wq.sparse24_w4a16_gemm if spec.bits == 4 else wq.sparse24_w8a16_gemm

    t = eager_and_graph(torch, timer, lambda: fn(x, vd, md, sd, spec.N, out=y), steps, warmup)
    ms = t["ms_per_step"]
    nbytes = vd.numel() + md.numel() + sd.numel() * 2 + m * spec.K * 2 + m * spec.N * 2
    flops = m * spec.N * spec.K   # nonzero multiply-adds x 2 = M*N*K for 2:4
    r = dict(M=m, **t, tokens_per_s=m / (ms * 1e-3), alg_bytes=int(nbytes), alg_flops=int(flops))
    r.update(rates(nbytes, flops, ms))
    return r


ROW_NAMES = ("mixtral-w4a16-actorder", "deepseekv2-w8a16", "mixtral-fp8-w8a8", "sparse24-w4a16", "sparse24-w8a16",
             "dense-w4a16", "quantize-w8")


def bench_row(name, torch, wq, gen, timer, steps, warmup, ms=None):
    """One of the other workloads at its batch sizes (or `ms`): layer time,
    stage times and both roofline fractions (HBM on algorithmic bytes, MFMA on
    algorithmic flops)."""
    out = []
    if name in ("mixtral-w4a16-actorder", "deepseekv2-w8a16", "mixtral-fp8-w8a8"):
        if name == "mixtral-fp8-w8a8":
            spec = gen.CFG_FP8  # the pages' comparison method, the same Mixtral shape and batch sizes
            log("bench: rows: generating and packing %s" % spec.name)
            fw = gen.make_fp8_weights(spec)
            packed = wq.pack_moe_fp8(fw.w1, fw.s1, fw.w2, fw.s2, torch.bfloat16, spec.a1, spec.a2)
            del fw
        else:
            spec = gen.CONFIGS[3 if name == "mixtral-w4a16-actorder" else 5]
            act = torch.float16 if spec.act == "f16" else torch.bfloat16
            log("bench: rows: generating and packing %s" % spec.name)
            wts = gen.make_moe_weights(spec)
            packed = wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2, act, spec.group_size, wts.g1, wts.g2)
            del wts
        for m in (ms or spec.m_sweep):
            _, r = measure_moe(torch, wq, gen, timer, spec, packed, m, steps, warmup)
            log("bench: rows: %s M=%d %.4f ms/step" % (spec.name, m, r["ms_per_step"]))
            out.append(dict(workload=spec.name, **rounded(r)))
        del packed
    elif name in ("sparse24-w4a16", "sparse24-w8a16"):
        spec = gen.CFG4 if name == "sparse24-w4a16" else gen.CFG4.with_(bits=8)  # 8-bit: the 2:4 support's variant
        log("bench: rows: generating and packing %s (%d-bit)" % (spec.name, spec.bits))
        sw = gen.make_sparse_weights(spec)
        vp, mp, sp = wq.pack_sparse24(sw.vals, sw.idx, sw.s, bits=spec.bits)
        dev = (torch.from_numpy(vp).cuda(), torch.from_numpy(mp).cuda(), torch.from_numpy(sp.view(np.int16)).cuda())
        for m in (ms or spec.m_sweep):
            r = measure_sparse(torch, wq, gen, timer, spec, dev, m, steps, warmup)
            log("bench: rows: %s %d-bit M=%d %.4f ms/step" % (spec.name, spec.bits, m, r["ms_per_step"]))
            out.append(dict(workload=spec.name if spec.bits == 4 else "yi34b-mlp-sparse24-w8a16", **rounded(r)))
        del dev
    elif name == "dense-w4a16":
        spec = gen.CFG4
        log("bench: rows: generating and packing the dense int4 layer")
        ddev = dense_weights(torch, wq, spec)
        for m in (ms or spec.m_sweep):
            r = measure_dense(torch, wq, gen, timer, spec, ddev, m, steps, warmup)
            log("bench: rows: dense M=%d %.4f ms/step" % (m, r["ms_per_step"]))
            out.append(dict(workload="yi34b-mlp-dense-w4a16", **rounded(r)))
        del ddev
    elif name == "quantize-w8":
        out.append(dict(workload="experts-int8-quantize-mixtral-w1", **rounded(measure_quant(torch, wq, timer, steps,
                                                                                             warmup))))
        log("bench: rows: quantizer %.4f ms" % out[-1]["ms_per_step"])
    else:
        raise ValueError("unknown row %r (one of %s)" % (name, ", ".join(ROW_NAMES)))
    torch.cuda.empty_cache()
    return out


def bench_rows(torch, wq, gen, timer, steps, warmup):
    rows = []
    for name in ROW_NAMES:
        rows += bench_row(name, torch, wq, gen, timer, steps, warmup)
    return rows


def dense_weights(torch, wq, spec):
    """Dense int4 weights of the 2:4 layer's shape (N x K, group-128 fp16
    scales), seeded uniform codes in [-8, 7] and scales in [0.005, 0.02]."""
    rng = np.random.default_rng([20240807, spec.K, spec.N])
    q = rng.integers(-8, 8, size=(1, spec.N, spec.K), dtype=np.int8)
    s = rng.uniform(0.005, 0.02, size=(1, spec.K // 128, spec.N)).astype(np.float16).view(np.uint16)
    packed, sp, _ = wq.pack_w4(q, s, 128)
    return torch.from_numpy(packed).cuda(), torch.from_numpy(sp.view(np.int16)).cuda()


def measure_dense(torch, wq, gen, timer, spec, dev, m, steps, warmup):
    """The dense int4 linear layer of the same shape as the 2:4 one (the pages
    set Marlin-24 beside dense Marlin): bytes = packed weights + scales + x + y."""
    wd, sd = dev
    x = torch.from_numpy(gen.make_sparse_x(spec, m).view(np.int16)).cuda().view(torch.float16)
    y = torch.empty((m, spec.N), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(1, wq.dense_gemm_workspace_bytes(m, spec.K, spec.N)), dtype=torch.uint8, device="cuda")

    t = eager_and_graph(torch, timer, lambda: wq.dense_w4a16_gemm(x, spec.N, wd, sd, 128, out=y, workspace=ws),
                        steps, warmup)
    ms = t["ms_per_step"]
    nbytes = wd.numel() + sd.numel() * 2 + m * spec.K * 2 + m * spec.N * 2
    flops = 2 * m * spec.N * spec.K
    r = dict(M=m, **t, tokens_per_s=m / (ms * 1e-3), alg_bytes=int(nbytes), alg_flops=int(flops))
    r.update(rates(nbytes, flops, ms))
    return r


def measure_quant(torch, wq, timer, steps, warmup):
    """The ExpertsInt8 load-time quantizer on Mixtral-8x7B's w1 (8 experts x
    28672 output columns x 4096 bf16 weights, seeded normal x 0.02): HBM-bound,
    2 bytes read and 1 written per weight."""
    E, n_out, k = 8, 2 * 14336, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(20240807)
    w = (torch.randn((E, n_out, k), generator=g, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
    q = torch.empty(w.shape, dtype=torch.int8, device="cuda")
    sc = torch.empty(w.shape[:-1], dtype=torch.bfloat16, device="cuda")

    def step(marks):
        wq.quantize_w8(w, q, sc)
        if marks:
            marks[0].record()

    spans, wall = timer.run(step, steps, warmup, 1)
    ms = float(spans[:, 0].mean())
    nbytes = E * n_out * k * 3 + E * n_out * 2
    r = dict(M=0, ms_per_step=ms, ms_per_step_median=float(np.median(spans[:, 0])), wall_ms_per_step=wall,
             alg_bytes=int(nbytes), alg_flops=0, shape=[E, n_out, k])
    r.update(rates(nbytes, 0, ms))
    del w, q, sc
    torch.cuda.empty_cache()
    return r


def summarize_counters(paths, calib_kernel="__amd_rocclr_copyBuffer", calib_bytes=None):
    """Counter summary of rocprofv3 --pmc CSV files (counter_collection.csv):
    per (kernel, grid size), the mean value per dispatch of every counter.
    With calib_bytes (the bytes one dispatch of calib_kernel moves), FETCH_SIZE
    and WRITE_SIZE (KiB) are also scaled by known_KiB / counted_KiB of that
    kernel (the calibration copy of --copy-calibration) and given in bytes."""
    import csv
    from collections import defaultdict
    acc = defaultdict(lambda: defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]))
                acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    scale = {}
    if calib_bytes:
        # the calibration copy is the calib_kernel dispatch with the largest count
        # (the runtime also copies small host buffers with it)
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            counted = [float(np.mean(cs[c])) for (name, _, _), cs in acc.items() if name.startswith(calib_kernel) and c in cs]
            if counted and max(counted) > 0:
                scale[c] = (calib_bytes / 1024.0) / max(counted)
    out = []
    for (name, grid, wg), counters in sorted(acc.items(), key=lambda kv: kv[0]):
        row = {"kernel": name, "grid": grid, "workgroup": wg}
        for c, v in sorted(counters.items()):
            row[c] = float(np.mean(v))
            row[c + "_dispatches"] = len(v)
            if c in scale:
                row[c + "_bytes"] = row[c] * 1024.0 * scale[c]
                row[c + "_scale"] = scale[c]
        out.append(row)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 5])
    ap.add_argument("--m", type=int, default=None, help="batch size (default: the largest of the config's sweep)")
    ap.add_argument("--no-sweep", action="store_true", help="time only --m of the chosen workload")
    ap.add_argument("--no-rows", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="how the last-level cache is emptied before every step (1 GiB read or written)")
    ap.add_argument("--row", choices=ROW_NAMES, default=None,
                    help="time only this one of the other workloads (at --m, else its batch sizes) and print its "
                         "results as one JSON line (for profiling a single kernel)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a device-to-device copy of MIB MiB twice: the known-size reference that "
                         "scales hardware byte counters (FETCH_SIZE / WRITE_SIZE) read under a profiler")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV", default=None,
                    help="print a per-kernel summary (one JSON line per kernel and grid) of rocprofv3 --pmc CSV "
                         "files and exit; FETCH_SIZE / WRITE_SIZE are scaled by the --copy-calibration copy "
                         "when --calib-mib gives its size")
    ap.add_argument("--calib-mib", type=int, default=None, help="size of the calibration copy (MiB)")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the oracle on this host for every configuration and batch size (about "
                         "--cpu-seconds each, on a sample of the batch where the whole would take longer) "
                         "and print one JSON line; no GPU is used")
    args = ap.parse_args(argv)

    if args.cpu_table:
        print(json.dumps({"cpu_table": cpu_table(args.cpu_seconds)}), flush=True)
        return 0

    if args.summarize_counters:
        for row in summarize_counters(args.summarize_counters,
                                      calib_bytes=(args.calib_mib << 20) if args.calib_mib else None):
            print(json.dumps(row))
        return 0

    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU; --gpus %d is not supported (the layer is not sharded "
              "across GPUs: expert- or tensor-parallel sharding is a design, not code)." % args.gpus,
              file=sys.stderr)
        return 2

    import torch
    import gen
    import weight_only_quantized_topk_amd as wq
    global PackedFp8MoE
    PackedFp8MoE = wq.PackedFp8MoE

    wq.load()  # fails loudly without the HIP library
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copied %d bytes twice (counter calibration)" % n)
        del src, dst
    timer = Timer(torch, args.flush)
    if args.row:
        res = bench_row(args.row, torch, wq, gen, timer, args.steps, args.warmup, [args.m] if args.m else None)
        print(json.dumps({"row": args.row, "results": res}), flush=True)
        return 0
    spec = gen.CONFIGS[args.config]
    M = args.m or max(spec.m_sweep)
    act = torch.float16 if spec.act == "f16" else torch.bfloat16
    log("bench: generating and packing %s" % spec.name)
    wts = gen.make_moe_weights(spec)
    packed = wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2, act, spec.group_size, wts.g1, wts.g2)
    torch.cuda.synchronize()

    log("bench: timing M=%d, %d steps after %d warmup" % (M, args.steps, args.warmup))
    toks, head = measure_moe(torch, wq, gen, timer, spec, packed, M, args.steps, args.warmup)
    log("bench: M=%d %.4f ms/step" % (M, head["ms_per_step"]))

    sweep = []
    if not args.no_sweep:
        for m in spec.m_sweep:
            if m == M:
                continue
            _, r = measure_moe(torch, wq, gen, timer, spec, packed, m, max(10, args.steps), args.warmup)
            log("bench: sweep M=%d %.4f ms/step" % (m, r["ms_per_step"]))
            sweep.append(r)
        sweep.append(head)
        sweep.sort(key=lambda r: r["M"])

    # roofline of the dominant kernel (the gate/up GEMM): HBM-bound at small M,
    # MFMA-bound at large M (arithmetic intensity vs the ridge point)
    intensity = head["gate_up_alg_flops"] / head["gate_up_alg_bytes"]
    peak_f = MFMA_PEAK_TFLOPS[spec.act]
    ridge = peak_f * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if intensity >= ridge:
        achieved = head["gate_up_TFLOPs"]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(achieved / peak_f, 4)}
    else:
        achieved = head["gate_up_GBps"]
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    large = head["block_size"] >= 64
    roof["kernel"] = "gemm_%s_kernel, gate/up stage (W%dA16)" % ("prefill" if large else "decode", spec.bits)
    roof["kernel_avg_ms"] = round(head["gate_up_ms"], 4)
    roof["alg_bytes_per_launch"] = int(head["gate_up_alg_bytes"])
    roof["alg_flops_per_launch"] = int(head["gate_up_alg_flops"])
    default_workload = args.config == 2 and M == 1024
    roof["traffic"] = stored_traffic() if (default_workload and large) else None

    rows = None
    if not args.no_rows:
        del packed, wts
        torch.cuda.empty_cache()
        rows = bench_rows(torch, wq, gen, timer, max(10, args.steps), args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        wts_cpu = gen.make_moe_weights(spec) if not args.no_rows else wts
        cpu = cpu_baseline(spec, wts_cpu, toks, args.cpu_seconds)

    res = {
        # the headline metric: layer tokens/s; the HBM GB/s (M <= 64) and
        # TFLOP/s (M >= 1024) figures are in "roofline", "sweep" and "rows"
        "metric": "fused-MoE W4/W8A16 tokens/s; HBM GB/s at M\u226464, TFLOP/s at M\u22651024",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "wall_ms_per_step": round(head["wall_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.act,
        "data": "synthetic",
        "config": {"workload": "%s MoE layer, E=%d top-%d K=%d N=%d, %s weights, M=%d tokens"
                               % (spec.name, spec.E, spec.topk, spec.K, spec.N,
                                  "int8 per-column" if spec.bits == 8 else "int4 group-128", M),
                   "M": M, "E": spec.E, "topk": spec.topk, "K": spec.K, "N": spec.N, "bits": spec.bits,
                   "block_size": head["block_size"], "touched_experts": head["touched_experts"],
                   "launch": head["launch"],
                   "cache": "1 GiB scratch %s before every step, outside the timed span"
                            % ("written" if args.flush == "write" else "read")},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": {"GBps": round(head["layer_GBps"], 1), "TFLOPs": round(head["layer_TFLOPs"], 2),
                  "alg_bytes": int(head["layer_alg_bytes"]), "alg_flops": int(head["layer_alg_flops"])},
        "sweep": [rounded(r) for r in sweep],
        "rows": rows,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
