"""Benchmark of the fused weight-only-quantized MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--m 1024]

A step is one pass of the hot path -- moe_route, moe_align, the fused gate/up
GEMM (SiLU*up epilogue) and the down GEMM with the routed weight and top-k
combine -- over one batch of M synthetic tokens whose inputs are already in
HBM.  The default workload is the Mixtral-8x7B-shaped W8A16 layer (E=8, top-2,
K=4096, N=14336, int8 per-column weights, bf16 activations) at M=1024, the
prompt length of the end-to-end latency workload in "[Kernel] W8A16 Int8
inside FusedMoE" (vLLM PR 7415, latency table).  The other batch sizes of that
layer's sweep are timed too and reported under "sweep".

Printed: one JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (the gate/up GEMM, timed with stream events over the timed
steps), and the CPU oracle timed on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # dense
SPARSE_NOTE = "2:4 counts nonzero flops against the dense peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def moe_alg_counts(spec, M, ids_np, packed):
    """Algorithmic bytes / flops of the gate/up GEMM launch and of the layer.
    Bytes: packed weights and scales of the experts the batch touches, the
    activations read and the outputs written (no padding rows, no re-reads)."""
    touched = int(np.unique(ids_np).size)
    T = M * spec.topk
    E = spec.E
    act = 2
    w1_bytes = packed.w1.numel() // E * touched
    s1_bytes = packed.s1.numel() * 2 // E * touched
    w2_bytes = packed.w2.numel() // E * touched
    s2_bytes = packed.s2.numel() * 2 // E * touched
    g1 = {
        "bytes": w1_bytes + s1_bytes + M * spec.K * act + T * spec.N * act,
        "flops": 2 * T * (2 * spec.N) * spec.K,
    }
    layer = {
        "bytes": w1_bytes + s1_bytes + w2_bytes + s2_bytes + 2 * M * spec.K * act,
        "flops": 6 * T * spec.N * spec.K,
    }
    return touched, g1, layer


def time_layer(torch, runner, x, lg, steps, warmup):
    """Warm up, then time exactly `steps` steps between two synchronisations;
    stream events after alignment / gate-up / down give per-stage durations."""
    for _ in range(warmup):
        runner(x, lg)
    torch.cuda.synchronize()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        runner(x, lg, marks=marks[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    g1 = np.array([m[0].elapsed_time(m[1]) for m in marks])     # ms
    g2 = np.array([m[1].elapsed_time(m[2]) for m in marks])
    return (t1 - t0) * 1e3 / steps, float(g1.mean()), float(g2.mean())


def cpu_baseline(spec, wts, toks, seconds):
    """The oracle, as it stands, on the first n tokens of the same batch (route +
    layer for those tokens), n chosen so the run takes about `seconds`."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
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
                      "accumulation, OpenMP over (token, slot, output row)" % (n, toks.M, dt)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 5])
    ap.add_argument("--m", type=int, default=None, help="batch size (default: the largest of the config's sweep)")
    ap.add_argument("--no-sweep", action="store_true", help="time only --m")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU (one MI355X per box); --gpus %d is not supported. "
              "Expert- or tensor-parallel sharding is described in the design notes but not run." % args.gpus,
              file=sys.stderr)
        return 2

    import torch
    import gen
    import weight_only_quantized_topk_amd as wq

    wq.load()  # fails loudly without the HIP library
    torch.cuda.set_device(0)
    spec = gen.CONFIGS[args.config]
    M = args.m or max(spec.m_sweep)
    act = torch.float16 if spec.act == "f16" else torch.bfloat16
    log("bench: generating and packing %s" % spec.name)
    wts = gen.make_moe_weights(spec)
    packed = wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2, act, spec.group_size, wts.g1, wts.g2)
    torch.cuda.synchronize()

    def measure(m, steps, warmup):
        toks = gen.make_tokens(spec, m)
        x = torch.from_numpy(toks.x.view(np.int16)).cuda().view(act)
        lg = torch.from_numpy(toks.logits).cuda()
        runner = wq.MoERunner(packed, m, spec.topk, spec.renormalize)
        ms, g1_ms, g2_ms = time_layer(torch, runner, x, lg, steps, warmup)
        ids_np = runner.ids.cpu().numpy()
        touched, g1, layer = moe_alg_counts(spec, m, ids_np, packed)
        return toks, ids_np, dict(M=m, ms_per_step=ms, tokens_per_s=m / (ms * 1e-3), gate_up_ms=g1_ms,
                                  down_ms=g2_ms, touched_experts=touched, block_size=runner.bs,
                                  gate_up_alg_bytes=g1["bytes"], gate_up_alg_flops=g1["flops"],
                                  layer_alg_bytes=layer["bytes"], layer_alg_flops=layer["flops"],
                                  gate_up_GBps=g1["bytes"] / (g1_ms * 1e-3) / 1e9,
                                  gate_up_TFLOPs=g1["flops"] / (g1_ms * 1e-3) / 1e12,
                                  layer_GBps=layer["bytes"] / (ms * 1e-3) / 1e9,
                                  layer_TFLOPs=layer["flops"] / (ms * 1e-3) / 1e12)

    log("bench: timing M=%d, %d steps after %d warmup" % (M, args.steps, args.warmup))
    toks, ids_np, head = measure(M, args.steps, args.warmup)
    log("bench: M=%d %.3f ms/step" % (M, head["ms_per_step"]))

    sweep = []
    if not args.no_sweep:
        for m in spec.m_sweep:
            if m == M:
                continue
            _, _, r = measure(m, max(10, args.steps), args.warmup)
            log("bench: sweep M=%d %.3f ms/step" % (m, r["ms_per_step"]))
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
    roof["kernel"] = "gemm_%s_kernel gate/up (W%dA16)" % ("prefill" if head["block_size"] >= 64 else "decode",
                                                        spec.bits)
    roof["kernel_avg_ms"] = round(head["gate_up_ms"], 4)
    roof["alg_bytes_per_launch"] = int(head["gate_up_alg_bytes"])
    roof["alg_flops_per_launch"] = int(head["gate_up_alg_flops"])
    roof["traffic"] = None

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(spec, wts, toks, args.cpu_seconds)

    res = {
        "metric": "fused-MoE W%dA16 tokens/s" % spec.bits,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.act,
        "data": "synthetic",
        "config": {"workload": "%s MoE layer, E=%d top-%d K=%d N=%d, %s weights, M=%d tokens"
                               % (spec.name, spec.E, spec.topk, spec.K, spec.N,
                                  "int8 per-column" if spec.bits == 8 else "int4 group-128", M),
                   "M": M, "E": spec.E, "topk": spec.topk, "K": spec.K, "N": spec.N, "bits": spec.bits,
                   "block_size": head["block_size"], "touched_experts": head["touched_experts"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": {"GBps": round(head["layer_GBps"], 1), "TFLOPs": round(head["layer_TFLOPs"], 2),
                  "alg_bytes": int(head["layer_alg_bytes"]), "alg_flops": int(head["layer_alg_flops"])},
        "sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in sweep],
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
