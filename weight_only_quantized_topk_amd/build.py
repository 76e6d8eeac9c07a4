"""Build libwqmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m weight_only_quantized_topk_amd.build

Each source is compiled with hipcc into _build/, then linked into
weight_only_quantized_topk_amd/libwqmoe.so next to this file; the streaming
read probe (csrc/stream_probe.hip) is built into the program stream_probe
beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwqmoe.so")
# a standalone program (not part of the library): the plain streaming-read
# bandwidth the weight-streaming kernels are read against
PROBE_SRC = "stream_probe.hip"
PROBE = os.path.join(HERE, "stream_probe")
SOURCES = ["abi.cpp", "route_align.hip", "gemm_decode.hip", "gemm_prefill.hip", "gemm_prefill_n256.hip", "sparse24.hip", "quant.hip", "dense_decode.hip", "gemm_tiny.hip", "gemm_fp8.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 arithmetic in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# per-source flags.  WQ_PREFILL_SCHED=iterative-ilp builds the large-batch
# GEMM (gemm_prefill.hip) under LLVM's iterative ILP scheduling strategy
# instead of the default one.  An A/B of the two on two MI355X boxes, three
# alternating runs each, found the default scheduler as fast or faster:
# Mixtral int8 M=1024 gate/up 0.450 vs 0.453 ms and 0.457 vs 0.459 ms, int4
# act-order M=4096 gate/up 1.754 vs 1.818 ms (layer 2.74 vs 2.86 ms).
PREFILL_SCHED = os.environ.get("WQ_PREFILL_SCHED", "default")
if PREFILL_SCHED not in ("iterative-ilp", "default"):
    raise ValueError("WQ_PREFILL_SCHED must be 'iterative-ilp' or 'default', got %r" % PREFILL_SCHED)
SOURCE_FLAGS = ({"gemm_prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}
                if PREFILL_SCHED == "iterative-ilp" else {})


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    ptmp = PROBE + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", ptmp, os.path.join(CSRC, PROBE_SRC)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (PROBE_SRC, r.stdout + r.stderr))
    os.replace(ptmp, PROBE)
    if verbose:
        print("built", LIB, "and", PROBE)
    return LIB


if __name__ == "__main__":
    build()
