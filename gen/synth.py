"""Seeded synthetic inputs for the weight-only-quantized top-k MoE layer and the
2:4-sparse W4A16 linear layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It draws canonical *logical* tensors only (integer codes, scales,
group indices, 2:4 keep positions, activations, router logits). It contains none
of the method's arithmetic: no dequantisation, no routing, no matmul.

Sources for the shapes and value distributions:
  * "[Kernel] W8A16 Int8 inside FusedMoE" (vLLM PR 7415), opening description:
    symmetric int8 per expert and per output column.
  * "Marlin moe integration" (nm-vllm PR 266), opening description: GPTQ 4-bit,
    group 128, with and without act-order.
  * "Add GPTQ Marlin 2:4 sparse structured support" (vLLM PR 4790), opening
    description: group size 128, 4-bit values, Yi-34B.
Workload sizes (Mixtral-8x7B, Yi-34B MLP, DeepSeek-V2 experts) follow the model
shapes those threads run.

Seeding: numpy PCG64 with SeedSequence([2026, config_id, M_or_0, stream]);
stream 0 = weights (M_or_0 = 0, so one weight set serves a whole M sweep),
1 = activations, 2 = router logits. Draw order for MoE weights: w1q, s1, g1,
w2q, s2, g2; for the sparse layer: keep positions, values, scales.

Float16 values are rounded from float32 draws with numpy's round-to-nearest-even
cast; bfloat16 values are rounded from float32 with round-to-nearest-even on the
bit pattern. Both sides of every comparison see identical rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

SEED_ROOT = 2026
STREAM_WEIGHTS, STREAM_X, STREAM_LOGITS = 0, 1, 2


# ----------------------------------------------------------------------------
# 16-bit float helpers (representation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns.
    Inputs are finite by construction here."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def round_to(act: str, a: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bit patterns of the 16-bit type `act` ('f16' | 'bf16')."""
    return f32_to_f16_bits(a) if act == "f16" else f32_to_bf16_bits(a)


def bits_to_f32(act: str, b: np.ndarray) -> np.ndarray:
    return f16_bits_to_f32(b) if act == "f16" else bf16_bits_to_f32(b)


def rng_for(config_id: int, m_or_0: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, config_id, m_or_0, stream])))


# ----------------------------------------------------------------------------
# MoE layer specification
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class MoESpec:
    """One MoE layer configuration.

    bits        4 (int4 codes in [-8, 7]) or 8 (int8 codes in [-127, 127])
    group_size  >0: scales per group of `group_size` input channels along each
                GEMM's reduction dimension; -1: one scale per output column
    act_order   GPTQ act-order: input channels quantised in a seeded permuted
                order; g_idx[k] = perm[k] // group_size
    act         activation and scale dtype: 'f16' or 'bf16'
    zipf_s      if set, add log(p_e) with p_e ~ (e+1)^-s to every router logit
    """
    name: str
    config_id: int
    bits: int
    E: int
    topk: int
    K: int
    N: int
    group_size: int
    act_order: bool
    act: str
    scale_lo: float
    scale_hi: float
    renormalize: bool = True
    zipf_s: Optional[float] = None
    m_sweep: Tuple[int, ...] = field(default_factory=tuple)

    @property
    def qmin(self) -> int:
        return -8 if self.bits == 4 else -127

    @property
    def qmax(self) -> int:
        return 7 if self.bits == 4 else 127

    def groups(self, k_in: int) -> int:
        return 1 if self.group_size == -1 else k_in // self.group_size

    def with_(self, **kw) -> "MoESpec":
        return replace(self, **kw)


@dataclass(frozen=True)
class SparseSpec:
    """2:4-structured-sparse W4A16 dense linear layer y = x W^T, W [N, K]."""
    name: str
    config_id: int
    K: int
    N: int
    group_size: int = 128
    act: str = "f16"
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    m_sweep: Tuple[int, ...] = field(default_factory=tuple)
    bits: int = 4                     # kept codes: 4-bit [-8, 7] or 8-bit [-128, 127]

    def with_(self, **kw) -> "SparseSpec":
        return replace(self, **kw)


CFG1 = MoESpec("tiny-w4a16-e4-top2", 1, bits=4, E=4, topk=2, K=256, N=512, group_size=128,
               act_order=False, act="f16", scale_lo=0.005, scale_hi=0.02, m_sweep=(16,))
CFG2 = MoESpec("mixtral8x7b-w8a16", 2, bits=8, E=8, topk=2, K=4096, N=14336, group_size=-1,
               act_order=False, act="bf16", scale_lo=1e-3, scale_hi=4e-3, m_sweep=(1, 4, 8, 64, 1024))
CFG3 = MoESpec("mixtral8x7b-w4a16-actorder", 3, bits=4, E=8, topk=2, K=4096, N=14336, group_size=128,
               act_order=True, act="f16", scale_lo=0.005, scale_hi=0.02, m_sweep=(1, 16, 256, 4096))
CFG4 = SparseSpec("yi34b-mlp-sparse24-w4a16", 4, K=7168, N=20480, group_size=128,
                  m_sweep=(1, 16, 128, 1024))
CFG5 = MoESpec("deepseekv2-w8a16-e160-top6", 5, bits=8, E=160, topk=6, K=5120, N=1536, group_size=-1,
               act_order=False, act="bf16", scale_lo=1e-3, scale_hi=4e-3, zipf_s=1.1, m_sweep=(64, 4096))

CONFIGS = {1: CFG1, 2: CFG2, 3: CFG3, 4: CFG4, 5: CFG5}


# ----------------------------------------------------------------------------
# MoE tensors
# ----------------------------------------------------------------------------
@dataclass
class MoEWeights:
    """Canonical logical weights.

    w1q [E, 2N, K] int8   rows [0, N) gate projection, rows [N, 2N) up projection
    s1  [E, G1, 2N] uint16 bits of `act` (G1 = 1 for per-column scales)
    g1  [E, K] int32 group of each input channel of w1, or None (g = k // gs)
    w2q [E, K, N] int8    down projection
    s2  [E, G2, K] uint16 bits
    g2  [E, N] int32 or None
    """
    spec: MoESpec
    w1q: np.ndarray
    s1: np.ndarray
    g1: Optional[np.ndarray]
    w2q: np.ndarray
    s2: np.ndarray
    g2: Optional[np.ndarray]

    def s1_f32(self) -> np.ndarray:
        return bits_to_f32(self.spec.act, self.s1)

    def s2_f32(self) -> np.ndarray:
        return bits_to_f32(self.spec.act, self.s2)


@dataclass
class Tokens:
    x: np.ndarray       # [M, K] uint16 bits of `act`
    logits: np.ndarray  # [M, E] float32
    act: str

    @property
    def M(self) -> int:
        return self.x.shape[0]

    def x_f32(self) -> np.ndarray:
        return bits_to_f32(self.act, self.x)


def _draw_codes(rng, shape, qmin, qmax) -> np.ndarray:
    return rng.integers(qmin, qmax + 1, size=shape, dtype=np.int8)


def _draw_scales(rng, shape, lo, hi, act) -> np.ndarray:
    return round_to(act, rng.uniform(lo, hi, size=shape).astype(np.float32))


def _draw_g_idx(rng, E, k_in, group_size) -> np.ndarray:
    """Per expert: a seeded random permutation of the input channels mapped to
    groups, so every group holds exactly `group_size` channels."""
    g = np.empty((E, k_in), dtype=np.int32)
    for e in range(E):
        g[e] = (rng.permutation(k_in) // group_size).astype(np.int32)
    return g


def make_moe_weights(spec: MoESpec, seed_config: Optional[int] = None) -> MoEWeights:
    cid = spec.config_id if seed_config is None else seed_config
    rng = rng_for(cid, 0, STREAM_WEIGHTS)
    E, K, N = spec.E, spec.K, spec.N
    G1, G2 = spec.groups(K), spec.groups(N)
    w1q = _draw_codes(rng, (E, 2 * N, K), spec.qmin, spec.qmax)
    s1 = _draw_scales(rng, (E, G1, 2 * N), spec.scale_lo, spec.scale_hi, spec.act)
    g1 = _draw_g_idx(rng, E, K, spec.group_size) if spec.act_order else None
    w2q = _draw_codes(rng, (E, K, N), spec.qmin, spec.qmax)
    s2 = _draw_scales(rng, (E, G2, K), spec.scale_lo, spec.scale_hi, spec.act)
    g2 = _draw_g_idx(rng, E, N, spec.group_size) if spec.act_order else None
    return MoEWeights(spec, w1q, s1, g1, w2q, s2, g2)


def zipf_log_bias(E: int, s: float) -> np.ndarray:
    """log p_e with p_e = (e+1)^-s / H_{E,s}: a skewed per-expert load prior,
    added to the router logits (expert 0 is the most loaded)."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def make_tokens(spec: MoESpec, M: int, seed_config: Optional[int] = None) -> Tokens:
    cid = spec.config_id if seed_config is None else seed_config
    rx = rng_for(cid, M, STREAM_X)
    rl = rng_for(cid, M, STREAM_LOGITS)
    x = round_to(spec.act, rx.standard_normal((M, spec.K), dtype=np.float32))
    logits = rl.standard_normal((M, spec.E), dtype=np.float32)
    if spec.zipf_s is not None:
        logits = (logits + zipf_log_bias(spec.E, spec.zipf_s)[None, :]).astype(np.float32)
    return Tokens(x, logits, spec.act)


# ----------------------------------------------------------------------------
# 2:4 sparse tensors
# ----------------------------------------------------------------------------
@dataclass
class SparseWeights:
    """Canonical 2:4 W4 weights, W logical [N, K].

    vals [N, K/2] int8   kept codes in [-8, 7], two per group of 4 along K,
                         in ascending position order (a kept code may be 0)
    idx  [N, K/2] uint8  position (0..3) of each kept code inside its group of 4;
                         the two positions of a group are distinct and ascending
    s    [K/gs, N] uint16 bits of `act`
    """
    spec: SparseSpec
    vals: np.ndarray
    idx: np.ndarray
    s: np.ndarray

    def s_f32(self) -> np.ndarray:
        return bits_to_f32(self.spec.act, self.s)


# the 6 ways to keep 2 of 4 positions, ascending pairs
_KEEP_PAIRS = np.array([(a, b) for a in range(4) for b in range(a + 1, 4)], dtype=np.uint8)


def make_sparse_weights(spec: SparseSpec, seed_config: Optional[int] = None) -> SparseWeights:
    cid = spec.config_id if seed_config is None else seed_config
    rng = rng_for(cid, 0, STREAM_WEIGHTS)
    N, K = spec.N, spec.K
    choice = rng.integers(0, 6, size=(N, K // 4), dtype=np.int8)
    idx = _KEEP_PAIRS[choice].reshape(N, K // 2)
    lim = 8 if spec.bits == 4 else 128
    vals = rng.integers(-lim, lim, size=(N, K // 2), dtype=np.int8)
    G = 1 if spec.group_size == -1 else K // spec.group_size
    s = _draw_scales(rng, (G, N), spec.scale_lo, spec.scale_hi, spec.act)
    return SparseWeights(spec, vals, np.ascontiguousarray(idx), s)


def make_sparse_x(spec: SparseSpec, M: int, seed_config: Optional[int] = None) -> np.ndarray:
    cid = spec.config_id if seed_config is None else seed_config
    rx = rng_for(cid, M, STREAM_X)
    return round_to(spec.act, rx.standard_normal((M, spec.K), dtype=np.float32))


# ----------------------------------------------------------------------------
# FP8 (E4M3) W8A8 MoE tensors
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Fp8MoESpec:
    """An FP8 W8A8 MoE layer: E4M3 weight codes with float32 per-column scales,
    static float32 activation scales a1 (layer input) and a2 (intermediate H).

    Weight codes are drawn as bit patterns: sign uniform, exponent field
    uniform in [exp_lo, exp_hi] (values 2^(e-7) (1 + m/8)), mantissa uniform;
    scales uniform in [scale_lo, scale_hi] as float32.  a1 and a2 are powers of
    two chosen so the largest |x| / a1 and |h| / a2 of the workload stay below
    448 (a calibrated static scale)."""
    name: str
    config_id: int
    E: int
    topk: int
    K: int
    N: int
    act: str
    scale_lo: float
    scale_hi: float
    exp_lo: int
    exp_hi: int
    a1: float
    a2: float
    renormalize: bool = True
    zipf_s: Optional[float] = None
    m_sweep: Tuple[int, ...] = field(default_factory=tuple)

    def with_(self, **kw) -> "Fp8MoESpec":
        return replace(self, **kw)


# the pages' FP8 rows run Mixtral-8x7B; same shape and batch sizes as the int8 layer
# (a1 = 2^-6: |x| <= 5.5 maps below 352; a2 = 2^-4: |h| of the 1024-token batch stays below 448 a2)
CFG_FP8 = Fp8MoESpec("mixtral8x7b-fp8-w8a8", 6, E=8, topk=2, K=4096, N=14336, act="bf16", scale_lo=1e-3,
                     scale_hi=4e-3, exp_lo=4, exp_hi=10, a1=2.0 ** -6, a2=2.0 ** -4, m_sweep=(1, 4, 8, 64, 1024))


@dataclass
class Fp8MoEWeights:
    """w1 [E, 2N, K] / w2 [E, K, N] E4M3 codes (uint8); s1 [E, 2N] / s2 [E, K] float32."""
    spec: Fp8MoESpec
    w1: np.ndarray
    s1: np.ndarray
    w2: np.ndarray
    s2: np.ndarray


def _draw_e4m3(rng, shape, exp_lo, exp_hi) -> np.ndarray:
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
    expo = rng.integers(exp_lo, exp_hi + 1, size=shape, dtype=np.uint8)
    mant = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign << 7) | (expo << 3) | mant


def make_fp8_weights(spec: Fp8MoESpec, seed_config: Optional[int] = None) -> Fp8MoEWeights:
    cid = spec.config_id if seed_config is None else seed_config
    rng = rng_for(cid, 0, STREAM_WEIGHTS)
    E, K, N = spec.E, spec.K, spec.N
    w1 = _draw_e4m3(rng, (E, 2 * N, K), spec.exp_lo, spec.exp_hi)
    s1 = rng.uniform(spec.scale_lo, spec.scale_hi, size=(E, 2 * N)).astype(np.float32)
    w2 = _draw_e4m3(rng, (E, K, N), spec.exp_lo, spec.exp_hi)
    s2 = rng.uniform(spec.scale_lo, spec.scale_hi, size=(E, K)).astype(np.float32)
    return Fp8MoEWeights(spec, w1, s1, w2, s2)
