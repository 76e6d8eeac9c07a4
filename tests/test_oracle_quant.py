"""Pins of the oracle's ExpertsInt8 load-time quantizer ("[Kernel] W8A16 Int8
inside FusedMoE", opening description: symmetric per-column per-expert int8,
scales extracted at startup).  The oracle computes s = max|w|/127 in float32,
rounds it to the 16-bit type (nearest-even), and q = round-half-even(w / s)
clamped to +-127.  Each check below fixes the result by something other than
the oracle's own code: a hand-derived example, the 16-bit casts of numpy and
torch, a brute-force search over all 255 codes, and invariants of the
definition."""
import numpy as np
import pytest
import torch

import gen
import oracle


def _w(act, shape, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    return gen.bits_to_f32(act, gen.round_to(act, (rng.standard_normal(shape) * scale).astype(np.float32)))


def test_hand_example_bf16():
    # max |w| = 1, 1/127 = 0.0078740157...; bf16 near it: 0x3C01 = 0.00787353515625
    # (step 2^-14 = 6.1e-5 between 0x3C00 = 0.0078125 and 0x3C02 = 0.0079345703125);
    # codes: 0.5 / s = 63.5035 -> 64, -1 / s = -127.0078 -> -127, 0.25 / s = 31.75 -> 32
    q, s = oracle.quant_w8(np.array([[0.5, -1.0, 0.25, 0.0]], np.float32), bf16=True)
    assert s[0] == np.float32(0.00787353515625)
    assert q.tolist() == [[64, -127, 32, 0]]


def test_zero_row():
    q, s = oracle.quant_w8(np.zeros((2, 16), np.float32), bf16=True)
    assert np.all(s == 0) and np.all(q == 0)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_scale_is_the_16bit_cast_of_max_over_127(act):
    w = _w(act, (64, 256), 11)
    _, s = oracle.quant_w8(w, bf16=(act == "bf16"))
    s32 = (np.abs(w).max(axis=1).astype(np.float32) / np.float32(127.0)).astype(np.float32)
    if act == "f16":
        ref = s32.astype(np.float16).astype(np.float32)
    else:
        ref = torch.from_numpy(s32).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(s, ref)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_codes_are_the_nearest_multiple_brute_force(act):
    """Every code is the integer in [-127, 127] nearest to w / s (exact
    arithmetic over all 255 candidates, ties to even); a disagreement is only
    allowed where the float32 quotient sits within rounding of a tie."""
    w = _w(act, (24, 128), 12)
    q, s = oracle.quant_w8(w, bf16=(act == "bf16"))
    cand = np.arange(-127, 128, dtype=np.float64)
    for r in range(w.shape[0]):
        err = np.abs(cand[None, :] * np.float64(s[r]) - w[r].astype(np.float64)[:, None])
        best = err.min(axis=1, keepdims=True)
        ties = err <= best * (1 + 1e-12)
        # among exact ties prefer the even code
        pick = np.where(ties & (np.abs(cand) % 2 == 0)[None, :], 1, 0) + ties
        ref = cand[np.argmax(pick, axis=1)].astype(np.int64)
        diff = np.nonzero(ref != q[r])[0]
        for i in diff:
            t = np.float64(w[r, i]) / np.float64(s[r])
            assert abs(abs(t - np.floor(t)) - 0.5) < 1e-5, (r, i, t, ref[i], q[r, i])


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_invariants(act):
    """max |q| = 127 on every nonzero row (the scale rounds to within half a
    16-bit step of max/127), and |q s - w| <= s / 2 everywhere (nothing is
    clipped beyond the rounding)."""
    w = _w(act, (40, 512), 13)
    w[3] = 0.0
    q, s = oracle.quant_w8(w, bf16=(act == "bf16"))
    nz = np.abs(w).max(axis=1) > 0
    assert np.all(np.abs(q[nz].astype(np.int32)).max(axis=1) == 127)
    assert np.all(q[~nz] == 0) and np.all(s[~nz] == 0)
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - w.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))


def test_symmetric():
    """q(-w) = -q(w) with the same scale (symmetric quantization)."""
    w = _w("bf16", (8, 64), 14)
    q1, s1 = oracle.quant_w8(w, bf16=True)
    q2, s2 = oracle.quant_w8(-w, bf16=True)
    assert np.array_equal(s1, s2) and np.array_equal(q1, -q2)
