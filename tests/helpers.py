"""Test helpers: decoders of the packed layouts (for packer round-trip tests),
the float tolerance of the parity tests, and device upload helpers."""
from __future__ import annotations

import numpy as np

REL_FRO = 5e-3      # relative Frobenius error bound
MAX_ABS = 3e-2      # max abs error bound, relative to max |ref|


def assert_close_fp(got, ref, what="", rel_fro=REL_FRO, max_abs=MAX_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / nref if nref > 0 else err
    mx = np.abs(got - ref).max() if got.size else 0.0
    lim = max_abs * (np.abs(ref).max() if ref.size else 0.0)
    assert rel <= rel_fro, "%s: relative Frobenius error %.3e > %.1e" % (what, rel, rel_fro)
    assert mx <= lim + 1e-30, "%s: max abs error %.3e > %.3e" % (what, mx, lim)
    return rel, mx


def _nibble_shift(j):
    return 4 * (j >> 1) + 16 * (j & 1)


def decode_w4(packed: np.ndarray, E: int, n_out: int, k_in: int) -> np.ndarray:
    """Packed int4 bytes -> codes [E, n_out, k_in] in packed row / channel order."""
    C = k_in // 128
    d = packed.view(np.uint32).reshape(E, n_out // 16, C, 64, 4)
    out = np.empty((E, n_out // 16, 16, C, 4, 4, 8), np.int8)   # e, t, row, c, s, lanegroup, j
    for l in range(64):
        for j in range(8):
            u = ((d[:, :, :, l, :] >> np.uint32(_nibble_shift(j))) & np.uint32(15)).astype(np.int16) - 8
            out[:, :, l % 16, :, :, l // 16, j] = u
    return out.reshape(E, n_out, k_in)


def decode_w8(packed: np.ndarray, E: int, n_out: int, k_in: int) -> np.ndarray:
    C = k_in // 64
    b = packed.reshape(E, n_out // 16, C, 64, 2, 8)
    out = np.empty((E, n_out // 16, 16, C, 2, 4, 8), np.int8)   # e, t, row, c, s, lanegroup, j
    for l in range(64):
        out[:, :, l % 16, :, :, l // 16, :] = b[:, :, :, l, :, :].view(np.int8)
    return out.reshape(E, n_out, k_in)


def logical_rows(n_out: int, interleave: bool, perm=None) -> np.ndarray:
    """Canonical row held by each packed row (one expert)."""
    p = np.arange(n_out)
    if not interleave:
        return p if perm is None else np.asarray(perm)[p]
    t = p // 16
    j, half, within = t // 2, t % 2, p % 16
    lr = 16 * j + within
    if perm is not None:
        lr = np.asarray(perm)[lr]
    return half * (n_out // 2) + lr


def decode_sparse24(vp: np.ndarray, mp: np.ndarray, N: int, K: int):
    """Packed 2:4 -> (vals [N, K/2], idx [N, K/2])."""
    C = K // 256
    d = vp.view(np.uint32).reshape(N // 16, C, 64, 4)
    m = mp.view(np.uint16).reshape(N // 16, C, 64, 4)
    vals = np.empty((N // 16, 16, C, 4, 4, 4, 2), np.int8)   # t, row, c, step, lanegroup, group b, h
    idx = np.empty_like(vals, dtype=np.uint8)
    for l in range(64):
        for b in range(4):
            for h in range(2):
                j = 2 * b + h
                vals[:, l % 16, :, :, l // 16, b, h] = (
                    ((d[:, :, l, :] >> np.uint32(_nibble_shift(j))) & np.uint32(15)).astype(np.int16) - 8)
                idx[:, l % 16, :, :, l // 16, b, h] = (m[:, :, l, :] >> np.uint16(4 * b + 2 * h)) & np.uint16(3)
    return vals.reshape(N, K // 2), idx.reshape(N, K // 2)
