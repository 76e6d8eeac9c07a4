"""Pins for the oracle's token sort and pad per expert: a hand-worked example,
the construction from numpy's stable argsort, and the invariants the padded
layout must satisfy."""
import json
import os

import numpy as np
import pytest

import gen
import oracle


def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "align_example.json")))
    ids = np.array(g["topk_ids"], np.int32)
    assert oracle.align_capacity(ids.size, g["E"], g["block_size"]) == g["capacity"]
    st, ex, nt = oracle.align(ids, g["E"], g["block_size"])
    assert st.tolist() == g["sorted_token_ids"]
    assert ex.tolist() == g["expert_ids"]
    assert nt == g["num_tokens_post_padded"]


def argsort_construction(flat, E, BS, cap):
    """Independent construction: numpy's stable argsort groups the flattened
    (token, slot) indices by expert in ascending order; each expert's run is then
    padded with the sentinel to a multiple of the block size."""
    T = flat.size
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    st = np.full(cap, T, np.int32)
    ex = np.full(cap // BS, -1, np.int32)
    pos = 0
    start = 0
    for e in range(E):
        c = counts[e]
        p = -(-c // BS) * BS
        st[pos:pos + c] = order[start:start + c]
        ex[pos // BS:(pos + p) // BS] = e
        pos += p
        start += c
    return st, ex, pos


def check_invariants(flat, E, BS, st, ex, nt):
    T = flat.size
    counts = np.bincount(flat, minlength=E)
    assert counts.sum() == T                                      # per-expert counts sum to M*topk
    assert nt == int((-(-counts // BS) * BS).sum())
    valid = st[st < T]
    assert sorted(valid.tolist()) == list(range(T))                 # each valid index exactly once
    assert (st[nt:] == T).all()
    used = ex[: nt // BS]
    assert (used >= 0).all() and (np.diff(used) >= 0).all()        # non-decreasing over used blocks
    assert (ex[nt // BS:] == -1).all()
    for b, e in enumerate(used):                                    # each block single-expert
        blk = st[b * BS:(b + 1) * BS]
        real = blk[blk < T]
        assert (flat[real] == e).all()
        # padding only after the real ids of a block
        if real.size < BS:
            assert (blk[real.size:] == T).all()
        assert (np.diff(real) > 0).all()                            # stable ascending order


@pytest.mark.parametrize("BS", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("cid,M", [(1, 16), (2, 1), (2, 64), (3, 16), (3, 256), (5, 64), (5, 4096)])
def test_matches_stable_argsort(cid, M, BS):
    spec = gen.CONFIGS[cid]
    toks = gen.make_tokens(spec, M)
    _, ids = oracle.route(toks.logits, spec.topk, spec.renormalize)
    flat = ids.reshape(-1)
    cap = oracle.align_capacity(flat.size, spec.E, BS)
    st, ex, nt = oracle.align(ids, spec.E, BS)
    st2, ex2, nt2 = argsort_construction(flat, spec.E, BS, cap)
    assert nt == nt2
    assert (st == st2).all()
    assert (ex == ex2).all()
    check_invariants(flat, spec.E, BS, st, ex, nt)


def test_capacity_is_reached():
    """Every expert with a single token: sum_e p_e reaches T + min(E,T)(BS-1)."""
    E, BS = 8, 16
    ids = np.arange(E, dtype=np.int32).reshape(4, 2)
    st, ex, nt = oracle.align(ids, E, BS)
    assert nt == oracle.align_capacity(ids.size, E, BS) == E * BS


def test_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 9]], np.int32), 4, 16)
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 1]], np.int32), 4, 16, capacity=16)
