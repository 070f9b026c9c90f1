"""Pins for the oracle's padded expert-major (low-latency) dispatch (CPU only).

Layout: page "[Not ready] MSCCLPP EP implementation #852" -- the LL
benchmark's receive buffer holds one fixed-size region per expert, and the
low-latency runtime is tested at capacities 1 and 2.  With one source the
buffer is [E, capacity, H], each region filled in (token, slot) order, and a
slot that finds its region full is dropped.  Independent references: a
hand-worked example, a numpy brute force (stable argsort by expert), the
reduction to the packed dispatch when nothing is dropped, conservation of
slots, the per-token FP8 cast, and the combine over the padded map.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_get_dispatch_02_amd.workloads import CONFIGS, make_workload, mask_slots
from test_oracle_layout_rows import ROUTINGS, _random_idx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(idx, E, cap):
    """Slot of every (t, j) and source token of every filled slot, by numpy:
    positions within an expert come from a stable argsort of the flat ids."""
    T, k = idx.shape
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=E + 1)
    start = np.concatenate([[0], np.cumsum(counts)])
    pos = np.empty_like(order)
    pos[order] = np.arange(len(order)) - start[key[order]]
    slot = np.where(valid & (pos < cap), key * cap + pos, -1).reshape(T, k)
    src = -np.ones(E * cap, np.int64)
    kept = slot.ravel() >= 0
    src[slot.ravel()[kept]] = np.nonzero(kept)[0] // k
    return slot, np.minimum(counts[:E], cap), src.reshape(E, cap)


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_example_ll.json")) as f:
        g = json.load(f)
    idx = np.array(g["topk_idx"], np.int64)
    w = np.array(g["topk_weights"], np.float32)
    E, cap = g["num_experts"], g["capacity"]
    T = idx.shape[0]
    x = (np.arange(T * 4, dtype=np.uint16) + 1).reshape(T, 4)
    d = oracle.dispatch_ll(x, idx, w, E, cap, sentinel=0xFFFF)
    np.testing.assert_array_equal(d["token_slot"], g["token_slot"])
    np.testing.assert_array_equal(d["recv_count"], g["recv_count"])
    for e in range(E):
        n = g["recv_count"][e]
        np.testing.assert_array_equal(d["recv_src_idx"][e, :n], g["recv_src_idx"][e][:n])
        np.testing.assert_array_equal(d["recv_topk_weights"][e, :n],
                                      np.array(g["recv_topk_weights"][e][:n], np.float32))
        np.testing.assert_array_equal(d["recv_x"][e, :n], x[g["recv_src_idx"][e][:n]])
        assert np.all(d["recv_x"][e, n:] == 0xFFFF) and np.all(d["recv_src_idx"][e, n:] == -2)


CAPS = [1, 2, 3, 7, None]          # None: capacity = T (nothing can be dropped)


@pytest.mark.parametrize("cap", CAPS)
@pytest.mark.parametrize("case", range(len(ROUTINGS)))
def test_matches_brute_force(case, cap):
    T, k, E, R, P, mf, dup, bad = ROUTINGS[case]
    cap = cap or max(T * k, 1)
    idx = _random_idx(T, k, E, mf, dup, bad, case)
    rng = np.random.default_rng(case)
    x = rng.integers(0, 65535, size=(T, 16)).astype(np.uint16)
    w = rng.random((T, k)).astype(np.float32)
    d = oracle.dispatch_ll(x, idx, w, E, cap, sentinel=0xABCD)
    slot, count, src = _brute(idx, E, cap)
    np.testing.assert_array_equal(d["token_slot"], slot)
    np.testing.assert_array_equal(d["recv_count"], count)
    filled = src >= 0
    np.testing.assert_array_equal(np.where(filled, d["recv_src_idx"], -1), src)
    assert np.all(d["recv_src_idx"][~filled] == -2)
    rx = d["recv_x"].reshape(E * cap, -1)
    np.testing.assert_array_equal(rx[filled.ravel()], x[src.ravel()[filled.ravel()]])
    assert np.all(rx[~filled.ravel()] == 0xABCD)
    ts = slot.ravel()
    rw = d["recv_topk_weights"].ravel()
    np.testing.assert_array_equal(rw[ts[ts >= 0]], w.ravel()[ts >= 0])


@pytest.mark.parametrize("name", ["tiny", "ll_fp8", "skewed"])
def test_no_drop_is_the_packed_dispatch_per_expert(name):
    """With capacity >= every expert's count, expert e's filled rows are the
    packed dispatch's rows expert_offset[e] .. expert_offset[e+1]-1."""
    wl = CONFIGS[name].scaled(T=min(CONFIGS[name].T, 600), H=128)
    x, idx, w = make_workload(wl)
    idx = mask_slots(idx, 0.1, 1)
    p = oracle.dispatch(x, idx, w, wl.E, wl.R)
    cnt = np.diff(p["recv_expert_offset"])
    cap = int(cnt.max())
    d = oracle.dispatch_ll(x, idx, w, wl.E, cap)
    np.testing.assert_array_equal(d["recv_count"], cnt)
    for e in range(wl.E):
        a, b = p["recv_expert_offset"][e], p["recv_expert_offset"][e + 1]
        np.testing.assert_array_equal(d["recv_x"][e, :b - a], p["recv_x"][a:b])
        np.testing.assert_array_equal(d["recv_src_idx"][e, :b - a], p["recv_src_idx"][a:b])
    valid = p["token_row"] >= 0
    e_of = np.where(valid, idx, 0)
    np.testing.assert_array_equal(d["token_slot"][valid],
                                  (e_of * cap + p["token_row"] - p["recv_expert_offset"][e_of])[valid])


@pytest.mark.parametrize("cap", [1, 2, 5])
def test_drops_are_the_latest_slots_and_conserved(cap):
    wl = CONFIGS["skewed"].scaled(T=400, H=8)
    x, idx, w = make_workload(wl)
    d = oracle.dispatch_ll(x, idx, w, wl.E, cap)
    valid = (idx >= 0) & (idx < wl.E)
    dropped = valid & (d["token_slot"] < 0)
    assert d["recv_count"].sum() + dropped.sum() == valid.sum()
    assert np.all(d["recv_count"] <= cap)
    # every kept slot of expert e precedes every dropped one in (t, j) order
    flat_e = np.where(valid, idx, -1).ravel()
    kept = d["token_slot"].ravel() >= 0
    for e in np.unique(flat_e[flat_e >= 0]):
        ke = np.nonzero(kept & (flat_e == e))[0]
        de = np.nonzero(~kept & (flat_e == e))[0]
        assert len(ke) == min(cap, len(ke) + len(de))
        if len(de):
            assert ke.max() < de.min()


def test_fp8_rows_hold_the_token_cast():
    wl = CONFIGS["ll_fp8"].scaled(T=64, H=512)
    x, idx, w = make_workload(wl)
    cap = 2
    d = oracle.dispatch_ll_fp8(x, idx, w, wl.E, cap)
    b = oracle.dispatch_ll(x, idx, w, wl.E, cap)
    np.testing.assert_array_equal(d["token_slot"], b["token_slot"])
    np.testing.assert_array_equal(d["recv_count"], b["recv_count"])
    q = d["recv_x_fp8"].reshape(wl.E * cap, -1)
    s = d["recv_scales"].reshape(wl.E * cap, -1)
    for t in range(wl.T):
        qt, st = oracle.quantize_row(x[t])
        for sl in d["token_slot"][t]:
            if sl >= 0:
                np.testing.assert_array_equal(q[sl], qt)
                np.testing.assert_array_equal(s[sl].view(np.uint32), st.view(np.uint32))
    unfilled = np.ones(wl.E * cap, bool)
    unfilled[d["token_slot"][d["token_slot"] >= 0]] = False
    assert np.all(np.isnan(s[unfilled])) and np.all(q[unfilled] == 0)


def test_combine_over_padded_map_equals_packed_combine():
    """Same expert outputs, two layouts: the weighted combine through
    token_slot equals the combine through the packed token_row bit for bit
    (nothing dropped), and a dropped slot contributes nothing."""
    wl = CONFIGS["tiny"]
    x, idx, w = make_workload(wl)
    p = oracle.dispatch(x, idx, w, wl.E, wl.R)
    cap = int(np.diff(p["recv_expert_offset"]).max())
    d = oracle.dispatch_ll(x, idx, w, wl.E, cap)
    ref = oracle.combine(p["recv_x"], p["token_row"], w)
    got = oracle.combine(d["recv_x"].reshape(wl.E * cap, -1), d["token_slot"], w)
    np.testing.assert_array_equal(got, ref)
    d1 = oracle.dispatch_ll(x, idx, w, wl.E, 1)
    kept_w = np.where(d1["token_slot"] >= 0, w, 0.0).astype(np.float32)
    got1 = oracle.combine(d1["recv_x"].reshape(wl.E, -1), d1["token_slot"], w)
    ref1 = oracle.combine(p["recv_x"], p["token_row"], kept_w)
    np.testing.assert_array_equal(got1, ref1)


def test_rejects_bad_capacity():
    idx = np.zeros((2, 2), np.int64)
    x = np.zeros((2, 8), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch_ll(x, idx, None, 4, 0)
