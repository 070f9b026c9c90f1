"""Seeded random shapes through every entry point, against the oracle.

Each case draws T, k, E, R (E a multiple of R), ranks per group, H (a
multiple of 128), a capacity, a routing with distinct or duplicate ids and
empty or out-of-range slots, with or without weights, and checks layout,
dispatch, FP8 dispatch, cached dispatch, rank-deduplicated dispatch, the
padded layout (bf16 and FP8) and the combines over each map: maps and bytes
bit-exact, FP8 codes within one step (scales bit-exact), combines bit-exact.
The shapes cross the kernels' internal limits: the one-launch small batch
(T*k <= 2048), the one-launch receive order (<= 49152 slots) and beyond, the
one-launch rank-deduplicated index (R, k <= 16) and beyond.  A second,
wider draw reaches top-64, 2048 experts, 64 ranks and 40000 tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_02_amd import ep
from parity import assert_fp8_codes
from test_gpu_parity import dev_bf16, host_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw(seed):
    rng = np.random.default_rng([7, seed])
    R = int(rng.choice([1, 2, 3, 4, 8, 16, 17, 32, 64]))
    epr = int(rng.choice([1, 2, 3, 8, 16]))
    E = min(R * epr, 2048 // R * R)
    k = int(rng.integers(1, min(E, 16) + 1)) if rng.random() < 0.9 else int(rng.integers(17, 25))
    T = int(rng.choice([1, 7, 64, 129, 300, 1000, 2500, 5000]))
    H = 128 * int(rng.choice([1, 2, 3, 8, 56]))
    if T * k > 8000:                      # keep the oracle's share to seconds
        H = min(H, 1024)
    P = int(rng.choice([d for d in range(1, R + 1) if R % d == 0]))
    if rng.random() < 0.5 and k <= E:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int64)
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int64)
    bad = rng.random((T, k)) < rng.choice([0.0, 0.05, 0.3])
    idx[bad] = rng.choice([-1, E, E + 5, -7], size=int(bad.sum()))
    x = (rng.standard_normal((T, H)).astype(np.float32) * rng.choice([1.0, 3.0]))
    x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = rng.random((T, k)).astype(np.float32) if rng.random() < 0.8 else None
    cap = int(rng.choice([1, 2, 5, max(1, T * k // max(E, 1))]))
    return T, k, E, R, P, H, idx, x, w, cap


def draw_wide(seed):
    """Wider shapes: top-k to 64, up to 2048 experts and 64 ranks, up to
    40000 tokens (H = 128 once T*k passes 4000, T*k at most 300000), half of
    the slots empty or out of range in some cases."""
    rng = np.random.default_rng([11, seed])
    R = int(rng.choice([1, 2, 5, 8, 16, 32, 33, 64]))
    epr = int(rng.choice([1, 2, 4, 8, 32]))
    E = min(R * epr, 2048 // R * R)
    k = int(rng.integers(1, min(E, 64) + 1)) if rng.random() < 0.7 else int(rng.integers(1, 65))
    T = int(rng.choice([1, 2, 31, 64, 65, 257, 2049, 4097, 9000, 16385, 40000]))
    H = 128 * int(rng.choice([1, 2, 7, 56]))
    if T * k > 4000:
        H = 128
    if T * k > 300000:
        T = max(1, 300000 // k)
    P = int(rng.choice([d for d in range(1, R + 1) if R % d == 0]))
    if rng.random() < 0.5 and k <= E:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int64)
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int64)
    bad = rng.random((T, k)) < rng.choice([0.0, 0.02, 0.5])
    idx[bad] = rng.choice([-1, E, E + 1000, -3], size=int(bad.sum()))
    x = (rng.standard_normal((T, H)).astype(np.float32) * rng.choice([1.0, 4.0]))
    x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = rng.random((T, k)).astype(np.float32) if rng.random() < 0.8 else None
    cap = int(rng.choice([1, 3, max(1, T * k // max(E, 1)), T]))
    return T, k, E, R, P, H, idx, x, w, cap


@pytest.mark.parametrize("seed", range(60))
def test_random_shapes_every_entry_point(seed):
    run_every_entry_point(f"random {seed}", *draw(seed))


@pytest.mark.parametrize("seed", range(40))
def test_wide_random_shapes_every_entry_point(seed):
    run_every_entry_point(f"wide {seed}", *draw_wide(seed))


def run_every_entry_point(label, T, k, E, R, P, H, idx, x, w, cap):
    print(f"[{label}] T={T} k={k} E={E} R={R} P={P} H={H} cap={cap} w={w is not None}", flush=True)
    xd, idxd = dev_bf16(x), torch.from_numpy(idx).to(DEV)
    wd = None if w is None else torch.from_numpy(w).to(DEV)

    lay = ep.ep_get_dispatch_layout(idxd, E, R, P)
    for key, ref in oracle.layout(idx, E, R, P).items():
        np.testing.assert_array_equal(lay[key].cpu().numpy(), ref, err_msg=key)

    ref = oracle.dispatch(x, idx, w, E, R)
    n = int(ref["recv_expert_offset"][-1])
    d = ep.ep_dispatch(xd, idxd, wd, E, R)
    for key in ("recv_expert_offset", "recv_rank_offset", "token_row"):
        np.testing.assert_array_equal(d[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(d["recv_src_idx"].cpu().numpy()[:n], ref["recv_src_idx"][:n])
    np.testing.assert_array_equal(host_bits(d["recv_x"])[:n], ref["recv_x"][:n])
    if w is not None:
        np.testing.assert_array_equal(d["recv_topk_weights"].cpu().numpy()[:n].view(np.uint32),
                                      ref["recv_topk_weights"][:n].view(np.uint32))
        got = host_bits(ep.ep_combine(d["recv_x"], d["token_row"], wd, num_rows=n))
        np.testing.assert_array_equal(got, oracle.combine(ref["recv_x"], ref["token_row"], w, num_rows=n))

    f = ep.ep_dispatch_fp8(xd, idxd, wd, E, R)
    ref8 = oracle.dispatch_fp8(x, idx, w, E, R)
    np.testing.assert_array_equal(f["token_row"].cpu().numpy(), ref8["token_row"])
    np.testing.assert_array_equal(f["recv_scales"].cpu().numpy()[:n].view(np.uint32),
                                  ref8["recv_scales"][:n].view(np.uint32))
    assert_fp8_codes(f["recv_x_fp8"].cpu().numpy()[:n], ref8["recv_x_fp8"][:n])

    c = ep.ep_dispatch_cached(xd, d["token_row"], n)
    np.testing.assert_array_equal(host_bits(c), ref["recv_x"][:n])

    h = ep.ep_dispatch_ht(xd, idxd, wd, E, R)
    rh = oracle.dispatch_ht(x, idx, w, E, R)
    nh = int(rh["recv_rank_offset"][-1])
    for key in ("recv_rank_offset", "token_rank_row"):
        np.testing.assert_array_equal(h[key].cpu().numpy(), rh[key], err_msg=key)
    np.testing.assert_array_equal(h["recv_topk_idx"].cpu().numpy()[:nh], rh["recv_topk_idx"][:nh])
    np.testing.assert_array_equal(host_bits(h["recv_x"])[:nh], rh["recv_x"][:nh])
    got = host_bits(ep.ep_combine(h["recv_x"], h["token_rank_row"], None, num_rows=nh))
    np.testing.assert_array_equal(got, oracle.combine(rh["recv_x"], rh["token_rank_row"], None, num_rows=nh))

    ll = ep.ep_dispatch_ll(xd, idxd, wd, E, cap)
    rl = oracle.dispatch_ll(x, idx, w, E, cap)
    np.testing.assert_array_equal(ll["token_slot"].cpu().numpy(), rl["token_slot"])
    np.testing.assert_array_equal(ll["recv_count"].cpu().numpy(), rl["recv_count"])
    filled = rl["recv_src_idx"] >= 0
    np.testing.assert_array_equal(ll["recv_src_idx"].cpu().numpy()[filled], rl["recv_src_idx"][filled])
    np.testing.assert_array_equal(host_bits(ll["recv_x"])[filled], rl["recv_x"][filled])
    l8 = ep.ep_dispatch_ll_fp8(xd, idxd, wd, E, cap)
    r8 = oracle.dispatch_ll_fp8(x, idx, w, E, cap)
    np.testing.assert_array_equal(l8["token_slot"].cpu().numpy(), r8["token_slot"])
    np.testing.assert_array_equal(l8["recv_scales"].cpu().numpy()[filled].view(np.uint32),
                                  r8["recv_scales"][filled].view(np.uint32))
    assert_fp8_codes(l8["recv_x_fp8"].cpu().numpy()[filled], r8["recv_x_fp8"][filled])
    if w is not None:
        y = rl["recv_x"].reshape(E * cap, H)
        got = host_bits(ep.ep_combine(ll["recv_x"].view(E * cap, H), ll["token_slot"], wd))
        np.testing.assert_array_equal(got, oracle.combine(y, rl["token_slot"], w))
