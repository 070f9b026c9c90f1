"""GPU parity of the padded expert-major (low-latency) dispatch, bf16 and FP8,
and of the combine through its slot map, against the oracle (page
"[Not ready] MSCCLPP EP implementation #852": the LL benchmark's per-expert
receive regions, the low-latency runtime's capacities).

Bar: slot map, counts, source tokens, weights and bf16 rows bit-exact; FP8
codes within one step of the oracle's (R16) and scales bit-exact; combine
bit-exact (same fp32 chain).  Slots an expert does not fill must keep their
sentinel.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_02_amd import ep
from combine_get_dispatch_02_amd.workloads import CONFIGS, make_workload, mask_slots, random_bf16
from parity import assert_combine, assert_fp8_codes
from test_gpu_parity import (SENT16, SENT8, assert_rows_hold_token_casts, dev_bf16, host_bits,
                              rows_as_tokens, token_casts)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def prefilled(T, k, H, E, cap, fp8, weights):
    o = dict(recv_count=torch.full((E,), -7, dtype=torch.int32, device=DEV),
             recv_src_idx=torch.full((E, cap), -2, dtype=torch.int32, device=DEV),
             recv_topk_weights=(torch.full((E, cap), float("nan"), dtype=torch.float32, device=DEV)
                                if weights else None),
             token_slot=torch.full((T, k), -9, dtype=torch.int32, device=DEV))
    if fp8:
        o["recv_x_fp8"] = torch.full((E, cap, H), SENT8, dtype=torch.uint8, device=DEV)
        o["recv_scales"] = torch.full((E, cap, H // 128), float("nan"), dtype=torch.float32, device=DEV)
    else:
        o["recv_x"] = torch.full((E, cap, H), SENT16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return o


def run_case(x, idx, w, E, cap, fp8, y_rng=None):
    T, k = idx.shape
    H = x.shape[1]
    ref = (oracle.dispatch_ll_fp8 if fp8 else oracle.dispatch_ll)(x, idx, w, E, cap)
    out = prefilled(T, k, H, E, cap, fp8, w is not None)
    fn = ep.ep_dispatch_ll_fp8 if fp8 else ep.ep_dispatch_ll
    d = fn(dev_bf16(x), torch.from_numpy(idx).to(DEV), None if w is None else torch.from_numpy(w).to(DEV),
           E, cap, out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d["token_slot"].cpu().numpy(), ref["token_slot"])
    np.testing.assert_array_equal(d["recv_count"].cpu().numpy(), ref["recv_count"])
    filled = ref["recv_src_idx"] >= 0
    src = d["recv_src_idx"].cpu().numpy()
    np.testing.assert_array_equal(src[filled], ref["recv_src_idx"][filled])
    assert np.all(src[~filled] == -2)
    if w is not None:
        rw = d["recv_topk_weights"].cpu().numpy()
        np.testing.assert_array_equal(rw[filled].view(np.uint32), ref["recv_topk_weights"][filled].view(np.uint32))
        assert np.all(np.isnan(rw[~filled]))
    if fp8:
        q = d["recv_x_fp8"].cpu().numpy()
        s = d["recv_scales"].cpu().numpy()
        assert_fp8_codes(q[filled], ref["recv_x_fp8"][filled])
        np.testing.assert_array_equal(s[filled].view(np.uint32), ref["recv_scales"][filled].view(np.uint32))
        assert np.all(q[~filled] == SENT8) and np.all(np.isnan(s[~filled]))
    else:
        rx = host_bits(d["recv_x"])
        np.testing.assert_array_equal(rx[filled], ref["recv_x"][filled])
        assert np.all(rx[~filled] == SENT16)
    if y_rng is not None:
        y = random_bf16(y_rng, E * cap, H)
        exp = oracle.combine(y, ref["token_slot"], w)
        got = host_bits(ep.ep_combine(dev_bf16(y), d["token_slot"],
                                      None if w is None else torch.from_numpy(w).to(DEV)))
        np.testing.assert_array_equal(got, exp)
    return d, ref


# (workload, T, H, capacity or None for T, mask fraction); T*k spans the
# one-launch path (<= 2048 slots) and the index + slot-map path above it.
CASES = [("ll_fp8", 128, 7168, None, 0.0), ("ll_fp8", 128, 7168, 2, 0.0), ("ll_fp8", 128, 1024, 1, 0.1),
         ("tiny", 128, 256, 3, 0.0), ("tiny", 128, 256, None, 0.05), ("dsv3", 300, 1024, 4, 0.0),
         ("dsv3", 300, 2048, 12, 0.05), ("dsv3", 257, 512, None, 0.0), ("skewed", 600, 512, 8, 0.0),
         ("skewed", 600, 512, 600, 0.0), ("large", 520, 256, 20, 0.1)]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-T{c[1]}-H{c[2]}-cap{c[3]}-m{c[4]}" for c in CASES])
def test_ll_parity_oracle_sized(case, fp8):
    name, T, H, cap, mask = case
    wl = CONFIGS[name].scaled(T=T, H=H)
    cap = cap or T
    print(f"[ll] {wl.describe()} cap={cap} mask={mask} fp8={fp8}", flush=True)
    x, idx, w = make_workload(wl, seed_extra=3)
    if mask:
        idx = mask_slots(idx, mask, 3)
    run_case(x, idx, w, wl.E, cap, fp8, y_rng=np.random.default_rng(T + cap))


@pytest.mark.parametrize("T,k,E,cap,H", [(40000, 8, 256, 200, 16), (33000, 8, 64, 4000, 16)])
def test_ll_two_kernel_index_path(T, k, E, cap, H):
    """T*k > 49152: the packed rows come from the two-launch receive-order path."""
    print(f"[ll-big] T={T} k={k} E={E} cap={cap} H={H}", flush=True)
    rng = np.random.default_rng(T)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int64)
    x = rng.integers(0, 0x7F00, size=(T, H)).astype(np.uint16)
    w = rng.random((T, k)).astype(np.float32)
    run_case(x, idx, w, E, cap, False)


@pytest.mark.parametrize("T,k,E,cap,H", [(1, 1, 1, 1, 128), (37, 3, 12, 2, 128), (9, 16, 8, 5, 256),
                                         (700, 8, 2048, 3, 128), (30, 64, 128, 3, 128),
                                         (100, 64, 2048, 2, 128)])
def test_ll_edge_shapes(T, k, E, cap, H):
    rng = np.random.default_rng(T * k + cap)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int64)          # duplicates allowed
    bad = rng.random((T, k)) < 0.1
    idx[bad] = rng.choice([-1, E, -5], size=bad.sum())
    x = rng.integers(0, 0x7F00, size=(T, H)).astype(np.uint16)
    w = rng.random((T, k)).astype(np.float32)
    for fp8 in (False, True):
        run_case(x, idx, w, E, cap, fp8, y_rng=rng)
        run_case(x, idx, None, E, cap, fp8)


def test_ll_empty_batch_and_all_empty_slots():
    for fp8 in (False, True):
        fn = ep.ep_dispatch_ll_fp8 if fp8 else ep.ep_dispatch_ll
        d = fn(torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV),
               torch.zeros((0, 4), dtype=torch.int64, device=DEV), None, 16, 3,
               out=prefilled(0, 4, 128, 16, 3, fp8, False))
        torch.cuda.synchronize()
        assert d["recv_count"].abs().sum().item() == 0
        d, _ = run_case(np.ones((9, 128), np.uint16), -np.ones((9, 3), np.int64), None, 6, 2, fp8)
        assert d["recv_count"].abs().sum().item() == 0


def test_ll_full_size_ll_workload_and_dsv3():
    """The LL workload at full size (T=128, H=7168) at capacity T, and the dsv3
    workload (T=4096, H=7168, k=8, E=256) at capacity 256 (2x the mean load):
    maps and counts bit-exact against the oracle (computed with H=8, since
    they do not depend on H); every filled bf16 slot against x at the oracle's
    source token, every filled FP8 slot against the oracle's cast of that
    token, and the combine over token_slot of every token against the
    oracle's."""
    for name, cap in (("ll_fp8", 128), ("dsv3", 256)):
        wl = CONFIGS[name]
        print(f"[ll-full] {wl.describe()} cap={cap}", flush=True)
        x, idx, w = make_workload(wl)
        ref = oracle.dispatch_ll(np.ascontiguousarray(x[:, :8]), idx, w, wl.E, cap)
        xd = dev_bf16(x)
        idxd = torch.from_numpy(idx).to(DEV)
        wd = torch.from_numpy(w).to(DEV)
        d = ep.ep_dispatch_ll(xd, idxd, wd, wl.E, cap)
        q = ep.ep_dispatch_ll_fp8(xd, idxd, wd, wl.E, cap)
        torch.cuda.synchronize()
        for o in (d, q):
            np.testing.assert_array_equal(o["token_slot"].cpu().numpy(), ref["token_slot"])
            np.testing.assert_array_equal(o["recv_count"].cpu().numpy(), ref["recv_count"])
        src_all = ref["recv_src_idx"].ravel()
        filled_rows = np.nonzero(src_all >= 0)[0]
        src = src_all[filled_rows]
        rows_d = torch.from_numpy(filled_rows.astype(np.int64)).to(DEV)
        src_d = torch.from_numpy(src.astype(np.int64)).to(DEV)
        assert torch.equal(d["recv_src_idx"].view(-1)[rows_d], src_d.to(torch.int32))
        assert torch.equal(d["recv_x"].view(wl.E * cap, wl.H)[rows_d].view(torch.int16),
                           xd[src_d].view(torch.int16))
        qtok, stok = token_casts(x)
        assert_rows_hold_token_casts(q["recv_x_fp8"].view(wl.E * cap, wl.H)[rows_d],
                                     q["recv_scales"].view(wl.E * cap, wl.H // 128)[rows_d],
                                     src, qtok, stok, f"{name} padded fp8")
        got = host_bits(ep.ep_combine(d["recv_x"].view(wl.E * cap, wl.H), d["token_slot"], wd))
        assert_combine(got, oracle.combine(x, rows_as_tokens(ref["token_slot"], src_all), w),
                       f"{name} combine over token_slot")
