"""GPU: repeat dispatch from a saved map (cached dispatch), and the whole path
captured in a HIP graph and replayed.

Cached dispatch follows the cached_notify of page "[Not ready] MSCCLPP EP
implementation #852" (Scope / Internode HT): a repeat dispatch with the same
routing reuses the earlier layout.  Expected values come from the oracle's
own cached scatter over the oracle's own map.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_02_amd import ep
from combine_get_dispatch_02_amd.workloads import CONFIGS, expert_outputs, make_workload, random_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,T,H", [("dsv3", 300, 7168), ("skewed", 257, 512), ("ll_fp8", 128, 7168),
                                      ("tiny", 128, 256)])
def test_cached_dispatch_matches_oracle(name, T, H):
    wl = CONFIGS[name].scaled(T=T, H=H)
    print(f"[cached] {wl.describe()}", flush=True)
    x, idx, w = make_workload(wl)
    ref = oracle.dispatch(x, idx, w, wl.E, wl.R)
    N = int(ref["recv_expert_offset"][-1])
    xd = dev_bf16(x)
    trow_d = torch.from_numpy(ref["token_row"]).to(DEV)
    # a second batch of activations routed the same way
    x2 = random_bf16(np.random.default_rng([5, T]), T, H)
    for xx in (x, x2):
        exp = oracle.dispatch_cached(xx, ref["token_row"], N)
        out = torch.full((N, H), 0x7FBF, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        got = host_bits(ep.ep_dispatch_cached(dev_bf16(xx), trow_d, N, out=out))
        np.testing.assert_array_equal(got, exp)
    if H % 128 == 0:
        q_exp, s_exp = oracle.dispatch_fp8_cached(x, ref["token_row"], N)
        o = dict(recv_x_fp8=torch.full((N, H), 0xA5, dtype=torch.uint8, device=DEV),
                 recv_scales=torch.full((N, H // 128), float("nan"), dtype=torch.float32, device=DEV))
        f = ep.ep_dispatch_fp8_cached(xd, trow_d, N, out=o)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(f["recv_x_fp8"].cpu().numpy(), q_exp)
        np.testing.assert_array_equal(f["recv_scales"].cpu().numpy().view(np.uint32), s_exp.view(np.uint32))


def test_cached_dispatch_skips_rows_out_of_range():
    rng = np.random.default_rng(9)
    T, k, H, rows = 200, 4, 64, 500
    x = rng.integers(0, 0x7F00, size=(T, H)).astype(np.uint16)
    trow = rng.permutation(T * k).astype(np.int32).reshape(T, k)      # 0..799, many >= rows
    trow[rng.random((T, k)) < 0.1] = -1
    sentinel = np.full((rows, H), 0x7FBF, np.uint16)
    exp = oracle.dispatch_cached(x, trow, rows, recv_x=sentinel.copy())
    out = torch.from_numpy(sentinel.view(np.int16)).to(DEV).view(torch.bfloat16)
    got = host_bits(ep.ep_dispatch_cached(dev_bf16(x), torch.from_numpy(trow).to(DEV), rows, out=out))
    np.testing.assert_array_equal(got, exp)


@pytest.mark.parametrize("name", ["ll_fp8", "dsv3"])
def test_whole_path_replays_in_hip_graph(name):
    """layout -> dispatch -> combine -> FP8 dispatch, then the rank-deduplicated
    dispatch and its unweighted combine and the padded-layout dispatches (bf16
    and FP8, capacity 4, so slots are dropped) and their combine, captured once
    and replayed with fresh activations and routing copied into the captured
    inputs; every replay must equal the eager path on the same inputs, bit for
    bit, with eager work and synchronisations between replays."""
    wl = CONFIGS[name] if name == "ll_fp8" else CONFIGS[name].scaled(T=512)
    x, idx, w = make_workload(wl)
    xd, idxd, wd = dev_bf16(x), torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)

    cap = 4

    def step():
        lay = ep.ep_get_dispatch_layout(idxd, wl.E, wl.R, wl.P)
        d = ep.ep_dispatch(xd, idxd, wd, wl.E, wl.R)
        c = ep.ep_combine(d["recv_x"], d["token_row"], wd)
        f = ep.ep_dispatch_fp8(xd, idxd, wd, wl.E, wl.R)
        h = ep.ep_dispatch_ht(xd, idxd, wd, wl.E, wl.R)
        hc = ep.ep_combine(h["recv_x"], h["token_rank_row"], None)
        ll = ep.ep_dispatch_ll(xd, idxd, wd, wl.E, cap)
        lc = ep.ep_combine(ll["recv_x"].view(wl.E * cap, -1), ll["token_slot"], wd)
        l8 = ep.ep_dispatch_ll_fp8(xd, idxd, wd, wl.E, cap)
        return lay, d, c, f, h, hc, ll, lc, l8

    def flat(res):
        lay, d, c, f, h, hc, ll, lc, l8 = res
        out = [lay[k].view(torch.uint8).clone() for k in sorted(lay)]
        out += [d[k].view(torch.uint8).clone() for k in sorted(d) if d[k] is not None and k != "recv_x"]
        n = int(d["recv_expert_offset"][-1].item())
        out.append(d["recv_x"][:n].view(torch.uint8).clone())
        out.append(c.view(torch.uint8).clone())
        out += [f[k][:n].view(torch.uint8).clone() for k in ("recv_x_fp8", "recv_scales")]
        nh = int(h["recv_rank_offset"][-1].item())
        out += [h[k].view(torch.uint8).clone() for k in ("recv_rank_offset", "token_rank_row")]
        out += [h[k][:nh].view(torch.uint8).clone()
                for k in ("recv_x", "recv_src_idx", "recv_topk_idx", "recv_topk_weights")]
        out.append(hc.view(torch.uint8).clone())
        slots = ll["token_slot"].flatten()
        slots = slots[slots >= 0].long()
        for o in (ll, l8):
            out += [o[k].view(torch.uint8).clone() for k in ("recv_count", "token_slot")]
        out.append(ll["recv_x"].view(wl.E * cap, -1)[slots].view(torch.uint8).clone())
        out.append(ll["recv_src_idx"].flatten()[slots].view(torch.uint8).clone())
        out.append(l8["recv_x_fp8"].view(wl.E * cap, -1)[slots].clone())
        out.append(l8["recv_scales"].view(wl.E * cap, -1)[slots].view(torch.uint8).clone())
        out.append(lc.view(torch.uint8).clone())
        return out

    step()                                   # warm up allocator and kernels outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            static = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        x2, idx2, w2 = make_workload(wl, seed_extra=rep + 1)
        xd.copy_(dev_bf16(x2))
        idxd.copy_(torch.from_numpy(idx2).to(DEV))
        wd.copy_(torch.from_numpy(w2).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = flat(static)
        eager = flat(step())                 # eager work between replays
        torch.cuda.synchronize()
        assert len(replayed) == len(eager)
        for a, b in zip(replayed, eager):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
