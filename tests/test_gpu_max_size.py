"""The largest batch one call accepts, on one GPU's HBM.

At H = 7168 and top-8 the bf16 copy launch holds at most
(2^32 - 1) / (7 segments * 8 waves * 64 lanes) = 1,198,372 tokens (a larger
batch is rejected on the host; tests/test_abi.py).  At that size the receive
buffer is 9.6 M rows, 137 GB, which MI355X's 288 GB hold.  Routing has
duplicate experts and 1 % empty slots; x is random bf16 generated on the GPU.

Checks, phase by phase (each phase frees its buffers before the next):
- layout, and dispatch's offsets, token_row, source map and weights: every
  element equal to the oracle's (the oracle's index work does not depend on
  H, so it runs with H = 8);
- every dispatched row equal to its source token (compared on the GPU);
- combine (identity experts, num_rows = filled rows) on 256 sampled tokens,
  bit-exact against the oracle's fp32 chain over the same rows;
- FP8 dispatch on 64 sampled tokens' rows against the oracle's cast;
- rank-deduplicated dispatch (two-launch index path): maps equal to the
  oracle's, every row equal to its token, its combine on sampled tokens;
- padded layout at the mean expert load (so slots are dropped): counts and
  slot map equal to the oracle's, every filled slot equal to its token.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_02_amd import ep
from parity import assert_fp8_codes
from test_gpu_parity import host_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H, K, E, R = 7168, 8, 256, 8
T = (2 ** 32 - 1) // (7 * 8 * 64)


def rows_equal_tokens(rows, src, xd, chunk=1 << 16):
    """rows[i] == xd[src[i]] for every i, compared on the GPU in chunks."""
    n = rows.shape[0]
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        a = rows[c0:c1].view(torch.int16)
        b = xd[src[c0:c1].long()].view(torch.int16)
        assert torch.equal(a, b), f"rows {c0}..{c1} differ from their tokens"


def sampled_combine_matches(y, token_row, w, out, tokens, num_rows):
    """oracle.combine over the sampled tokens' own rows (fetched from the GPU)."""
    tr = token_row[tokens]                                  # [S, k] host
    valid = (tr >= 0) & (tr < num_rows)
    uniq = np.unique(tr[valid])
    local = np.full(tr.shape, -1, np.int32)
    local[valid] = np.searchsorted(uniq, tr[valid]).astype(np.int32)
    y_local = host_bits(y[torch.from_numpy(uniq.astype(np.int64)).to(DEV)])
    exp = oracle.combine(y_local, local, None if w is None else w[tokens])
    got = host_bits(out[torch.from_numpy(tokens.astype(np.int64)).to(DEV)])
    np.testing.assert_array_equal(got, exp)


def test_largest_batch_one_launch_accepts():
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    need = 2 * T * K * H + 3 * 2 * T * H + (64 << 20)
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    print(f"[max size] T={T} H={H} k={K} E={E} R={R}: {T * K} slots, "
          f"recv {T * K * H * 2 / 1e9:.1f} GB", flush=True)
    rng = np.random.default_rng(1198372)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    idx[rng.random((T, K)) < 0.01] = -1
    w = rng.random((T, K)).astype(np.float32)
    idxd, wd = torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(7)
    xd = torch.randn((T, H), device=DEV, dtype=torch.bfloat16, generator=g)
    x8 = np.zeros((T, 8), np.uint16)                        # index work does not depend on H
    samples = rng.choice(T, size=256, replace=False)

    # layout
    lay = ep.ep_get_dispatch_layout(idxd, E, R)
    for key, v in oracle.layout(idx, E, R, 8).items():
        np.testing.assert_array_equal(lay[key].cpu().numpy(), v, err_msg=key)
    del lay

    # dispatch + combine
    ref = oracle.dispatch(x8, idx, w, E, R)
    N = int(ref["recv_expert_offset"][-1])
    d = ep.ep_dispatch(xd, idxd, wd, E, R)
    torch.cuda.synchronize()
    for key in ("recv_expert_offset", "recv_rank_offset", "token_row"):
        np.testing.assert_array_equal(d[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(d["recv_src_idx"][:N].cpu().numpy(), ref["recv_src_idx"][:N])
    np.testing.assert_array_equal(d["recv_topk_weights"][:N].cpu().numpy().view(np.uint32),
                                  ref["recv_topk_weights"][:N].view(np.uint32))
    rows_equal_tokens(d["recv_x"][:N], d["recv_src_idx"][:N], xd)
    out = ep.ep_combine(d["recv_x"], d["token_row"], wd, num_rows=N)
    torch.cuda.synchronize()
    sampled_combine_matches(d["recv_x"], ref["token_row"], w, out, samples, N)
    token_row = ref["token_row"]
    del d, out, ref
    torch.cuda.empty_cache()

    # FP8 dispatch: sampled tokens' rows against the oracle's cast
    f = ep.ep_dispatch_fp8(xd, idxd, wd, E, R)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f["token_row"].cpu().numpy(), token_row)
    for t in samples[:64]:
        qt, st = oracle.quantize_row(host_bits(xd[int(t)]))
        for r in token_row[t][token_row[t] >= 0]:
            assert_fp8_codes(f["recv_x_fp8"][int(r)].cpu().numpy(), qt)
            np.testing.assert_array_equal(f["recv_scales"][int(r)].cpu().numpy().view(np.uint32),
                                          st.view(np.uint32))
    del f
    torch.cuda.empty_cache()

    # rank-deduplicated dispatch and its unweighted combine
    rh = oracle.dispatch_ht(x8, idx, w, E, R)
    nh = int(rh["recv_rank_offset"][-1])
    h = ep.ep_dispatch_ht(xd, idxd, wd, E, R)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h["recv_rank_offset"].cpu().numpy(), rh["recv_rank_offset"])
    np.testing.assert_array_equal(h["token_rank_row"].cpu().numpy(), rh["token_rank_row"])
    np.testing.assert_array_equal(h["recv_src_idx"][:nh].cpu().numpy(), rh["recv_src_idx"][:nh])
    np.testing.assert_array_equal(h["recv_topk_idx"][:nh].cpu().numpy(), rh["recv_topk_idx"][:nh])
    rows_equal_tokens(h["recv_x"][:nh], h["recv_src_idx"][:nh], xd)
    ch = ep.ep_combine(h["recv_x"], h["token_rank_row"], None, num_rows=nh)
    torch.cuda.synchronize()
    sampled_combine_matches(h["recv_x"], rh["token_rank_row"], None, ch, samples, nh)
    del h, ch, rh
    torch.cuda.empty_cache()

    # padded layout at the mean expert load: slots are dropped
    cap = T * K // E
    rl = oracle.dispatch_ll(x8, idx, w, E, cap)
    assert rl["recv_count"].sum() < int((idx >= 0).sum())
    l = ep.ep_dispatch_ll(xd, idxd, wd, E, cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(l["recv_count"].cpu().numpy(), rl["recv_count"])
    np.testing.assert_array_equal(l["token_slot"].cpu().numpy(), rl["token_slot"])
    filled = torch.from_numpy((rl["recv_src_idx"] >= 0).reshape(-1)).to(DEV)
    src = l["recv_src_idx"].view(-1)[filled]
    np.testing.assert_array_equal(src.cpu().numpy(), rl["recv_src_idx"].reshape(-1)[filled.cpu().numpy()])
    slots = torch.nonzero(filled).squeeze(1)
    flat = l["recv_x"].view(E * cap, H)
    for c0 in range(0, slots.numel(), 1 << 16):
        sl = slots[c0:c0 + (1 << 16)]
        assert torch.equal(flat[sl].view(torch.int16), xd[src[c0:c0 + (1 << 16)].long()].view(torch.int16))
