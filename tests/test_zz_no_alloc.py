"""ep_dispatch_noalloc (the dispatch with the library's fixed device scratch,
for callers that cannot allocate) against ep_dispatch with a workspace: every
output bit-identical, on two calls in a row -- the second with a smaller
batch, so it runs on the scratch the first one left behind -- and a batch
whose scratch need exceeds the fixed array is refused before any work."""
import numpy as np
import pytest
import torch

from combine_get_dispatch_02_amd import ep
from combine_get_dispatch_02_amd.workloads import CONFIGS, make_workload, mask_slots

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH = 1 << 20


def _dev(x, idx, w):
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return xd, torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)


def _filled(T, k, H, E, R, fill):
    N = T * k
    return dict(recv_x=torch.full((N, H), fill, dtype=torch.int16, device=DEV).view(torch.bfloat16),
                recv_src_idx=torch.full((N,), fill, dtype=torch.int32, device=DEV),
                recv_topk_weights=torch.full((N,), float(fill), dtype=torch.float32, device=DEV),
                recv_expert_offset=torch.full((E + 1,), fill, dtype=torch.int32, device=DEV),
                recv_rank_offset=torch.full((R + 1,), fill, dtype=torch.int32, device=DEV),
                token_row=torch.full((T, k), fill, dtype=torch.int32, device=DEV))


def _same(a, b):
    for key in a:
        ta, tb = a[key], b[key]
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), key


# first call: two receive-order launches (T*k > 2^15, per-tile histograms in
# the scratch); second, smaller: one fused launch; third: the one-launch
# small-batch path (no scratch use)
CALLS = [("dsv3", 8192, 1024, 0.02), ("skewed", 3000, 512, 0.0), ("ll_fp8", 100, 1024, 0.0)]


def test_noalloc_matches_dispatch_on_consecutive_calls():
    for name, T, H, mask in CALLS:
        wl = CONFIGS[name].scaled(T=T, H=H)
        print(f"[noalloc] {wl.describe()} mask={mask}", flush=True)
        x, idx, w = make_workload(wl, seed_extra=3)
        if mask:
            idx = mask_slots(idx, mask, 5)
        xd, idxd, wd = _dev(x, idx, w)
        assert ep.ep_dispatch_workspace_bytes(T, wl.k, wl.E) <= SCRATCH
        ref = ep.ep_dispatch(xd, idxd, wd, wl.E, wl.R, out=_filled(T, wl.k, H, wl.E, wl.R, -3))
        got = ep.ep_dispatch_noalloc(xd, idxd, wd, wl.E, wl.R, out=_filled(T, wl.k, H, wl.E, wl.R, -3))
        torch.cuda.synchronize()
        _same(ref, got)


def test_noalloc_refuses_batches_beyond_the_scratch():
    T, k, E, R, H = 8192, 64, 2048, 64, 8
    assert ep.ep_dispatch_workspace_bytes(T, k, E) > SCRATCH
    rng = np.random.default_rng(1)
    idx = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :k].astype(np.int64)
    x = np.zeros((T, H), np.uint16)
    w = np.ones((T, k), np.float32)
    xd, idxd, wd = _dev(x, idx, w)
    out = _filled(T, k, H, E, R, -3)
    with pytest.raises(ep.EPError, match="scratch"):
        ep.ep_dispatch_noalloc(xd, idxd, wd, E, R, out=out)
    torch.cuda.synchronize()
    assert bool((out["token_row"] == -3).all())          # nothing was enqueued
