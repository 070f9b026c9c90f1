"""Python binding of libep.so (include/ep.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  torch is
used for device memory (outputs and workspace are torch tensors on the input's
device) and for the stream (torch's current stream of that device); every
step of the computation runs in the HIP kernels behind the C ABI.  There is
no fallback: if libep.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

EP_OK = 0
_lib: Optional[ctypes.CDLL] = None


class EPError(RuntimeError):
    """A libep.so entry point returned a status other than EP_OK."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(detail)


def lib() -> ctypes.CDLL:
    """Load libep.so once (from this package's directory) and declare signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m combine_get_dispatch_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.ep_status_string.argtypes = [i32]
    L.ep_status_string.restype = ctypes.c_char_p
    L.ep_last_error.argtypes = []
    L.ep_last_error.restype = ctypes.c_char_p
    L.ep_version.argtypes = []
    L.ep_version.restype = ctypes.c_char_p
    L.ep_layout_workspace_bytes.argtypes = [i64, i32, i32, i32]
    L.ep_layout_workspace_bytes.restype = sz
    L.ep_dispatch_workspace_bytes.argtypes = [i64, i32, i32]
    L.ep_dispatch_workspace_bytes.restype = sz
    L.ep_get_dispatch_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    L.ep_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    L.ep_dispatch_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, sz, P]
    L.ep_dispatch_noalloc.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P]
    L.ep_combine.argtypes = [P, i64, P, P, i64, i32, i32, P, P]
    L.ep_dispatch_cached.argtypes = [P, P, i64, i32, i32, P, i64, P]
    L.ep_dispatch_ht_workspace_bytes.argtypes = [i64, i32]
    L.ep_dispatch_ht_workspace_bytes.restype = sz
    L.ep_dispatch_ht.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    L.ep_dispatch_fp8_cached.argtypes = [P, P, i64, i32, i32, P, P, i64, P]
    L.ep_dispatch_ll_workspace_bytes.argtypes = [i64, i32, i32]
    L.ep_dispatch_ll_workspace_bytes.restype = sz
    L.ep_dispatch_ll.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, sz, P]
    L.ep_dispatch_ll_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    for f in ("ep_get_dispatch_layout", "ep_dispatch", "ep_dispatch_noalloc", "ep_dispatch_fp8", "ep_combine",
              "ep_dispatch_cached", "ep_dispatch_fp8_cached", "ep_dispatch_ht", "ep_dispatch_ll",
              "ep_dispatch_ll_fp8"):
        getattr(L, f).restype = i32
    _lib = L
    return L


def _check(status: int, fn: str) -> None:
    if status != EP_OK:
        L = lib()
        raise EPError(status, f"{fn}: {L.ep_status_string(status).decode()}: "
                              f"{L.ep_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dev: Optional[torch.device] = None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(out: Dict[str, Optional[torch.Tensor]], dev: torch.device, spec) -> None:
    """Caller-supplied outputs: spec rows are (name, shape, dtype, required,
    capacity).  A capacity buffer needs at least shape[0] rows and exactly the
    trailing shape; any other array needs exactly `shape`.  The kernels write
    through raw pointers, so a smaller or mistyped tensor is refused here."""
    for name, shape, dtype, required, capacity in spec:
        t = out.get(name)
        if t is None:
            if required:
                raise ValueError(f"out is missing {name}")
            continue
        _need(t, name, dtype, dev)
        got = tuple(t.shape)
        ok = (len(got) == len(shape) and got[0] >= shape[0] and got[1:] == tuple(shape[1:])) if capacity \
            else got == tuple(shape)
        if not ok:
            want = f"[>= {shape[0]}{''.join(', ' + str(d) for d in shape[1:])}]" if capacity else str(list(shape))
            raise ValueError(f"out[{name!r}] has shape {list(got)}, needs {want}")


def _dispatch_spec(T, k, E, R, H, recv_name, recv_dtype, recv_cols, scales):
    N = T * k
    spec = [(recv_name, (N, recv_cols), recv_dtype, True, True),
            ("recv_src_idx", (N,), torch.int32, True, True),
            ("recv_topk_weights", (N,), torch.float32, False, True),
            ("recv_expert_offset", (E + 1,), torch.int32, True, False),
            ("recv_rank_offset", (R + 1,), torch.int32, False, False),
            ("token_row", (T, k), torch.int32, True, False)]
    if scales:
        spec.append(("recv_scales", (N, H // 128), torch.float32, True, True))
    return spec


def ep_layout_workspace_bytes(num_tokens: int, num_experts: int, num_ranks: int,
                              ranks_per_group: int) -> int:
    return int(lib().ep_layout_workspace_bytes(num_tokens, num_experts, num_ranks, ranks_per_group))


def ep_dispatch_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().ep_dispatch_workspace_bytes(num_tokens, num_topk, num_experts))


def _workspace(nbytes: int, dev: torch.device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        _need(ws, "workspace", torch.uint8, dev)
        if ws.numel() < nbytes:
            raise ValueError(f"workspace has {ws.numel()} bytes, needs {nbytes}")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)


def ep_get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                           ranks_per_group: Optional[int] = None, *,
                           out: Optional[Dict[str, torch.Tensor]] = None,
                           workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Routing histogram: num_tokens_per_rank [R], num_tokens_per_group [R/P],
    num_tokens_per_expert [E] (int32) and is_token_in_rank [T,R] (uint8).
    ranks_per_group defaults to min(8, num_ranks)."""
    _need(topk_idx, "topk_idx", torch.int64)
    dev = topk_idx.device
    T, k = topk_idx.shape
    P = min(8, num_ranks) if ranks_per_group is None else ranks_per_group
    G = num_ranks // P if P > 0 else 0
    if out is None:
        out = dict(
            num_tokens_per_rank=torch.empty(num_ranks, dtype=torch.int32, device=dev),
            num_tokens_per_group=torch.empty(max(G, 1), dtype=torch.int32, device=dev)[:G],
            num_tokens_per_expert=torch.empty(num_experts, dtype=torch.int32, device=dev),
            is_token_in_rank=torch.empty((T, num_ranks), dtype=torch.uint8, device=dev),
        )
    else:
        _check_out(out, dev, [("num_tokens_per_rank", (num_ranks,), torch.int32, True, False),
                              ("num_tokens_per_group", (G,), torch.int32, False, False),
                              ("num_tokens_per_expert", (num_experts,), torch.int32, True, False),
                              ("is_token_in_rank", (T, num_ranks), torch.uint8, True, False)])
    ws = _workspace(ep_layout_workspace_bytes(T, num_experts, num_ranks, max(P, 1)), dev, workspace)
    with torch.cuda.device(dev):
        st = lib().ep_get_dispatch_layout(
            _ptr(topk_idx), T, k, num_experts, num_ranks, P,
            _ptr(out["num_tokens_per_rank"]), _ptr(out["num_tokens_per_group"]),
            _ptr(out["num_tokens_per_expert"]), _ptr(out["is_token_in_rank"]),
            _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ep_get_dispatch_layout")
    return out


def _dispatch_outputs(T: int, k: int, E: int, R: int, dev, weights: bool) -> Dict[str, torch.Tensor]:
    N = T * k
    return dict(
        recv_src_idx=torch.empty(N, dtype=torch.int32, device=dev),
        recv_topk_weights=torch.empty(N, dtype=torch.float32, device=dev) if weights else None,
        recv_expert_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
        recv_rank_offset=torch.empty(R + 1, dtype=torch.int32, device=dev),
        token_row=torch.empty((T, k), dtype=torch.int32, device=dev),
    )


def ep_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                num_experts: int, num_ranks: int, *,
                out: Optional[Dict[str, torch.Tensor]] = None,
                workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """bf16 dispatch: recv_x [T*k, H] bf16 (capacity; recv_expert_offset[E] rows
    filled), recv_src_idx, recv_topk_weights, recv_expert_offset [E+1],
    recv_rank_offset [R+1], token_row [T,k]."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int64, dev)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, dev)
    T, H = x.shape
    k = topk_idx.shape[1]
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on num_tokens")
    if out is None:
        out = _dispatch_outputs(T, k, num_experts, num_ranks, dev, topk_weights is not None)
        out["recv_x"] = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    else:
        _check_out(out, dev, _dispatch_spec(T, k, num_experts, num_ranks, H, "recv_x",
                                            torch.bfloat16, H, False))
    ws = _workspace(ep_dispatch_workspace_bytes(T, k, num_experts), dev, workspace)
    with torch.cuda.device(dev):
        st = lib().ep_dispatch(
            _ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k, num_experts, num_ranks,
            _ptr(out["recv_x"]), _ptr(out["recv_src_idx"]), _ptr(out.get("recv_topk_weights")),
            _ptr(out["recv_expert_offset"]), _ptr(out.get("recv_rank_offset")),
            _ptr(out["token_row"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ep_dispatch")
    return out


def ep_dispatch_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                        num_experts: int, num_ranks: int, *,
                        out: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """ep_dispatch with the library's fixed device scratch instead of a
    workspace: the caller passes every output (the dict ep_dispatch returns),
    so nothing is allocated on this path."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int64, dev)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, dev)
    T, H = x.shape
    k = topk_idx.shape[1]
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on num_tokens")
    _check_out(out, dev, _dispatch_spec(T, k, num_experts, num_ranks, H, "recv_x",
                                        torch.bfloat16, H, False))
    with torch.cuda.device(dev):
        st = lib().ep_dispatch_noalloc(
            _ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k, num_experts, num_ranks,
            _ptr(out["recv_x"]), _ptr(out["recv_src_idx"]), _ptr(out.get("recv_topk_weights")),
            _ptr(out["recv_expert_offset"]), _ptr(out.get("recv_rank_offset")),
            _ptr(out["token_row"]), _stream(dev))
    _check(st, "ep_dispatch_noalloc")
    return out


def ep_dispatch_fp8(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                    num_experts: int, num_ranks: int, *,
                    out: Optional[Dict[str, torch.Tensor]] = None,
                    workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """FP8 dispatch: recv_x_fp8 [T*k, H] uint8 (OCP E4M3FN codes) and
    recv_scales [T*k, H/128] fp32, plus the same maps as ep_dispatch."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int64, dev)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, dev)
    T, H = x.shape
    k = topk_idx.shape[1]
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on num_tokens")
    if out is None:
        out = _dispatch_outputs(T, k, num_experts, num_ranks, dev, topk_weights is not None)
        out["recv_x_fp8"] = torch.empty((T * k, H), dtype=torch.uint8, device=dev)
        out["recv_scales"] = torch.empty((T * k, H // 128), dtype=torch.float32, device=dev)
    else:
        _check_out(out, dev, _dispatch_spec(T, k, num_experts, num_ranks, H, "recv_x_fp8",
                                            torch.uint8, H, True))
    ws = _workspace(ep_dispatch_workspace_bytes(T, k, num_experts), dev, workspace)
    with torch.cuda.device(dev):
        st = lib().ep_dispatch_fp8(
            _ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k, num_experts, num_ranks,
            _ptr(out["recv_x_fp8"]), _ptr(out["recv_scales"]), _ptr(out["recv_src_idx"]),
            _ptr(out.get("recv_topk_weights")), _ptr(out["recv_expert_offset"]),
            _ptr(out.get("recv_rank_offset")), _ptr(out["token_row"]), _ptr(ws), ws.numel(),
            _stream(dev))
    _check(st, "ep_dispatch_fp8")
    return out


def ep_dispatch_cached(x: torch.Tensor, token_row: torch.Tensor, recv_rows: int, *,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Repeat bf16 dispatch with a saved map: recv_x[token_row[t, j]] = x[t]
    for rows in [0, recv_rows).  Returns recv_x [recv_rows, H] bf16 (rows
    no slot maps to are left as they were: uninitialised unless `out` is given)."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(token_row, "token_row", torch.int32, dev)
    T, H = x.shape
    k = token_row.shape[1]
    if token_row.shape[0] != T:
        raise ValueError("x and token_row disagree on num_tokens")
    if out is None:
        out = torch.empty((recv_rows, H), dtype=torch.bfloat16, device=dev)
    elif tuple(out.shape) != (recv_rows, H):
        raise ValueError("out must be [recv_rows, H]")
    else:
        _need(out, "out", torch.bfloat16, dev)
    with torch.cuda.device(dev):
        st = lib().ep_dispatch_cached(_ptr(x), _ptr(token_row), T, H, k, _ptr(out), recv_rows,
                                      _stream(dev))
    _check(st, "ep_dispatch_cached")
    return out


def ep_dispatch_fp8_cached(x: torch.Tensor, token_row: torch.Tensor, recv_rows: int, *,
                           out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Repeat FP8 dispatch with a saved map: recv_x_fp8 [recv_rows, H] codes and
    recv_scales [recv_rows, H/128]."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(token_row, "token_row", torch.int32, dev)
    T, H = x.shape
    k = token_row.shape[1]
    if token_row.shape[0] != T:
        raise ValueError("x and token_row disagree on num_tokens")
    if out is None:
        out = dict(recv_x_fp8=torch.empty((recv_rows, H), dtype=torch.uint8, device=dev),
                   recv_scales=torch.empty((recv_rows, H // 128), dtype=torch.float32, device=dev))
    else:
        _check_out(out, dev, [("recv_x_fp8", (recv_rows, H), torch.uint8, True, True),
                              ("recv_scales", (recv_rows, H // 128), torch.float32, True, True)])
    with torch.cuda.device(dev):
        st = lib().ep_dispatch_fp8_cached(_ptr(x), _ptr(token_row), T, H, k, _ptr(out["recv_x_fp8"]),
                                          _ptr(out["recv_scales"]), recv_rows, _stream(dev))
    _check(st, "ep_dispatch_fp8_cached")
    return out


def ep_dispatch_ht_workspace_bytes(num_tokens: int, num_ranks: int) -> int:
    return int(lib().ep_dispatch_ht_workspace_bytes(num_tokens, num_ranks))


def ep_dispatch_ht(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                   num_experts: int, num_ranks: int, *,
                   out: Optional[Dict[str, torch.Tensor]] = None,
                   workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Rank-deduplicated dispatch: recv_x [T*R, H] (recv_rank_offset[R] rows
    filled), recv_src_idx, recv_topk_idx [T*R, k] int64 (local ids, -1
    elsewhere), recv_topk_weights [T*R, k], recv_rank_offset [R+1] and
    token_rank_row [T, R]; combine with ep_combine(y, token_rank_row, None)."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int64, dev)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, dev)
    T, H = x.shape
    k = topk_idx.shape[1]
    R = num_ranks
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on num_tokens")
    if out is None:
        cap = T * R
        out = dict(recv_x=torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
                   recv_src_idx=torch.empty(cap, dtype=torch.int32, device=dev),
                   recv_topk_idx=torch.empty((cap, k), dtype=torch.int64, device=dev),
                   recv_topk_weights=(torch.empty((cap, k), dtype=torch.float32, device=dev)
                                      if topk_weights is not None else None),
                   recv_rank_offset=torch.empty(R + 1, dtype=torch.int32, device=dev),
                   token_rank_row=torch.empty((T, R), dtype=torch.int32, device=dev))
    else:
        cap = T * R
        _check_out(out, dev, [("recv_x", (cap, H), torch.bfloat16, True, True),
                              ("recv_src_idx", (cap,), torch.int32, True, True),
                              ("recv_topk_idx", (cap, k), torch.int64, True, True),
                              ("recv_topk_weights", (cap, k), torch.float32, False, True),
                              ("recv_rank_offset", (R + 1,), torch.int32, True, False),
                              ("token_rank_row", (T, R), torch.int32, True, False)])
    ws = _workspace(ep_dispatch_ht_workspace_bytes(T, R), dev, workspace)
    with torch.cuda.device(dev):
        st = lib().ep_dispatch_ht(
            _ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k, num_experts, R,
            _ptr(out["recv_x"]), _ptr(out["recv_src_idx"]), _ptr(out["recv_topk_idx"]),
            _ptr(out.get("recv_topk_weights")), _ptr(out["recv_rank_offset"]),
            _ptr(out["token_rank_row"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ep_dispatch_ht")
    return out


def ep_dispatch_ll_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().ep_dispatch_ll_workspace_bytes(num_tokens, num_topk, num_experts))


def _ll(fp8: bool, x, topk_idx, topk_weights, num_experts, capacity, out, workspace):
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int64, dev)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, dev)
    T, H = x.shape
    k = topk_idx.shape[1]
    E = num_experts
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on num_tokens")
    if out is None:
        out = dict(recv_count=torch.empty(E, dtype=torch.int32, device=dev),
                   recv_src_idx=torch.empty((E, capacity), dtype=torch.int32, device=dev),
                   recv_topk_weights=(torch.empty((E, capacity), dtype=torch.float32, device=dev)
                                      if topk_weights is not None else None),
                   token_slot=torch.empty((T, k), dtype=torch.int32, device=dev))
        if fp8:
            out["recv_x_fp8"] = torch.empty((E, capacity, H), dtype=torch.uint8, device=dev)
            out["recv_scales"] = torch.empty((E, capacity, H // 128), dtype=torch.float32, device=dev)
        else:
            out["recv_x"] = torch.empty((E, capacity, H), dtype=torch.bfloat16, device=dev)
    else:
        spec = [("recv_count", (E,), torch.int32, True, False),
                ("recv_src_idx", (E, capacity), torch.int32, True, False),
                ("recv_topk_weights", (E, capacity), torch.float32, False, False),
                ("token_slot", (T, k), torch.int32, True, False)]
        if fp8:
            spec += [("recv_x_fp8", (E, capacity, H), torch.uint8, True, False),
                     ("recv_scales", (E, capacity, H // 128), torch.float32, True, False)]
        else:
            spec.append(("recv_x", (E, capacity, H), torch.bfloat16, True, False))
        _check_out(out, dev, spec)
    ws = _workspace(ep_dispatch_ll_workspace_bytes(T, k, E), dev, workspace)
    L = lib()
    with torch.cuda.device(dev):
        if fp8:
            st = L.ep_dispatch_ll_fp8(
                _ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k, E, capacity,
                _ptr(out["recv_x_fp8"]), _ptr(out["recv_scales"]), _ptr(out["recv_count"]),
                _ptr(out["recv_src_idx"]), _ptr(out.get("recv_topk_weights")),
                _ptr(out["token_slot"]), _ptr(ws), ws.numel(), _stream(dev))
        else:
            st = L.ep_dispatch_ll(
                _ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k, E, capacity,
                _ptr(out["recv_x"]), _ptr(out["recv_count"]), _ptr(out["recv_src_idx"]),
                _ptr(out.get("recv_topk_weights")), _ptr(out["token_slot"]), _ptr(ws), ws.numel(),
                _stream(dev))
    _check(st, "ep_dispatch_ll_fp8" if fp8 else "ep_dispatch_ll")
    return out


def ep_dispatch_ll(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                   num_experts: int, capacity: int, *,
                   out: Optional[Dict[str, torch.Tensor]] = None,
                   workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Padded expert-major dispatch: recv_x [E, capacity, H] (recv_count[e]
    rows of expert e filled), recv_count [E], recv_src_idx [E, capacity],
    recv_topk_weights [E, capacity], token_slot [T, k] (-1: empty or dropped).
    Combine with ep_combine(y.view(E * capacity, H), token_slot, weights)."""
    return _ll(False, x, topk_idx, topk_weights, num_experts, capacity, out, workspace)


def ep_dispatch_ll_fp8(x: torch.Tensor, topk_idx: torch.Tensor,
                       topk_weights: Optional[torch.Tensor], num_experts: int, capacity: int, *,
                       out: Optional[Dict[str, torch.Tensor]] = None,
                       workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """As ep_dispatch_ll with the FP8 cast of ep_dispatch_fp8: recv_x_fp8
    [E, capacity, H] uint8 (E4M3FN codes) and recv_scales [E, capacity, H/128]."""
    return _ll(True, x, topk_idx, topk_weights, num_experts, capacity, out, workspace)


def ep_combine(expert_out: torch.Tensor, token_row: torch.Tensor,
               topk_weights: Optional[torch.Tensor], num_rows: Optional[int] = None, *,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Weighted top-k gather-sum: combined_x [T, H] bf16.  num_rows defaults to
    expert_out.shape[0]; slots whose row is outside [0, num_rows) are skipped.
    topk_weights None: every weight is 1 (the combine of ep_dispatch_ht's
    per-rank rows, with token_rank_row as the map)."""
    _need(expert_out, "expert_out", torch.bfloat16)
    dev = expert_out.device
    _need(token_row, "token_row", torch.int32, dev)
    T, k = token_row.shape
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, dev)
        if tuple(topk_weights.shape) != (T, k):
            raise ValueError("topk_weights must have the shape of token_row")
    H = expert_out.shape[1]
    rows = expert_out.shape[0] if num_rows is None else int(num_rows)
    if rows > expert_out.shape[0]:
        raise ValueError("num_rows exceeds expert_out rows")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        _check_out({"out": out}, dev, [("out", (T, H), torch.bfloat16, True, False)])
    with torch.cuda.device(dev):
        st = lib().ep_combine(_ptr(expert_out), rows, _ptr(token_row), _ptr(topk_weights), T, H,
                              k, _ptr(out), _stream(dev))
    _check(st, "ep_combine")
    return out


def version() -> str:
    return lib().ep_version().decode()
