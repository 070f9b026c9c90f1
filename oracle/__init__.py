"""CPU oracle for MoE EP dispatch / combine -- TEST INFRASTRUCTURE.

Thin ctypes wrappers over ``ep_oracle.c`` (plain sequential C, built with gcc
``-O2 -ffp-contract=off``).  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports it and shares no
code with it.

Every function takes and returns numpy arrays on the host.  The definitions
themselves (and the page passages they follow) are documented in
``ep_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")
_lib: Optional[ctypes.CDLL] = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
          "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no HIP, no shared code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P]
    lib.oracle_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_dispatch_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P]
    lib.oracle_combine.argtypes = [P, i64, P, P, i64, i32, i32, P]
    lib.oracle_dispatch_cached.argtypes = [P, P, i64, i32, i32, P, i64]
    lib.oracle_dispatch_ht.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_dispatch_fp8_cached.argtypes = [P, P, i64, i32, i32, P, P, i64]
    lib.oracle_dispatch_ll.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P]
    lib.oracle_dispatch_ll_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_quantize_row.argtypes = [P, i32, P, P]
    lib.oracle_e4m3_encode_array.argtypes = [P, i64, P]
    lib.oracle_bf16_rne_array.argtypes = [P, i64, P]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_float
    for f in ("oracle_layout", "oracle_dispatch", "oracle_dispatch_fp8", "oracle_combine",
              "oracle_quantize_row", "oracle_dispatch_cached", "oracle_dispatch_fp8_cached",
              "oracle_dispatch_ht", "oracle_dispatch_ll", "oracle_dispatch_ll_fp8"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _use_library(path: Optional[str]) -> None:
    """Point the wrappers at another build of the oracle (``None``: the default).
    Used only by the mutation tests, which build deliberately broken copies of
    ep_oracle.c to show that the pins catch them."""
    global _lib
    _lib = None
    if path is not None:
        _load()                       # resolve argtypes on the default first
        lib = ctypes.CDLL(path)
        for f in ("oracle_layout", "oracle_dispatch", "oracle_dispatch_fp8", "oracle_combine",
                  "oracle_quantize_row", "oracle_e4m3_encode_array", "oracle_bf16_rne_array",
                  "oracle_e4m3_decode", "oracle_dispatch_cached", "oracle_dispatch_fp8_cached",
                  "oracle_dispatch_ht", "oracle_dispatch_ll", "oracle_dispatch_ll_fp8"):
            getattr(lib, f).argtypes = getattr(_lib, f).argtypes
            getattr(lib, f).restype = getattr(_lib, f).restype
        _lib = lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: invalid argument (rc={rc})")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int, ranks_per_group: int):
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    G = num_ranks // max(1, ranks_per_group)
    per_rank = np.zeros(num_ranks, np.int32)
    per_group = np.zeros(max(G, 1), np.int32)
    per_expert = np.zeros(num_experts, np.int32)
    in_rank = np.zeros((T, num_ranks), np.uint8)
    rc = _load().oracle_layout(_p(idx), T, k, num_experts, num_ranks, ranks_per_group,
                               _p(per_rank), _p(per_group), _p(per_expert), _p(in_rank))
    _check(rc, "oracle_layout")
    return dict(num_tokens_per_rank=per_rank, num_tokens_per_group=per_group[:G],
                num_tokens_per_expert=per_expert, is_token_in_rank=in_rank)


def dispatch(x: np.ndarray, topk_idx: np.ndarray, topk_weights: Optional[np.ndarray],
             num_experts: int, num_ranks: int, sentinel: Optional[int] = None):
    """x: bf16 bits [T,H] uint16.  Returns recv buffers sized at capacity T*k rows."""
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    H = x.shape[1]
    N = T * k
    fill16 = 0 if sentinel is None else sentinel
    recv_x = np.full((N, H), fill16, np.uint16)
    src = np.full(N, -2, np.int32)
    recv_w = np.full(N, np.nan, np.float32) if topk_weights is not None else None
    eoff = np.zeros(num_experts + 1, np.int32)
    roff = np.zeros(num_ranks + 1, np.int32)
    trow = np.zeros((T, k), np.int32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rc = _load().oracle_dispatch(_p(x), _p(idx), _p(w), T, H, k, num_experts, num_ranks,
                                 _p(recv_x), _p(src), _p(recv_w), _p(eoff), _p(roff), _p(trow))
    _check(rc, "oracle_dispatch")
    return dict(recv_x=recv_x, recv_src_idx=src, recv_topk_weights=recv_w,
                recv_expert_offset=eoff, recv_rank_offset=roff, token_row=trow)


def dispatch_ht(x: np.ndarray, topk_idx: np.ndarray, topk_weights: Optional[np.ndarray],
                num_experts: int, num_ranks: int):
    """Rank-deduplicated dispatch; receive buffers at capacity T*R rows."""
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    H = x.shape[1]
    R = num_ranks
    cap = T * R
    recv_x = np.zeros((cap, H), np.uint16)
    src = np.full(cap, -2, np.int32)
    ridx = np.full((cap, k), -9, np.int64)
    rw = np.full((cap, k), np.nan, np.float32) if topk_weights is not None else None
    roff = np.zeros(R + 1, np.int32)
    trr = np.zeros((T, R), np.int32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rc = _load().oracle_dispatch_ht(_p(x), _p(idx), _p(w), T, H, k, num_experts, R, _p(recv_x),
                                    _p(src), _p(ridx), _p(rw), _p(roff), _p(trr))
    _check(rc, "oracle_dispatch_ht")
    return dict(recv_x=recv_x, recv_src_idx=src, recv_topk_idx=ridx, recv_topk_weights=rw,
                recv_rank_offset=roff, token_rank_row=trr)


def dispatch_ll(x: np.ndarray, topk_idx: np.ndarray, topk_weights: Optional[np.ndarray],
                num_experts: int, capacity: int, sentinel: int = 0):
    """Padded expert-major dispatch: recv_x [E, capacity, H]; rows an expert
    does not fill keep `sentinel` (src -2, weights NaN)."""
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    H = x.shape[1]
    E = num_experts
    recv_x = np.full((E, capacity, H), sentinel, np.uint16)
    cnt = np.full(E, -7, np.int32)
    src = np.full((E, capacity), -2, np.int32)
    rw = np.full((E, capacity), np.nan, np.float32) if topk_weights is not None else None
    slot = np.zeros((T, k), np.int32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rc = _load().oracle_dispatch_ll(_p(x), _p(idx), _p(w), T, H, k, E, capacity, _p(recv_x),
                                    _p(cnt), _p(src), _p(rw), _p(slot))
    _check(rc, "oracle_dispatch_ll")
    return dict(recv_x=recv_x, recv_count=cnt, recv_src_idx=src, recv_topk_weights=rw,
                token_slot=slot)


def dispatch_ll_fp8(x: np.ndarray, topk_idx: np.ndarray, topk_weights: Optional[np.ndarray],
                    num_experts: int, capacity: int):
    """Padded expert-major FP8 dispatch: codes [E, capacity, H], scales
    [E, capacity, H/128]; unfilled rows keep codes 0 and scales NaN."""
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    H = x.shape[1]
    E = num_experts
    q = np.zeros((E, capacity, H), np.uint8)
    sc = np.full((E, capacity, H // 128), np.nan, np.float32)
    cnt = np.full(E, -7, np.int32)
    src = np.full((E, capacity), -2, np.int32)
    rw = np.full((E, capacity), np.nan, np.float32) if topk_weights is not None else None
    slot = np.zeros((T, k), np.int32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rc = _load().oracle_dispatch_ll_fp8(_p(x), _p(idx), _p(w), T, H, k, E, capacity, _p(q), _p(sc),
                                        _p(cnt), _p(src), _p(rw), _p(slot))
    _check(rc, "oracle_dispatch_ll_fp8")
    return dict(recv_x_fp8=q, recv_scales=sc, recv_count=cnt, recv_src_idx=src,
                recv_topk_weights=rw, token_slot=slot)


def dispatch_fp8(x: np.ndarray, topk_idx: np.ndarray, topk_weights: Optional[np.ndarray],
                 num_experts: int, num_ranks: int):
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    H = x.shape[1]
    N = T * k
    recv_q = np.zeros((N, H), np.uint8)
    recv_s = np.full((N, H // 128), np.nan, np.float32)
    src = np.full(N, -2, np.int32)
    recv_w = np.full(N, np.nan, np.float32) if topk_weights is not None else None
    eoff = np.zeros(num_experts + 1, np.int32)
    roff = np.zeros(num_ranks + 1, np.int32)
    trow = np.zeros((T, k), np.int32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rc = _load().oracle_dispatch_fp8(_p(x), _p(idx), _p(w), T, H, k, num_experts, num_ranks,
                                     _p(recv_q), _p(recv_s), _p(src), _p(recv_w), _p(eoff),
                                     _p(roff), _p(trow))
    _check(rc, "oracle_dispatch_fp8")
    return dict(recv_x_fp8=recv_q, recv_scales=recv_s, recv_src_idx=src,
                recv_topk_weights=recv_w, recv_expert_offset=eoff, recv_rank_offset=roff,
                token_row=trow)


def dispatch_cached(x: np.ndarray, token_row: np.ndarray, num_rows: int,
                    recv_x: Optional[np.ndarray] = None):
    """recv_x[token_row[t,j]] = x[t] for rows in [0, num_rows); other rows of
    recv_x (zeros, or the given array) are left as they are."""
    x = _c(x, np.uint16)
    trow = _c(token_row, np.int32)
    T, k = trow.shape
    H = x.shape[1]
    out = np.zeros((num_rows, H), np.uint16) if recv_x is None else recv_x
    rc = _load().oracle_dispatch_cached(_p(x), _p(trow), T, H, k, _p(out), num_rows)
    _check(rc, "oracle_dispatch_cached")
    return out


def dispatch_fp8_cached(x: np.ndarray, token_row: np.ndarray, num_rows: int):
    x = _c(x, np.uint16)
    trow = _c(token_row, np.int32)
    T, k = trow.shape
    H = x.shape[1]
    q = np.zeros((num_rows, H), np.uint8)
    s = np.full((num_rows, H // 128), np.nan, np.float32)
    rc = _load().oracle_dispatch_fp8_cached(_p(x), _p(trow), T, H, k, _p(q), _p(s), num_rows)
    _check(rc, "oracle_dispatch_fp8_cached")
    return q, s


def quantize_row(xrow: np.ndarray):
    """Per-128-channel FP8 cast of one token: returns (codes[H] uint8, scales[H/128] fp32)."""
    xrow = _c(xrow, np.uint16)
    H = xrow.shape[0]
    q = np.zeros(H, np.uint8)
    s = np.zeros(max(H // 128, 1), np.float32)
    _check(_load().oracle_quantize_row(_p(xrow), H, _p(q), _p(s)), "oracle_quantize_row")
    return q, s[: H // 128]


def combine(expert_out: np.ndarray, token_row: np.ndarray, topk_weights: Optional[np.ndarray],
            num_rows: Optional[int] = None):
    """Weighted gather-sum; topk_weights None means every weight is 1."""
    y = _c(expert_out, np.uint16)
    trow = _c(token_row, np.int32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    T, k = trow.shape
    H = y.shape[1]
    rows = y.shape[0] if num_rows is None else num_rows
    out = np.zeros((T, H), np.uint16)
    rc = _load().oracle_combine(_p(y), rows, _p(trow), _p(w), T, H, k, _p(out))
    _check(rc, "oracle_combine")
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.zeros(v.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(code))


def bf16_rne(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.zeros(v.shape, np.uint16)
    _load().oracle_bf16_rne_array(_p(v), v.size, _p(out))
    return out
