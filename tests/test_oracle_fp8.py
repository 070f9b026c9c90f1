"""Pins for the oracle's FP8 (OCP E4M3FN) encoder and per-128-channel cast.

Independent references: torch's CPU float8_e4m3fn conversion (a library
routine; it rounds to nearest-even but turns values >= 480 into NaN rather than
saturating, so it is only consulted below 464), the format's closed-form
decode, hand-computed codes, and error bounds that any correct round-to-nearest
quantiser meets.  The method (low-latency dispatch with kUseFP8 on page
"[Not ready] MSCCLPP EP implementation #852") casts each token to FP8 with one
fp32 scale per 128 channels, the scale being amax / 448.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_02_amd.workloads import CONFIGS, make_workload, bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_decode(codes)
    got = np.array([oracle.e4m3_decode(int(c)) for c in codes], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2       # 0x7F, 0xFF
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)


def test_midpoints_round_to_even_code():
    pos = np.arange(0, 0x7E, dtype=np.uint8)            # adjacent pairs (c, c+1)
    lo, hi = torch_decode(pos).astype(np.float64), torch_decode(pos + 1).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)             # exact in fp32
    expect = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(mid), expect)
    np.testing.assert_array_equal(oracle.e4m3_encode(-mid), expect | 0x80)
    # one fp32 ulp either side of the midpoint decides by distance
    below = np.nextafter(mid, np.float32(-np.inf))
    above = np.nextafter(mid, np.float32(np.inf))
    np.testing.assert_array_equal(oracle.e4m3_encode(below[1:]), pos[1:])
    np.testing.assert_array_equal(oracle.e4m3_encode(above), pos + 1)


def test_matches_torch_below_464():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-14, np.log2(463.9), size=200000)).astype(np.float32)
    v = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11,
                                       448.0, 450.0, 463.9, -463.9, 1e-30, 1e-45])])
    np.testing.assert_array_equal(oracle.e4m3_encode(v), torch_e4m3(v))


def test_saturates_above_448():
    v = np.float32([448.0, 464.0, 480.0, 1e9, np.inf, -500.0, -np.inf])
    np.testing.assert_array_equal(oracle.e4m3_encode(v), [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert oracle.e4m3_encode(np.float32([np.nan]))[0] & 0x7F == 0x7F


def test_hand_computed_block():
    """Codes worked by hand (golden fixture)."""
    with open(os.path.join(GOLDEN, "fp8_block.json")) as f:
        g = json.load(f)
    x = np.zeros(128, np.float32)
    for i, v in g["nonzero_inputs"]:
        x[i] = v
    xb = bf16_bits(x)
    q, s = oracle.quantize_row(xb)
    assert s[0] == np.float32(g["scale"])
    for i, c in g["codes"]:
        assert q[i] == c, (i, q[i], c)
    assert np.all(np.delete(q, [i for i, _ in g["codes"]]) == 0)


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("sigma,seed", [(2.0, 0), (1.0, 1), (1e-3, 2), (300.0, 3)])
def test_quantize_row_bounds(sigma, seed):
    """Per block: the amax element encodes to +-448, the scale is amax/448 in
    fp32, and every code is within half a step of x/s (relative 2^-4 in the
    normal range, 2^-10 * s absolute in the subnormal range), with a small fp32
    slack for the division x / s."""
    rng = np.random.default_rng(seed)
    H = 1024
    xb = bf16_bits(rng.standard_normal(H).astype(np.float32) * np.float32(sigma))
    q, s = oracle.quantize_row(xb)
    x = _f32(xb).reshape(-1, 128)
    a = np.abs(x).max(1)
    np.testing.assert_array_equal(s, (a / np.float32(448.0)).astype(np.float32))
    qb = q.reshape(-1, 128)
    dec = torch_decode(qb.ravel()).reshape(qb.shape).astype(np.float64)
    for c in range(x.shape[0]):
        am = np.argmax(np.abs(x[c]))
        assert qb[c, am] & 0x7F == 0x7E
        assert (qb[c, am] >> 7) == (x[c, am] < 0)
        xs = x[c].astype(np.float64) / float(s[c])
        err = np.abs(dec[c] - xs)
        normal = np.abs(xs) >= 2.0 ** -6
        slack = 1 + 2.0 ** -20
        assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xs[normal]) * slack + 1e-30)
        assert np.all(err[~normal] <= 2.0 ** -10 * slack)
        assert np.all(np.sign(dec[c][dec[c] != 0]) == np.sign(xs[dec[c] != 0]))


def test_zero_and_signed_zero_blocks():
    x = np.zeros(256, np.float32)
    x[128] = -0.0
    x[129] = 1.0
    x[130] = -0.0
    q, s = oracle.quantize_row(bf16_bits(x))
    assert s[0] == 0.0 and np.all(q[:128] == 0x00)           # all-zero block: scale 0, codes 0
    assert q[129] == 0x7E and q[128] == 0x80 and q[130] == 0x80


def test_tiny_amax_keeps_denormal_scale():
    # smallest bf16 subnormal 2^-133: the scale is an fp32 denormal, not 0
    x = np.zeros(128, np.uint16)
    x[5] = 0x0001
    x[6] = 0x8001
    q, s = oracle.quantize_row(x)
    assert s[0] > 0 and s[0] == np.float32(2.0 ** -133) / np.float32(448.0)
    assert q[5] == 0x7E and q[6] == 0xFE


def test_non_finite_blocks():
    """Non-finite activations (the page defines none; the reading kept is plain
    IEEE arithmetic on a NaN-free amax): NaN never raises or poisons the block
    amax; every NaN, of either sign, quiet or signalling, encodes as 0x7F when
    the block scale is positive; an infinite amax gives an infinite scale, so
    finite channels become signed zeros and the infinities NaN (inf / inf)."""
    x = np.zeros(512, np.uint16)
    one, two, three, five = 0x3F80, 0x4000, 0x4040, 0x40A0
    x[0], x[1] = one, two
    x[2], x[3], x[4], x[5] = 0x7FC0, 0xFFC0, 0x7F81, 0xFF81      # +-qNaN, +-sNaN
    x[128], x[129], x[130], x[131] = 0x7F80, 0xFF80, three, 0x8000 | five   # +inf, -inf, 3, -5
    x[256] = 0xFFC0                                              # only a NaN: amax 0
    x[384], x[385] = 0x7F7F, 0x7FC0                              # bf16 max with a NaN
    q, s = oracle.quantize_row(x)
    assert s[0] == np.float32(2.0) / np.float32(448.0)
    assert q[0] == 0x76 and q[1] == 0x7E                         # 224 = 1.75 * 2^7, 448
    assert np.all(q[2:6] == 0x7F) and np.all(q[6:128] == 0x00)
    assert np.isinf(s[1]) and s[1] > 0
    assert q[128] == 0x7F and q[129] == 0x7F and q[130] == 0x00 and q[131] == 0x80
    assert np.all(q[132:256] == 0x00)
    assert s[2] == 0.0 and np.all(q[256:384] == 0x00)            # scale 0: all codes 0
    assert s[3] == np.float32(3.3895313892515355e38) / np.float32(448.0)
    assert q[384] == 0x7E and q[385] == 0x7F and np.all(q[386:] == 0x00)


def test_fp8_dispatch_rows_hold_token_cast():
    wl = CONFIGS["ll_fp8"].scaled(T=24, H=512)
    x, idx, w = make_workload(wl)
    d = oracle.dispatch_fp8(x, idx, w, wl.E, wl.R)
    b = oracle.dispatch(x, idx, w, wl.E, wl.R)
    for key in ("token_row", "recv_src_idx", "recv_expert_offset", "recv_rank_offset"):
        np.testing.assert_array_equal(d[key], b[key])
    for t in range(wl.T):
        q, s = oracle.quantize_row(x[t])
        for r in d["token_row"][t]:
            np.testing.assert_array_equal(d["recv_x_fp8"][r], q)
            np.testing.assert_array_equal(d["recv_scales"][r], s)


def test_fp8_cached_dispatch_matches_fp8_dispatch():
    wl = CONFIGS["ll_fp8"].scaled(T=20, H=384)
    x, idx, w = make_workload(wl)
    d = oracle.dispatch_fp8(x, idx, w, wl.E, wl.R)
    N = int(d["recv_expert_offset"][-1])
    q, s = oracle.dispatch_fp8_cached(x, d["token_row"], N)
    np.testing.assert_array_equal(q, d["recv_x_fp8"][:N])
    np.testing.assert_array_equal(s.view(np.uint32), d["recv_scales"][:N].view(np.uint32))
