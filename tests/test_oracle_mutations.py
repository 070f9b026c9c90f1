"""Planted-mistake check for the oracle's pins (CPU only).

Each case copies ep_oracle.c, plants one plausible mistake (a dropped term, a
wrong sign, index or tie rule, a transposed operand), builds the copy with gcc
into a temporary directory and runs the pins against it: at least one pin must
fail.  This shows that the pins in the other oracle tests constrain every part
of the oracle, not just that the oracle agrees with itself.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_combine as tc
import test_oracle_fp8 as tf
import test_oracle_ht as th
import test_oracle_ll as tll
import test_oracle_layout_rows as tl

SRC = os.path.join(os.path.dirname(oracle.__file__), "ep_oracle.c")


def _layout_pins():
    for i in range(len(tl.ROUTINGS)):
        tl.test_layout_matches_bincount(i)
    for name in ("hand_example.json", "hand_example_masked.json"):
        tl.test_hand_worked_example(name)


def _row_pins():
    for i in range(len(tl.ROUTINGS)):
        tl.test_rows_are_stable_argsort(i)
    tl.test_weights_travel_with_rows()
    for name in ("hand_example.json", "hand_example_masked.json"):
        tl.test_hand_worked_example(name)


def _cached_pins():
    for i in range(len(tl.ROUTINGS)):
        tl.test_cached_dispatch_reproduces_dispatch(i)
    tf.test_fp8_cached_dispatch_matches_fp8_dispatch()


def _ht_pins():
    th.test_hand_worked_example()
    for i in range(len(tl.ROUTINGS)):
        th.test_matches_brute_force(i)
    for name in ("tiny", "large"):
        th.test_weights_and_slots_conserved(name)
    th.test_unweighted_combine_closed_form()


def _ll_pins():
    tll.test_hand_worked_example()
    for i in range(len(tl.ROUTINGS)):
        for cap in tll.CAPS:
            tll.test_matches_brute_force(i, cap)
    for name in ("tiny", "ll_fp8"):
        tll.test_no_drop_is_the_packed_dispatch_per_expert(name)
    for cap in (1, 2, 5):
        tll.test_drops_are_the_latest_slots_and_conserved(cap)
    tll.test_fp8_rows_hold_the_token_cast()
    tll.test_combine_over_padded_map_equals_packed_combine()


def _fp8_pins():
    tf.test_decode_all_codes_against_torch()
    tf.test_encode_roundtrips_every_finite_code()
    tf.test_midpoints_round_to_even_code()
    tf.test_matches_torch_below_464()
    tf.test_saturates_above_448()
    tf.test_hand_computed_block()
    for s, seed in [(2.0, 0), (1e-3, 2)]:
        tf.test_quantize_row_bounds(s, seed)
    tf.test_zero_and_signed_zero_blocks()
    tf.test_tiny_amax_keeps_denormal_scale()
    tf.test_non_finite_blocks()
    tf.test_fp8_dispatch_rows_hold_token_cast()


def _combine_pins():
    tc.test_bf16_rne_matches_torch()
    tc.test_weight_one_k1_returns_rows()
    tc.test_power_of_two_weights_identity_experts_exact(4, 0.25)
    tc.test_identity_experts_give_x_times_sum_w()
    for name, mask in [("tiny", 0.0), ("skewed", 0.15)]:
        tc.test_random_experts_within_fma_chain_bound(name, mask)
    tc.test_masked_and_out_of_range_rows_skipped()
    tc.test_signed_zero_start()
    tc.test_hand_computed_order_and_fma()


MUTATIONS = {
    # layout
    "rank_map_modulo": ("is_token_in_rank[t * R + e / epr] = 1;",
                        "is_token_in_rank[t * R + e % R] = 1;", _layout_pins),
    "group_and_not_or": ("touched |= is_token_in_rank", "touched &= is_token_in_rank", _layout_pins),
    "group_off_by_one": ("for (int r = g * P; r < (g + 1) * P; ++r)",
                         "for (int r = g * P; r <= (g + 1) * P && r < R; ++r)", _layout_pins),
    "count_masked_slots": ("if (!slot_valid(e, E)) continue;\n            num_tokens_per_expert[e] += 1;",
                           "if (e < 0) continue;\n            num_tokens_per_expert[e % E] += 1;",
                           _layout_pins),
    # receive order
    "unstable_rows_reverse_j": ("for (int64_t t = 0; t < T; ++t)\n        for (int j = 0; j < k; ++j) {\n            int64_t e = topk_idx[t * k + j];\n            if (!slot_valid(e, E)) { token_row",
                                "for (int64_t t = 0; t < T; ++t)\n        for (int j = k - 1; j >= 0; --j) {\n            int64_t e = topk_idx[t * k + j];\n            if (!slot_valid(e, E)) { token_row",
                                _row_pins),
    "rank_offset_index": ("rank_offset[r] = expert_offset[r * epr];",
                          "rank_offset[r] = expert_offset[r];", _row_pins),
    "copy_wrong_token": ("memcpy(recv_x + (int64_t)row * H, x + t * (int64_t)H,",
                         "memcpy(recv_x + (int64_t)row * H, x + ((t + 1) % T) * (int64_t)H,", _row_pins),
    "copy_short_row": ("x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);",
                       "x + t * (int64_t)H, sizeof(uint16_t) * (size_t)(H - 1));", _row_pins),
    "weight_transposed": ("recv_topk_weights[row] = topk_weights[t * k + j];\n        }\n    return ORC_OK;\n}\n\n/* Per-token",
                          "recv_topk_weights[row] = topk_weights[j * T + t];\n        }\n    return ORC_OK;\n}\n\n/* Per-token",
                          _row_pins),
    # FP8
    "e4m3_ties_down": ("else code = (lo & 1) ? hi : lo;", "else code = lo;", _fp8_pins),
    "e4m3_no_saturation": ("if (a >= e4m3_table[126]) return (uint8_t)(sign | 126);",
                           "if (a >= 464.0f) return (uint8_t)(sign | 127);", _fp8_pins),
    "e4m3_subnormal_scale": ("return ldexpf((float)M, -9);", "return ldexpf((float)M, -10);", _fp8_pins),
    "e4m3_sign_dropped": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = 0x00;", _fp8_pins),
    "amax_signed": ("float v = fabsf(bf16_to_f32(xrow[h]));", "float v = bf16_to_f32(xrow[h]);", _fp8_pins),
    "scale_447": ("float s = a / 448.0f;", "float s = a / 447.0f;", _fp8_pins),
    "amax_nan_poisons": ("if (v > a) a = v;", "if (!(v <= a)) a = v;", _fp8_pins),
    "e4m3_nan_keeps_sign": ("if (isnan(v)) return 0x7F;", "if (isnan(v)) return signbit(v) ? 0xFF : 0x7F;",
                            _fp8_pins),
    "scale_reciprocal_multiply": ("oracle_e4m3_encode(bf16_to_f32(xrow[h]) / s)",
                                  "oracle_e4m3_encode(bf16_to_f32(xrow[h]) * s)", _fp8_pins),
    # combine and bf16 rounding
    "bf16_ties_up": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
                     "if (dropped >= 0x8000u) kept += 1u;", _combine_pins),
    "bf16_truncate": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
                      "(void)dropped;", _combine_pins),
    "combine_drop_last_term": ("for (int j = 0; j < k; ++j) {\n                int32_t row = token_row[t * k + j];\n                if (row < 0 || (int64_t)row >= num_rows) continue;",
                               "for (int j = 0; j < k - 1; ++j) {\n                int32_t row = token_row[t * k + j];\n                if (row < 0 || (int64_t)row >= num_rows) continue;",
                               _combine_pins),
    "combine_weight_index": ("const float wj = topk_weights ? topk_weights[t * k + j] : 1.0f;",
                             "const float wj = topk_weights ? topk_weights[j] : 1.0f;", _combine_pins),
    "combine_sign": ("acc = fmaf(wj,", "acc = fmaf(-wj,", _combine_pins),
    "combine_negzero_start": ("float acc = 0.0f;\n            for (int j = 0; j < k; ++j) {\n                int32_t row",
                              "float acc = -0.0f;\n            for (int j = 0; j < k; ++j) {\n                int32_t row",
                              _combine_pins),
    "combine_reverse_j": ("for (int j = 0; j < k; ++j) {\n                int32_t row = token_row[t * k + j];\n                if (row < 0 || (int64_t)row >= num_rows) continue;",
                          "for (int j = k - 1; j >= 0; --j) {\n                int32_t row = token_row[t * k + j];\n                if (row < 0 || (int64_t)row >= num_rows) continue;",
                          _combine_pins),
    "combine_mul_then_add": ("acc = fmaf(wj, bf16_to_f32(expert_out[(int64_t)row * H + h]), acc);",
                             "{ float p = wj * bf16_to_f32(expert_out[(int64_t)row * H + h]); acc = acc + p; }",
                             _combine_pins),
    "combine_fp64_accumulator": ("float acc = 0.0f;\n            for (int j = 0; j < k; ++j) {\n                int32_t row = token_row[t * k + j];\n                if (row < 0 || (int64_t)row >= num_rows) continue;\n                const float wj = topk_weights ? topk_weights[t * k + j] : 1.0f;\n                acc = fmaf(wj, bf16_to_f32(expert_out[(int64_t)row * H + h]), acc);",
                                 "double acc = 0.0;\n            for (int j = 0; j < k; ++j) {\n                int32_t row = token_row[t * k + j];\n                if (row < 0 || (int64_t)row >= num_rows) continue;\n                const float wj = topk_weights ? topk_weights[t * k + j] : 1.0f;\n                acc = fma((double)wj, (double)bf16_to_f32(expert_out[(int64_t)row * H + h]), acc);",
                                 _combine_pins),
    "combine_no_range_guard": ("if (row < 0 || (int64_t)row >= num_rows) continue;\n                const float wj",
                               "if (row < 0) continue;\n                if (row >= num_rows) row = num_rows - 1;\n                const float wj",
                               _combine_pins),
    # cached dispatch
    "cached_no_range_guard": ("if (row < 0 || (int64_t)row >= num_rows) continue;\n            memcpy(recv_x",
                              "if (row < 0) continue;\n            if (row >= num_rows) row = num_rows - 1;\n            memcpy(recv_x",
                              _cached_pins),
    "cached_wrong_source": ("memcpy(recv_x + (int64_t)row * H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);\n        }\n    return ORC_OK;\n}\n\n/* Cached FP8",
                            "memcpy(recv_x + (int64_t)row * H, x + (T - 1 - t) * (int64_t)H, sizeof(uint16_t) * (size_t)H);\n        }\n    return ORC_OK;\n}\n\n/* Cached FP8",
                            _cached_pins),
    "cached_fp8_scale_row": ("recv_scales + (int64_t)row * nb);\n        }\n    return ORC_OK;",
                             "recv_scales + (int64_t)t * nb);\n        }\n    return ORC_OK;",
                             _cached_pins),
    # rank-deduplicated dispatch
    "ht_token_major_rows": ("    for (int r = 0; r < R; ++r) {\n        int32_t row = recv_rank_offset[r];\n        for (int64_t t = 0; t < T; ++t) {",
                            "    for (int r = 0; r < R; ++r) {\n        int32_t row = recv_rank_offset[R - 1 - r];\n        for (int64_t t = 0; t < T; ++t) {",
                            _ht_pins),
    "ht_weights_not_masked": ("(local && topk_weights) ? topk_weights[t * k + j] : 0.0f;",
                              "topk_weights ? topk_weights[t * k + j] : 0.0f;", _ht_pins),
    "ht_local_by_modulo": ("int local = slot_valid(e, E) && e / epr == r;",
                           "int local = slot_valid(e, E) && e % R == r;", _ht_pins),
    "ht_offset_off_by_one": ("for (int64_t t = 0; t < T; ++t)\n        for (int r = 0; r < R; ++r) recv_rank_offset[r + 1] += token_rank_row[t * R + r];",
                             "for (int64_t t = 1; t < T; ++t)\n        for (int r = 0; r < R; ++r) recv_rank_offset[r + 1] += token_rank_row[t * R + r];",
                             _ht_pins),
    "combine_unweighted_zero": ("const float wj = topk_weights ? topk_weights[t * k + j] : 1.0f;",
                                "const float wj = topk_weights ? topk_weights[t * k + j] : 0.5f;", _ht_pins),
    # padded expert-major (low-latency) dispatch
    "ll_capacity_off_by_one": ("if (pos >= capacity) continue;", "if (pos > capacity) continue;", _ll_pins),
    "ll_position_major": ("int32_t slot = (int32_t)(e * capacity + pos);",
                          "int32_t slot = (int32_t)(pos * E + e);", _ll_pins),
    "ll_count_unclamped": ("if (pos >= capacity) continue;",
                           "recv_count[e] = (int32_t)(pos + 1);\n            if (pos >= capacity) continue;",
                           _ll_pins),
    "ll_weight_first_slot": ("recv_topk_weights[slot] = topk_weights[t * k + j];",
                             "recv_topk_weights[slot] = topk_weights[t * k];", _ll_pins),
    "ll_fp8_scale_row": ("recv_scales + (int64_t)slot * nb);",
                         "recv_scales + (int64_t)(slot / 2) * nb);", _ll_pins),
    "bf16_widen_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;", _combine_pins),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    find, repl, pins = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(find) >= 1, f"mutation anchor not found: {name}"
    mutated = src.replace(find, repl, 1)
    csrc = tmp_path / "ep_oracle_mut.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-w", "-o", str(lib), str(csrc), "-lm"])
    oracle._use_library(str(lib))
    try:
        with pytest.raises((AssertionError, oracle.OracleError)):
            pins()
    finally:
        oracle._use_library(None)


def test_unmutated_oracle_passes_all_pins():
    for pins in (_layout_pins, _row_pins, _fp8_pins, _combine_pins, _cached_pins, _ht_pins, _ll_pins):
        pins()
