/*
 * ep_oracle.c -- CPU oracle for MoE expert-parallel dispatch / combine.
 *
 * TEST INFRASTRUCTURE.  This file is the plain, sequential, obviously-correct
 * definition that the HIP path is checked against.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never calls it.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no fast-math), so
 * every floating-point operation below is one IEEE binary32 operation in the
 * order written.
 *
 * Sources (all on the page "[Not ready] MSCCLPP EP implementation #852"):
 *   - PR body, "Scope / Intranode": get_dispatch_layout, intranode dispatch
 *     and combine over the x / topk_idx / topk_weights tensor ABI.
 *   - PR body, "Scope / Internode HT": the two-level (RDMA-rank = group)
 *     variant of the layout.
 *   - commit fixing internode HT combine: combine must consume the
 *     receiver-side prefix sums that dispatch produced (here: token_row).
 *   - low-latency port commit: dispatch<kUseFP8,...> casts each token to FP8
 *     with per-128-channel scales before sending.
 * Where the page leaves a step open (expert->rank map, group size, order of
 * rows inside an expert, FP8 format and arithmetic order, summation order),
 * the plainest reading is taken and stated at the function that uses it.
 *
 * Return codes: 0 = ok, 1 = invalid argument.  Outputs are untouched on error.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1

/* A slot (t,j) routes somewhere iff its expert id is in [0, E).  Any other
 * value (the conventional -1, or anything out of range) is an empty slot. */
static int slot_valid(int64_t e, int E) { return e >= 0 && e < (int64_t)E; }

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even, on the magnitude: the two
 * bf16 neighbours of f are its truncation and the next value away from zero;
 * the 16 dropped bits decide (above half: up, below: down, exactly half: the
 * neighbour whose last kept bit is 0).  NaN stays NaN (quiet). */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* ---------------------------------------------------------------------------
 * OCP OFP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 *   E = 0      : subnormal, value M/8 * 2^-6
 *   E = 1..15  : normal, value (1 + M/8) * 2^(E-7); E=15,M=7 is NaN
 * so the non-negative finite values are codes 0x00..0x7E, largest 448.
 * Encoding used by the method: round to the nearest representable value,
 * ties to the code with even mantissa, saturating beyond 448.  (The page
 * names no FP8 format; the scale rule "amax / 448" fixes E4M3 with 448 as
 * its largest finite value, which is OCP E4M3FN, not the 240-max FNUZ.)
 * ------------------------------------------------------------------------- */
static float e4m3_table[127];
static int e4m3_table_ready = 0;

static float e4m3_code_value(int code)     /* code in 0..126, sign clear */
{
    int E = code >> 3, M = code & 7;
    if (E == 0) return ldexpf((float)M, -9);          /* M/8 * 2^-6 */
    return ldexpf((float)(8 + M), E - 10);            /* (8+M)/8 * 2^(E-7) */
}

static void e4m3_init(void)
{
    if (e4m3_table_ready) return;
    for (int c = 0; c < 127; ++c) e4m3_table[c] = e4m3_code_value(c);
    e4m3_table_ready = 1;
}

float oracle_e4m3_decode(uint8_t code)
{
    e4m3_init();
    if ((code & 0x7F) == 0x7F) return NAN;
    float v = e4m3_table[code & 0x7F];
    return (code & 0x80) ? -v : v;
}

uint8_t oracle_e4m3_encode(float v)
{
    e4m3_init();
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a >= e4m3_table[126]) return (uint8_t)(sign | 126);   /* saturate at 448 */
    /* Largest code whose value is <= a (binary search over the sorted table). */
    int lo = 0, hi = 126;                       /* table[lo] <= a < table[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_table[mid] <= a) lo = mid; else hi = mid;
    }
    /* Midpoint of two adjacent codes has at most 5 significant bits: exact. */
    float half = (e4m3_table[lo] + e4m3_table[hi]) * 0.5f;
    int code;
    if (a < half) code = lo;
    else if (a > half) code = hi;
    else code = (lo & 1) ? hi : lo;             /* tie: even mantissa bit */
    return (uint8_t)(sign | code);
}

void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_bf16_rne_array(const float* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(v[i]);
}

/* ---------------------------------------------------------------------------
 * Layout (get_dispatch_layout).  Experts are split into R contiguous blocks
 * of E/R, so rank(e) = e / (E/R); ranks into G = R/P groups of P consecutive
 * ranks (the two-level layout groups the ranks of one node).
 *   num_tokens_per_expert[e] = number of valid slots (t,j) routed to e
 *   is_token_in_rank[t,r]    = 1 iff some valid slot of t lands on rank r
 *   num_tokens_per_rank[r]   = number of tokens t with is_token_in_rank[t,r]
 *   num_tokens_per_group[g]  = number of tokens touching any rank of group g
 * ------------------------------------------------------------------------- */
static int check_routing_args(int64_t T, int k, int E, int R)
{
    if (T < 0 || k < 1 || E < 1 || R < 1) return 0;
    if (E % R != 0) return 0;
    return 1;
}

int oracle_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R, int P,
                  int32_t* num_tokens_per_rank, int32_t* num_tokens_per_group,
                  int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank)
{
    if (!check_routing_args(T, k, E, R) || P < 1 || R % P != 0) return ORC_EINVAL;
    if ((T > 0 && !topk_idx) || !num_tokens_per_rank || !num_tokens_per_expert ||
        (T > 0 && !is_token_in_rank))
        return ORC_EINVAL;
    const int epr = E / R, G = R / P;

    for (int e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;
    for (int r = 0; r < R; ++r) num_tokens_per_rank[r] = 0;
    if (num_tokens_per_group)
        for (int g = 0; g < G; ++g) num_tokens_per_group[g] = 0;
    for (int64_t i = 0; i < T * (int64_t)R; ++i) is_token_in_rank[i] = 0;

    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (!slot_valid(e, E)) continue;
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[t * R + e / epr] = 1;
        }
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) num_tokens_per_rank[r] += is_token_in_rank[t * R + r];
    if (num_tokens_per_group)
        for (int64_t t = 0; t < T; ++t)
            for (int g = 0; g < G; ++g) {
                int touched = 0;
                for (int r = g * P; r < (g + 1) * P; ++r) touched |= is_token_in_rank[t * R + r];
                num_tokens_per_group[g] += touched;
            }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Receive order shared by both dispatch variants.  Each valid slot (t,j) gets
 * one receive row.  Rows are grouped by expert in ascending expert order (so
 * every rank's experts form one contiguous range, rank-major), and inside an
 * expert by (t, j) ascending (one source, so no per-source-rank order is
 * left to keep): a stable counting sort keyed by expert over the slots in
 * lexicographic order.
 *   recv_expert_offset[e] = first row of expert e, [E] = total valid slots
 *   recv_rank_offset[r]   = recv_expert_offset[r * E/R], r = 0..R
 *   token_row[t,j]        = row of slot (t,j), -1 for an empty slot
 *   recv_src_idx[row]     = source token t of that row
 * ------------------------------------------------------------------------- */
static void assign_rows(const int64_t* topk_idx, int64_t T, int k, int E, int R,
                        int32_t* expert_offset, int32_t* rank_offset, int32_t* token_row,
                        int32_t* recv_src_idx)
{
    const int epr = E / R;
    for (int e = 0; e <= E; ++e) expert_offset[e] = 0;
    for (int64_t s = 0; s < T * (int64_t)k; ++s)
        if (slot_valid(topk_idx[s], E)) expert_offset[topk_idx[s] + 1] += 1;
    for (int e = 0; e < E; ++e) expert_offset[e + 1] += expert_offset[e];
    if (rank_offset)
        for (int r = 0; r <= R; ++r) rank_offset[r] = expert_offset[r * epr];

    /* cursor[e] walks expert e's row range. */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) abort();
    for (int e = 0; e < E; ++e) cursor[e] = expert_offset[e];
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (!slot_valid(e, E)) { token_row[t * k + j] = -1; continue; }
            int32_t row = cursor[e]++;
            token_row[t * k + j] = row;
            recv_src_idx[row] = (int32_t)t;
        }
    free(cursor);
}

static int check_dispatch_args(const void* x, const int64_t* topk_idx, int64_t T, int H,
                               int k, int E, int R, const void* recv, const int32_t* src,
                               const int32_t* eoff, const int32_t* trow)
{
    if (!check_routing_args(T, k, E, R) || H < 1) return 0;
    if (T * (int64_t)k > INT32_MAX) return 0;
    if (!eoff) return 0;
    if (T > 0 && (!x || !topk_idx || !recv || !src || !trow)) return 0;
    return 1;
}

/* ep_dispatch (bf16): recv_x[row(t,j), :] = x[t, :] bit for bit; the routing
 * weight of the slot travels with it (recv_topk_weights[row] = w[t,j]). */
int oracle_dispatch(const uint16_t* x, const int64_t* topk_idx, const float* topk_weights,
                    int64_t T, int H, int k, int E, int R,
                    uint16_t* recv_x, int32_t* recv_src_idx, float* recv_topk_weights,
                    int32_t* recv_expert_offset, int32_t* recv_rank_offset, int32_t* token_row)
{
    if (!check_dispatch_args(x, topk_idx, T, H, k, E, R, recv_x, recv_src_idx,
                             recv_expert_offset, token_row))
        return ORC_EINVAL;
    assign_rows(topk_idx, T, k, E, R, recv_expert_offset, recv_rank_offset, token_row,
                recv_src_idx);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t row = token_row[t * k + j];
            if (row < 0) continue;
            memcpy(recv_x + (int64_t)row * H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
            if (topk_weights && recv_topk_weights) recv_topk_weights[row] = topk_weights[t * k + j];
        }
    return ORC_OK;
}

/* Per-token FP8 cast with one fp32 scale per 128 channels (low-latency
 * dispatch with kUseFP8).  For block c of token t (the page gives no
 * arithmetic; this is the plainest one: a true division by the scale, and an
 * all-zero block gets scale 0 and zero codes):
 *   a = max |x| over the block's 128 channels that are not NaN (in fp32;
 *       bf16 -> fp32 is exact; NaN fails the comparison and is passed over)
 *   s = a / 448                       (one IEEE fp32 division)
 *   q = E4M3(x / s)   if s > 0, else all codes 0x00
 * so a NaN channel gets the NaN code 0x7F when s > 0, and an infinite a gives
 * s = inf (finite channels -> signed zero, infinite ones inf/inf = NaN).
 * H must be a multiple of 128. */
int oracle_quantize_row(const uint16_t* xrow, int H, uint8_t* q, float* scales)
{
    if (H < 128 || H % 128 != 0 || !xrow || !q || !scales) return ORC_EINVAL;
    for (int c = 0; c < H / 128; ++c) {
        float a = 0.0f;
        for (int h = 128 * c; h < 128 * (c + 1); ++h) {
            float v = fabsf(bf16_to_f32(xrow[h]));
            if (v > a) a = v;
        }
        float s = a / 448.0f;
        scales[c] = s;
        for (int h = 128 * c; h < 128 * (c + 1); ++h)
            q[h] = (s > 0.0f) ? oracle_e4m3_encode(bf16_to_f32(xrow[h]) / s) : (uint8_t)0x00;
    }
    return ORC_OK;
}

/* ep_dispatch_fp8: same receive order as oracle_dispatch; each row holds the
 * token's codes [H] and scales [H/128]; the scales are repeated in every row
 * of the token so that each rank's range is self-contained. */
int oracle_dispatch_fp8(const uint16_t* x, const int64_t* topk_idx, const float* topk_weights,
                        int64_t T, int H, int k, int E, int R,
                        uint8_t* recv_x_fp8, float* recv_scales, int32_t* recv_src_idx,
                        float* recv_topk_weights, int32_t* recv_expert_offset,
                        int32_t* recv_rank_offset, int32_t* token_row)
{
    if (!check_dispatch_args(x, topk_idx, T, H, k, E, R, recv_x_fp8, recv_src_idx,
                             recv_expert_offset, token_row))
        return ORC_EINVAL;
    if (H % 128 != 0 || (T > 0 && !recv_scales)) return ORC_EINVAL;
    assign_rows(topk_idx, T, k, E, R, recv_expert_offset, recv_rank_offset, token_row,
                recv_src_idx);
    const int nb = H / 128;
    for (int64_t t = 0; t < T; ++t) {
        int first = -1;
        for (int j = 0; j < k; ++j) {
            int32_t row = token_row[t * k + j];
            if (row < 0) continue;
            if (first < 0) {
                oracle_quantize_row(x + t * (int64_t)H, H, recv_x_fp8 + (int64_t)row * H,
                                    recv_scales + (int64_t)row * nb);
                first = row;
            } else {
                memcpy(recv_x_fp8 + (int64_t)row * H, recv_x_fp8 + (int64_t)first * H, (size_t)H);
                memcpy(recv_scales + (int64_t)row * nb, recv_scales + (int64_t)first * nb,
                       sizeof(float) * (size_t)nb);
            }
            if (topk_weights && recv_topk_weights) recv_topk_weights[row] = topk_weights[t * k + j];
        }
    }
    return ORC_OK;
}

/* Cached dispatch: reuse the receive map of an earlier dispatch (page
 * "[Not ready] MSCCLPP EP implementation #852", PR body "Scope / Internode
 * HT": cached_notify reuses a previous dispatch's layout for a repeat
 * dispatch).  For every slot whose row r = token_row[t,j] lies in
 * [0, num_rows): recv_x[r, :] = x[t, :]; other slots are skipped. */
int oracle_dispatch_cached(const uint16_t* x, const int32_t* token_row, int64_t T, int H, int k,
                           uint16_t* recv_x, int64_t num_rows)
{
    if (T < 0 || H < 1 || k < 1 || num_rows < 0) return ORC_EINVAL;
    if (T > 0 && (!x || !token_row || (num_rows > 0 && !recv_x))) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t row = token_row[t * k + j];
            if (row < 0 || (int64_t)row >= num_rows) continue;
            memcpy(recv_x + (int64_t)row * H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
        }
    return ORC_OK;
}

/* Cached FP8 dispatch: the per-token cast of oracle_quantize_row written to
 * every row of the reused map that lies in [0, num_rows). */
int oracle_dispatch_fp8_cached(const uint16_t* x, const int32_t* token_row, int64_t T, int H,
                               int k, uint8_t* recv_x_fp8, float* recv_scales, int64_t num_rows)
{
    if (T < 0 || H < 128 || H % 128 != 0 || k < 1 || num_rows < 0) return ORC_EINVAL;
    if (T > 0 && (!x || !token_row || (num_rows > 0 && (!recv_x_fp8 || !recv_scales))))
        return ORC_EINVAL;
    const int nb = H / 128;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t row = token_row[t * k + j];
            if (row < 0 || (int64_t)row >= num_rows) continue;
            oracle_quantize_row(x + t * (int64_t)H, H, recv_x_fp8 + (int64_t)row * H,
                                recv_scales + (int64_t)row * nb);
        }
    return ORC_OK;
}

/* Low-latency padded receive layout: page "[Not ready] MSCCLPP EP
 * implementation #852" -- the LL benchmark's receive buffer (the commit that
 * stops cloning the ~58 MB dispatch receive buffer: one expert region per
 * local expert, each sized for a fixed number of tokens per source) and the
 * low-latency runtime's rank-major / expert-major tests at capacities 1 and 2.
 * With one source the receive buffer is [E, capacity, H]: expert e owns rows
 * e*capacity .. e*capacity + capacity - 1, filled from the front in (t, j)
 * order; a slot that finds its expert's region full is dropped.
 *   recv_count[e]               = min(#valid slots with expert e, capacity)
 *   token_slot[t, j]            = e*capacity + (its position among expert e's
 *                                 slots in (t, j) order) if that position is
 *                                 below capacity, else -1 (also -1 if empty)
 *   recv_x[slot, :]             = x[t, :]
 *   recv_src_idx[slot]          = t
 *   recv_topk_weights[slot]     = topk_weights[t, j]
 * Rows from recv_count[e] to capacity - 1 of each expert are not written. */
static int check_ll_args(const void* x, const int64_t* topk_idx, int64_t T, int H, int k, int E,
                         int capacity, const void* recv, const int32_t* recv_count,
                         const int32_t* recv_src_idx, const int32_t* token_slot)
{
    if (T < 0 || H < 1 || k < 1 || E < 1 || capacity < 1) return 0;
    if ((int64_t)E * capacity > INT32_MAX) return 0;
    if (!recv_count) return 0;
    if (T > 0 && (!x || !topk_idx || !recv || !recv_src_idx || !token_slot)) return 0;
    return 1;
}

static void assign_ll_slots(const int64_t* topk_idx, int64_t T, int k, int E, int capacity,
                            int32_t* recv_count, int32_t* token_slot, int32_t* recv_src_idx,
                            const float* topk_weights, float* recv_topk_weights)
{
    for (int e = 0; e < E; ++e) recv_count[e] = 0;
    int64_t* seen = (int64_t*)calloc((size_t)E, sizeof(int64_t));   /* slots met so far */
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            token_slot[t * k + j] = -1;
            if (!slot_valid(e, E)) continue;
            int64_t pos = seen[e]++;
            if (pos >= capacity) continue;
            int32_t slot = (int32_t)(e * capacity + pos);
            token_slot[t * k + j] = slot;
            recv_count[e] = (int32_t)(pos + 1);
            recv_src_idx[slot] = (int32_t)t;
            if (topk_weights && recv_topk_weights) recv_topk_weights[slot] = topk_weights[t * k + j];
        }
    free(seen);
}

int oracle_dispatch_ll(const uint16_t* x, const int64_t* topk_idx, const float* topk_weights,
                       int64_t T, int H, int k, int E, int capacity, uint16_t* recv_x,
                       int32_t* recv_count, int32_t* recv_src_idx, float* recv_topk_weights,
                       int32_t* token_slot)
{
    if (!check_ll_args(x, topk_idx, T, H, k, E, capacity, recv_x, recv_count, recv_src_idx,
                       token_slot))
        return ORC_EINVAL;
    assign_ll_slots(topk_idx, T, k, E, capacity, recv_count, token_slot, recv_src_idx,
                    topk_weights, recv_topk_weights);
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t slot = token_slot[t * k + j];
            if (slot < 0) continue;
            memcpy(recv_x + (int64_t)slot * H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
        }
    return ORC_OK;
}

/* The same padded layout holding the per-token FP8 cast of
 * oracle_quantize_row: codes [E, capacity, H], scales [E, capacity, H/128]. */
int oracle_dispatch_ll_fp8(const uint16_t* x, const int64_t* topk_idx, const float* topk_weights,
                           int64_t T, int H, int k, int E, int capacity, uint8_t* recv_x_fp8,
                           float* recv_scales, int32_t* recv_count, int32_t* recv_src_idx,
                           float* recv_topk_weights, int32_t* token_slot)
{
    if (!check_ll_args(x, topk_idx, T, H, k, E, capacity, recv_x_fp8, recv_count, recv_src_idx,
                       token_slot))
        return ORC_EINVAL;
    if (H % 128 != 0 || (T > 0 && !recv_scales)) return ORC_EINVAL;
    assign_ll_slots(topk_idx, T, k, E, capacity, recv_count, token_slot, recv_src_idx,
                    topk_weights, recv_topk_weights);
    const int nb = H / 128;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t slot = token_slot[t * k + j];
            if (slot < 0) continue;
            oracle_quantize_row(x + t * (int64_t)H, H, recv_x_fp8 + (int64_t)slot * H,
                                recv_scales + (int64_t)slot * nb);
        }
    return ORC_OK;
}

/* High-throughput (rank-deduplicated) dispatch: page "[Not ready] MSCCLPP EP
 * implementation #852", PR body "Scope / Intranode" (intranode dispatch sends
 * each token once to every rank that hosts at least one of its experts; the
 * receiving rank gets the token's top-k ids remapped to its local experts).
 * One receive row per (t, r) with is_token_in_rank[t, r] = 1, ordered by rank,
 * then token ascending:
 *   recv_rank_offset[r]   = first row of rank r, [R] = rows
 *   token_rank_row[t, r]  = row of (t, r), or -1
 *   recv_x[row]           = x[t]
 *   recv_src_idx[row]     = t
 *   recv_topk_idx[row, j] = topk_idx[t, j] - r*E/R if that expert is on rank r, else -1
 *   recv_topk_weights[row, j] = topk_weights[t, j] on the same condition, else 0
 * (The page leaves the weights of non-local slots unspecified; zero is the
 * reading taken, so a rank can sum its row's weights directly.) */
int oracle_dispatch_ht(const uint16_t* x, const int64_t* topk_idx, const float* topk_weights,
                       int64_t T, int H, int k, int E, int R, uint16_t* recv_x,
                       int32_t* recv_src_idx, int64_t* recv_topk_idx, float* recv_topk_weights,
                       int32_t* recv_rank_offset, int32_t* token_rank_row)
{
    if (!check_routing_args(T, k, E, R) || H < 1) return ORC_EINVAL;
    if (T * (int64_t)R > INT32_MAX || !recv_rank_offset) return ORC_EINVAL;
    if (T > 0 && (!x || !topk_idx || !recv_x || !recv_src_idx || !recv_topk_idx || !token_rank_row))
        return ORC_EINVAL;
    const int epr = E / R;
    for (int64_t i = 0; i < T * (int64_t)R; ++i) token_rank_row[i] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (slot_valid(e, E)) token_rank_row[t * R + e / epr] = 1;   /* is_token_in_rank */
        }
    for (int r = 0; r <= R; ++r) recv_rank_offset[r] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) recv_rank_offset[r + 1] += token_rank_row[t * R + r];
    for (int r = 0; r < R; ++r) recv_rank_offset[r + 1] += recv_rank_offset[r];
    for (int r = 0; r < R; ++r) {
        int32_t row = recv_rank_offset[r];
        for (int64_t t = 0; t < T; ++t) {
            if (!token_rank_row[t * R + r]) { token_rank_row[t * R + r] = -1; continue; }
            token_rank_row[t * R + r] = row;
            recv_src_idx[row] = (int32_t)t;
            memcpy(recv_x + (int64_t)row * H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
            for (int j = 0; j < k; ++j) {
                int64_t e = topk_idx[t * k + j];
                int local = slot_valid(e, E) && e / epr == r;
                recv_topk_idx[(int64_t)row * k + j] = local ? e - (int64_t)r * epr : -1;
                if (recv_topk_weights)
                    recv_topk_weights[(int64_t)row * k + j] =
                        (local && topk_weights) ? topk_weights[t * k + j] : 0.0f;
            }
            ++row;
        }
    }
    return ORC_OK;
}

/* ep_combine: for each token t and channel h, an fp32 accumulator starts at
 * +0 and takes one fused multiply-add per valid slot in fixed top-k (j)
 * order:  acc = fma(w[t,j], y[token_row[t,j], h], acc);  out = bf16_RNE(acc).
 * A slot whose row is negative or >= num_rows contributes nothing.  Without
 * weights (NULL) every weight is 1: the plain fp32 sum in j order, which is the
 * high-throughput combine over a token's per-rank rows (token_rank_row). */
int oracle_combine(const uint16_t* expert_out, int64_t num_rows, const int32_t* token_row,
                   const float* topk_weights, int64_t T, int H, int k, uint16_t* combined_x)
{
    if (T < 0 || H < 1 || k < 1 || num_rows < 0) return ORC_EINVAL;
    if (T > 0 && (!token_row || !combined_x)) return ORC_EINVAL;
    if (T > 0 && num_rows > 0 && !expert_out) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int32_t row = token_row[t * k + j];
                if (row < 0 || (int64_t)row >= num_rows) continue;
                const float wj = topk_weights ? topk_weights[t * k + j] : 1.0f;
                acc = fmaf(wj, bf16_to_f32(expert_out[(int64_t)row * H + h]), acc);
            }
            combined_x[t * (int64_t)H + h] = oracle_bf16_rne(acc);
        }
    return ORC_OK;
}
