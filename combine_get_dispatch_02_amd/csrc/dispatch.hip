// dispatch.hip -- receive order and data movement of ep_dispatch /
// ep_dispatch_fp8 on gfx950.
//
// Page "[Not ready] MSCCLPP EP implementation #852": intranode dispatch
// (PR body, "Scope / Intranode") places each token's hidden vector in the
// receive buffers of the ranks its experts live on; the low-latency dispatch
// (low-latency port commit, dispatch<kUseFP8,...>) optionally casts each
// token to FP8 with one scale per 128 channels on the way.  On one GPU the
// ranks are contiguous ranges of one receive buffer, rows grouped by expert
// and, inside an expert, ordered by (token, slot).
//
// Kernels (all deterministic; no global atomics):
//   tile_hist    per tile of >= 64 tokens (at most 64 tiles at the benchmark
//                sizes), per-expert slot counts (LDS atomics)
//   rows         per tile: per-expert prefix over earlier tiles + block scan
//                over experts -> tile base rows; each lane holds its slots'
//                ids in registers; the stable rank of every slot inside the
//                tile from wave64 ballot matching, by up to 16 waves (as LDS
//                allows); writes token_row, recv_src_idx, recv_topk_weights
//                and the offsets
//   rows_fused   tile_hist and rows in one launch (every block sweeps all
//                ids), up to kFusedMaxSlots slots
//   copy_bf16    one block per (token, 2 KB column segment; 1 KB when the
//                index launch has read x into the Infinity Cache), one wave
//                per destination row: x[t] shared through L2, one 16-byte
//                non-temporal store per vector per lane per row
//   copy_fp8     one wave per (token, 512 channels); per 128-channel block
//                amax over 16 lanes, scale amax/448, E4M3FN codes, 8-byte
//                code stores + scale stores to each of the token's rows
//   dispatch_small_{bf16,fp8}   for T*k <= kSmallSlots: the copy kernels with
//                the receive order derived inside each block (one launch)
#include "ep_device.h"
#include "ep_launch.h"

namespace ep {
namespace {

constexpr int kHistThreads = 256;    // tile_hist block
constexpr int kHistSlotsPerLane = kMaxTileSlots / kHistThreads;
constexpr int kHistBatch = 64;
// LDS budget of the ranking launch of the two-launch receive order.
constexpr size_t kRankMaxLds = 48 * 1024;
// Fused receive-order kernel: every block histograms all T*k slots itself.
constexpr int kFusedThreads = 1024;
// Loads per thread per sweep step.  8 measured ~1 us faster per ep_dispatch
// than 32 at 4096 x 8 slots, despite more round trips: the smaller unrolled
// batch costs less.  With 16-byte loads (two ids each, when topk_idx is
// 16-byte aligned) the same 8 loads cover 16 slots, and the kernel is 1.6 us
// shorter at 4096 x 8 slots than with 8-byte loads (14.5 vs 16.1 us by
// kernel trace, x prefetch included); 4 or 16 pair loads were slower.
constexpr int kFusedBatch = 8;
// Two-launch receive order: up to this many slots the x prefetch is split
// between the histogram and ranking launches.
constexpr int64_t kSplitPrefetchSlots = int64_t(1) << 17;
typedef long long i64x2 __attribute__((ext_vector_type(2)));

// Per-tile expert histogram: hist[tile][e] = valid slots of the tile's tokens
// routed to e (LDS atomics; integer sums do not depend on order).
// Blocks past the tiles (if any) read part of x through the caches instead
// (see prefetch_vectors).
__global__ __launch_bounds__(kHistThreads) void tile_hist_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int tile_tokens,
    int32_t* __restrict__ hist, int ntiles, const u32x4* __restrict__ pf_src, int64_t pf_vecs,
    uint32_t* __restrict__ pf_sink) {
    if (static_cast<int>(blockIdx.x) >= ntiles) {   // whole block: x prefetch only
        prefetch_vectors<kHistThreads>(pf_src, pf_vecs, static_cast<int>(blockIdx.x) - ntiles,
                                       static_cast<int>(gridDim.x) - ntiles, pf_sink);
        return;
    }
    extern __shared__ int32_t h[];
    for (int e = threadIdx.x; e < E; e += kHistThreads) h[e] = 0;
    __syncthreads();
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tile_tokens;
    const int nt = static_cast<int>(T - t0 < tile_tokens ? T - t0 : tile_tokens);
    const int S = nt * k;                 // <= kMaxTileSlots = kHistSlotsPerLane * kHistThreads
    const int64_t* ids = topk_idx + t0 * k;
    // All of a thread's ids are requested before any is counted (indices
    // clamped to the tile's last slot: no branch around a load, which would
    // make the compiler wait for each in turn).
    int64_t v[kHistSlotsPerLane];
#pragma unroll
    for (int i = 0; i < kHistSlotsPerLane; ++i) {
        const int s = i * kHistThreads + static_cast<int>(threadIdx.x);
        v[i] = ids[s < S ? s : S - 1];
    }
#pragma unroll
    for (int i = 0; i < kHistSlotsPerLane; ++i) {
        const int s = i * kHistThreads + static_cast<int>(threadIdx.x);
        if (s < S && v[i] >= 0 && v[i] < E) atomicAdd(&h[v[i]], 1);
    }
    __syncthreads();
    int32_t* out = hist + static_cast<int64_t>(blockIdx.x) * E;
    for (int e = threadIdx.x; e < E; e += kHistThreads) out[e] = h[e];
}

// In-place exclusive scan of a[0..n) held in LDS by a block of NT threads,
// n <= 8 * NT.  Every thread gets the total.  Caller synchronises before;
// this syncs after.
template <int NT>
__device__ int block_exclusive_scan(int32_t* a, int n, int32_t* wave_tot) {
    const int ipt = (n + NT - 1) / NT;
    const int b = threadIdx.x * ipt;
    int sum = 0;
    for (int i = 0; i < ipt; ++i)
        if (b + i < n) sum += a[b + i];
    int incl = sum;
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    const int wave = threadIdx.x / kWave;
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        base += (w < wave) ? wave_tot[w] : 0;
        total += wave_tot[w];
    }
    int run = base + incl - sum;
    for (int i = 0; i < ipt; ++i)
        if (b + i < n) {
            const int v = a[b + i];
            a[b + i] = run;
            run += v;
        }
    __syncthreads();
    return total;
}

// The tile's slots are ranked by the block's first NR threads (NR / 64
// waves; NR is chosen per launch, see index_rankers): wave w owns slots
// [w*Q, (w+1)*Q) (Q a multiple of 64), lane l of it the slots w*Q + 64*i + l,
// whose raw ids and weights it loads into registers here.
template <int NR>
__device__ __forceinline__ void load_tile_slots(const int64_t* __restrict__ topk_idx,
                                                const float* __restrict__ topk_weights,
                                                bool want_w, int64_t s0, int S, int Q,
                                                int64_t (&raw)[kMaxTileSlots / NR],
                                                float (&wt)[kMaxTileSlots / NR]) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const bool ranker = threadIdx.x < NR;
#pragma unroll
    for (int i = 0; i < kMaxTileSlots / NR; ++i) {
        const int s = wave * Q + i * kWave + lane;
        const bool in = ranker && i * kWave < Q && s < S;
        raw[i] = in ? topk_idx[s0 + s] : -1;
        wt[i] = (in && want_w) ? topk_weights[s0 + s] : 0.0f;
    }
}

// Shared tail of both receive-order paths.  base[e] (LDS) holds the first row
// of expert e for this tile.  Each ranking wave counts its range per expert,
// the waves' cursors are seeded in wave order, then each wave walks its range
// 64 slots at a time, in order: a slot's row = its wave's cursor for the
// expert + the number of lower lanes with the same expert (wave64 ballot
// matching); the highest such lane then advances the cursor (LDS accesses of
// one wave complete in program order).  With cap > 0 (padded layout) base[e]
// holds positions within expert e instead of rows, and a slot's row becomes
// e*cap + position, or -1 from position cap on.  Called by every thread of the
// block.
template <int NR>
__device__ __forceinline__ void rank_tile(const int (&ids)[kMaxTileSlots / NR],
                                          const float (&wt)[kMaxTileSlots / NR], const int32_t* base,
                                          int32_t* wc, int E, int S, int Q, int64_t s0, int64_t t0,
                                          int k, int nbits, int32_t* __restrict__ token_row,
                                          int32_t* __restrict__ recv_src_idx,
                                          float* __restrict__ recv_w, int cap) {
    constexpr int kRankWaves = NR / kWave;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const bool ranker = threadIdx.x < NR;
    for (int i = threadIdx.x; i < kRankWaves * E; i += blockDim.x) wc[i] = 0;
    __syncthreads();
    int32_t* my = wc + (ranker ? wave : 0) * E;
    if (ranker) {
#pragma unroll
        for (int i = 0; i < kMaxTileSlots / NR; ++i)
            if (ids[i] >= 0) atomicAdd(&my[ids[i]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = base[e];
        for (int w = 0; w < kRankWaves; ++w) {
            const int v = wc[w * E + e];
            wc[w * E + e] = run;
            run += v;
        }
    }
    __syncthreads();
    if (!ranker) return;
#pragma unroll
    for (int i = 0; i < kMaxTileSlots / NR; ++i) {
        if (i * kWave >= Q) break;
        const int s = wave * Q + i * kWave + lane;
        const bool in = s < S;
        const int e = ids[i];
        const bool valid = e >= 0;
        const uint64_t peers = match_key(valid ? e : 0, valid, nbits);
        int row = -1;
        if (valid) row = my[e] + __popcll(peers & lanes_below());
        if (valid && (peers >> lane) == 1) my[e] += __popcll(peers);
        if (cap > 0 && row >= 0) row = row < cap ? e * cap + row : -1;   // padded slot
        if (in) {
            const int64_t gs = s0 + s;
            token_row[gs] = row;
            if (row >= 0) {
                recv_src_idx[row] = static_cast<int32_t>(t0) +
                                    static_cast<int32_t>(static_cast<unsigned>(s) / static_cast<unsigned>(k));
                if (recv_w) recv_w[row] = wt[i];
            }
        }
    }
}

__device__ __forceinline__ void write_offsets(const int32_t* eoff, int total, int E, int R,
                                              int32_t* __restrict__ expert_offset,
                                              int32_t* __restrict__ rank_offset) {
    const int epr = E / R;
    for (int e = threadIdx.x; e <= E; e += blockDim.x) expert_offset[e] = e < E ? eoff[e] : total;
    if (rank_offset)
        for (int r = threadIdx.x; r <= R; r += blockDim.x) rank_offset[r] = r < R ? eoff[r * epr] : total;
}

// Two-kernel path, second kernel: one block per tile.  Per expert, the tile
// histograms of all tiles (-> expert offsets) and of the tiles before this
// one (-> this tile's base rows).  Blocks of NR threads, all of them
// ranking.  LDS: base[E], wc[NR/64][E], wave_tot[NR/64].
template <int NR>
__global__ __launch_bounds__(NR) void rows_kernel(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int64_t T,
    int k, int E, int R, int tile_tokens, int ntiles, int nbits, const int32_t* __restrict__ hist,
    int32_t* __restrict__ token_row, int32_t* __restrict__ recv_src_idx,
    float* __restrict__ recv_w, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ rank_offset, int cap, int32_t* __restrict__ recv_count,
    const u32x4* __restrict__ pf_src, int64_t pf_vecs, uint32_t* __restrict__ pf_sink) {
    if (static_cast<int>(blockIdx.x) >= ntiles) {   // whole block: x prefetch only
        prefetch_vectors<NR>(pf_src, pf_vecs, static_cast<int>(blockIdx.x) - ntiles,
                             static_cast<int>(gridDim.x) - ntiles, pf_sink);
        return;
    }
    constexpr int kLane = kMaxTileSlots / NR;      // slots per ranking lane
    extern __shared__ int32_t lds[];
    int32_t* base = lds;
    int32_t* wc = lds + E;
    int32_t* wave_tot = lds + (1 + NR / kWave) * E;
    const int c = blockIdx.x;
    const int64_t t0 = static_cast<int64_t>(c) * tile_tokens;
    const int nt = static_cast<int>(T - t0 < tile_tokens ? T - t0 : tile_tokens);
    const int S = nt * k;
    const int64_t s0 = t0 * k;
    const int Q = (S + NR - 1) / NR * kWave;

    int64_t raw[kLane];
    float wt[kLane];
    load_tile_slots<NR>(topk_idx, topk_weights, recv_w != nullptr, s0, S, Q, raw, wt);
    // The histograms were written by blocks on every XCD, so most come from
    // beyond this XCD's L2: issue them kHistBatch at a time.
    for (int e = threadIdx.x; e < E; e += NR) {
        int tot = 0, pre = 0;
        for (int c0 = 0; c0 < ntiles; c0 += kHistBatch) {
            int v[kHistBatch];
#pragma unroll
            for (int i = 0; i < kHistBatch; ++i)
                v[i] = (c0 + i < ntiles) ? hist[static_cast<int64_t>(c0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kHistBatch; ++i) {
                tot += v[i];
                pre += (c0 + i < c) ? v[i] : 0;
            }
        }
        base[e] = tot;
        wc[e] = pre;
    }
    int ids[kLane];
#pragma unroll
    for (int i = 0; i < kLane; ++i)
        ids[i] = (raw[i] >= 0 && raw[i] < E) ? static_cast<int>(raw[i]) : -1;
    __syncthreads();
    if (cap > 0) {        // padded layout: counts, and positions within each expert
        for (int e = threadIdx.x; e < E; e += NR) {
            if (c == 0) recv_count[e] = min(base[e], cap);
            base[e] = wc[e];
        }
    } else {
        const int total = block_exclusive_scan<NR>(base, E, wave_tot);
        if (c == 0) write_offsets(base, total, E, R, expert_offset, rank_offset);
        for (int e = threadIdx.x; e < E; e += NR) base[e] += wc[e];
    }
    __syncthreads();
    rank_tile<NR>(ids, wt, base, wc, E, S, Q, s0, t0, k, nbits, token_row, recv_src_idx, recv_w, cap);
}

// Fused path (one launch): one block of kFusedThreads per tile.  Every block
// sweeps all T*k slots and builds, in LDS, the per-expert counts of the slots
// before its tile (pre) and of the rest; their sum scanned over experts gives
// the expert offsets and pre gives the tile's base rows.  The sweep is
// redundant across blocks (each reads all ids, mostly from L2), but needs no
// inter-block communication and no second launch.  A dependent global round
// trip costs microseconds here, so the kernel makes exactly one: the tile's
// weights are requested first, the sweep's loads next, and the threads that
// load the tile's own ids keep them in LDS for the ranking.
// The first NR threads rank the tile.
// LDS: pre[E], rest[E], wc[NR/64][E], wave_tot[kFusedThreads/64],
//      tile_ids[tile slots], tile_w[tile slots].
// The launch carries extra blocks past the tiles that read the first
// pf_vecs 16-byte vectors of x once through the caches while the tile blocks
// rank: the index work uses a quarter of the CUs for ~12 us, and the copy
// that follows then finds that part of x in the 256 MB Infinity Cache
// instead of HBM (x is still read from HBM exactly once).
constexpr int kFusedWeights = kMaxTileSlots / kFusedThreads;

// One id of the sweep: counted in LDS among the slots before the tile (pre)
// or the others (rest), and kept in LDS when it belongs to the tile.
__device__ __forceinline__ void sweep_count(int64_t v, unsigned sl, unsigned lo, unsigned hi, int E,
                                            int32_t* pre, int32_t* rest, int32_t* tile_ids) {
    const bool valid = v >= 0 && v < E;
    if (valid) atomicAdd(sl < lo ? &pre[v] : &rest[v], 1);
    if (sl >= lo && sl < hi) tile_ids[sl - lo] = valid ? static_cast<int32_t>(v) : -1;
}

// kPairs: topk_idx is 16-byte aligned and each load brings two consecutive
// ids (slots 2p, 2p+1).  NR <= kFusedThreads: the ranking threads.
template <bool kPairs, int NR>
__global__ __launch_bounds__(kFusedThreads) void rows_fused_kernel(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int64_t T,
    int k, int E, int R, int tile_tokens, int nbits, int32_t* __restrict__ token_row,
    int32_t* __restrict__ recv_src_idx, float* __restrict__ recv_w,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ rank_offset, int ntiles, int cap,
    int32_t* __restrict__ recv_count, const u32x4* __restrict__ pf_src, int64_t pf_vecs,
    uint32_t* __restrict__ pf_sink) {
    if (static_cast<int>(blockIdx.x) >= ntiles) {   // whole block: no tile work, no barrier
        prefetch_vectors<kFusedThreads>(pf_src, pf_vecs, static_cast<int>(blockIdx.x) - ntiles,
                                        static_cast<int>(gridDim.x) - ntiles, pf_sink);
        return;
    }
    extern __shared__ int32_t lds[];
    int32_t* pre = lds;
    int32_t* rest = lds + E;
    int32_t* wc = lds + 2 * E;
    int32_t* wave_tot = lds + (2 + NR / kWave) * E;
    int32_t* tile_ids = wave_tot + kFusedThreads / kWave;
    float* tile_w = reinterpret_cast<float*>(tile_ids + tile_tokens * k);
    const int c = blockIdx.x;
    const int64_t t0 = static_cast<int64_t>(c) * tile_tokens;
    const int nt = static_cast<int>(T - t0 < tile_tokens ? T - t0 : tile_tokens);
    const int S = nt * k;
    const int64_t s0 = t0 * k;
    const int Q = (S + NR - 1) / NR * kWave;
    const bool want_w = recv_w != nullptr;

    // The tile's weights: requested before the sweep so both share one round trip.
    float wpre[kFusedWeights];
#pragma unroll
    for (int i = 0; i < kFusedWeights; ++i) {
        const int sl = i * kFusedThreads + threadIdx.x;
        wpre[i] = (want_w && sl < S) ? topk_weights[s0 + sl] : 0.0f;
    }
    for (int e = threadIdx.x; e < E; e += kFusedThreads) {
        pre[e] = 0;
        rest[e] = 0;
    }
    __syncthreads();
    // T*k <= kFusedMaxSlots here, so 32-bit unsigned slot indices suffice.
    const unsigned total_slots = static_cast<unsigned>(T * k);
    const unsigned lo = static_cast<unsigned>(s0);
    const unsigned hi = lo + static_cast<unsigned>(S);
    // Addresses are a scalar base plus a 32-bit byte offset (one VGPR of
    // address per load).
    const char* ids_base = reinterpret_cast<const char*>(topk_idx);
    const uint64_t uE = static_cast<uint64_t>(E);     // valid: an id below E read as unsigned
    const unsigned wv = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave));
    if (kPairs) {
        for (unsigned b0 = 0; b0 < total_slots; b0 += 2 * kFusedThreads * kFusedBatch) {
            i64x2 v[kFusedBatch];
#pragma unroll
            for (int i = 0; i < kFusedBatch; ++i) {
                const unsigned sl = b0 + 2 * (i * kFusedThreads + threadIdx.x);
                if (sl + 1 < total_slots) {
                    v[i] = *reinterpret_cast<const i64x2*>(ids_base + sl * 8u);
                } else {
                    v[i][0] = sl < total_slots ? *reinterpret_cast<const int64_t*>(ids_base + sl * 8u) : -1;
                    v[i][1] = -1;
                }
            }
#pragma unroll
            for (int i = 0; i < kFusedBatch; ++i) {
                // The wave's 128 slots [ws, ws + 128) lie before the tile,
                // after it, inside it, or (at most twice per sweep) across one
                // of its ends; only the last case is sorted per lane.
                const unsigned ws = b0 + 2u * (i * kFusedThreads + wv * kWave);
                const uint64_t e0 = static_cast<uint64_t>(v[i][0]), e1 = static_cast<uint64_t>(v[i][1]);
                if (ws + 2 * kWave <= lo || ws >= hi) {
                    int32_t* h = ws < lo ? pre : rest;
                    if (e0 < uE) atomicAdd(&h[e0], 1);
                    if (e1 < uE) atomicAdd(&h[e1], 1);
                } else if (ws >= lo && ws + 2 * kWave <= hi) {
                    if (e0 < uE) atomicAdd(&rest[e0], 1);
                    if (e1 < uE) atomicAdd(&rest[e1], 1);
                    const unsigned sl = b0 + 2 * (i * kFusedThreads + threadIdx.x) - lo;
                    tile_ids[sl] = e0 < uE ? static_cast<int32_t>(e0) : -1;
                    tile_ids[sl + 1] = e1 < uE ? static_cast<int32_t>(e1) : -1;
                } else {
                    const unsigned sl = b0 + 2 * (i * kFusedThreads + threadIdx.x);
                    sweep_count(v[i][0], sl, lo, hi, E, pre, rest, tile_ids);
                    sweep_count(v[i][1], sl + 1, lo, hi, E, pre, rest, tile_ids);
                }
            }
        }
    } else {
        for (unsigned b0 = 0; b0 < total_slots; b0 += kFusedThreads * kFusedBatch) {
            int64_t v[kFusedBatch];
#pragma unroll
            for (int i = 0; i < kFusedBatch; ++i) {
                const unsigned sl = b0 + i * kFusedThreads + threadIdx.x;
                v[i] = sl < total_slots ? *reinterpret_cast<const int64_t*>(ids_base + sl * 8u) : -1;
            }
#pragma unroll
            for (int i = 0; i < kFusedBatch; ++i)
                sweep_count(v[i], b0 + i * kFusedThreads + threadIdx.x, lo, hi, E, pre, rest, tile_ids);
        }
    }
#pragma unroll
    for (int i = 0; i < kFusedWeights; ++i) {
        const int sl = i * kFusedThreads + threadIdx.x;
        if (sl < S) tile_w[sl] = wpre[i];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kFusedThreads) rest[e] += pre[e];
    __syncthreads();
    if (cap > 0) {        // padded layout: counts; pre already holds positions
        if (c == 0)
            for (int e = threadIdx.x; e < E; e += kFusedThreads) recv_count[e] = min(rest[e], cap);
    } else {
        const int total = block_exclusive_scan<kFusedThreads>(rest, E, wave_tot);
        if (c == 0) write_offsets(rest, total, E, R, expert_offset, rank_offset);
        for (int e = threadIdx.x; e < E; e += kFusedThreads) pre[e] += rest[e];
    }
    // The ranking waves pick up their slots from LDS.
    int ids[kMaxTileSlots / NR];
    float wt[kMaxTileSlots / NR];
    {
        const int lane = lane_id();
        const int wave = threadIdx.x / kWave;
        const bool ranker = threadIdx.x < NR;
#pragma unroll
        for (int i = 0; i < kMaxTileSlots / NR; ++i) {
            const int s = wave * Q + i * kWave + lane;
            const bool in = ranker && i * kWave < Q && s < S;
            ids[i] = in ? tile_ids[s] : -1;
            wt[i] = in ? tile_w[s] : 0.0f;
        }
    }
    __syncthreads();
    rank_tile<NR>(ids, wt, pre, wc, E, S, Q, s0, t0, k, nbits, token_row, recv_src_idx, recv_w, cap);
}

__global__ void zero_offsets_kernel(int32_t* expert_offset, int E, int32_t* rank_offset, int R) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) expert_offset[i] = 0;
    if (rank_offset)
        for (int i = threadIdx.x; i <= R; i += blockDim.x) rank_offset[i] = 0;
}

// Wave index made explicitly uniform (an SGPR) so per-tile indices stay scalar.
__device__ __forceinline__ int64_t wave_index() {
    return static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) +
           __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

// bf16 copy: one block per (token t, column segment of CV*64 16-byte vectors,
// CV KB), one wave per destination row.  The block has kb = min(k, 8) waves;
// wave w writes rows j = w, w + kb, ... of the token.  Every wave loads the
// same segment of x[t] with plain (cached) loads, so the kb waves of the
// block (same CU, same XCD) share it through L2 and HBM reads it once; each
// lane then issues CV 16-byte non-temporal stores per row.  On MI355X this
// drains a 1:k fan-out faster than one wave storing one load to all k rows
// (measured: ~6% at 4096 x 7168, k = 8); longer runs per wave (4 or 7
// vectors per lane) were markedly slower.  CV = 2 (kCopyVec) reads x from
// HBM best; CV = 1 is faster once the index launch has read x into the
// Infinity Cache (at 4096 x 7168, top-8: 87.6 against 89.7 us, kernel trace,
// three alternating pairs) but much slower from HBM (133 against 96 us), and
// slower for the rank-deduplicated copy either way.
template <int CV>
__global__ __launch_bounds__(512) void copy_bf16_kernel(const u32x4* __restrict__ x,
                                                        const int32_t* __restrict__ token_row,
                                                        u32x4* __restrict__ recv, int64_t num_rows,
                                                        int V, int k, int kb, int segs) {
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t t = blockIdx.x / segs;
    const int seg = static_cast<int>(blockIdx.x - t * segs);
    const int v0 = seg * (CV * kWave) + lane;
    // The wave's first destination row (w < kb <= k) is requested together
    // with x, so the two round trips overlap.
    const int r0 = token_row[t * k + w];
    u32x4 val[CV];
#pragma unroll
    for (int u = 0; u < CV; ++u) {
        const int v = v0 + u * kWave;
        if (v < V) val[u] = x[t * V + v];
    }
    // A segment wholly inside the row is stored without a per-lane guard: a
    // branch around each store made the compiler wait for the previous store
    // to complete before issuing the next.
    const bool full = (seg + 1) * (CV * kWave) <= V;
    auto store_row = [&](int r) {
        if (r < 0 || r >= num_rows) return;
        u32x4* dst = recv + static_cast<int64_t>(r) * V;
        if (full) {
#pragma unroll
            for (int u = 0; u < CV; ++u) __builtin_nontemporal_store(val[u], dst + v0 + u * kWave);
        } else {
#pragma unroll
            for (int u = 0; u < CV; ++u) {
                const int v = v0 + u * kWave;
                if (v < V) __builtin_nontemporal_store(val[u], dst + v);
            }
        }
    };
    store_row(r0);
    for (int j = w + kb; j < k; j += kb) store_row(token_row[t * k + j]);
}

// Quantise the 8 consecutive bf16 channels a lane holds (one 16-byte vector)
// as part of a 128-channel block shared by 16 aligned lanes: block amax by
// four xor-shuffles, scale = amax / 448 (one correctly rounded fp32
// division), codes = E4M3FN(x / scale), or all zero when the scale is 0.
// amax is the largest magnitude that is not NaN: magnitudes are compared as
// integers (the order of non-negative floats, +inf included), with NaN bit
// patterns counted as 0, so the result does not depend on how a float max
// treats quiet or signalling NaNs.
// Every lane of the wave must call it (the shuffles span the wave).
__device__ __forceinline__ u32x2 quantize8(u32x4 a, float& scale) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(a[i]);
        f[2 * i + 1] = bf16_hi(a[i]);
    }
    uint32_t amax = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t m = __float_as_uint(f[i]) & 0x7FFFFFFFu;
        amax = max(amax, m > 0x7F800000u ? 0u : m);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
        amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), o, kWave)));
    const float s = __uint_as_float(amax) / 448.0f;
    u32x2 q = {0u, 0u};
    if (s > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i / 4] |= e4m3fn_encode(f[i] / s) << (8 * (i % 4));
    }
    scale = s;
    return q;
}

// FP8 copy: a lane owns 8 consecutive channels (one 16-byte bf16 vector),
// 16 lanes one 128-channel block, a wave 512 channels of one token; each row
// gets 8 bytes of codes per lane.  Half-width waves (more, smaller ones)
// measured faster than 1024 channels per wave: 53.1 against 55.6 us with x
// cached and 61.9 against 62.8 us from HBM at 4096 x 7168, top-8 (events,
// caches evicted, two rounds); 256 channels per wave (4-byte code stores)
// took 71-74 us.
__global__ __launch_bounds__(256) void copy_fp8_kernel(const u32x4* __restrict__ x,
                                                       const int32_t* __restrict__ token_row,
                                                       uint8_t* __restrict__ recv_q,
                                                       float* __restrict__ recv_scales,
                                                       int64_t num_rows, int H, int k,
                                                       int tiles_per_token, int64_t num_tiles) {
    const int lane = lane_id();
    const int V = H / 8;
    const int nb = H / 128;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
    for (int64_t tile = wave_index(); tile < num_tiles; tile += nwaves) {
        const int64_t t = tile / tiles_per_token;
        const int ch0 = static_cast<int>(tile - t * tiles_per_token) * 512 + lane * 8;
        const bool active = ch0 < H;
        // The token's rows are requested together with x (lane j < k holds
        // row j; the index is clamped, not branched on, so the load does not
        // wait for x).
        int my_row = token_row[t * k + (lane < k ? lane : k - 1)];
        u32x4 a = {0u, 0u, 0u, 0u};
        if (active) a = __builtin_nontemporal_load(x + t * V + ch0 / 8);
        float s;
        const u32x2 q = quantize8(a, s);
        if (lane >= k || my_row >= num_rows) my_row = -1;
        for (int j = 0; j < k; ++j) {
            const int r = read_lane(my_row, j);
            if (r < 0) continue;
            if (active) {
                __builtin_nontemporal_store(
                    q, reinterpret_cast<u32x2*>(recv_q + static_cast<int64_t>(r) * H + ch0));
                if ((lane & 15) == 0) recv_scales[static_cast<int64_t>(r) * nb + ch0 / 128] = s;
            }
        }
    }
}

// ---- small batches: receive order and copy in one launch -------------------
// For T*k <= kSmallSlots every copy block derives the rows of its own token:
// it counts all T*k ids in LDS (those before the token, and all), scans the
// totals over experts, and ranks the token's k slots among themselves.  The
// ids are a few KB and L2-resident after the first blocks, so this costs one
// round trip that overlaps the block's x loads, and no index launch precedes
// the copy.  The token's first block writes its token_row / recv_src_idx /
// recv_topk_weights; block 0 writes the offsets.
// With cap > 0 the same blocks fill the padded expert-major layout instead:
// the slot of (t, j) is e*cap + (its position among expert e's slots), or -1
// from position cap on, and block 0 writes recv_count[e] = min(count, cap).
// LDS: cnt_pre[E], cnt_all[E], wave_tot[16], own[EP_MAX_TOPK], rows[EP_MAX_TOPK].
constexpr int kSmallMaxK = 64;
constexpr int kSmallBatch = 4;     // id loads per thread per step of the small-batch sweep

__device__ int block_exclusive_scan_rt(int32_t* a, int n, int32_t* wave_tot) {
    const int nthreads = blockDim.x;
    const int ipt = (n + nthreads - 1) / nthreads;
    const int b = threadIdx.x * ipt;
    int sum = 0;
    for (int i = 0; i < ipt; ++i)
        if (b + i < n) sum += a[b + i];
    int incl = sum;
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    const int wave = threadIdx.x / kWave;
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < nthreads / kWave; ++w) {
        base += (w < wave) ? wave_tot[w] : 0;
        total += wave_tot[w];
    }
    int run = base + incl - sum;
    for (int i = 0; i < ipt; ++i)
        if (b + i < n) {
            const int v = a[b + i];
            a[b + i] = run;
            run += v;
        }
    __syncthreads();
    return total;
}

// Rows of token t into rows_out[0..k) (LDS, -1 for an empty slot).  Called by
// every thread of the block.
__device__ void small_token_rows(const int64_t* __restrict__ topk_idx,
                                 const float* __restrict__ topk_weights, int64_t T, int k, int E,
                                 int R, int cap, int64_t t, bool write_maps, bool write_offs,
                                 int32_t* __restrict__ token_row,
                                 int32_t* __restrict__ recv_src_idx, float* __restrict__ recv_w,
                                 int32_t* __restrict__ expert_offset,
                                 int32_t* __restrict__ rank_offset,
                                 int32_t* __restrict__ recv_count, int32_t* lds,
                                 int32_t* rows_out) {
    int32_t* cnt_pre = lds;
    int32_t* cnt_all = lds + E;
    int32_t* wave_tot = lds + 2 * E;
    int32_t* own = wave_tot + 16;
    const int j = threadIdx.x;
    // The token's weights (needed only by its first block) and the first
    // batch of ids are requested before anything waits, so they share one
    // round trip with the caller's x loads: kSmallBatch loads per thread,
    // indices clamped to the last slot (no branch around a load, which would
    // make the compiler wait for it).
    const float wj = (write_maps && recv_w && j < k) ? topk_weights[t * k + j] : 0.0f;
    const int total_slots = static_cast<int>(T * k);
    const int first = static_cast<int>(t * k);
    const int step = kSmallBatch * static_cast<int>(blockDim.x);
    int64_t v[kSmallBatch];
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) {
        const int sl = u * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x);
        v[u] = topk_idx[sl < total_slots ? sl : total_slots - 1];
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        cnt_pre[e] = 0;
        cnt_all[e] = 0;
    }
    __syncthreads();
    for (int s0 = 0; s0 < total_slots; s0 += step) {
        if (s0 > 0) {
#pragma unroll
            for (int u = 0; u < kSmallBatch; ++u) {
                const int sl = s0 + u * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x);
                v[u] = topk_idx[sl < total_slots ? sl : total_slots - 1];
            }
        }
#pragma unroll
        for (int u = 0; u < kSmallBatch; ++u) {
            const int sl = s0 + u * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x);
            if (sl >= total_slots) continue;
            const int64_t e = v[u];
            const bool valid = e >= 0 && e < E;
            if (valid) {
                atomicAdd(&cnt_all[e], 1);
                if (sl < first) atomicAdd(&cnt_pre[e], 1);
            }
            if (sl >= first && sl < first + k) own[sl - first] = valid ? static_cast<int32_t>(e) : -1;
        }
    }
    __syncthreads();
    if (cap > 0) {
        if (write_offs)
            for (int e = threadIdx.x; e < E; e += blockDim.x) recv_count[e] = min(cnt_all[e], cap);
    } else {
        const int total = block_exclusive_scan_rt(cnt_all, E, wave_tot);
        if (write_offs) write_offsets(cnt_all, total, E, R, expert_offset, rank_offset);
    }
    if (j < k) {
        const int e = own[j];
        int row = -1;
        if (e >= 0) {
            int before = 0;
            for (int q = 0; q < j; ++q) before += own[q] == e;
            const int pos = cnt_pre[e] + before;
            if (cap <= 0) row = cnt_all[e] + pos;
            else if (pos < cap) row = e * cap + pos;
        }
        rows_out[j] = row;
        if (write_maps) {
            token_row[t * k + j] = row;
            if (row >= 0) {
                recv_src_idx[row] = static_cast<int32_t>(t);
                if (recv_w) recv_w[row] = wj;
            }
        }
    }
    __syncthreads();
}

// bf16, small batches: the copy_bf16 block shape, rows derived in-block.
__global__ __launch_bounds__(512) void dispatch_small_bf16_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, int64_t T, int k, int E, int R, int cap, int V,
    int kb, int segs, u32x4* __restrict__ recv, int32_t* __restrict__ token_row,
    int32_t* __restrict__ recv_src_idx, float* __restrict__ recv_w,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ recv_count) {
    extern __shared__ int32_t lds[];
    int32_t* rows = lds + 2 * E + 16 + kSmallMaxK;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t t = blockIdx.x / segs;
    const int seg = static_cast<int>(blockIdx.x - t * segs);
    const int v0 = seg * (kCopyVec * kWave) + lane;
    // Both x loads issued before either is waited on: the vector index is
    // clamped to the row (lanes past its end store nothing).
    u32x4 val[kCopyVec];
#pragma unroll
    for (int u = 0; u < kCopyVec; ++u) {
        const int v = v0 + u * kWave;
        val[u] = x[t * V + (v < V ? v : V - 1)];
    }
    small_token_rows(topk_idx, topk_weights, T, k, E, R, cap, t, seg == 0, blockIdx.x == 0,
                     token_row, recv_src_idx, recv_w, expert_offset, rank_offset, recv_count, lds,
                     rows);
    // A segment wholly inside the row is stored without a per-lane guard (a
    // branch around each store makes the compiler wait for the one before).
    const bool full = (seg + 1) * (kCopyVec * kWave) <= V;
    for (int j = w; j < k; j += kb) {
        const int r = rows[j];
        if (r < 0) continue;
        u32x4* dst = recv + static_cast<int64_t>(r) * V;
        if (full) {
#pragma unroll
            for (int u = 0; u < kCopyVec; ++u) __builtin_nontemporal_store(val[u], dst + v0 + u * kWave);
        } else {
#pragma unroll
            for (int u = 0; u < kCopyVec; ++u) {
                const int v = v0 + u * kWave;
                if (v < V) __builtin_nontemporal_store(val[u], dst + v);
            }
        }
    }
}

// FP8, small batches: block = 8 waves = (token, 4096-channel segment), each
// wave quantises 512 channels (as copy_fp8) and stores them to every row of
// the token.
__global__ __launch_bounds__(512) void dispatch_small_fp8_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, int64_t T, int k, int E, int R, int cap, int H,
    int segs, uint8_t* __restrict__ recv_q, float* __restrict__ recv_scales,
    int32_t* __restrict__ token_row, int32_t* __restrict__ recv_src_idx,
    float* __restrict__ recv_w, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ rank_offset, int32_t* __restrict__ recv_count) {
    extern __shared__ int32_t lds[];
    int32_t* rows = lds + 2 * E + 16 + kSmallMaxK;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t t = blockIdx.x / segs;
    const int seg = static_cast<int>(blockIdx.x - t * segs);
    const int V = H / 8;
    const int nb = H / 128;
    const int ch0 = seg * 4096 + w * 512 + lane * 8;
    const bool active = ch0 < H;
    u32x4 a = {0u, 0u, 0u, 0u};
    if (active) a = __builtin_nontemporal_load(x + t * V + ch0 / 8);
    small_token_rows(topk_idx, topk_weights, T, k, E, R, cap, t, seg == 0, blockIdx.x == 0,
                     token_row, recv_src_idx, recv_w, expert_offset, rank_offset, recv_count, lds,
                     rows);
    float s;
    const u32x2 q = quantize8(a, s);
    if (!active) return;
    for (int j = 0; j < k; ++j) {
        const int r = rows[j];
        if (r < 0) continue;
        __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(recv_q + static_cast<int64_t>(r) * H + ch0));
        if ((lane & 15) == 0) recv_scales[static_cast<int64_t>(r) * nb + ch0 / 128] = s;
    }
}

}  // namespace

// Ranking threads per tile block of the receive-order kernels.  Each ranking
// wave walks its share of the tile 64 slots at a time, one dependent LDS
// update per step, so more waves per tile finish sooner: at 32768 x top-8 of
// 256 experts (64 tiles of 4096 slots) the ranking launch takes 21.6 us with
// 256 threads, 15.0 with 512 and 13.5 with 1024; the one-launch receive order
// at 4096 x top-8 12.1 us with 256 and 11.2 with 512 or 1024 (kernel trace,
// no x prefetch).  Every ranking wave keeps a counter per expert in LDS, so
// NR is the largest of 1024, 512 and 256 for which those counters and the
// kernel's other fixed_ints words fit the budget.
static int index_rankers(size_t fixed_ints, int E, size_t budget) {
    for (int nr = 1024; nr > 256; nr /= 2)
        if ((fixed_ints + static_cast<size_t>(nr / kWave) * E) * sizeof(int32_t) <= budget) return nr;
    return 256;
}

// Tokens per tile of the receive-order kernels: a multiple of 64, at least 64,
// large enough that there are at most kMaxTiles tiles (each tile sums the
// histograms of the tiles before it), and small enough that a tile's ids fit
// the kMaxTileSlots LDS budget.
static int index_tile_tokens(int64_t T, int k) {
    int64_t tt = ceil_div(T, kMaxTiles);
    tt = ceil_div(tt < 64 ? 64 : tt, 64) * 64;
    int64_t cap = (kMaxTileSlots / k) / 64 * 64;
    if (cap < 64) cap = 64;
    return static_cast<int>(tt < cap ? tt : cap);
}

// Workspace: the per-tile histograms of the two-launch path, then 256 bytes
// where the x-prefetch blocks store their folded words.
static size_t index_hist_bytes(int64_t T, int k, int E) {
    const int64_t ntiles = T > 0 ? ceil_div(T, index_tile_tokens(T, k)) : 0;
    return round_up(static_cast<size_t>(ntiles) * static_cast<size_t>(E) * sizeof(int32_t), 256);
}

size_t index_workspace_bytes(int64_t T, int k, int E) { return index_hist_bytes(T, k, E) + 256; }

hipError_t launch_dispatch_index(const int64_t* topk_idx, const float* topk_weights, int64_t T,
                                 int k, int E, int R, int32_t* recv_src_idx, float* recv_w,
                                 int32_t* expert_offset, int32_t* rank_offset,
                                 int32_t* token_row, void* workspace, const void* x,
                                 int64_t x_bytes, int cap, int32_t* recv_count, hipStream_t stream) {
    if (T == 0) {
        hipLaunchKernelGGL(zero_offsets_kernel, dim3(1), dim3(256), 0, stream, expert_offset, E,
                           rank_offset, R);
        return hipGetLastError();
    }
    const int tt = index_tile_tokens(T, k);
    const int ntiles = static_cast<int>(ceil_div(T, tt));
    const int nbits = E > 1 ? 32 - __builtin_clz(static_cast<unsigned>(E - 1)) : 0;
    const float* w_in = recv_w ? topk_weights : nullptr;
    float* w_out = topk_weights ? recv_w : nullptr;
    const int64_t pf_bytes = x ? (x_bytes < kPrefetchMaxBytes ? x_bytes : kPrefetchMaxBytes) : 0;
    uint32_t* pf_sink = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + index_hist_bytes(T, k, E));
    const size_t fused_fixed = 2 * static_cast<size_t>(E) + kFusedThreads / kWave + 2 * static_cast<size_t>(tt) * k;
    const int fused_nr = index_rankers(fused_fixed, E, kFusedMaxLds);
    const size_t fused_lds = (fused_fixed + static_cast<size_t>(fused_nr / kWave) * E) * sizeof(int32_t);
    if (T * k <= kFusedMaxSlots && fused_lds <= kFusedMaxLds) {
        const size_t lds = fused_lds;
        // Prefetch blocks only while that part of x fits the cache comfortably.
        const int pf_blocks = pf_bytes > 0 ? prefetch_blocks(pf_bytes) : 0;
        const bool pairs = (reinterpret_cast<uintptr_t>(topk_idx) & 15u) == 0;
        auto kern = fused_nr == 1024 ? (pairs ? rows_fused_kernel<true, 1024> : rows_fused_kernel<false, 1024>)
                  : fused_nr == 512  ? (pairs ? rows_fused_kernel<true, 512> : rows_fused_kernel<false, 512>)
                                     : (pairs ? rows_fused_kernel<true, 256> : rows_fused_kernel<false, 256>);
        hipLaunchKernelGGL(kern, dim3(ntiles + pf_blocks), dim3(kFusedThreads), lds, stream,
                           topk_idx, w_in, T, k, E, R, tt, nbits, token_row, recv_src_idx, w_out,
                           expert_offset, rank_offset, ntiles, cap, recv_count,
                           static_cast<const u32x4*>(x), pf_bytes / 16, pf_sink);
        return hipGetLastError();
    }
    int32_t* hist = static_cast<int32_t*>(workspace);
    // The x prefetch: up to kSplitPrefetchSlots slots, half of it rides on the
    // histogram launch and half on the ranking launch (at 8192 x top-6 this
    // made ep_dispatch 94.0 -> 91.8 us); above, the histogram launch has
    // tiles of up to 4096 slots of its own and all of it goes with the
    // ranking launch (at 32768 x top-8 the split measured 3 us slower).
    const int64_t pf_a = T * k <= kSplitPrefetchSlots ? (pf_bytes / 2) / 16 * 16 : 0;
    const int pf_blocks_a = pf_a > 0 ? (1024 / kHistThreads) * prefetch_blocks(pf_a) : 0;
    hipLaunchKernelGGL(tile_hist_kernel, dim3(ntiles + pf_blocks_a), dim3(kHistThreads),
                       static_cast<size_t>(E) * sizeof(int32_t), stream, topk_idx, T, k, E, tt, hist,
                       ntiles, static_cast<const u32x4*>(x), pf_a / 16, pf_sink);
    const int nr = index_rankers(static_cast<size_t>(E) + kFusedThreads / kWave, E, kRankMaxLds);
    const size_t lds = (static_cast<size_t>(1 + nr / kWave) * E + nr / kWave) * sizeof(int32_t);
    // The ranking launch carries the rest of the x prefetch (in blocks of nr threads).
    const int64_t pf_b = pf_bytes - pf_a;
    const int pf_blocks = pf_b > 0 ? (1024 / nr) * prefetch_blocks(pf_b) : 0;
    const u32x4* pf_src_b = pf_b > 0 ? reinterpret_cast<const u32x4*>(static_cast<const char*>(x) + pf_a) : nullptr;
    auto rows = nr == 1024 ? rows_kernel<1024> : nr == 512 ? rows_kernel<512> : rows_kernel<256>;
    hipLaunchKernelGGL(rows, dim3(ntiles + pf_blocks), dim3(nr), lds, stream, topk_idx,
                       w_in, T, k, E, R, tt, ntiles, nbits, hist, token_row, recv_src_idx, w_out,
                       expert_offset, rank_offset, cap, recv_count, pf_src_b, pf_b / 16, pf_sink);
    return hipGetLastError();
}

static size_t small_lds_bytes(int E) {
    return (2 * static_cast<size_t>(E) + 16 + 2 * kSmallMaxK) * sizeof(int32_t);
}

bool dispatch_is_small(int64_t T, int k) { return T > 0 && T * k <= kSmallSlots; }

bool copy_launch_fits(int64_t T, int H, int fanout) {
    const int64_t segs = ceil_div(H / 8, kCopyVec * kWave);
    const int64_t kb = fanout < 8 ? fanout : 8;
    return T * segs * kb * kWave <= kMaxLaunchThreads;
}

hipError_t launch_dispatch_small_bf16(const void* x, const int64_t* topk_idx,
                                      const float* topk_weights, int64_t T, int H, int k, int E,
                                      int R, int cap, void* recv_x, int32_t* recv_src_idx,
                                      float* recv_w, int32_t* expert_offset, int32_t* rank_offset,
                                      int32_t* recv_count, int32_t* token_row,
                                      hipStream_t stream) {
    const int V = H / 8;
    const int segs = static_cast<int>(ceil_div(V, kCopyVec * kWave));
    const int kb = k < 8 ? k : 8;
    hipLaunchKernelGGL(dispatch_small_bf16_kernel, dim3(static_cast<unsigned>(T * segs)),
                       dim3(kb * kWave), small_lds_bytes(E), stream, static_cast<const u32x4*>(x),
                       topk_idx, (recv_w ? topk_weights : nullptr), T, k, E, R, cap, V, kb, segs,
                       static_cast<u32x4*>(recv_x), token_row, recv_src_idx,
                       (topk_weights ? recv_w : nullptr), expert_offset, rank_offset, recv_count);
    return hipGetLastError();
}

hipError_t launch_dispatch_small_fp8(const void* x, const int64_t* topk_idx,
                                     const float* topk_weights, int64_t T, int H, int k, int E,
                                     int R, int cap, uint8_t* recv_q, float* recv_scales,
                                     int32_t* recv_src_idx, float* recv_w,
                                     int32_t* expert_offset, int32_t* rank_offset,
                                     int32_t* recv_count, int32_t* token_row,
                                     hipStream_t stream) {
    const int segs = static_cast<int>(ceil_div(H, 4096));
    hipLaunchKernelGGL(dispatch_small_fp8_kernel, dim3(static_cast<unsigned>(T * segs)), dim3(512),
                       small_lds_bytes(E), stream, static_cast<const u32x4*>(x), topk_idx,
                       (recv_w ? topk_weights : nullptr), T, k, E, R, cap, H, segs, recv_q,
                       recv_scales, token_row, recv_src_idx, (topk_weights ? recv_w : nullptr),
                       expert_offset, rank_offset, recv_count);
    return hipGetLastError();
}

hipError_t launch_dispatch_copy_bf16(const void* x, const int32_t* token_row, void* recv_x,
                                     int64_t num_rows, int64_t T, int H, int k,
                                     hipStream_t stream, bool x_cached, int max_waves) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int kb = k < max_waves ? k : max_waves;
    const int64_t segs1 = ceil_div(V, kWave);
    if (x_cached && T * segs1 * kb * kWave <= kMaxLaunchThreads) {
        hipLaunchKernelGGL(copy_bf16_kernel<1>, dim3(static_cast<unsigned>(T * segs1)), dim3(kb * kWave),
                           0, stream, static_cast<const u32x4*>(x), token_row,
                           static_cast<u32x4*>(recv_x), num_rows, V, k, kb, static_cast<int>(segs1));
        return hipGetLastError();
    }
    const int segs = static_cast<int>(ceil_div(V, kCopyVec * kWave));
    hipLaunchKernelGGL(copy_bf16_kernel<kCopyVec>, dim3(static_cast<unsigned>(T * segs)),
                       dim3(kb * kWave), 0, stream, static_cast<const u32x4*>(x), token_row,
                       static_cast<u32x4*>(recv_x), num_rows, V, k, kb, segs);
    return hipGetLastError();
}

hipError_t launch_dispatch_copy_fp8(const void* x, const int32_t* token_row, uint8_t* recv_q,
                                    float* recv_scales, int64_t num_rows, int64_t T, int H, int k,
                                    hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int tiles_per_token = static_cast<int>(ceil_div(H, 512));
    const int64_t num_tiles = T * tiles_per_token;
    const int64_t blocks = ceil_div(num_tiles, 4);
    const int64_t cap = kMaxLaunchThreads / 256;
    const unsigned grid = static_cast<unsigned>(blocks < cap ? blocks : cap);
    hipLaunchKernelGGL(copy_fp8_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4*>(x), token_row, recv_q, recv_scales, num_rows, H, k,
                       tiles_per_token, num_tiles);
    return hipGetLastError();
}

}  // namespace ep
