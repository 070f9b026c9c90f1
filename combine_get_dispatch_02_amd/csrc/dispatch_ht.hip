// dispatch_ht.hip -- rank-deduplicated ("high-throughput") dispatch on gfx950.
//
// Page "[Not ready] MSCCLPP EP implementation #852", PR body "Scope /
// Intranode": the intranode dispatch sends each token once to every rank that
// hosts one of its experts, and the receiving rank sees the token's top-k ids
// remapped to its local experts.  Here the ranks are contiguous ranges of one
// receive buffer: one row per (token t, rank r) with t routed to r, ordered by
// rank and then token.
//
// Up to 2048 slots (T * k) and 512 tokens: one launch (ht_small, index and
// copy per (token, segment) block, as the packed small-batch dispatch).
// Up to 8192 tokens, 16 ranks, top-16 and 65536 (token, rank) pairs: two
// launches, deterministic, no global atomics:
//   ht_fused      one block of 1024 threads per 64-token tile: every block
//                 sweeps all tokens (one token per thread per step), builds
//                 each token's rank mask from an LDS table of rank bits, and
//                 counts, per rank, the tokens before its tile and in all,
//                 with one ballot per rank per wave (no atomics); a scan over
//                 ranks gives recv_rank_offset and the tile's base rows; one
//                 wave ranks the tile's tokens by ballots; token_rank_row and
//                 each row's source token and remapped ids and weights are
//                 written from LDS, one token per wave.  Extra blocks read x
//                 through the caches meanwhile (see prefetch_vectors).
//   copy          as below.
// Otherwise three launches:
//   ht_tile_hist  one token per thread, 128 tokens per tile: the token's rank
//                 mask (R <= 64) from its k ids; per-tile, per-rank counts
//   ht_rows       per tile: per-rank sums over all tiles and the earlier ones,
//                 a 64-lane scan over ranks (-> recv_rank_offset), the rank of
//                 each token among the tile's tokens routed to the same rank
//                 from one ballot per rank per wave; writes token_rank_row and
//                 each row's source token and remapped top-k ids and weights
//                 (one thread per (token, slot): the k threads of a token
//                 store each row's k entries together); extra blocks read x
//                 through the caches meanwhile, as in ht_fused
//   copy          the bf16 copy kernel of ep_dispatch, driven by the [T, R]
//                 map token_rank_row instead of the [T, k] token_row
#include "../../include/ep.h"
#include "ep_device.h"
#include "ep_ids.h"
#include "ep_launch.h"

namespace ep {
namespace {

constexpr int kHtTile = 128;          // tokens per tile of the multi-launch path
constexpr int kHtWaves = kHtTile / kWave;
constexpr int kHtRowsThreads = 512;   // threads per ht_rows block (kHtWaves of them own the tokens)

// Ranks of valid expert ids: rank_of (ep_ids.h), a multiply-high by
// magic = rank_magic(E / R).
__device__ __forceinline__ uint64_t rank_mask(const int64_t* __restrict__ ids, int k, int E, uint32_t magic) {
    uint64_t m = 0;
    for (int j0 = 0; j0 < k; j0 += kIdBatch) {
        int64_t v[kIdBatch];
        load_ids(ids, j0, k, v);
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u)
            if (v[u] >= 0 && v[u] < E) m |= uint64_t(1) << rank_of(v[u], magic);
    }
    return m;
}

__global__ __launch_bounds__(kHtTile) void ht_tile_hist_kernel(const int64_t* __restrict__ topk_idx,
                                                              int64_t T, int k, int E, int R,
                                                              uint32_t magic,
                                                              int32_t* __restrict__ hist) {
    __shared__ int32_t h[EP_MAX_RANKS];
    if (threadIdx.x < R) h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kHtTile + threadIdx.x;
    if (t < T) {
        for (uint64_t b = rank_mask(topk_idx + t * k, k, E, magic); b; b &= b - 1)
            atomicAdd(&h[__builtin_ctzll(b)], 1);
    }
    __syncthreads();
    if (threadIdx.x < R) hist[static_cast<int64_t>(blockIdx.x) * R + threadIdx.x] = h[threadIdx.x];
}

constexpr int kHtStageRanks = 32;
constexpr int kHtStagePitch = kHtStageRanks + 1;
constexpr int kHtHistLoads = 16;      // tile histogram entries per thread per round trip
constexpr int kHtRecBatch = 8;        // slots whose ids a thread loads per round trip
// Second launch of the multi-launch path: one block of kHtRowsThreads
// threads per tile of kHtTile tokens, thread t < kHtTile owning token t,
// then the x-prefetch blocks (if any).
//   1. Per rank: its tokens in all tiles (-> recv_rank_offset) and in the
//      tiles before this one, summed from the per-tile histograms by
//      kHtRowsThreads / R threads per rank (kHtHistLoads loads each per round
//      trip, requested together with the tile's ids), then over those threads
//      in LDS, then scanned over ranks by one wave.
//   2. The rank of each token among the tile's tokens routed to the same
//      rank: one ballot per rank per token wave.
//   3. Per chunk of up to 32 ranks: the rows go to LDS (pitch 33 words: no
//      bank conflicts), then out to token_rank_row in order (contiguous when
//      R <= 32, 128-byte runs per token otherwise), and each row's records
//      -- source token, the k remapped ids and weights -- are written by one
//      thread per (token, slot): k consecutive threads store a row's k
//      entries together.  The record stores are most of the launch's time,
//      hence the threads beyond the tile's tokens: at 32768 tokens x top-8
//      over 32 ranks the launch takes 16.6 us with 128-token tiles of 512
//      threads, against 24.1 us with 256-token tiles of 256 threads and
//      17.2-20.4 us for 64/128/256-token tiles of 256-1024 threads (kernel
//      trace); without the records it took 13.5 us, and the former separate
//      records launch 9.5 us.
__global__ __launch_bounds__(kHtRowsThreads) void ht_rows_kernel(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int64_t T, int k,
    int E, int R, uint32_t magic, uint32_t kmagic, int ntiles, const int32_t* __restrict__ hist,
    int32_t* __restrict__ token_rank_row, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ recv_src_idx, int64_t* __restrict__ recv_topk_idx,
    float* __restrict__ recv_w, const u32x4* __restrict__ pf_src, int64_t pf_vecs,
    uint32_t* __restrict__ pf_sink) {
    if (static_cast<int>(blockIdx.x) >= ntiles) {   // whole block: x prefetch only
        prefetch_vectors<kHtRowsThreads>(pf_src, pf_vecs, static_cast<int>(blockIdx.x) - ntiles,
                                         static_cast<int>(gridDim.x) - ntiles, pf_sink);
        return;
    }
    __shared__ int32_t wcnt[kHtWaves][EP_MAX_RANKS];       // per-wave counts -> first rows
    __shared__ int32_t part_tot[kHtRowsThreads], part_pre[kHtRowsThreads];
    __shared__ uint64_t tok_mask[kHtTile];
    __shared__ int32_t stage[kHtTile * kHtStagePitch];
    const int c = blockIdx.x;
    const int tid = static_cast<int>(threadIdx.x);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int epr = E / R;
    const int64_t t0 = static_cast<int64_t>(c) * kHtTile;
    const int nt = static_cast<int>(T - t0 < kHtTile ? T - t0 : kHtTile);

    // 1. Histogram sums: thread (g, r) = (tid / R, tid % R) takes tiles g, g + G, ...
    const int G = kHtRowsThreads / R;
    const int hr = tid % R;
    const int hg = tid / R;
    int tot = 0, pre = 0;
    int hv[kHtHistLoads];
    const bool summer = hg < G;
    int c0 = hg;
#pragma unroll
    for (int i = 0; i < kHtHistLoads; ++i) {
        const int cc = c0 + i * G;
        hv[i] = (summer && cc < ntiles) ? hist[static_cast<int64_t>(cc) * R + hr] : 0;
    }
    const int64_t t = t0 + tid;
    const uint64_t m = (tid < kHtTile && t < T) ? rank_mask(topk_idx + t * k, k, E, magic) : 0;
    if (tid < kHtTile) tok_mask[tid] = m;
    for (;;) {
#pragma unroll
        for (int i = 0; i < kHtHistLoads; ++i) {
            const int cc = c0 + i * G;
            tot += hv[i];
            pre += cc < c ? hv[i] : 0;
        }
        c0 += kHtHistLoads * G;
        if (!summer || c0 >= ntiles) break;
#pragma unroll
        for (int i = 0; i < kHtHistLoads; ++i) {
            const int cc = c0 + i * G;
            hv[i] = cc < ntiles ? hist[static_cast<int64_t>(cc) * R + hr] : 0;
        }
    }
    part_tot[tid] = summer ? tot : 0;
    part_pre[tid] = summer ? pre : 0;
    // 2. In-tile ranks: one ballot per rank per token wave.
    if (wave < kHtWaves)
        for (int r = 0; r < R; ++r) {
            const uint64_t b = ballot((m >> r) & 1);
            if (lane == 0) wcnt[wave][r] = __popcll(b);
        }
    __syncthreads();
    if (tid < kWave) {
        const int r = lane;
        int rt = 0, rp = 0;
        if (r < R)
            for (int g = 0; g < G; ++g) {
                rt += part_tot[g * R + r];
                rp += part_pre[g * R + r];
            }
        // exclusive scan of the totals over ranks (one lane per rank)
        int incl = rt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += u;
        }
        const int excl = incl - rt;
        if (r < R) {
            int run = excl + rp;
            for (int w = 0; w < kHtWaves; ++w) {
                const int v = wcnt[w][r];
                wcnt[w][r] = run;
                run += v;
            }
        }
        if (c == 0) {
            if (r < R) rank_offset[r] = excl;
            if (r == R - 1) rank_offset[R] = incl;
        }
    }
    __syncthreads();
    // 3. Rows, up to 32 ranks at a time.  Lanes past the last token have
    // m == 0 and add nothing to a ballot.
    const bool want_w = recv_w != nullptr && topk_weights != nullptr;
    for (int r0 = 0; r0 < R; r0 += kHtStageRanks) {
        const int nr = R - r0 < kHtStageRanks ? R - r0 : kHtStageRanks;
        if (wave < kHtWaves)
            for (int rr = 0; rr < nr; ++rr) {
                const int r = r0 + rr;
                const uint64_t b = ballot((m >> r) & 1);
                int row = -1;
                if ((m >> r) & 1) row = wcnt[wave][r] + __popcll(b & lanes_below());
                stage[tid * kHtStagePitch + rr] = row;
            }
        __syncthreads();
        for (int i = tid; i < nt * nr; i += kHtRowsThreads) {
            const int tl = i / nr;
            const int rr = i - tl * nr;
            token_rank_row[(t0 + tl) * R + r0 + rr] = stage[tl * kHtStagePitch + rr];
        }
        // Records of the chunk's rows: thread i takes slot j of token tl, for
        // every rank of the chunk that the token reaches.
        // The slots' ids and weights are loaded kHtRecBatch at a time (the
        // tile's slots are contiguous; indices clamped, not branched on), so
        // one round trip serves kHtRecBatch slots.
        const uint64_t chunk = (uint64_t(1) << nr) - 1;            // nr <= 32
        const int ns = nt * k;
        const int64_t s0 = t0 * k;
        for (int i0 = tid; i0 < ns; i0 += kHtRowsThreads * kHtRecBatch) {
            int64_t ev[kHtRecBatch];
            float wv[kHtRecBatch];
#pragma unroll
            for (int u = 0; u < kHtRecBatch; ++u) {
                const int i = i0 + u * kHtRowsThreads;
                const int64_t gs = s0 + (i < ns ? i : ns - 1);
                ev[u] = topk_idx[gs];
                wv[u] = want_w ? topk_weights[gs] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kHtRecBatch; ++u) {
                const int i = i0 + u * kHtRowsThreads;
                if (i >= ns) break;
                const uint32_t tl = kmagic ? __umulhi(static_cast<uint32_t>(i), kmagic) : static_cast<uint32_t>(i);
                const int j = i - static_cast<int>(tl) * k;
                const int64_t e = ev[u];
                const int rj = (e >= 0 && e < E) ? rank_of(e, magic) : -1;
                for (uint64_t mm = (tok_mask[tl] >> r0) & chunk; mm; mm &= mm - 1) {
                    const int rr = __builtin_ctzll(mm);
                    const int row = stage[tl * kHtStagePitch + rr];
                    const int r = r0 + rr;
                    const bool local = r == rj;
                    recv_topk_idx[static_cast<int64_t>(row) * k + j] = local ? e - static_cast<int64_t>(r) * epr : -1;
                    if (recv_w) recv_w[static_cast<int64_t>(row) * k + j] = local ? wv[u] : 0.0f;
                    if (j == 0) recv_src_idx[row] = static_cast<int32_t>(t0 + tl);
                }
            }
        }
        __syncthreads();
    }
}

constexpr int kHtFusedThreads = 1024;
constexpr int kHtFusedWaves = kHtFusedThreads / kWave;
constexpr int kHtFusedTile = kWave;                // tokens per tile: one ranking wave
constexpr int kHtFusedMaxR = 16;
constexpr int kHtFusedMaxK = 16;
// The fused sweep costs each block work in proportion to T (and to R), so
// from some size on the two launches beat it, once the second of them also
// carries the x prefetch (index + copy by kernel trace, top-8 of 256 experts,
// ht_fused against ht_tile_hist + ht_rows): 69.4 against 70.4 us at 4096
// tokens over 8 ranks, 139.4 against 139.2 at 8192 (57.8 against 57.9 at
// 8192 x top-6 of 64), 104.4 against 99.3 at 8192 over 16 ranks (hidden
// 4096), 224.9 against 217.4 at 12288 and 336.3 against 319.8 at 16384 over
// 16 ranks (hidden 7168, no prefetch: x too large), 97.7 against 79.6 at
// 16384 over 8 ranks (hidden 2048).
constexpr int64_t kHtFusedMaxTokens = 8192;
constexpr int64_t kHtFusedMaxTokenRanks = 65536;

// KMAX >= k slots per token; NQ tokens per thread per sweep step.  One token
// per step is fastest on MI355X even where it takes four steps (4096
// tokens): 19.9 us against 22.4 us with four tokens (and 10.9 against 17.7
// us at 128 tokens), the larger unrolled id arrays costing more than the
// extra round trips.  kPairs (k even, topk_idx 16-byte aligned): a token's
// ids are read two per 16-byte load; at 4096 tokens x top-8 the kernel then
// takes 17.1 instead of 19.6 us (kernel trace, x prefetch included).
typedef long long i64x2 __attribute__((ext_vector_type(2)));
template <int KMAX, int NQ, bool kPairs>
__global__ __launch_bounds__(kHtFusedThreads) void ht_fused_kernel(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int64_t T,
    int k, int E, int R, uint32_t magic, int ntiles, int32_t* __restrict__ token_rank_row,
    int32_t* __restrict__ recv_src_idx, int64_t* __restrict__ recv_topk_idx,
    float* __restrict__ recv_w, int32_t* __restrict__ rank_offset, const u32x4* __restrict__ pf_src,
    int64_t pf_vecs, uint32_t* __restrict__ pf_sink) {
    if (static_cast<int>(blockIdx.x) >= ntiles) {   // whole block: no tile work, no barrier
        prefetch_vectors<kHtFusedThreads>(pf_src, pf_vecs, static_cast<int>(blockIdx.x) - ntiles,
                                          static_cast<int>(gridDim.x) - ntiles, pf_sink);
        return;
    }
    __shared__ int32_t cnt_all[kHtFusedWaves][kHtFusedMaxR];
    __shared__ int32_t cnt_pre[kHtFusedWaves][kHtFusedMaxR];
    __shared__ int32_t tile_ids[kHtFusedTile * kHtFusedMaxK];   // -1 for an empty slot
    __shared__ float tile_w[kHtFusedTile * kHtFusedMaxK];
    __shared__ int32_t tile_row[kHtFusedTile * kHtFusedMaxR];
    __shared__ uint32_t rank_bit[EP_MAX_EXPERTS + 1];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int epr = E / R;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kHtFusedTile;
    const int nt = static_cast<int>(T - lo < kHtFusedTile ? T - lo : kHtFusedTile);
    const bool want_w = recv_w != nullptr && topk_weights != nullptr;

    // The tile's weights are requested first, so they share the sweep's
    // round trip (a load feeding an LDS store inside the sweep would wait on
    // its own).
    const int wsl = threadIdx.x;                  // kHtFusedTile * KMAX <= kHtFusedThreads
    const float wreg = (want_w && wsl < nt * k) ? topk_weights[lo * k + wsl] : 0.0f;
    // rank_bit[e] = 1 << (rank of expert e); rank_bit[E] = 0 stands for
    // every invalid id (any value outside [0, E), read as unsigned): one LDS
    // read per id builds a token's rank mask.
    for (int e = threadIdx.x; e <= E; e += kHtFusedThreads)
        rank_bit[e] = e < E ? 1u << rank_of(e, magic) : 0u;
    const uint64_t uE = static_cast<uint64_t>(E);
    // Sweep: per rank, the wave's tokens in all tiles and before this one,
    // from one ballot per rank per step into wave-uniform (scalar)
    // accumulators; lane r takes rank r's at the end.
    int acc_all[kHtFusedMaxR], acc_pre[kHtFusedMaxR];
#pragma unroll
    for (int r = 0; r < kHtFusedMaxR; ++r) {
        acc_all[r] = 0;
        acc_pre[r] = 0;
    }
    __syncthreads();
    for (int64_t t0 = 0; t0 < T; t0 += static_cast<int64_t>(NQ) * kHtFusedThreads) {
        int64_t ids[NQ][KMAX];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t t = t0 + q * kHtFusedThreads + threadIdx.x;
            if (kPairs) {
#pragma unroll
                for (int j = 0; j < KMAX; j += 2) {
                    i64x2 pr = {-1, -1};
                    if (t < T && j < k) pr = *reinterpret_cast<const i64x2*>(topk_idx + t * k + j);
                    ids[q][j] = pr[0];
                    ids[q][j + 1] = pr[1];
                }
            } else {
#pragma unroll
                for (int j = 0; j < KMAX; ++j)
                    ids[q][j] = (t < T && j < k) ? topk_idx[t * k + j] : -1;
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            // A wave's 64 tokens start at a multiple of 64, as the tile does,
            // so "in the tile" and "before the tile" hold for the whole wave.
            const int64_t wt0 = t0 + q * kHtFusedThreads + static_cast<int64_t>(wave) * kWave;
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                const uint64_t u = static_cast<uint64_t>(ids[q][j]);   // slots j >= k hold -1
                m |= rank_bit[u < uE ? u : uE];
            }
            if (wt0 == lo && lane < nt) {
#pragma unroll
                for (int j = 0; j < KMAX; ++j) {
                    const uint64_t u = static_cast<uint64_t>(ids[q][j]);
                    if (j < k) tile_ids[lane * k + j] = u < uE ? static_cast<int32_t>(u) : -1;
                }
            }
            const bool wave_before = wt0 < lo;
#pragma unroll
            for (int r = 0; r < kHtFusedMaxR; ++r) {
                if (r < R) {
                    const int c = __popcll(ballot((m >> r) & 1u));
                    acc_all[r] += c;
                    if (wave_before) acc_pre[r] += c;
                }
            }
        }
    }
    int my_all = 0, my_pre = 0;
#pragma unroll
    for (int r = 0; r < kHtFusedMaxR; ++r)
        if (lane == r) {
            my_all = acc_all[r];
            my_pre = acc_pre[r];
        }
    if (lane < R) {
        cnt_all[wave][lane] = my_all;
        cnt_pre[wave][lane] = my_pre;
    }
    if (want_w && wsl < nt * k) tile_w[wsl] = wreg;
    __syncthreads();
    if (wave == 0) {
        // Lane r: rank r's tokens in all tiles and before this one; a scan
        // over the lanes gives the ranks' first rows.
        int tot = 0, pre = 0;
        if (lane < R)
            for (int w = 0; w < kHtFusedWaves; ++w) {
                tot += cnt_all[w][lane];
                pre += cnt_pre[w][lane];
            }
        int incl = tot;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += u;
        }
        const int base = incl - tot + pre;        // this tile's first row in rank `lane`
        if (blockIdx.x == 0) {
            if (lane < R) rank_offset[lane] = incl - tot;
            if (lane == R - 1) rank_offset[R] = incl;
        }
        // Rank the tile's tokens: lane = token.
        uint32_t m = 0;
        if (lane < nt)
            for (int j = 0; j < k; ++j) {
                const int e = tile_ids[lane * k + j];
                if (e >= 0) m |= 1u << rank_of(e, magic);
            }
        for (int r = 0; r < R; ++r) {
            const uint64_t b = ballot((m >> r) & 1u);
            const int row = read_lane(base, r) + __popcll(b & lanes_below());
            if (lane < nt) tile_row[lane * R + r] = ((m >> r) & 1u) ? row : -1;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt * R; i += kHtFusedThreads) token_rank_row[lo * R + i] = tile_row[i];
    // Per-row records: one token per wave, lanes over its (rank, slot) pairs,
    // so a row's k ids and weights are contiguous stores.
    const int per_token = R * k;
    for (int tl = wave; tl < nt; tl += kHtFusedWaves) {
        for (int c = lane; c < per_token; c += kWave) {
            const int r = c / k;
            const int j = c - r * k;
            const int row = tile_row[tl * R + r];
            if (row < 0) continue;
            const int e = tile_ids[tl * k + j];
            const bool local = e >= 0 && rank_of(e, magic) == r;
            recv_topk_idx[static_cast<int64_t>(row) * k + j] = local ? e - r * epr : -1;
            if (recv_w) recv_w[static_cast<int64_t>(row) * k + j] = (local && want_w) ? tile_w[tl * k + j] : 0.0f;
            if (j == 0) recv_src_idx[row] = static_cast<int32_t>(lo + tl);
        }
    }
}

// Small batches (T * k <= kSmallSlots): index and copy in one launch.  One
// block per (token t, 2 KB column segment), as in the packed small-batch
// dispatch.  Every block counts the rank masks of all tokens (one token per
// thread, one ballot per rank per wave) into per-rank totals and the counts
// of the tokens before t; a 64-lane scan over ranks gives recv_rank_offset
// and t's row in each rank it reaches.  Wave w copies x[t]'s segment to the
// rows of ranks w, w + 8, ...; the token's first block writes its
// token_rank_row entries and the records of its rows; block 0 writes the
// offsets.  The x segment and the ids are requested before anything waits.
constexpr int kHtSmallThreads = 512;
constexpr int kHtSmallWaves = kHtSmallThreads / kWave;
__global__ __launch_bounds__(kHtSmallThreads) void ht_small_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_weights, int64_t T, int k, int E, int R, uint32_t magic, int V, int segs,
    u32x4* __restrict__ recv, int32_t* __restrict__ token_rank_row,
    int32_t* __restrict__ recv_src_idx, int64_t* __restrict__ recv_topk_idx,
    float* __restrict__ recv_w, int32_t* __restrict__ rank_offset) {
    __shared__ int32_t cnt_all[kHtSmallWaves][EP_MAX_RANKS];
    __shared__ int32_t cnt_pre[kHtSmallWaves][EP_MAX_RANKS];
    __shared__ int32_t rows[EP_MAX_RANKS];
    __shared__ uint64_t tok_mask;
    const int tid = static_cast<int>(threadIdx.x);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t t = blockIdx.x / segs;
    const int seg = static_cast<int>(blockIdx.x - t * segs);
    const int v0 = seg * (kCopyVec * kWave) + lane;
    const int epr = E / R;
    u32x4 val[kCopyVec];
#pragma unroll
    for (int u = 0; u < kCopyVec; ++u) {
        const int v = v0 + u * kWave;
        val[u] = x[t * V + (v < V ? v : V - 1)];
    }
    // Sweep: thread i takes token i (T <= kHtSmallThreads).
    const uint64_t m = tid < T ? rank_mask(topk_idx + static_cast<int64_t>(tid) * k, k, E, magic) : 0;
    int my_all = 0, my_pre = 0;
    for (int r = 0; r < R; ++r) {
        const bool bit = (m >> r) & 1u;
        const int a = __popcll(ballot(bit));
        const int p = __popcll(ballot(bit && tid < t));
        if (lane == r) {
            my_all = a;
            my_pre = p;
        }
    }
    if (lane < R) {
        cnt_all[wave][lane] = my_all;
        cnt_pre[wave][lane] = my_pre;
    }
    if (tid == t) tok_mask = m;
    __syncthreads();
    if (wave == 0) {
        int tot = 0, pre = 0;
        if (lane < R)
            for (int w = 0; w < kHtSmallWaves; ++w) {
                tot += cnt_all[w][lane];
                pre += cnt_pre[w][lane];
            }
        int incl = tot;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += u;
        }
        const int excl = incl - tot;
        if (blockIdx.x == 0) {
            if (lane < R) rank_offset[lane] = excl;
            if (lane == R - 1) rank_offset[R] = incl;
        }
        if (lane < R) rows[lane] = ((tok_mask >> lane) & 1u) ? excl + pre : -1;
    }
    __syncthreads();
    const bool full = (seg + 1) * (kCopyVec * kWave) <= V;
    for (int r = wave; r < R; r += kHtSmallWaves) {
        const int row = rows[r];
        if (row < 0) continue;
        u32x4* dst = recv + static_cast<int64_t>(row) * V;
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
    if (seg != 0) return;
    if (tid < R) token_rank_row[t * R + tid] = rows[tid];
    const bool want_w = recv_w != nullptr && topk_weights != nullptr;
    for (int c = tid; c < R * k; c += kHtSmallThreads) {
        const int r = c / k;
        const int j = c - r * k;
        const int row = rows[r];
        if (row < 0) continue;
        const int64_t e = topk_idx[t * k + j];
        const bool local = e >= 0 && e < E && rank_of(e, magic) == r;
        recv_topk_idx[static_cast<int64_t>(row) * k + j] = local ? e - static_cast<int64_t>(r) * epr : -1;
        if (recv_w) recv_w[static_cast<int64_t>(row) * k + j] = (local && want_w) ? topk_weights[t * k + j] : 0.0f;
        if (j == 0) recv_src_idx[row] = static_cast<int32_t>(t);
    }
}

// Waves per block of the rank-deduplicated copy.  A token reaches few of R
// ranks, so most of its R slots are empty; beyond 8 ranks, 4 waves that each
// walk R/4 slots beat 8 that each walk R/8: at 32768 tokens over 32 ranks
// the copy takes 686 against 743 us (1 or 2 waves: 786 / 742 us; 16: 1052
// us), while at 8 ranks 4 and 8 waves are within 0.5 us (kernel trace).
inline int ht_copy_waves(int R) { return R > 8 ? 4 : 8; }

__global__ void ht_zero_offsets_kernel(int32_t* rank_offset, int R) {
    if (static_cast<int>(threadIdx.x) <= R) rank_offset[threadIdx.x] = 0;
}

}  // namespace

// The per-tile rank counts of the three-launch path, then 256 bytes where
// the x-prefetch blocks store their folded words (ht_fused uses the first
// 256 bytes for those).
static size_t ht_hist_bytes(int64_t T, int R) {
    const size_t b = static_cast<size_t>(ceil_div(T, kHtTile)) * static_cast<size_t>(R) * sizeof(int32_t);
    return round_up(b > 0 ? b : 1, 256);
}

size_t ht_workspace_bytes(int64_t T, int R) { return ht_hist_bytes(T, R) + 256; }

hipError_t launch_dispatch_ht(const void* x, const int64_t* topk_idx, const float* topk_weights,
                              int64_t T, int H, int k, int E, int R, void* recv_x,
                              int32_t* recv_src_idx, int64_t* recv_topk_idx, float* recv_w,
                              int32_t* rank_offset, int32_t* token_rank_row, void* workspace,
                              hipStream_t stream) {
    if (T == 0) {
        hipLaunchKernelGGL(ht_zero_offsets_kernel, dim3(1), dim3(2 * kWave), 0, stream, rank_offset, R);
        return hipGetLastError();
    }
    const uint32_t magic = rank_magic(E / R);
    const int64_t small_segs = ceil_div(H / 8, kCopyVec * kWave);
    if (T <= kHtSmallThreads && T * k <= kSmallSlots &&
        T * small_segs * kHtSmallThreads <= kMaxLaunchThreads) {
        const int V = H / 8;
        const int segs = static_cast<int>(small_segs);
        hipLaunchKernelGGL(ht_small_kernel, dim3(static_cast<unsigned>(T * segs)), dim3(kHtSmallThreads),
                           0, stream, static_cast<const u32x4*>(x), topk_idx, topk_weights, T, k, E, R, magic,
                           V, segs, static_cast<u32x4*>(recv_x), token_rank_row, recv_src_idx,
                           recv_topk_idx, recv_w, rank_offset);
        return hipGetLastError();
    }
    const int64_t x_bytes = T * static_cast<int64_t>(H) * 2;
    const int64_t pf_bytes = !prefetch_pays(x_bytes, false) ? 0
                             : x_bytes < kPrefetchMaxBytes ? x_bytes : kPrefetchMaxBytes;
    if (T <= kHtFusedMaxTokens && T * R <= kHtFusedMaxTokenRanks && R <= kHtFusedMaxR &&
        k <= kHtFusedMaxK) {
        const int ntiles = static_cast<int>(ceil_div(T, kHtFusedTile));
        const int pf_blocks = pf_bytes > 0 ? prefetch_blocks(pf_bytes) : 0;
        const bool pairs = k % 2 == 0 && (reinterpret_cast<uintptr_t>(topk_idx) & 15u) == 0;
        auto kern = k <= 8 ? (pairs ? ht_fused_kernel<8, 1, true> : ht_fused_kernel<8, 1, false>)
                           : (pairs ? ht_fused_kernel<16, 1, true> : ht_fused_kernel<16, 1, false>);
        hipLaunchKernelGGL(kern, dim3(ntiles + pf_blocks), dim3(kHtFusedThreads), 0, stream, topk_idx,
                           topk_weights, T, k, E, R, magic, ntiles, token_rank_row, recv_src_idx,
                           recv_topk_idx, recv_w, rank_offset, static_cast<const u32x4*>(x),
                           pf_bytes / 16, static_cast<uint32_t*>(workspace));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_dispatch_copy_bf16(x, token_rank_row, recv_x, T * R, T, H, R, stream, false,
                                         ht_copy_waves(R));
    }
    const int ntiles = static_cast<int>(ceil_div(T, kHtTile));
    int32_t* hist = static_cast<int32_t*>(workspace);
    hipLaunchKernelGGL(ht_tile_hist_kernel, dim3(ntiles), dim3(kHtTile), 0, stream, topk_idx, T, k,
                       E, R, magic, hist);
    // The x prefetch rides on the ranking launch, in blocks of kHtRowsThreads.
    const int pf_blocks = pf_bytes > 0 ? (1024 / kHtRowsThreads) * prefetch_blocks(pf_bytes) : 0;
    uint32_t* pf_sink = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + ht_hist_bytes(T, R));
    hipLaunchKernelGGL(ht_rows_kernel, dim3(ntiles + pf_blocks), dim3(kHtRowsThreads), 0, stream, topk_idx,
                       (recv_w ? topk_weights : nullptr), T, k, E, R, magic, rank_magic(k), ntiles,
                       hist, token_rank_row, rank_offset, recv_src_idx, recv_topk_idx, recv_w,
                       static_cast<const u32x4*>(x), pf_bytes / 16, pf_sink);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dispatch_copy_bf16(x, token_rank_row, recv_x, T * R, T, H, R, stream, false,
                                     ht_copy_waves(R));
}

}  // namespace ep
