// ep_launch.h -- internal kernel launchers of libep.so (host side).
//
// The C ABI in include/ep.h validates arguments and then calls these; each
// launcher only sizes its grid and enqueues on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Tokens per block of the layout histogram kernel (one token per thread).
constexpr int kLayoutTokensPerBlock = 256;
// Receive-order computation: tokens are cut into tiles (at most kMaxTiles of
// them while a tile's slots fit kMaxTileSlots); rows are ranked inside a tile
// with wave ballots, and tiles are chained by per-expert prefix sums.
constexpr int kMaxTiles = 64;
constexpr int kMaxTileSlots = 4096;
// Up to this many slots (T*k) one fused launch computes the receive order;
// beyond it, a histogram launch feeds the ranking launch.  Every fused block
// sweeps all T*k ids, so its cost grows with the batch: measured on MI355X
// (kernel trace, top-8 of 256 experts, no x prefetch, as at hidden 7168 from
// 6144 tokens on), the fused launch takes 13.8 / 15.9 / 20.6 us at
// 49152 / 65536 / 98304 slots against 4.8 + 9.4 / 4.8 + 9.4 / 4.8 + 10.5 us
// for the two launches (12.9 against 4.8 + 8.5 us at 8192 x top-6 of 64).
constexpr int64_t kFusedMaxSlots = int64_t(3) << 14;
constexpr size_t kFusedMaxLds = 64 * 1024;
// Up to this many slots (T*k) each copy block derives its own token's rows and
// ep_dispatch / ep_dispatch_fp8 are a single launch.
constexpr int64_t kSmallSlots = 2048;
// Index launches that run for ~10 us on part of the chip carry this many
// extra blocks reading up to kPrefetchMaxBytes of x through the caches (well
// inside the 256 MB Infinity Cache), for the copy that follows.
constexpr int kPrefetchBlocks = 192;
constexpr int64_t kPrefetchMaxBytes = int64_t(64) << 20;
// The prefetch pays only while it covers most of x, and less so the more the
// copy writes per byte of x it reads (index + copy, kernel trace, caches
// evicted first, top-8 of 256 experts unless noted).  bf16 copy: -4 us with
// 58.7 MB of x, -8 us with 67 MB (top-6 of 64), but +3.7 / +8 / +14 us with
// 117 / 176 / 470 MB; FP8 copy: -4.7 us at 58.7 MB, -2 us at 117 MB, none
// at 470 MB; the rank-deduplicated copy (5.3 rows per token): -13 us at
// 117 MB, none at 235 MB.  So up to kPrefetchMaxXBf16 bytes of x for the
// bf16 copy and kPrefetchMaxXOther for the FP8 and rank-deduplicated ones.
constexpr int64_t kPrefetchMaxXBf16 = int64_t(80) << 20;
constexpr int64_t kPrefetchMaxXOther = int64_t(128) << 20;
inline bool prefetch_pays(int64_t x_bytes, bool bf16_fanout) {
    return x_bytes <= (bf16_fanout ? kPrefetchMaxXBf16 : kPrefetchMaxXOther);
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }
// Prefetch blocks of 1024 threads (8 vectors each per step) for x_bytes of x.
inline int prefetch_blocks(int64_t x_bytes) {
    const int64_t bytes = x_bytes < kPrefetchMaxBytes ? x_bytes : kPrefetchMaxBytes;
    const int64_t b = ceil_div(bytes / 16, 1024 * 8);
    return static_cast<int>(b < kPrefetchBlocks ? b : kPrefetchBlocks);
}

// ---- layout -----------------------------------------------------------------
size_t layout_workspace_bytes(int64_t T, int E, int R, int G);
hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R, int P,
                         int32_t* per_rank, int32_t* per_group, int32_t* per_expert,
                         uint8_t* in_rank, void* workspace, hipStream_t stream);

// ---- receive order (shared by both dispatch variants) -------------------------
size_t index_workspace_bytes(int64_t T, int k, int E);
// x / x_bytes (may be NULL / 0): the dispatched tokens, of which the ranking
// launch reads up to 64 MB through the caches while it ranks (its folded
// words go to the workspace's last 256 bytes), so the copy that follows finds
// them cached.
// cap == 0: packed receive order (expert_offset / rank_offset written);
// cap > 0: padded [E, cap] slots (token_row holds slots, recv_count written,
// recv_src_idx / recv_w indexed by slot).
hipError_t launch_dispatch_index(const int64_t* topk_idx, const float* topk_weights, int64_t T,
                                 int k, int E, int R, int32_t* recv_src_idx, float* recv_w,
                                 int32_t* expert_offset, int32_t* rank_offset,
                                 int32_t* token_row, void* workspace, const void* x,
                                 int64_t x_bytes, int cap, int32_t* recv_count, hipStream_t stream);

// ---- small batches: receive order + copy in one launch -------------------------
bool dispatch_is_small(int64_t T, int k);

// A dispatch packet carries the grid's work-item count per dimension in 32
// bits, so one launch holds at most this many threads in x.  Grid-stride
// kernels cap their grid below it; the one-block-per-(token, segment) bf16
// copies cannot, and their callers reject shapes beyond it.
constexpr int64_t kMaxLaunchThreads = 0xFFFFFFFFll;
// 16-byte vectors per lane per destination row in the bf16 copies (2 KB of a
// row per wave) when x comes from HBM; copy_launch_fits checks that shape
// (the 1 KB form used once x is cached falls back to it when its twice as
// many blocks would not fit one launch).
constexpr int kCopyVec = 2;
bool copy_launch_fits(int64_t T, int H, int fanout);
// cap == 0: packed receive order (expert_offset / rank_offset written);
// cap > 0: padded [E, cap] slots (recv_count written, token_row = slots).
hipError_t launch_dispatch_small_bf16(const void* x, const int64_t* topk_idx,
                                      const float* topk_weights, int64_t T, int H, int k, int E,
                                      int R, int cap, void* recv_x, int32_t* recv_src_idx,
                                      float* recv_w, int32_t* expert_offset, int32_t* rank_offset,
                                      int32_t* recv_count, int32_t* token_row,
                                      hipStream_t stream);
hipError_t launch_dispatch_small_fp8(const void* x, const int64_t* topk_idx,
                                     const float* topk_weights, int64_t T, int H, int k, int E,
                                     int R, int cap, uint8_t* recv_q, float* recv_scales,
                                     int32_t* recv_src_idx, float* recv_w,
                                     int32_t* expert_offset, int32_t* rank_offset,
                                     int32_t* recv_count, int32_t* token_row,
                                     hipStream_t stream);

// ---- rank-deduplicated (high-throughput) dispatch -------------------------------
size_t ht_workspace_bytes(int64_t T, int R);
hipError_t launch_dispatch_ht(const void* x, const int64_t* topk_idx, const float* topk_weights,
                              int64_t T, int H, int k, int E, int R, void* recv_x,
                              int32_t* recv_src_idx, int64_t* recv_topk_idx, float* recv_w,
                              int32_t* rank_offset, int32_t* token_rank_row, void* workspace,
                              hipStream_t stream);

// ---- padded expert-major (low-latency) dispatch ----------------------------------
size_t ll_workspace_bytes(int64_t T, int k, int E);
// recv_q_or_x: bf16 rows [E*cap, H] when recv_scales is NULL, else FP8 codes
// [E*cap, H] with scales [E*cap, H/128].
hipError_t launch_dispatch_ll(const void* x, const int64_t* topk_idx, const float* topk_weights,
                              int64_t T, int H, int k, int E, int cap, void* recv_q_or_x,
                              float* recv_scales, int32_t* recv_count, int32_t* recv_src_idx,
                              float* recv_w, int32_t* token_slot, void* workspace,
                              hipStream_t stream);

// ---- data movement ------------------------------------------------------------
// Copy kernels: every slot whose row lies in [0, num_rows) receives x[t]
// (bf16) or its FP8 cast; other slots are skipped.  x_cached: x was just read
// through the caches by the index launch (its prefetch), which the bf16 copy
// then reads in 1 KB instead of 2 KB segments.  max_waves (<= 8): waves per
// bf16 copy block, each taking every max_waves-th of a token's k slots.
hipError_t launch_dispatch_copy_bf16(const void* x, const int32_t* token_row, void* recv_x,
                                     int64_t num_rows, int64_t T, int H, int k,
                                     hipStream_t stream, bool x_cached = false, int max_waves = 8);
hipError_t launch_dispatch_copy_fp8(const void* x, const int32_t* token_row, uint8_t* recv_q,
                                    float* recv_scales, int64_t num_rows, int64_t T, int H, int k,
                                    hipStream_t stream);
hipError_t launch_combine(const void* expert_out, int64_t num_rows, const int32_t* token_row,
                          const float* topk_weights, int64_t T, int H, int k, void* out,
                          hipStream_t stream);

}  // namespace ep
