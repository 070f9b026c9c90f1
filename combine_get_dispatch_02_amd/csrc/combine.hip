// combine.hip -- ep_combine on gfx950.
//
// Page "[Not ready] MSCCLPP EP implementation #852": intranode combine (PR
// body, "Scope / Intranode") brings every expert output back to its source
// token and sums them weighted by topk_weights; the commit fixing internode
// HT combine states that combine must follow the receiver-side layout that
// dispatch produced -- here token_row[t, j].
//
// One wave per (token, 1 KB column tile: one 16-byte vector per lane).  The
// wave reads the token's k rows, KB at a time, accumulates
// acc = fma(w[t,j], y[row(t,j)], acc) in fp32 for j = 0..k-1 in that fixed
// order (v_fma_f32, one rounding per step), and stores bf16 rounded to
// nearest even.  The result is therefore independent of the launch shape.
// Without weights every weight is 1: the high-throughput combine of a token's
// per-rank rows.  That case has its own instantiation, which loads no weights
// and adds (acc + y rounds exactly as fma(1, y, acc) does).
//
// Large batches (at least 6144 tiles) read one row at a time per wave
// (KB = 1), small ones all rows at once (KB = 8).  Bound by the DRAM side of the scattered row reads,
// large batches gain from many small waves each with one row in flight: at
// 4096 tokens x 7168, top-8 of 256 experts the kernel takes 89.3 us with 1 KB
// tiles and one row per wave, against 90.4 us with 2 KB tiles and one row
// (the earlier form), 91.2-91.8 us with 2, 4 or 8 rows of 1 KB in flight
// and 111.6 us with 7 KB tiles; at 32768 tokens 720 against 746 us (kernel
// trace, caches evicted).
#include "ep_device.h"
#include "ep_launch.h"

namespace ep {
namespace {

__device__ __forceinline__ int64_t wave_index() {
    return static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) +
           __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

template <int KB, bool kWeighted>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y,
                                                      int64_t num_rows,
                                                      const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_weights,
                                                      u32x4* __restrict__ out, int V, int k,
                                                      int tiles_per_token, int64_t num_tiles) {
    const int lane = lane_id();
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
    for (int64_t tile = wave_index(); tile < num_tiles; tile += nwaves) {
        const int64_t t = tile / tiles_per_token;
        const int v0 = static_cast<int>(tile - t * tiles_per_token) * kWave + lane;
        // Lanes past the row's end read its last vector and store nothing.
        const int vc = v0 < V ? v0 : V - 1;
        int my_row = -1;
        float my_w = 0.0f;
        if (lane < k) {
            my_row = token_row[t * k + lane];
            if (kWeighted) my_w = topk_weights[t * k + lane];
            if (my_row < 0 || static_cast<int64_t>(my_row) >= num_rows) my_row = -1;
        }
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

        for (int j0 = 0; j0 < k; j0 += KB) {
            u32x4 val[KB];
            int rows[KB];
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
                const int j = j0 + jj;
                rows[jj] = j < k ? read_lane(my_row, j) : -1;
                // One row at a time: an empty slot (a wave-uniform test) is
                // skipped, no load.  Several rows: every row's load is issued
                // unconditionally, so all KB rows are in flight before any is
                // waited on (a branch or select around each row's load makes
                // the compiler wait for it before the next); an empty slot
                // reads row 0 of y -- or, when y has no rows, the wave's own
                // output segment, which only this wave writes, after its
                // loads -- and never accumulates it.
                if (KB == 1 && rows[jj] < 0) continue;
                const u32x4* src = num_rows > 0 ? y + static_cast<int64_t>(rows[jj] >= 0 ? rows[jj] : 0) * V
                                                : out + t * V;
                val[jj] = __builtin_nontemporal_load(src + vc);
            }
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
                if (rows[jj] < 0) continue;
                if (kWeighted) {
                    const float wj = read_lane(my_w, j0 + jj);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = __builtin_fmaf(wj, bf16_lo(val[jj][i]), acc[2 * i]);
                        acc[2 * i + 1] = __builtin_fmaf(wj, bf16_hi(val[jj][i]), acc[2 * i + 1]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] += bf16_lo(val[jj][i]);
                        acc[2 * i + 1] += bf16_hi(val[jj][i]);
                    }
                }
            }
        }
        if (v0 < V) {
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = bf16_rne(acc[2 * i]) | (bf16_rne(acc[2 * i + 1]) << 16);
            __builtin_nontemporal_store(o, out + t * V + v0);
        }
    }
}

template <int KB, bool kWeighted>
hipError_t launch_kb(const void* y, int64_t num_rows, const int32_t* token_row, const float* w,
                     void* out, int64_t T, int V, int k, hipStream_t stream) {
    const int tiles_per_token = static_cast<int>(ceil_div(V, kWave));
    const int64_t num_tiles = T * tiles_per_token;
    const int64_t blocks = ceil_div(num_tiles, 4);
    const int64_t cap = kMaxLaunchThreads / 256;
    const unsigned grid = static_cast<unsigned>(blocks < cap ? blocks : cap);
    hipLaunchKernelGGL((combine_kernel<KB, kWeighted>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4*>(y), num_rows, token_row, w,
                       static_cast<u32x4*>(out), V, k, tiles_per_token, num_tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* expert_out, int64_t num_rows, const int32_t* token_row,
                          const float* topk_weights, int64_t T, int H, int k, void* out,
                          hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    // Large: at least 6144 1 KB tiles (4096 x 7168 has 57344).  At H = 7168,
    // top-8 the one-row form is 1.4 us slower at 256 tokens (3584 tiles) and
    // 0.5 us faster at 512 (7168 tiles) than the all-rows one.
    const bool large = T * ceil_div(V, kWave) >= 6144;
    if (topk_weights)
        return large ? launch_kb<1, true>(expert_out, num_rows, token_row, topk_weights, out, T, V, k, stream)
                     : launch_kb<8, true>(expert_out, num_rows, token_row, topk_weights, out, T, V, k, stream);
    return large ? launch_kb<1, false>(expert_out, num_rows, token_row, nullptr, out, T, V, k, stream)
                 : launch_kb<8, false>(expert_out, num_rows, token_row, nullptr, out, T, V, k, stream);
}

}  // namespace ep
