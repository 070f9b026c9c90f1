// layout.hip -- get_dispatch_layout on gfx950.
//
// Routing histogram of page "[Not ready] MSCCLPP EP implementation #852",
// PR body "Scope / Intranode" (get_dispatch_layout) and "Scope / Internode
// HT" (the per-RDMA-rank count, here a group of P consecutive ranks).
//
// Two launches, no atomics on global memory and no zero-fill (one when the
// batch fits a single block of 256 tokens):
//   1. layout_partial: one token per thread, 256 tokens per block.  Each block
//      builds its expert / rank / group histograms in LDS (experts by LDS
//      atomics; ranks and groups by one wave64 ballot per rank or group, whose
//      popcount lane r of the wave accumulates, then one LDS add per lane),
//      writes the is_token_in_rank rows of its tokens, and stores its
//      histograms in the workspace.
//   2. layout_reduce: one thread per output counter sums the per-block
//      histograms (integer sums: the result does not depend on order).
#include "ep_device.h"
#include "ep_ids.h"
#include "ep_launch.h"

namespace ep {
namespace {

// kFinal: the whole batch is this one block (T <= kLayoutTokensPerBlock), so
// its histograms are the final counts and no reduce launch follows.
template <bool kFinal>
__global__ __launch_bounds__(kLayoutTokensPerBlock) void layout_partial_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, int P, uint32_t magic,
    uint8_t* __restrict__ in_rank, int32_t* __restrict__ partial,
    int32_t* __restrict__ per_expert, int32_t* __restrict__ per_rank,
    int32_t* __restrict__ per_group) {
    extern __shared__ int32_t lds[];
    const int G = R / P;
    const int nh = E + R + G;
    int32_t* h_e = lds;
    int32_t* h_r = lds + E;
    int32_t* h_g = h_r + R;
    uint64_t* masks = reinterpret_cast<uint64_t*>(lds + ((nh + 1) & ~1));

    for (int i = threadIdx.x; i < nh; i += blockDim.x) lds[i] = 0;
    __syncthreads();

    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kLayoutTokensPerBlock;
    const int64_t t = t0 + threadIdx.x;
    uint64_t m = 0;  // ranks this token reaches (R <= 64)
    if (t < T) {
        const int64_t* row = topk_idx + t * k;
        for (int j0 = 0; j0 < k; j0 += kIdBatch) {
            int64_t v[kIdBatch];
            load_ids(row, j0, k, v);
#pragma unroll
            for (int u = 0; u < kIdBatch; ++u) {
                const int64_t e = v[u];
                if (e >= 0 && e < E) {
                    atomicAdd(&h_e[e], 1);
                    m |= uint64_t(1) << rank_of(e, magic);   // magic = rank_magic(E / R)
                }
            }
        }
    }
    masks[threadIdx.x] = m;
    uint64_t gm = 0;
    for (uint64_t b = m; b; b &= b - 1) gm |= uint64_t(1) << (__builtin_ctzll(b) / P);
    // Tokens of this wave reaching rank r (group g): popcount of one ballot,
    // kept by lane r (g).  R, G <= 64.
    const int lane = lane_id();
    int my_r = 0, my_g = 0;
    for (int r = 0; r < R; ++r) {
        const int c = __popcll(ballot((m >> r) & 1u));
        if (lane == r) my_r = c;
    }
    for (int g = 0; g < G; ++g) {
        const int c = __popcll(ballot((gm >> g) & 1u));
        if (lane == g) my_g = c;
    }
    if (lane < R && my_r) atomicAdd(&h_r[lane], my_r);
    if (lane < G && my_g) atomicAdd(&h_g[lane], my_g);
    __syncthreads();

    // is_token_in_rank rows of this block are nt * R consecutive bytes.
    const int nt = static_cast<int>(T - t0 < kLayoutTokensPerBlock ? T - t0 : kLayoutTokensPerBlock);
    uint8_t* out = in_rank + t0 * R;
    for (int i = threadIdx.x; i < nt * R; i += blockDim.x) {
        const int tl = i / R;
        const int r = i - tl * R;
        out[i] = static_cast<uint8_t>((masks[tl] >> r) & 1);
    }
    if (kFinal) {
        for (int i = threadIdx.x; i < nh; i += blockDim.x) {
            if (i < E)
                per_expert[i] = lds[i];
            else if (i < E + R)
                per_rank[i - E] = lds[i];
            else if (per_group)
                per_group[i - E - R] = lds[i];
        }
        return;
    }
    int32_t* p = partial + static_cast<int64_t>(blockIdx.x) * nh;
    for (int i = threadIdx.x; i < nh; i += blockDim.x) p[i] = lds[i];
}

__global__ __launch_bounds__(256) void layout_reduce_kernel(const int32_t* __restrict__ partial,
                                                            int nblk, int E, int R, int G,
                                                            int32_t* __restrict__ per_expert,
                                                            int32_t* __restrict__ per_rank,
                                                            int32_t* __restrict__ per_group) {
    const int nh = E + R + G;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nh) return;
    int32_t s = 0;
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) s += partial[static_cast<int64_t>(b) * nh + i];
    if (i < E)
        per_expert[i] = s;
    else if (i < E + R)
        per_rank[i - E] = s;
    else if (per_group)
        per_group[i - E - R] = s;
}

}  // namespace

size_t layout_workspace_bytes(int64_t T, int E, int R, int G) {
    const int64_t nblk = ceil_div(T, kLayoutTokensPerBlock);
    return round_up(static_cast<size_t>(nblk) * static_cast<size_t>(E + R + G) * sizeof(int32_t), 256);
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R, int P,
                         int32_t* per_rank, int32_t* per_group, int32_t* per_expert,
                         uint8_t* in_rank, void* workspace, hipStream_t stream) {
    const int G = R / P;
    const int nh = E + R + G;
    const int64_t nblk = ceil_div(T, kLayoutTokensPerBlock);
    int32_t* partial = static_cast<int32_t*>(workspace);
    const size_t lds = (static_cast<size_t>((nh + 1) & ~1)) * sizeof(int32_t) +
                       kLayoutTokensPerBlock * sizeof(uint64_t);
    if (nblk == 1) {
        hipLaunchKernelGGL(layout_partial_kernel<true>, dim3(1), dim3(kLayoutTokensPerBlock), lds,
                           stream, topk_idx, T, k, E, R, P, rank_magic(E / R), in_rank, partial,
                           per_expert, per_rank, per_group);
        return hipGetLastError();
    }
    if (nblk > 0) {
        hipLaunchKernelGGL(layout_partial_kernel<false>, dim3(static_cast<unsigned>(nblk)),
                           dim3(kLayoutTokensPerBlock), lds, stream, topk_idx, T, k, E, R, P,
                           rank_magic(E / R), in_rank, partial, per_expert, per_rank, per_group);
    }
    hipLaunchKernelGGL(layout_reduce_kernel, dim3(static_cast<unsigned>(ceil_div(nh, 256))),
                       dim3(256), 0, stream, partial, static_cast<int>(nblk), E, R, G, per_expert,
                       per_rank, per_group);
    return hipGetLastError();
}

}  // namespace ep
