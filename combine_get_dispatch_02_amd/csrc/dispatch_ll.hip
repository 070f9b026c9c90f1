// dispatch_ll.hip -- padded expert-major ("low-latency") dispatch on gfx950.
//
// Page "[Not ready] MSCCLPP EP implementation #852": the LL benchmark's
// receive buffer is one fixed-size region per expert (the commit that stops
// cloning it inside the timed loop), and the low-latency runtime is tested at
// capacities 1 and 2.  With one source the buffer is [E, cap, H]: expert e
// owns slots e*cap .. e*cap + cap - 1, filled in (token, slot) order, and a
// slot that finds its region full is dropped (token_slot = -1).  This is the
// shape a grouped expert GEMM consumes directly (one [cap, H] operand per
// expert, recv_count[e] valid rows).
//
// T*k <= 2048: one launch -- the small-batch dispatch kernels rank each
// token's slots in-block and write the padded slots directly.
// Larger batches: the receive-order kernels of ep_dispatch in their padded
// mode (a slot's position within its expert, without the expert offset,
// becomes e*cap + position, or -1 from cap on; block 0 writes the counts),
// then the copy kernels of ep_dispatch fill the slots, skipping dropped ones.
#include "ep_device.h"
#include "ep_launch.h"

namespace ep {
namespace {

__global__ void ll_zero_counts_kernel(int32_t* __restrict__ recv_count, int E) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) recv_count[e] = 0;
}

}  // namespace

size_t ll_workspace_bytes(int64_t T, int k, int E) { return index_workspace_bytes(T, k, E); }

hipError_t launch_dispatch_ll(const void* x, const int64_t* topk_idx, const float* topk_weights,
                              int64_t T, int H, int k, int E, int cap, void* recv_q_or_x,
                              float* recv_scales, int32_t* recv_count, int32_t* recv_src_idx,
                              float* recv_w, int32_t* token_slot, void* workspace,
                              hipStream_t stream) {
    if (T == 0) {
        hipLaunchKernelGGL(ll_zero_counts_kernel, dim3(1), dim3(256), 0, stream, recv_count, E);
        return hipGetLastError();
    }
    const bool fp8 = recv_scales != nullptr;
    if (dispatch_is_small(T, k)) {
        if (fp8)
            return launch_dispatch_small_fp8(x, topk_idx, topk_weights, T, H, k, E, 1, cap,
                                             static_cast<uint8_t*>(recv_q_or_x), recv_scales,
                                             recv_src_idx, recv_w, nullptr, nullptr, recv_count,
                                             token_slot, stream);
        return launch_dispatch_small_bf16(x, topk_idx, topk_weights, T, H, k, E, 1, cap, recv_q_or_x,
                                          recv_src_idx, recv_w, nullptr, nullptr, recv_count,
                                          token_slot, stream);
    }
    const int64_t x_bytes = T * static_cast<int64_t>(H) * 2;
    const hipError_t e = launch_dispatch_index(topk_idx, topk_weights, T, k, E, 1, recv_src_idx,
                                               recv_w, nullptr, nullptr, token_slot, workspace,
                                               prefetch_pays(x_bytes, !fp8) ? x : nullptr, x_bytes,
                                               cap, recv_count, stream);
    if (e != hipSuccess) return e;
    const int64_t rows = static_cast<int64_t>(E) * cap;
    if (fp8)
        return launch_dispatch_copy_fp8(x, token_slot, static_cast<uint8_t*>(recv_q_or_x), recv_scales,
                                        rows, T, H, k, stream);
    return launch_dispatch_copy_bf16(x, token_slot, recv_q_or_x, rows, T, H, k, stream,
                                     prefetch_pays(x_bytes, true));
}

}  // namespace ep
