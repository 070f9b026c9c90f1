// ep_api.hip -- the C ABI of include/ep.h: argument validation, workspace
// sizing, status codes, and the launch sequence of every entry point.
//
// Validation happens on the host before anything is enqueued, so an invalid
// call leaves every output untouched and can never make a kernel index out
// of the buffers described in ep.h.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/ep.h"
#include "ep_launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return EP_OK;
    return fail(EP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Routing arguments shared by every entry point that reads topk_idx.
int check_routing(const char* fn, const int64_t* topk_idx, int64_t T, int k, int E, int R) {
    if (T < 0) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_tokens < 0", fn);
    if (k < 1) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_topk < 1", fn);
    if (k > EP_MAX_TOPK) return fail(EP_ERR_UNSUPPORTED, "%s: num_topk > %d", fn, EP_MAX_TOPK);
    if (E < 1 || R < 1) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_experts and num_ranks must be >= 1", fn);
    if (R > EP_MAX_RANKS) return fail(EP_ERR_UNSUPPORTED, "%s: num_ranks > %d", fn, EP_MAX_RANKS);
    if (E > EP_MAX_EXPERTS) return fail(EP_ERR_UNSUPPORTED, "%s: num_experts > %d", fn, EP_MAX_EXPERTS);
    if (E % R != 0) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_experts %% num_ranks != 0", fn);
    if (T > 0 && !topk_idx) return fail(EP_ERR_INVALID_ARGUMENT, "%s: topk_idx is NULL", fn);
    if (T * static_cast<int64_t>(k) > INT32_MAX)
        return fail(EP_ERR_UNSUPPORTED, "%s: num_tokens * num_topk >= 2^31", fn);
    return EP_OK;
}

// The kernels keep 32-bit counters in the workspace.
int check_workspace(const char* fn, int64_t T, const void* ws, size_t ws_bytes, size_t need) {
    if (T > 0 && (!ws || ws_bytes < need))
        return fail(EP_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes", fn, need);
    if (T > 0 && (reinterpret_cast<uintptr_t>(ws) & 3u))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: workspace must be 4-byte aligned", fn);
    return EP_OK;
}

int check_dispatch_args(const char* fn, const void* x, const int64_t* topk_idx, int64_t T, int H,
                        int k, int E, int R, const void* recv, const int32_t* recv_src_idx,
                        const int32_t* expert_offset, const int32_t* token_row) {
    int s = check_routing(fn, topk_idx, T, k, E, R);
    if (s != EP_OK) return s;
    if (H < 8 || H % 8 != 0) return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden must be a positive multiple of 8", fn);
    if (!expert_offset) return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_expert_offset is NULL", fn);
    if (T > 0 && (!x || !recv || !recv_src_idx || !token_row))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    if (T > 0 && (!aligned16(x) || !aligned16(recv)))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: x and the receive buffer must be 16-byte aligned", fn);
    return EP_OK;
}

int check_dispatch_common(const char* fn, const void* x, const int64_t* topk_idx, int64_t T,
                          int H, int k, int E, int R, const void* recv, const int32_t* recv_src_idx,
                          const int32_t* expert_offset, const int32_t* token_row, const void* ws,
                          size_t ws_bytes) {
    int s = check_dispatch_args(fn, x, topk_idx, T, H, k, E, R, recv, recv_src_idx, expert_offset,
                                token_row);
    if (s != EP_OK) return s;
    return check_workspace(fn, T, ws, ws_bytes, ep::index_workspace_bytes(T, k, E));
}

// The launch sequence of ep_dispatch (arguments already validated): small
// batches in one launch, else the receive-order launch(es) then the copy.
int dispatch_bf16(const char* fn, const void* x, const int64_t* topk_idx, const float* topk_weights,
                  int64_t T, int H, int k, int E, int R, void* recv_x, int32_t* recv_src_idx,
                  float* recv_w, int32_t* expert_offset, int32_t* rank_offset, int32_t* token_row,
                  void* workspace, hipStream_t st) {
    if (!ep::copy_launch_fits(T, H, k))
        return fail(EP_ERR_UNSUPPORTED, "%s: num_tokens * hidden too large for one copy launch", fn);
    if (ep::dispatch_is_small(T, k))
        return hip_status(ep::launch_dispatch_small_bf16(x, topk_idx, topk_weights, T, H, k, E, R, 0,
                                                         recv_x, recv_src_idx, recv_w, expert_offset,
                                                         rank_offset, nullptr, token_row, st),
                          fn);
    const int64_t x_bytes = T * static_cast<int64_t>(H) * 2;
    int s = hip_status(ep::launch_dispatch_index(topk_idx, topk_weights, T, k, E, R, recv_src_idx,
                                                 recv_w, expert_offset, rank_offset, token_row,
                                                 workspace,
                                                 ep::prefetch_pays(x_bytes, true) ? x : nullptr,
                                                 x_bytes, 0, nullptr, st),
                       fn);
    if (s != EP_OK) return s;
    return hip_status(ep::launch_dispatch_copy_bf16(x, token_row, recv_x, T * k, T, H, k, st,
                                                    ep::prefetch_pays(x_bytes, true)),
                      fn);
}

// ---- fixed device scratch of ep_dispatch_noalloc ------------------------------
// For callers that cannot allocate, the receive-order scratch of ep_dispatch
// lives in the file-scope array `scratch` below: kScratchBytes per GPU, held
// until the process ends.  On the host the array's name is only a stand-in,
// not a device address; host code uses the address hipGetSymbolAddress
// returns for the current device, looked up once per device and kept in
// g_scratch.  Nothing in it must start at zero: the receive-order kernels
// write every histogram word they later read, and the prefetch words are
// write-only.  Calls that overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = EP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// This device's address of `scratch`; the stream must belong to the current
// device (the array's address differs per device).
int scratch_for_stream(const char* fn, hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(EP_ERR_UNSUPPORTED, "%s: device %d beyond the %d the scratch table holds", fn, dev,
                    kMaxScratchDevices);
    if (st) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(st, &sdev);
        if (e != hipSuccess) return hip_status(e, fn);
        if (sdev != dev)
            return fail(EP_ERR_INVALID_ARGUMENT, "%s: the stream belongs to device %d, the current device is %d",
                        fn, static_cast<int>(sdev), dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        if (!p) return fail(EP_ERR_HIP, "%s: no device address for the scratch array", fn);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return EP_OK;
}

}  // namespace

extern "C" {

const char* ep_status_string(int status) {
    switch (status) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARGUMENT: return "EP_ERR_INVALID_ARGUMENT";
        case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
        case EP_ERR_WORKSPACE_TOO_SMALL: return "EP_ERR_WORKSPACE_TOO_SMALL";
        case EP_ERR_HIP: return "EP_ERR_HIP";
        default: return "EP_ERR_UNKNOWN";
    }
}

const char* ep_last_error(void) { return g_last_error; }

const char* ep_version(void) { return "ep-mi355x 0.1 gfx950"; }

size_t ep_layout_workspace_bytes(int64_t num_tokens, int num_experts, int num_ranks,
                                 int ranks_per_group) {
    if (num_tokens < 0 || num_experts < 1 || num_ranks < 1 || ranks_per_group < 1) return 0;
    return ep::layout_workspace_bytes(num_tokens, num_experts, num_ranks,
                                      num_ranks / ranks_per_group);
}

int ep_get_dispatch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, int num_ranks, int ranks_per_group,
                           int32_t* num_tokens_per_rank, int32_t* num_tokens_per_group,
                           int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ep_get_dispatch_layout";
    int s = check_routing(fn, topk_idx, num_tokens, num_topk, num_experts, num_ranks);
    if (s != EP_OK) return s;
    if (ranks_per_group < 1 || num_ranks % ranks_per_group != 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_ranks %% ranks_per_group != 0", fn);
    if (!num_tokens_per_rank || !num_tokens_per_expert || (num_tokens > 0 && !is_token_in_rank))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    const size_t need = ep::layout_workspace_bytes(num_tokens, num_experts, num_ranks,
                                                   num_ranks / ranks_per_group);
    s = check_workspace(fn, num_tokens, workspace, workspace_bytes, need);
    if (s != EP_OK) return s;
    return hip_status(ep::launch_layout(topk_idx, num_tokens, num_topk, num_experts, num_ranks,
                                        ranks_per_group, num_tokens_per_rank,
                                        num_tokens_per_group, num_tokens_per_expert,
                                        is_token_in_rank, workspace,
                                        static_cast<hipStream_t>(stream)),
                      fn);
}

size_t ep_dispatch_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts) {
    if (num_tokens < 0 || num_topk < 1 || num_experts < 1) return 0;
    return ep::index_workspace_bytes(num_tokens, num_topk, num_experts);
}

int ep_dispatch(const void* x, const int64_t* topk_idx, const float* topk_weights,
                int64_t num_tokens, int hidden, int num_topk, int num_experts, int num_ranks,
                void* recv_x, int32_t* recv_src_idx, float* recv_topk_weights,
                int32_t* recv_expert_offset, int32_t* recv_rank_offset, int32_t* token_row,
                void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ep_dispatch";
    int s = check_dispatch_common(fn, x, topk_idx, num_tokens, hidden, num_topk, num_experts,
                                  num_ranks, recv_x, recv_src_idx, recv_expert_offset, token_row,
                                  workspace, workspace_bytes);
    if (s != EP_OK) return s;
    return dispatch_bf16(fn, x, topk_idx, topk_weights, num_tokens, hidden, num_topk, num_experts,
                         num_ranks, recv_x, recv_src_idx, recv_topk_weights, recv_expert_offset,
                         recv_rank_offset, token_row, workspace, static_cast<hipStream_t>(stream));
}

int ep_dispatch_noalloc(const void* x, const int64_t* topk_idx, const float* topk_weights,
                        int64_t num_tokens, int hidden, int num_topk, int num_experts,
                        int num_ranks, void* recv_x, int32_t* recv_src_idx,
                        float* recv_topk_weights, int32_t* recv_expert_offset,
                        int32_t* recv_rank_offset, int32_t* token_row, void* stream) {
    const char* fn = "ep_dispatch_noalloc";
    hipStream_t st = static_cast<hipStream_t>(stream);
    int s = check_dispatch_args(fn, x, topk_idx, num_tokens, hidden, num_topk, num_experts,
                                num_ranks, recv_x, recv_src_idx, recv_expert_offset, token_row);
    if (s != EP_OK) return s;
    const size_t need = ep::index_workspace_bytes(num_tokens, num_topk, num_experts);
    if (need > kScratchBytes)
        return fail(EP_ERR_UNSUPPORTED,
                    "%s: this batch needs %zu bytes of receive-order scratch; the fixed device "
                    "array holds %zu (use ep_dispatch with a workspace)",
                    fn, need, kScratchBytes);
    void* ws = nullptr;
    if (num_tokens > 0) {
        s = scratch_for_stream(fn, st, &ws);
        if (s != EP_OK) return s;
    }
    return dispatch_bf16(fn, x, topk_idx, topk_weights, num_tokens, hidden, num_topk, num_experts,
                         num_ranks, recv_x, recv_src_idx, recv_topk_weights, recv_expert_offset,
                         recv_rank_offset, token_row, ws, st);
}

int ep_dispatch_fp8(const void* x, const int64_t* topk_idx, const float* topk_weights,
                    int64_t num_tokens, int hidden, int num_topk, int num_experts,
                    int num_ranks, uint8_t* recv_x_fp8, float* recv_scales,
                    int32_t* recv_src_idx, float* recv_topk_weights,
                    int32_t* recv_expert_offset, int32_t* recv_rank_offset,
                    int32_t* token_row, void* workspace, size_t workspace_bytes,
                    void* stream) {
    const char* fn = "ep_dispatch_fp8";
    int s = check_dispatch_common(fn, x, topk_idx, num_tokens, hidden, num_topk, num_experts,
                                  num_ranks, recv_x_fp8, recv_src_idx, recv_expert_offset,
                                  token_row, workspace, workspace_bytes);
    if (s != EP_OK) return s;
    if (hidden % 128 != 0) return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden %% 128 != 0", fn);
    if (num_tokens > 0 && !recv_scales)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_scales is NULL", fn);
    if (num_tokens > 0 && (reinterpret_cast<uintptr_t>(recv_scales) & 3u))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_scales must be 4-byte aligned", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ep::dispatch_is_small(num_tokens, num_topk))
        return hip_status(ep::launch_dispatch_small_fp8(x, topk_idx, topk_weights, num_tokens, hidden,
                                                        num_topk, num_experts, num_ranks, 0, recv_x_fp8,
                                                        recv_scales, recv_src_idx, recv_topk_weights,
                                                        recv_expert_offset, recv_rank_offset,
                                                        nullptr, token_row, st),
                          fn);
    const int64_t x_bytes = num_tokens * static_cast<int64_t>(hidden) * 2;
    s = hip_status(ep::launch_dispatch_index(topk_idx, topk_weights, num_tokens, num_topk,
                                             num_experts, num_ranks, recv_src_idx,
                                             recv_topk_weights, recv_expert_offset,
                                             recv_rank_offset, token_row, workspace,
                                             ep::prefetch_pays(x_bytes, false) ? x : nullptr,
                                             x_bytes, 0, nullptr, st),
                   fn);
    if (s != EP_OK) return s;
    return hip_status(ep::launch_dispatch_copy_fp8(x, token_row, recv_x_fp8, recv_scales,
                                                   num_tokens * num_topk, num_tokens, hidden,
                                                   num_topk, st),
                      fn);
}

int ep_dispatch_cached(const void* x, const int32_t* token_row, int64_t num_tokens, int hidden,
                       int num_topk, void* recv_x, int64_t recv_rows, void* stream) {
    const char* fn = "ep_dispatch_cached";
    if (num_tokens < 0 || recv_rows < 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_tokens and recv_rows must be >= 0", fn);
    if (num_topk < 1) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_topk < 1", fn);
    if (num_topk > EP_MAX_TOPK) return fail(EP_ERR_UNSUPPORTED, "%s: num_topk > %d", fn, EP_MAX_TOPK);
    if (hidden < 8 || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden must be a positive multiple of 8", fn);
    if (num_tokens > 0 && (!x || !token_row))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    if (num_tokens > 0 && recv_rows > 0 && !recv_x)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_x is NULL", fn);
    if (num_tokens > 0 && (!aligned16(x) || (recv_rows > 0 && !aligned16(recv_x))))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: x and recv_x must be 16-byte aligned", fn);
    if (!ep::copy_launch_fits(num_tokens, hidden, num_topk))
        return fail(EP_ERR_UNSUPPORTED, "%s: num_tokens * hidden too large for one copy launch", fn);
    if (num_tokens == 0 || recv_rows == 0) return EP_OK;
    return hip_status(ep::launch_dispatch_copy_bf16(x, token_row, recv_x, recv_rows, num_tokens,
                                                    hidden, num_topk, static_cast<hipStream_t>(stream)),
                      fn);
}

int ep_dispatch_fp8_cached(const void* x, const int32_t* token_row, int64_t num_tokens,
                           int hidden, int num_topk, uint8_t* recv_x_fp8, float* recv_scales,
                           int64_t recv_rows, void* stream) {
    const char* fn = "ep_dispatch_fp8_cached";
    if (num_tokens < 0 || recv_rows < 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_tokens and recv_rows must be >= 0", fn);
    if (num_topk < 1) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_topk < 1", fn);
    if (num_topk > EP_MAX_TOPK) return fail(EP_ERR_UNSUPPORTED, "%s: num_topk > %d", fn, EP_MAX_TOPK);
    if (hidden < 128 || hidden % 128 != 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden must be a positive multiple of 128", fn);
    if (num_tokens > 0 && (!x || !token_row))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    if (num_tokens > 0 && recv_rows > 0 && (!recv_x_fp8 || !recv_scales))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_x_fp8 / recv_scales is NULL", fn);
    if (num_tokens > 0 && (!aligned16(x) || (recv_rows > 0 && (!aligned16(recv_x_fp8) ||
                                                               (reinterpret_cast<uintptr_t>(recv_scales) & 3u)))))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: misaligned x / recv_x_fp8 / recv_scales", fn);
    if (num_tokens == 0 || recv_rows == 0) return EP_OK;
    return hip_status(ep::launch_dispatch_copy_fp8(x, token_row, recv_x_fp8, recv_scales, recv_rows,
                                                   num_tokens, hidden, num_topk,
                                                   static_cast<hipStream_t>(stream)),
                      fn);
}

size_t ep_dispatch_ht_workspace_bytes(int64_t num_tokens, int num_ranks) {
    if (num_tokens < 0 || num_ranks < 1) return 0;
    return ep::ht_workspace_bytes(num_tokens, num_ranks);
}

int ep_dispatch_ht(const void* x, const int64_t* topk_idx, const float* topk_weights,
                   int64_t num_tokens, int hidden, int num_topk, int num_experts, int num_ranks,
                   void* recv_x, int32_t* recv_src_idx, int64_t* recv_topk_idx,
                   float* recv_topk_weights, int32_t* recv_rank_offset, int32_t* token_rank_row,
                   void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ep_dispatch_ht";
    int s = check_routing(fn, topk_idx, num_tokens, num_topk, num_experts, num_ranks);
    if (s != EP_OK) return s;
    if (hidden < 8 || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden must be a positive multiple of 8", fn);
    if (num_tokens * static_cast<int64_t>(num_ranks) > INT32_MAX)
        return fail(EP_ERR_UNSUPPORTED, "%s: num_tokens * num_ranks >= 2^31", fn);
    if (!ep::copy_launch_fits(num_tokens, hidden, num_ranks))
        return fail(EP_ERR_UNSUPPORTED, "%s: num_tokens * hidden too large for one copy launch", fn);
    if (!recv_rank_offset) return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_rank_offset is NULL", fn);
    if (num_tokens > 0 && (!x || !recv_x || !recv_src_idx || !recv_topk_idx || !token_rank_row))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    if (num_tokens > 0 && (!aligned16(x) || !aligned16(recv_x)))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: x and recv_x must be 16-byte aligned", fn);
    const size_t need = ep::ht_workspace_bytes(num_tokens, num_ranks);
    s = check_workspace(fn, num_tokens, workspace, workspace_bytes, need);
    if (s != EP_OK) return s;
    return hip_status(ep::launch_dispatch_ht(x, topk_idx, topk_weights, num_tokens, hidden, num_topk,
                                             num_experts, num_ranks, recv_x, recv_src_idx,
                                             recv_topk_idx, recv_topk_weights, recv_rank_offset,
                                             token_rank_row, workspace, static_cast<hipStream_t>(stream)),
                      fn);
}

size_t ep_dispatch_ll_workspace_bytes(int64_t num_tokens, int num_topk, int num_experts) {
    if (num_tokens < 0 || num_topk < 1 || num_experts < 1) return 0;
    return ep::ll_workspace_bytes(num_tokens, num_topk, num_experts);
}

static int dispatch_ll_common(const char* fn, bool fp8, const void* x, const int64_t* topk_idx,
                              const float* topk_weights, int64_t T, int H, int k, int E, int cap,
                              void* recv, float* recv_scales, int32_t* recv_count,
                              int32_t* recv_src_idx, float* recv_w, int32_t* token_slot,
                              void* workspace, size_t workspace_bytes, void* stream) {
    int s = check_routing(fn, topk_idx, T, k, E, 1);
    if (s != EP_OK) return s;
    if (cap < 1) return fail(EP_ERR_INVALID_ARGUMENT, "%s: capacity < 1", fn);
    if (static_cast<int64_t>(E) * cap > INT32_MAX)
        return fail(EP_ERR_UNSUPPORTED, "%s: num_experts * capacity >= 2^31", fn);
    if (fp8 ? (H < 128 || H % 128 != 0) : (H < 8 || H % 8 != 0))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden must be a positive multiple of %d", fn,
                    fp8 ? 128 : 8);
    if (!recv_count) return fail(EP_ERR_INVALID_ARGUMENT, "%s: recv_count is NULL", fn);
    if (T > 0 && (!x || !recv || !recv_src_idx || !token_slot || (fp8 && !recv_scales)))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    if (T > 0 && (!aligned16(x) || !aligned16(recv) ||
                  (fp8 && (reinterpret_cast<uintptr_t>(recv_scales) & 3u))))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: misaligned x / receive buffer / scales", fn);
    if (!fp8 && !ep::copy_launch_fits(T, H, k))
        return fail(EP_ERR_UNSUPPORTED, "%s: num_tokens * hidden too large for one copy launch", fn);
    const size_t need = ep::ll_workspace_bytes(T, k, E);
    s = check_workspace(fn, T, workspace, workspace_bytes, need);
    if (s != EP_OK) return s;
    return hip_status(ep::launch_dispatch_ll(x, topk_idx, topk_weights, T, H, k, E, cap, recv,
                                             fp8 ? recv_scales : nullptr, recv_count,
                                             recv_src_idx, recv_w, token_slot, workspace,
                                             static_cast<hipStream_t>(stream)),
                      fn);
}

int ep_dispatch_ll(const void* x, const int64_t* topk_idx, const float* topk_weights,
                   int64_t num_tokens, int hidden, int num_topk, int num_experts, int capacity,
                   void* recv_x, int32_t* recv_count, int32_t* recv_src_idx,
                   float* recv_topk_weights, int32_t* token_slot, void* workspace,
                   size_t workspace_bytes, void* stream) {
    return dispatch_ll_common("ep_dispatch_ll", false, x, topk_idx, topk_weights, num_tokens, hidden,
                              num_topk, num_experts, capacity, recv_x, nullptr, recv_count,
                              recv_src_idx, recv_topk_weights, token_slot, workspace,
                              workspace_bytes, stream);
}

int ep_dispatch_ll_fp8(const void* x, const int64_t* topk_idx, const float* topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, int num_experts,
                       int capacity, uint8_t* recv_x_fp8, float* recv_scales,
                       int32_t* recv_count, int32_t* recv_src_idx, float* recv_topk_weights,
                       int32_t* token_slot, void* workspace, size_t workspace_bytes,
                       void* stream) {
    return dispatch_ll_common("ep_dispatch_ll_fp8", true, x, topk_idx, topk_weights, num_tokens,
                              hidden, num_topk, num_experts, capacity, recv_x_fp8, recv_scales,
                              recv_count, recv_src_idx, recv_topk_weights, token_slot, workspace,
                              workspace_bytes, stream);
}

int ep_combine(const void* expert_out, int64_t num_rows, const int32_t* token_row,
               const float* topk_weights, int64_t num_tokens, int hidden, int num_topk,
               void* combined_x, void* stream) {
    const char* fn = "ep_combine";
    if (num_tokens < 0 || num_rows < 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_tokens and num_rows must be >= 0", fn);
    if (num_topk < 1) return fail(EP_ERR_INVALID_ARGUMENT, "%s: num_topk < 1", fn);
    if (num_topk > EP_MAX_TOPK) return fail(EP_ERR_UNSUPPORTED, "%s: num_topk > %d", fn, EP_MAX_TOPK);
    if (hidden < 8 || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: hidden must be a positive multiple of 8", fn);
    if (num_tokens > 0 && (!token_row || !combined_x))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: a required pointer is NULL", fn);
    if (num_tokens > 0 && num_rows > 0 && !expert_out)
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: expert_out is NULL", fn);
    if (num_tokens > 0 && (!aligned16(combined_x) || (num_rows > 0 && !aligned16(expert_out))))
        return fail(EP_ERR_INVALID_ARGUMENT, "%s: expert_out and combined_x must be 16-byte aligned", fn);
    return hip_status(ep::launch_combine(expert_out, num_rows, token_row, topk_weights,
                                         num_tokens, hidden, num_topk, combined_x,
                                         static_cast<hipStream_t>(stream)),
                      fn);
}

}  // extern "C"
