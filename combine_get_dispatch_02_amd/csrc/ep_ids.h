// ep_ids.h -- batched loads of one token's routing ids (gfx950).
//
// A loop that loads topk_idx[t*k + j] and uses it before the next load (an
// LDS atomic, a mask update) waits for every load in turn: k dependent round
// trips per token.  load_ids issues a batch of kIdBatch loads before any is
// used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kIdBatch = 8;

// v[u] = ids[j0 + u] for j0 + u < k, else -1 (an empty slot).  Every load
// is issued, at an index clamped to k - 1 (k >= 1), so that no branch around a
// load makes the compiler wait for it before the next one.
__device__ __forceinline__ void load_ids(const int64_t* __restrict__ ids, int j0, int k,
                                         int64_t (&v)[kIdBatch]) {
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) v[u] = ids[j0 + u < k ? j0 + u : k - 1];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u)
        if (j0 + u >= k) v[u] = -1;
}

}  // namespace ep
