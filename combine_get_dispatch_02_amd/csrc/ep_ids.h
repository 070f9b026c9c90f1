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

// The rank of a valid expert id, e / epr (epr = E / R experts per rank), as
// one multiply-high instead of the ~10 instructions of a 32-bit division:
// with magic = ceil(2^32 / epr) for epr >= 2, write magic * epr = 2^32 + d,
// 0 <= d < epr; then e * magic / 2^32 = e / epr + e * d / (epr * 2^32), and
// the excess stays below 1 / epr -- so the floor is unchanged -- whenever
// e * epr < 2^32, which 0 <= e < E <= 2048 guarantees.  epr == 1 has
// magic 0: every expert is its own rank.
inline uint32_t rank_magic(int epr) {
    if (epr <= 1) return 0u;
    return static_cast<uint32_t>(((uint64_t(1) << 32) + static_cast<uint64_t>(epr) - 1) /
                                 static_cast<uint64_t>(epr));
}

__device__ __forceinline__ int rank_of(int64_t e, uint32_t magic) {
    const uint32_t u = static_cast<uint32_t>(e);
    return static_cast<int>(magic ? __umulhi(u, magic) : u);
}

}  // namespace ep
