// ep_device.h -- device helpers shared by the gfx950 kernels of libep.so.
//
// Wave64 primitives (ballot-based key matching), bf16 rounding and the OCP
// E4M3FN encoder, all written for CDNA4 (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

// 16-byte vector used for every global load/store on the data path.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Mask of the lanes below the calling one.
__device__ __forceinline__ uint64_t lanes_below() {
    return (uint64_t(1) << lane_id()) - 1;
}

// Lanes of the wave whose `key` equals the caller's, among lanes with `active`
// set: one ballot per key bit (nbits = bits needed for the largest key).
// Inactive lanes get 0.
__device__ __forceinline__ uint64_t match_key(int key, bool active, int nbits) {
    uint64_t peers = ballot(active);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = ballot(active && bit);
        peers &= bit ? ones : ~ones;
    }
    return active ? peers : 0;
}

// Broadcast lane `src` (wave-uniform) of a 32-bit value to every lane.
__device__ __forceinline__ int read_lane(int v, int src) {
    return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ float read_lane(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even: adding 0x7FFF plus the last kept
// bit carries exactly when the dropped half is above one half, or equal to
// one half with an odd kept part.  NaN is kept quiet.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E4M3FN code (sign | 4-bit exponent, bias 7 | 3-bit mantissa),
// round to nearest even, saturating to +-448 (0x7E) above the largest finite
// value.  Normal range (|f| >= 2^-6): round the fp32 mantissa to 3 bits and
// rebias the exponent from 127 to 7.  Below 2^-6 the codes are the multiples
// of 2^-9, so the code is |f| * 512 rounded to an integer (0..8; 8 is the
// smallest normal, code 0x08).  Every NaN, whatever its sign and payload,
// becomes 0x7F, so the code does not depend on how a division propagated it.
__device__ __forceinline__ uint32_t e4m3fn_encode(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;                         // NaN
    uint32_t code;
    if (a >= 0x43E00000u) {                                    // >= 448.0f, inf
        code = 0x7Eu;
    } else if (a >= 0x3C800000u) {                             // >= 2^-6
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    } else {
        code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
    }
    return code | sign;
}

// Read src[0 .. nvec) once through the caches, as block pf_block of
// pf_blocks blocks of NT threads (a grid-stride sweep, 8 loads in flight per
// thread).  The values are folded into one word per block and stored to
// sink[pf_block % 64] (scratch, >= 256 bytes) so the loads are kept.  Used by
// index kernels to bring the tokens into the Infinity Cache while they rank,
// ahead of the copy that reads them.
template <int NT>
__device__ __forceinline__ void prefetch_vectors(const u32x4* __restrict__ src, int64_t nvec,
                                                 int pf_block, int pf_blocks,
                                                 uint32_t* __restrict__ sink) {
    constexpr int kUnroll = 8;
    uint32_t acc = 0;
    const int64_t stride = static_cast<int64_t>(pf_blocks) * NT;
    int64_t i = static_cast<int64_t>(pf_block) * NT + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < nvec; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (threadIdx.x == 0) sink[pf_block & 63] = acc;
}

}  // namespace ep
