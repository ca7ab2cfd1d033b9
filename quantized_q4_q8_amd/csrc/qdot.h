// Device helpers of the Q4_0 x Q8_0 block dot shared by the GEMV kernels, the
// expert GEMV and the persistent decode kernel: the integer block dot of one
// 32-block (and of a row-scaled int2 block), the byte sum that applies the
// nibble offset, the SwiGLU of two matmul outputs, the streaming weight loads
// and the all-rows wave reduction.
// The product is the block form of kenji.blog's llama.cpp guide, section 2.2.
#pragma once

#include "common.h"

namespace qk {

__device__ __forceinline__ int dot_block(const uint4 w, const uint4 x0, const uint4 x1, int s) {
    const uint32_t m4 = 0x0F0F0F0Fu;
    s = __builtin_amdgcn_sdot4((int)(w.x & m4), (int)x0.x, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.y & m4), (int)x0.y, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.z & m4), (int)x0.z, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.w & m4), (int)x0.w, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.x >> 4) & m4), (int)x1.x, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.y >> 4) & m4), (int)x1.y, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.z >> 4) & m4), (int)x1.z, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.w >> 4) & m4), (int)x1.w, s, false);
    return s;
}

__device__ __forceinline__ int byte_sum(const uint4 x0, const uint4 x1) {
    const int ones = 0x01010101;
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)x0.x, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x0.y, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x0.z, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x0.w, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x1.x, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x1.y, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x1.z, ones, s, false);
    s = __builtin_amdgcn_sdot4((int)x1.w, ones, s, false);
    return s;
}

// swish(g) * u of fp32 matmul outputs, in fp64, rounded once
__device__ __forceinline__ float swiglu1(float g, float u) {
    const double gd = (double)g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}

// Row-scaled int2 block (8 bytes in w.x, w.y): byte j holds elements j, j + 8,
// j + 16, j + 24 in bits 0-1, 2-3, 4-5, 6-7, so shifting the two words by 0,
// 2, 4, 6 and masking gives elements 0-7, 8-15, 16-23, 24-31 in order.
__device__ __forceinline__ int dot_block2(const uint4 w, const uint4 x0, const uint4 x1, int s) {
    const uint32_t m2 = 0x03030303u;
    s = __builtin_amdgcn_sdot4((int)(w.x & m2), (int)x0.x, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.y & m2), (int)x0.y, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.x >> 2) & m2), (int)x0.z, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.y >> 2) & m2), (int)x0.w, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.x >> 4) & m2), (int)x1.x, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.y >> 4) & m2), (int)x1.y, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.x >> 6) & m2), (int)x1.z, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.y >> 6) & m2), (int)x1.w, s, false);
    return s;
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// 16-byte weight load marked non-temporal: weights stream through once per
// call and should not displace the activations from the caches.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// The same for an 8-byte block (row-scaled int2).
__device__ __forceinline__ uint2 load_stream8(const uint8_t* p) {
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    return make_uint2(v.x, v.y);
}


// Sums of N values per lane over the 64 lanes of a wave, all N at once.  Two
// "transposed" butterfly steps across rows (lane offsets 32 and 16) halve
// the value count each: a lane keeps the half its offset bit selects and adds
// the partner's copy of it.  The remaining N / 4 values (at least one) are
// then summed over the rest of the wave, ending with DPP steps inside each
// 16-lane row, so every lane of a row holds the same complete sums.  Row
// (b5, b4) of the wave (lane bits 5 and 4) holds value indices
// b5 * N/2 + b4 * N/4 + k, k < max(N/4, 1) (for N < 4 the index is b5 when
// N = 2, 0 when N = 1).  The order of additions is fixed, so the result is
// deterministic.
// The first value index whose sums row_sums leaves in the 16-lane row of
// `lane` (see row_sums).
template <int N>
__device__ __forceinline__ int row_sums_base(int lane) {
    int base = 0;
    if (N >= 2 && (lane & 32) != 0) base += N / 2;
    if (N >= 4 && (lane & 16) != 0) base += N / 4;
    return base;
}

template <int N>
__device__ __forceinline__ int row_sums(double (&v)[N], int lane) {
    if (N >= 2) {
        constexpr int h = N / 2;
        const bool up = (lane & 32) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const double send = up ? v[i] : v[i + h];
            const double keep = up ? v[i + h] : v[i];
            v[i] = keep + __shfl_xor(send, 32, WAVE);
        }
    }
    if (N >= 4) {
        constexpr int h = N / 4;
        const bool up = (lane & 16) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const double send = up ? v[i] : v[i + h];
            const double keep = up ? v[i + h] : v[i];
            v[i] = keep + __shfl_xor(send, 16, WAVE);
        }
    }
    constexpr int NV = N >= 4 ? N / 4 : 1;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        if (N == 1) v[k] += __shfl_xor(v[k], 32, WAVE);
        if (N <= 2) v[k] += __shfl_xor(v[k], 16, WAVE);
        v[k] = group_sum<16>(v[k]);
    }
    return row_sums_base<N>(lane);
}

}  // namespace qk
