// Q8_0 / Q4_0 quantizers and the exact per-block int32 dot products.
//
// Block quantization follows kenji.blog's llama.cpp guide, section 2.2
// (one scale per block from the block's largest magnitude; weights use
// delta = max|w| / 7 with codes in [-8, 7]) and the TinyLLaMA-in-C++ guide,
// section 6.1 (32 values and one fp16 scale per block).  Activations use the
// Q8_0 rule: d = max|x| / 127, codes rounded half away from zero.
#include "common.h"

namespace qk {

// One thread per 8 consecutive values; four threads per block.  x, x_q and
// x_d are flat over [rows][k] since rows are contiguous.
__global__ __launch_bounds__(256) void k_quantize_q8_0(const float* __restrict__ x,
                                                       int64_t nblocks, int8_t* __restrict__ xq,
                                                       uint16_t* __restrict__ xd) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = t >> 2;
    const int sub = (int)(t & 3);
    // Whole quads stay together: nblocks * 4 threads are live, the rest of
    // the last workgroup is masked after the shuffles.
    const bool live = blk < nblocks;
    float v[8];
    if (live) {
        const float4* p = reinterpret_cast<const float4*>(x + blk * QBLK + sub * 8);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    uint32_t lo, hi;
    float d;
    q8_quad(v, lo, hi, d);
    if (!live) return;
    *reinterpret_cast<uint2*>(xq + blk * QBLK + sub * 8) = make_uint2(lo, hi);
    if (sub == 0) xd[blk] = f2h(d);
}

// One thread per Q4_0 block (weights are quantized once, off the hot path).
__global__ __launch_bounds__(256) void k_quantize_q4_0(const float* __restrict__ w,
                                                       int64_t nblocks, uint8_t* __restrict__ wq,
                                                       uint16_t* __restrict__ wd) {
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    const float4* p = reinterpret_cast<const float4*>(w + blk * QBLK);
    float v[QBLK];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 a = p[i];
        v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QBLK; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float delta = amax / 7.0f;
    uint32_t nib[QBLK];
#pragma unroll
    for (int i = 0; i < QBLK; ++i) {
        if (delta == 0.0f) {
            nib[i] = 8;
        } else {
            float c = roundf(v[i] / delta);
            c = fminf(7.0f, fmaxf(-8.0f, c));
            nib[i] = (uint32_t)((int)c + 8);
        }
    }
    uint32_t words[4];
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        uint32_t word = 0;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            const int j = 4 * wi + bi;  // byte j: element j low, element j + 16 high
            word |= (nib[j] | (nib[j + 16] << 4)) << (8 * bi);
        }
        words[wi] = word;
    }
    *reinterpret_cast<uint4*>(wq + blk * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    wd[blk] = f2h(delta);
}

// isum[t][r][b] = sum_j (nibble - 8) * x_q, one thread per (t, r, b).
__global__ __launch_bounds__(256) void k_block_dots(const uint8_t* __restrict__ wq, int64_t n,
                                                    int64_t k, const int8_t* __restrict__ xq,
                                                    int64_t m, int32_t* __restrict__ isum) {
    const int64_t nb = k / QBLK;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m * n * nb) return;
    const int64_t b = i % nb;
    const int64_t r = (i / nb) % n;
    const int64_t t = i / (nb * n);
    const uint4 w = *reinterpret_cast<const uint4*>(wq + r * (k / 2) + b * 16);
    const uint4 x0 = *reinterpret_cast<const uint4*>(xq + t * k + b * QBLK);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xq + t * k + b * QBLK + 16);
    const uint32_t m4 = 0x0F0F0F0Fu;
    // nibbles are in [0, 15], valid non-negative int8 lanes for sdot4
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)(w.x & m4), (int)x0.x, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.y & m4), (int)x0.y, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.z & m4), (int)x0.z, s, false);
    s = __builtin_amdgcn_sdot4((int)(w.w & m4), (int)x0.w, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.x >> 4) & m4), (int)x1.x, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.y >> 4) & m4), (int)x1.y, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.z >> 4) & m4), (int)x1.z, s, false);
    s = __builtin_amdgcn_sdot4((int)((w.w >> 4) & m4), (int)x1.w, s, false);
    int sx = 0;
    const int ones = 0x01010101;
    sx = __builtin_amdgcn_sdot4((int)x0.x, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x0.y, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x0.z, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x0.w, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x1.x, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x1.y, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x1.z, ones, sx, false);
    sx = __builtin_amdgcn_sdot4((int)x1.w, ones, sx, false);
    isum[i] = s - 8 * sx;
}

int launch_quantize_q8(const float* x, int64_t rows, int64_t k, int8_t* xq, uint16_t* xd,
                       hipStream_t s) {
    if (rows == 0) return QK_OK;
    const int64_t nblocks = rows * (k / QBLK);
    const int64_t grid = (nblocks * 4 + 255) / 256;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)grid), dim3(256), 0, s, x, nblocks, xq, xd);
    return qk_launch_status();
}

}  // namespace qk

using namespace qk;

extern "C" int quantize_q8_0(const float* x, int64_t rows, int64_t k, int8_t* x_q,
                             uint16_t* x_d, void* stream) {
    QK_REQUIRE(rows >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    if (rows == 0) return QK_OK;
    QK_REQUIRE(x && x_q && x_d, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(x, 16) && QK_ALIGNED(x_q, 8) && QK_ALIGNED(x_d, 2), QK_EALIGN);
    return launch_quantize_q8(x, rows, k, x_q, x_d, (hipStream_t)stream);
}

extern "C" int qk_quantize_q4_0(const float* w, int64_t n, int64_t k, uint8_t* w_q,
                                uint16_t* w_d, void* stream) {
    QK_REQUIRE(n >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    if (n == 0) return QK_OK;
    QK_REQUIRE(w && w_q && w_d, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w, 16) && QK_ALIGNED(w_q, 16) && QK_ALIGNED(w_d, 2), QK_EALIGN);
    const int64_t nblocks = n * (k / QBLK);
    hipLaunchKernelGGL(k_quantize_q4_0, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, w, nblocks, w_q, w_d);
    return qk_launch_status();
}

extern "C" int qk_block_dots_q4_0_q8_0(const uint8_t* w_q, int64_t n, int64_t k,
                                       const int8_t* x_q, int64_t m, int32_t* isum,
                                       void* stream) {
    QK_REQUIRE(n >= 0 && m >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    if (n == 0 || m == 0) return QK_OK;
    QK_REQUIRE(w_q && x_q && isum, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w_q, 16) && QK_ALIGNED(x_q, 16) && QK_ALIGNED(isum, 4), QK_EALIGN);
    const int64_t total = m * n * (k / QBLK);
    hipLaunchKernelGGL(k_block_dots, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, w_q, n, k, x_q, m, isum);
    return qk_launch_status();
}

extern "C" int qk_q4_0_from_blocks(const void* aos18, int64_t n, int64_t k, uint8_t* w_q,
                                   uint16_t* w_d) {
    QK_REQUIRE(n >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    QK_REQUIRE(n == 0 || (aos18 && w_q && w_d), QK_EINVAL);
    const uint8_t* src = static_cast<const uint8_t*>(aos18);
    const int64_t nb = k / QBLK;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = src + (r * nb + b) * 18;
            w_d[r * nb + b] = (uint16_t)(blk[0] | (blk[1] << 8));
            for (int j = 0; j < 16; ++j) w_q[r * (k / 2) + b * 16 + j] = blk[2 + j];
        }
    return QK_OK;
}
