// Row-scaled int4 / int2 weights: the quantizer and the matmul with Q8_0
// activations.
//
// kerneldigest.dev, "Colibri: running 744B MoE models on consumer hardware by
// streaming experts": the engine requantizes to its own int4 container with
// one scale per row (model-conversion flow) and its integer kernels pack int4
// and int2 codes (layer table).  For b bits, delta = max|w_row| / (2^(b-1) - 1)
// in fp32 (/7 as for Q4_0, /1 for int2, whose codes are then -1, 0, 1);
// codes are rounded half away from zero, clamped to [-2^(b-1), 2^(b-1) - 1]
// and stored as code + 2^(b-1).  Per 32-element group the int4 codes keep the
// Q4_0 nibble order (byte j: element j low, j + 16 high) and the int2 codes
// put elements j, j + 8, j + 16, j + 24 in bits 0-1, 2-3, 4-5, 6-7 of byte j.
// The matmul is the GEMV of the Q4_0 path with the block scale dropped from
// the block sum (dx * isum, exact in fp64) and the row's scale applied once to
// the row's total.
#include "internal.h"

namespace qk {

namespace {

// One workgroup per row: the row's max |w| (exact), then one thread per
// 32-element group packs its codes.
template <int BITS>
__global__ __launch_bounds__(256) void k_quantize_rowq(const float* __restrict__ w, int64_t k,
                                                       uint8_t* __restrict__ wq,
                                                       float* __restrict__ wr) {
    constexpr int HI = (1 << (BITS - 1)) - 1, LO = -(1 << (BITS - 1));
    constexpr int GB = BITS * QBLK / 8;   // bytes per group
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const float* __restrict__ row = w + r * k;
    const int tid = threadIdx.x;
    float amax = 0.0f;
    for (int64_t i = tid * 4; i < k; i += 256 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + i);
        amax = fmaxf(fmaxf(amax, fabsf(v.x)), fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = group_max<WAVE>(amax);
    if ((tid & (WAVE - 1)) == 0) red[tid / WAVE] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float delta = amax / (float)HI;

    const int64_t ng = k / QBLK;
    for (int64_t gi = tid; gi < ng; gi += 256) {
        const float4* p = reinterpret_cast<const float4*>(row + gi * QBLK);
        uint32_t c[QBLK];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 a = p[i];
            const float v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float q = 0.0f;
                if (delta != 0.0f) q = fminf((float)HI, fmaxf((float)LO, roundf(v[e] / delta)));
                c[4 * i + e] = (uint32_t)((int)q - LO);
            }
        }
        uint32_t words[GB / 4];
#pragma unroll
        for (int wi = 0; wi < GB / 4; ++wi) {
            uint32_t word = 0;
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
                const int j = 4 * wi + bi;   // byte j of the group
                const uint32_t byte = BITS == 4 ? (c[j] | (c[j + 16] << 4))
                                                : (c[j] | (c[j + 8] << 2) | (c[j + 16] << 4) | (c[j + 24] << 6));
                word |= byte << (8 * bi);
            }
            words[wi] = word;
        }
        uint8_t* dst = wq + r * (k / QBLK) * GB + gi * GB;
        if (BITS == 4)
            *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        else
            *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
    }
    if (tid == 0) wr[r] = delta;
}

}  // namespace

}  // namespace qk

using namespace qk;

extern "C" int qk_quantize_rowq(int32_t bits, const float* w, int64_t n, int64_t k, uint8_t* w_q,
                                float* w_r, void* stream) {
    QK_REQUIRE(bits == 4 || bits == 2, QK_EINVAL);
    QK_REQUIRE(n >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    QK_REQUIRE(n <= INT32_MAX, QK_EINVAL);
    if (n == 0) return QK_OK;
    QK_REQUIRE(w && w_q && w_r, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w, 16) && QK_ALIGNED(w_q, 16) && QK_ALIGNED(w_r, 4), QK_EALIGN);
    if (bits == 4)
        hipLaunchKernelGGL(k_quantize_rowq<4>, dim3((unsigned)n), dim3(256), 0, (hipStream_t)stream,
                           w, k, w_q, w_r);
    else
        hipLaunchKernelGGL(k_quantize_rowq<2>, dim3((unsigned)n), dim3(256), 0, (hipStream_t)stream,
                           w, k, w_q, w_r);
    return qk_launch_status();
}

extern "C" int qk_qmatmul_rowq_q8_0(int32_t bits, const uint8_t* w_q, const float* w_r, int64_t n,
                                    int64_t k, const int8_t* x_q, const uint16_t* x_d, int64_t m,
                                    float* y, void* stream) {
    QK_REQUIRE(bits == 4 || bits == 2, QK_EINVAL);
    QK_REQUIRE(n >= 0 && m >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    QK_REQUIRE(m <= INT32_MAX && n <= INT32_MAX / 2, QK_EINVAL);
    if (n == 0 || m == 0) return QK_OK;
    QK_REQUIRE(w_q && w_r && x_q && x_d && y, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w_q, 16) && QK_ALIGNED(w_r, 4) && QK_ALIGNED(x_q, 16) &&
                   QK_ALIGNED(x_d, 2) && QK_ALIGNED(y, 4),
               QK_EALIGN);
    QK_REQUIRE(gemv_fits(k), QK_ESHAPE);
    GemvArgs a{};
    a.fmt = bits == 4 ? FMT_Q4_ROW : FMT_Q2_ROW;
    a.wq = w_q; a.wr = w_r; a.n = n; a.k = k;
    a.xq = x_q; a.xd = x_d; a.m = (int32_t)m; a.groups = 1;
    a.y = y; a.ldy = n; a.residual = nullptr; a.ldr = 0; a.ffn = 0;
    a.max_cols = (int32_t)std::min<int64_t>(m, 8);
    return launch_gemv(a, EPI_STORE, (hipStream_t)stream);
}
