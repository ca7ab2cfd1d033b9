// Q4_0 x Q8_0 matmul for few activation columns (decode GEMV and the grouped
// expert GEMVs of the MoE layer).
//
// The product is the block form of kenji.blog's llama.cpp guide, section 2.2:
// y = sum over blocks of delta_w * delta_x * (exact int32 sum of q_w * q_x),
// with the decode step being a matrix-vector product (same guide, 2.1).
//
// Design (CDNA4, wave64): LPR lanes share one weight row, lane i of a row
// handles blocks i, i + LPR, ...; each lane reads a block's 16 nibble bytes
// with one 128-bit load (a wave reads 1 KiB of a row contiguously) plus its
// fp16 scale.  All weight loads of an unrolled step are issued before any
// arithmetic so each wave keeps ROWS * U 16-byte loads in flight.  Nibbles
// are unpacked in registers with a mask and a shift; v_dot4_i32_i8 forms the
// block's integer sum from the unsigned nibbles and the int8 activations, and
// the -8 offset is applied once per block as -8 * sum(x) (computed per
// activation block, shared by every row).  Row sums finish with a butterfly
// over the LPR lanes.  No LDS, no barriers.
#include "internal.h"

namespace qk {

namespace {

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

__device__ __forceinline__ float swish(float z) { return z / (1.0f + expf(-z)); }

}  // namespace

template <int M, int LPR, int ROWS, int U, int EPI>
__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a) {
    constexpr int RL = WAVE / LPR;                            // rows per wave pass
    constexpr int LROWS = (EPI == EPI_SWIGLU) ? ROWS / 2 : ROWS;  // output rows per pass
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int lr = lane / LPR;
    const int li = lane % LPR;
    const int g = blockIdx.y;

    const int64_t nlog = (EPI == EPI_SWIGLU) ? a.ffn : a.n;
    const int64_t lbase = ((int64_t)blockIdx.x * 4 + wave) * LROWS * RL;
    if (lbase >= nlog) return;

    int c0 = 0, nc = a.m;
    if (a.col_off) {
        c0 = a.col_off[g];
        nc = a.col_off[g + 1] - c0;
    }
    if (nc <= 0) return;

    const int64_t k = a.k, nb = k / QBLK, kh = k / 2;
    const uint8_t* __restrict__ wq = a.wq + (int64_t)g * a.wq_gstride;
    const uint16_t* __restrict__ wd = a.wd + (int64_t)g * a.wd_gstride;

    int64_t orow[ROWS], prow[ROWS];
    bool rv[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        orow[r] = lbase + (r % LROWS) * RL + lr;
        rv[r] = orow[r] < nlog;
        prow[r] = (EPI == EPI_SWIGLU && r >= LROWS) ? orow[r] + a.ffn : orow[r];
    }

    for (int cc = 0; cc < nc; cc += M) {
        float acc[ROWS][M];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

        int xr[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int col = cc + m < nc ? cc + m : nc - 1;  // clamp: extra columns are discarded
            xr[m] = a.col_idx ? a.col_idx[c0 + col] : c0 + col;
        }

        for (int64_t b0 = 0; b0 < nb; b0 += (int64_t)LPR * U) {
            uint4 w[ROWS][U];
            float dw[ROWS][U];
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t b = b0 + u * LPR + li;
                    if (rv[r] && b < nb) {
                        w[r][u] = *reinterpret_cast<const uint4*>(wq + prow[r] * kh + b * 16);
                        dw[r][u] = h2f(wd[prow[r] * nb + b]);
                    } else {
                        w[r][u] = make_uint4(0, 0, 0, 0);
                        dw[r][u] = 0.0f;
                    }
                }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t b = b0 + u * LPR + li;
                if (b >= nb) break;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int8_t* xp = a.xq + (int64_t)xr[m] * k + b * QBLK;
                    const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
                    const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 16);
                    const float dx = h2f(a.xd[(int64_t)xr[m] * nb + b]);
                    const int s0 = -8 * byte_sum(x0, x1);
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        const int s = dot_block(w[r][u], x0, x1, s0);
                        acc[r][m] = fmaf(dw[r][u] * dx, (float)s, acc[r][m]);
                    }
                }
            }
        }

#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = group_sum<LPR>(acc[r][m]);

        if (li == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if (cc + m >= nc) break;
                const int64_t ocol = c0 + cc + m;
                if (EPI == EPI_STORE) {
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        if (!rv[r]) continue;
                        float v = acc[r][m];
                        if (a.residual) v += a.residual[ocol * a.ldr + prow[r]];
                        a.y[ocol * a.ldy + prow[r]] = v;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < LROWS; ++r) {
                        if (!rv[r]) continue;
                        a.y[ocol * a.ldy + orow[r]] = swish(acc[r][m]) * acc[r + LROWS][m];
                    }
                }
            }
        }
    }
}

namespace {

template <int M, int LPR, int ROWS, int EPI>
void launch_cfg(const GemvArgs& a, hipStream_t s) {
    constexpr int U = M == 1 ? 4 : (M <= 4 ? 2 : 1);
    constexpr int RL = WAVE / LPR;
    constexpr int LROWS = (EPI == EPI_SWIGLU) ? ROWS / 2 : ROWS;
    const int64_t nlog = (EPI == EPI_SWIGLU) ? a.ffn : a.n;
    const int64_t per_wg = 4 * (int64_t)LROWS * RL;
    dim3 grid((unsigned)((nlog + per_wg - 1) / per_wg), (unsigned)a.groups);
    hipLaunchKernelGGL((k_gemv<M, LPR, ROWS, U, EPI>), grid, dim3(256), 0, s, a);
}

template <int M, int LPR, int EPI>
void launch_rows(const GemvArgs& a, hipStream_t s) {
    const int64_t nlog = (EPI == EPI_SWIGLU) ? a.ffn : a.n;
    const int64_t rl = WAVE / LPR;
    // Four output rows per wave pass for tall matrices, two otherwise, so that
    // small matrices still spread over all 256 CUs.
    const bool tall = nlog / rl >= (EPI == EPI_SWIGLU ? 4096 : 8192);
    if (EPI == EPI_SWIGLU) {
        if (tall) launch_cfg<M, LPR, 4, EPI>(a, s);
        else launch_cfg<M, LPR, 2, EPI>(a, s);
    } else {
        if (tall) launch_cfg<M, LPR, 4, EPI>(a, s);
        else launch_cfg<M, LPR, 2, EPI>(a, s);
    }
}

template <int M, int EPI>
void launch_lpr(const GemvArgs& a, hipStream_t s) {
    if (a.k / QBLK >= 48) launch_rows<M, 64, EPI>(a, s);
    else launch_rows<M, 16, EPI>(a, s);
}

template <int EPI>
void launch_m(const GemvArgs& a, hipStream_t s) {
    if (a.max_cols <= 1) launch_lpr<1, EPI>(a, s);
    else if (a.max_cols <= 4) launch_lpr<4, EPI>(a, s);
    else launch_lpr<8, EPI>(a, s);
}

}  // namespace

int launch_gemv(const GemvArgs& a, int epi, hipStream_t s) {
    if (epi == EPI_SWIGLU) launch_m<EPI_SWIGLU>(a, s);
    else launch_m<EPI_STORE>(a, s);
    return qk_launch_status();
}

}  // namespace qk

using namespace qk;

extern "C" int qmatmul_q4_0_q8_0(const uint8_t* w_q, const uint16_t* w_d, int64_t n, int64_t k,
                                 const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y,
                                 void* stream) {
    QK_REQUIRE(n >= 0 && m >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    QK_REQUIRE(m <= INT32_MAX && n <= INT32_MAX / 2, QK_EINVAL);
    if (n == 0 || m == 0) return QK_OK;
    QK_REQUIRE(w_q && w_d && x_q && x_d && y, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w_q, 16) && QK_ALIGNED(x_q, 16) && QK_ALIGNED(w_d, 2) &&
                   QK_ALIGNED(x_d, 2) && QK_ALIGNED(y, 4),
               QK_EALIGN);
    GemvArgs a{};
    a.wq = w_q; a.wd = w_d; a.n = n; a.k = k;
    a.xq = x_q; a.xd = x_d; a.m = (int32_t)m; a.groups = 1;
    a.y = y; a.ldy = n; a.residual = nullptr; a.ldr = 0; a.ffn = 0;
    a.max_cols = (int32_t)m;
    if (m > 8) return launch_gemm(a, EPI_STORE, (hipStream_t)stream);
    return launch_gemv(a, EPI_STORE, (hipStream_t)stream);
}

extern "C" int qk_gate_up_swiglu(const uint8_t* w_q, const uint16_t* w_d, int64_t ffn, int64_t k,
                                 const int8_t* x_q, const uint16_t* x_d, int64_t m, float* h,
                                 void* stream) {
    QK_REQUIRE(ffn >= 0 && m >= 0 && k > 0, QK_EINVAL);
    QK_REQUIRE(k % QBLK == 0, QK_ESHAPE);
    QK_REQUIRE(m <= INT32_MAX && ffn <= INT32_MAX / 4, QK_EINVAL);
    if (ffn == 0 || m == 0) return QK_OK;
    QK_REQUIRE(w_q && w_d && x_q && x_d && h, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w_q, 16) && QK_ALIGNED(x_q, 16) && QK_ALIGNED(w_d, 2) &&
                   QK_ALIGNED(x_d, 2) && QK_ALIGNED(h, 4),
               QK_EALIGN);
    GemvArgs a{};
    a.wq = w_q; a.wd = w_d; a.n = 2 * ffn; a.k = k;
    a.xq = x_q; a.xd = x_d; a.m = (int32_t)m; a.groups = 1;
    a.y = h; a.ldy = ffn; a.residual = nullptr; a.ldr = 0; a.ffn = ffn;
    a.max_cols = (int32_t)m;
    if (m > 8) return launch_gemm(a, EPI_SWIGLU, (hipStream_t)stream);
    return launch_gemv(a, EPI_SWIGLU, (hipStream_t)stream);
}
