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

// swish(g) * u of fp32 matmul outputs, in fp64, rounded once
__device__ __forceinline__ float swiglu1(float g, float u) {
    const double gd = (double)g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// 16-byte weight load marked non-temporal: weights stream through once per
// call and should not displace the activations from the caches.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace

// Workgroup-wide RMSNorm / Q8_0 of one activation row into LDS.  Each lane
// takes 8 consecutive values per 2048-value chunk (four lanes per Q8_0 block),
// with the same arithmetic as the standalone quantizer.  The row's global
// loads are issued by `load_row` before the caller issues its weight loads,
// so that waiting on them leaves the weight loads in flight.
constexpr int PRO_CHUNKS = 3;  // rows up to 3 * 2048 values

template <int KC>
struct RowRegs {
    float v[KC][8];
    float g[KC][8];
};

template <int PRO, int KC>
__device__ __forceinline__ void load_row(RowRegs<KC>& R, const float* __restrict__ x,
                                         const float* __restrict__ gamma, int64_t k) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        const int64_t i = (int64_t)c * 2048 + threadIdx.x * 8;
        const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float4 a = zero, b = zero, ga = zero, gb = zero;
        if (i < k) {
            a = *reinterpret_cast<const float4*>(x + i);
            b = *reinterpret_cast<const float4*>(x + i + 4);
            if (PRO == PRO_RMSNORM) {
                ga = *reinterpret_cast<const float4*>(gamma + i);
                gb = *reinterpret_cast<const float4*>(gamma + i + 4);
            }
        }
        R.v[c][0] = a.x; R.v[c][1] = a.y; R.v[c][2] = a.z; R.v[c][3] = a.w;
        R.v[c][4] = b.x; R.v[c][5] = b.y; R.v[c][6] = b.z; R.v[c][7] = b.w;
        R.g[c][0] = ga.x; R.g[c][1] = ga.y; R.g[c][2] = ga.z; R.g[c][3] = ga.w;
        R.g[c][4] = gb.x; R.g[c][5] = gb.y; R.g[c][6] = gb.z; R.g[c][7] = gb.w;
    }
}

// LDS barrier that waits only for LDS traffic, so global loads issued before
// it stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int PRO, int KC>
__device__ __forceinline__ void stage_row(const RowRegs<KC>& R, int64_t k, float eps, double* red,
                                          int8_t* lxq, float* lxd) {
    double inv = 1.0;
    if (PRO == PRO_RMSNORM) {
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fma((double)R.v[c][e], (double)R.v[c][e], ss);
        ss = group_sum<WAVE>(ss);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
        lds_barrier();
        const double total = red[0] + red[1] + red[2] + red[3];
        inv = 1.0 / sqrt(total / (double)k + (double)eps);
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        const int64_t i = (int64_t)c * 2048 + threadIdx.x * 8;
        if ((int64_t)c * 2048 < k) {   // uniform over the workgroup
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (PRO == PRO_RMSNORM) ? (float)((double)R.v[c][e] * inv * (double)R.g[c][e])
                                            : R.v[c][e];
            uint32_t lo, hi;
            float d;
            q8_quad(v, lo, hi, d);
            if (i < k) {
                *reinterpret_cast<uint2*>(lxq + i) = make_uint2(lo, hi);
                if ((threadIdx.x & 3) == 0) lxd[i / QBLK] = h2f(f2h(d));
            }
        }
    }
}

template <int M, int LPR, int ROWS, int U, int EPI, int PRO, int KC>
__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ double red[4];
    constexpr int RL = WAVE / LPR;                                // row groups per wave
    constexpr int LROWS = (EPI == EPI_SWIGLU) ? ROWS / 2 : ROWS;  // output rows per row group
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int lr = lane / LPR;
    const int li = lane % LPR;
    const int g = blockIdx.y;

    if (a.zero_ptr && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;

    const int64_t nlog = (EPI == EPI_SWIGLU) ? a.ffn : a.n;
    const int64_t wg_base = (int64_t)blockIdx.x * 4 * LROWS * RL;
    const int64_t lbase = wg_base + (int64_t)wave * LROWS * RL;

    int c0 = 0, nc = a.m;
    if (a.col_off) {
        c0 = a.col_off[g];
        nc = a.col_off[g + 1] - c0;
    }
    if (nc <= 0) return;   // uniform over the workgroup

    const int64_t k = a.k, nb = k / QBLK, kh = k / 2;
    const uint8_t* __restrict__ wq = a.wq + (int64_t)g * a.wq_gstride;
    const uint16_t* __restrict__ wd = a.wd + (int64_t)g * a.wd_gstride;

    int64_t orow[ROWS], prow[ROWS];
    bool rv[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        orow[r] = lbase + lr * LROWS + (r % LROWS);
        rv[r] = orow[r] < nlog;
        prow[r] = (EPI == EPI_SWIGLU && r >= LROWS) ? orow[r] + a.ffn : orow[r];
    }

    // LDS: staged activations [M][k] codes, [M][k/32] scales, then the QKV
    // cos/sin table [M][pairs of this workgroup][2] (fp64)
    int8_t* lxq = reinterpret_cast<int8_t*>(smem);
    float* lxd = reinterpret_cast<float*>(smem + (size_t)M * k);
    double* lcs = reinterpret_cast<double*>(smem + (((size_t)M * k + (size_t)M * nb * 4 + 7) & ~(size_t)7));
    constexpr int WG_PAIRS = 4 * LROWS * RL / 2;

    for (int cc = 0; cc < nc; cc += M) {
        const int mc = nc - cc < M ? nc - cc : M;
        int xr[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int col = cc + m < nc ? cc + m : nc - 1;  // clamp: extra columns are discarded
            xr[m] = a.col_idx ? a.col_idx[c0 + col] : c0 + col;
        }

        uint4 w[ROWS][U];
        float dw[ROWS][U];
        auto load_w = [&](int64_t b0) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t b = b0 + u * LPR + li;
                    if (rv[r] && b < nb) {
                        w[r][u] = load_stream16(wq + prow[r] * kh + b * 16);
                        dw[r][u] = h2f(wd[prow[r] * nb + b]);
                    } else {
                        w[r][u] = make_uint4(0, 0, 0, 0);
                        dw[r][u] = 0.0f;
                    }
                }
        };

        if (PRO != PRO_NONE) {
            if (cc > 0) lds_barrier();   // previous chunk finished reading LDS
            RowRegs<KC> R;
            load_row<PRO, KC>(R, a.xf + (int64_t)xr[0] * k, a.gamma, k);
            load_w(0);                    // weight loads go out behind the row loads
            stage_row<PRO, KC>(R, k, a.eps, red, lxq, lxd);
#pragma unroll
            for (int m = 1; m < M; ++m) {
                if (m >= mc) break;       // uniform over the workgroup
                lds_barrier();            // `red` reused
                load_row<PRO, KC>(R, a.xf + (int64_t)xr[m] * k, a.gamma, k);
                stage_row<PRO, KC>(R, k, a.eps, red, lxq + (size_t)m * k, lxd + (size_t)m * nb);
            }
            if (EPI == EPI_QKV) {
                // cos/sin of this workgroup's q/k row pairs, per column, in fp64
                for (int i = threadIdx.x; i < mc * WG_PAIRS; i += 256) {
                    const int m = i / WG_PAIRS, pr = i % WG_PAIRS;
                    const int64_t row = wg_base + 2 * pr;
                    double cs = 1.0, sn = 0.0;
                    if (row < a.q_rows + a.kv_rows) {
                        const int64_t pair = (row % a.hd) / 2;
                        const double theta = pow((double)a.rope_base, -2.0 * (double)pair / (double)a.hd);
                        sincos((double)a.pos[c0 + cc + m] * theta, &sn, &cs);
                    }
                    lcs[2 * i] = cs;
                    lcs[2 * i + 1] = sn;
                }
            }
            lds_barrier();
        } else {
            load_w(0);
        }

        double acc[ROWS][M];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0;

        for (int64_t b0 = 0; b0 < nb; b0 += (int64_t)LPR * U) {
            if (b0 > 0) load_w(b0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t b = b0 + u * LPR + li;
                if (b >= nb) break;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    uint4 x0, x1;
                    float dx;
                    if (PRO != PRO_NONE) {
                        const int8_t* xp = lxq + (size_t)m * k + b * QBLK;
                        x0 = *reinterpret_cast<const uint4*>(xp);
                        x1 = *reinterpret_cast<const uint4*>(xp + 16);
                        dx = lxd[(size_t)m * nb + b];
                    } else {
                        const int8_t* xp = a.xq + (int64_t)xr[m] * k + b * QBLK;
                        x0 = *reinterpret_cast<const uint4*>(xp);
                        x1 = *reinterpret_cast<const uint4*>(xp + 16);
                        dx = h2f(a.xd[(int64_t)xr[m] * nb + b]);
                    }
                    const int s0 = -8 * byte_sum(x0, x1);
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        // dw * dx is exact in fp32 (two fp16 values); times the
                        // int32 block dot it is exact in fp64
                        const int s = dot_block(w[r][u], x0, x1, s0);
                        acc[r][m] = fma((double)(dw[r][u] * dx), (double)s, acc[r][m]);
                    }
                }
            }
        }

#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = group_sum<LPR>(acc[r][m]);

        if (EPI == EPI_ARGMAX) {
            // logits, then the workgroup's best (value, lowest row) per column
            float* bv = reinterpret_cast<float*>(lcs);          // [4 * RL][M], after the staged x
            int* bi = reinterpret_cast<int*>(bv + 4 * RL * M);
            if (li == 0) {
                const int slot = wave * RL + lr;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float best = -INFINITY;
                    int besti = INT32_MAX;
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        if (!rv[r] || cc + m >= nc) continue;
                        const float v = (float)acc[r][m];
                        a.y[(int64_t)(c0 + cc + m) * a.ldy + prow[r]] = v;
                        if (v > best || (v == best && (int)prow[r] < besti)) {
                            best = v;
                            besti = (int)prow[r];
                        }
                    }
                    bv[slot * M + m] = best;
                    bi[slot * M + m] = besti;
                }
            }
            lds_barrier();
            if (threadIdx.x < M && (int)threadIdx.x < mc) {
                const int m = threadIdx.x;
                float best = -INFINITY;
                int besti = INT32_MAX;
                for (int sl = 0; sl < 4 * RL; ++sl) {
                    const float v = bv[sl * M + m];
                    const int i = bi[sl * M + m];
                    if (v > best || (v == best && i < besti)) {
                        best = v;
                        besti = i;
                    }
                }
                a.part_val[(int64_t)(cc + m) * gridDim.x + blockIdx.x] = best;
                a.part_idx[(int64_t)(cc + m) * gridDim.x + blockIdx.x] = besti;
            }
            lds_barrier();
        } else if (li == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if (cc + m >= nc) break;
                const int64_t ocol = c0 + cc + m;
                if (EPI == EPI_STORE) {
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        if (!rv[r]) continue;
                        float v = (float)acc[r][m];
                        if (a.residual) v = a.residual[ocol * a.ldr + prow[r]] + v;
                        a.y[ocol * a.ldy + prow[r]] = v;
                    }
                } else if (EPI == EPI_SWIGLU) {
#pragma unroll
                    for (int r = 0; r < LROWS; ++r) {
                        if (!rv[r]) continue;
                        a.y[ocol * a.ldy + orow[r]] = swiglu1((float)acc[r][m], (float)acc[r + LROWS][m]);
                    }
                } else {  // EPI_QKV: rows orow[r], orow[r] + 1 form one RoPE pair
#pragma unroll
                    for (int r = 0; r < ROWS; r += 2) {
                        if (!rv[r]) continue;
                        const int64_t row = orow[r];
                        const int pr = (int)((row - wg_base) / 2);
                        const double c = lcs[2 * (m * WG_PAIRS + pr)], sn = lcs[2 * (m * WG_PAIRS + pr) + 1];
                        const double x1 = (double)(float)acc[r][m], x2 = (double)(float)acc[r + 1][m];
                        const int p = a.pos[ocol];
                        if (row < a.q_rows) {
                            a.q_out[ocol * a.q_rows + row] = (float)(x1 * c - x2 * sn);
                            a.q_out[ocol * a.q_rows + row + 1] = (float)(x1 * sn + x2 * c);
                        } else if (p >= 0 && p < a.cap) {
                            const bool is_k = row < a.q_rows + a.kv_rows;
                            const int64_t rr = row - a.q_rows - (is_k ? 0 : a.kv_rows);
                            const int64_t gh = rr / a.hd, d = rr % a.hd;
                            const int64_t dst = (((int64_t)a.seq[ocol] * a.n_kv + gh) * a.cap + p) * a.hd + d;
                            uint16_t* cache = is_k ? a.kc : a.vc;
                            const float o1 = (float)(is_k ? x1 * c - x2 * sn : x1);
                            const float o2 = (float)(is_k ? x1 * sn + x2 * c : x2);
                            cache[dst] = f2h(o1);
                            cache[dst + 1] = f2h(o2);
                        }
                    }
                }
            }
        }
    }
}

// idx[c] = row of the largest partial of column c (ties to the lowest row).
__global__ __launch_bounds__(256) void k_argmax_partials(const float* __restrict__ pv,
                                                         const int32_t* __restrict__ pi,
                                                         int64_t nparts, int32_t* __restrict__ idx) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int64_t c = blockIdx.x;
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int64_t i = threadIdx.x; i < nparts; i += 256) {
        const float v = pv[c * nparts + i];
        const int j = pi[c * nparts + i];
        if (v > bv || (v == bv && j < bi)) { bv = v; bi = j; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, WAVE);
        const int oi = __shfl_xor(bi, o, WAVE);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w)
            if (sv[w] > bv || (sv[w] == bv && si[w] < bi)) { bv = sv[w]; bi = si[w]; }
        idx[c] = bi == INT32_MAX ? 0 : bi;
    }
}

int launch_argmax_partials(const float* part_val, const int32_t* part_idx, int64_t nparts,
                           int64_t cols, int32_t* idx, hipStream_t s) {
    if (cols == 0) return QK_OK;
    hipLaunchKernelGGL(k_argmax_partials, dim3((unsigned)cols), dim3(256), 0, s, part_val,
                       part_idx, nparts, idx);
    return qk_launch_status();
}

namespace {

int pick_m(int64_t max_cols) { return max_cols <= 1 ? 1 : (max_cols <= 4 ? 4 : 8); }
int pick_lpr(int64_t k) { return k / QBLK >= 48 ? 64 : 16; }

// Rows per row group: four for tall matrices, two otherwise (and always two
// for the RoPE pairs of EPI_QKV), so that small matrices still spread over all
// 256 CUs.
int pick_rows(int epi, int64_t nlog, int lpr) {
    const int64_t rl = WAVE / lpr;
    if (epi == EPI_QKV) return 2;
    if (epi == EPI_SWIGLU) return nlog / rl >= 4096 ? 4 : 2;
    return nlog / rl >= 8192 ? 4 : 2;
}

size_t lds_bytes(int pro, int epi, int M, int64_t k, int lpr, int rows) {
    const int rl = WAVE / lpr;
    const int lrows = epi == EPI_SWIGLU ? rows / 2 : rows;
    size_t b = 0;
    if (pro != PRO_NONE) b = (size_t)M * k + (size_t)M * (k / QBLK) * 4;
    b = (b + 7) & ~(size_t)7;
    if (epi == EPI_QKV) b += (size_t)M * (4 * lrows * rl / 2) * 16;
    if (epi == EPI_ARGMAX) b += (size_t)4 * rl * M * 8;
    return b;
}

// Blocks per lane loaded together: enough to cover a row in one step for the
// common K (one for K <= 32 * LPR, three for K <= 96 * LPR at M = 1), fewer
// for wide M where the activations take the registers.
int pick_u(int M, int64_t k, int lpr) {
    const int64_t need = (k / QBLK + lpr - 1) / lpr;
    if (M == 1) return need <= 1 ? 1 : 3;
    if (M == 4) return need <= 1 ? 1 : 2;
    return 1;
}

template <int M, int LPR, int ROWS, int EPI, int PRO, int U, int KC>
void launch_cfg(const GemvArgs& a, hipStream_t s) {
    constexpr int RL = WAVE / LPR;
    constexpr int LROWS = (EPI == EPI_SWIGLU) ? ROWS / 2 : ROWS;
    const int64_t nlog = (EPI == EPI_SWIGLU) ? a.ffn : a.n;
    const int64_t per_wg = 4 * (int64_t)LROWS * RL;
    dim3 grid((unsigned)((nlog + per_wg - 1) / per_wg), (unsigned)a.groups);
    const size_t lds = lds_bytes(PRO, EPI, M, a.k, LPR, ROWS);
    hipLaunchKernelGGL((k_gemv<M, LPR, ROWS, U, EPI, PRO, KC>), grid, dim3(256), lds, s, a);
}

template <int M, int LPR, int EPI, int PRO, int U, int KC>
void launch_rows_kc(const GemvArgs& a, hipStream_t s) {
    const int64_t nlog = (EPI == EPI_SWIGLU) ? a.ffn : a.n;
    if constexpr (EPI == EPI_QKV) {
        launch_cfg<M, LPR, 2, EPI, PRO, U, KC>(a, s);
    } else {
        if (pick_rows(EPI, nlog, LPR) == 4) launch_cfg<M, LPR, 4, EPI, PRO, U, KC>(a, s);
        else launch_cfg<M, LPR, 2, EPI, PRO, U, KC>(a, s);
    }
}

// Prologue chunks (2048 values each) held in registers: one for K <= 2048.
template <int M, int LPR, int EPI, int PRO, int U>
void launch_rows(const GemvArgs& a, hipStream_t s) {
    if constexpr (PRO == PRO_NONE) {
        launch_rows_kc<M, LPR, EPI, PRO, U, 1>(a, s);
    } else {
        if (a.k <= 2048) launch_rows_kc<M, LPR, EPI, PRO, U, 1>(a, s);
        else launch_rows_kc<M, LPR, EPI, PRO, U, PRO_CHUNKS>(a, s);
    }
}

template <int M, int LPR, int EPI, int PRO>
void launch_u(const GemvArgs& a, hipStream_t s) {
    constexpr int UHI = M == 1 ? 3 : (M == 4 ? 2 : 1);
    if (pick_u(M, a.k, LPR) == 1) launch_rows<M, LPR, EPI, PRO, 1>(a, s);
    else launch_rows<M, LPR, EPI, PRO, UHI>(a, s);
}

template <int M, int EPI, int PRO>
void launch_lpr(const GemvArgs& a, hipStream_t s) {
    if (pick_lpr(a.k) == 64) launch_u<M, 64, EPI, PRO>(a, s);
    else launch_u<M, 16, EPI, PRO>(a, s);
}

template <int EPI, int PRO>
void launch_m(const GemvArgs& a, hipStream_t s) {
    switch (pick_m(a.max_cols)) {
        case 1: launch_lpr<1, EPI, PRO>(a, s); break;
        case 4: launch_lpr<4, EPI, PRO>(a, s); break;
        default: launch_lpr<8, EPI, PRO>(a, s); break;
    }
}

}  // namespace

bool gemv_prologue_fits(int64_t k, int64_t max_cols) {
    const int M = pick_m(max_cols);
    return k <= (int64_t)PRO_CHUNKS * 2048 &&
           lds_bytes(PRO_RMSNORM, EPI_QKV, M, k, pick_lpr(k), 2) <= 60 * 1024;
}

int64_t gemv_argmax_parts(int64_t n, int64_t k, int64_t max_cols) {
    (void)max_cols;
    const int lpr = pick_lpr(k);
    const int rows = pick_rows(EPI_ARGMAX, n, lpr);
    const int64_t per_wg = 4 * (int64_t)rows * (WAVE / lpr);
    return (n + per_wg - 1) / per_wg;
}

int launch_gemv(const GemvArgs& a, int epi, hipStream_t s, int pro) {
    if (pro != PRO_NONE && !gemv_prologue_fits(a.k, a.max_cols)) return QK_ESHAPE;
    if (epi == EPI_SWIGLU) {
        if (pro == PRO_RMSNORM) launch_m<EPI_SWIGLU, PRO_RMSNORM>(a, s);
        else launch_m<EPI_SWIGLU, PRO_NONE>(a, s);
    } else if (epi == EPI_QKV) {
        launch_m<EPI_QKV, PRO_RMSNORM>(a, s);
    } else if (epi == EPI_ARGMAX) {
        launch_m<EPI_ARGMAX, PRO_RMSNORM>(a, s);
    } else {
        if (pro == PRO_Q8) launch_m<EPI_STORE, PRO_Q8>(a, s);
        else launch_m<EPI_STORE, PRO_NONE>(a, s);
    }
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
