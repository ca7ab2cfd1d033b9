// Q4_0 x Q8_0 matmul for few activation columns (decode GEMV and the grouped
// expert GEMVs of the MoE layer).
//
// The product is the block form of kenji.blog's llama.cpp guide, section 2.2:
// y = sum over blocks of delta_w * delta_x * (exact int32 sum of q_w * q_x),
// with the decode step being a matrix-vector product (same guide, 2.1).
//
// Design (CDNA4, wave64): a wave owns a few weight rows (one output unit by
// default) and its 64 lanes split each row: lane i handles blocks i, i + 64,
// ..., reading a block's 16 nibble bytes with one 128-bit load (a wave reads
// 1 KiB of a row contiguously) plus its fp16 scale.  All weight loads of a
// step are issued before anything waits, so every wave has its whole share
// in flight; when the share is one step, later column passes reuse the
// registers instead of loading again.  The activation columns are staged
// once per workgroup in LDS
// (as Q8_0 codes and fp32 scales, either copied from the input or built by
// a fused RMSNorm / Q8_0 prologue).  Nibbles are unpacked in registers with a
// mask and a shift; v_dot4_i32_i8 forms the block's integer sum from the
// unsigned nibbles and the int8 activations, and the -8 offset is applied
// once per block as -8 * sum(x).  The wave's row sums are reduced together
// (row_sums) and the epilogue runs in the lanes that hold them.
#include "internal.h"
#include "qdot.h"

#include <type_traits>

namespace qk {

// Workgroup-wide RMSNorm / Q8_0 of one activation row into LDS.  Each lane
// takes 8 consecutive values per 2048-value chunk (four lanes per Q8_0 block),
// with the same arithmetic as the standalone quantizer.  By default
// `load_row` loads under a bounds test, so the row has arrived before the
// caller's weight loads go out; the norm and the LDS staging then overlap
// the weight loads.  For the gate/up GEMV (704 workgroups on the decode
// shape) issuing the weights before the row arrives measured slower: the
// row, read by every workgroup, then queues behind the weight misses.  The
// QKV and down GEMVs (160 and 256 workgroups) load the row unconditionally
// (UNC, clamped indexes) so their weights go out with it: decode +0.6 %.
constexpr int PRO_CHUNKS = 3;  // rows up to 3 * 2048 values

template <int KC>
struct RowRegs {
    float v[KC][8];
    float g[KC][8];
};

template <int PRO, int KC, bool UNC = false>
__device__ __forceinline__ void load_row(RowRegs<KC>& R, const float* __restrict__ x,
                                         const float* __restrict__ gamma, int64_t k) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        const int64_t i = (int64_t)c * 2048 + threadIdx.x * 8;
        const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float4 a = zero, b = zero, ga = zero, gb = zero;
        if constexpr (UNC) {
            const int64_t ii = i < k ? i : 0;
            a = *reinterpret_cast<const float4*>(x + ii);
            b = *reinterpret_cast<const float4*>(x + ii + 4);
            if (PRO == PRO_RMSNORM) {
                ga = *reinterpret_cast<const float4*>(gamma + ii);
                gb = *reinterpret_cast<const float4*>(gamma + ii + 4);
            }
            if (i >= k) a = b = ga = gb = zero;
        } else if (i < k) {
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

// Physical rows per output unit: SwiGLU units are (gate row, up row), QKV
// units are RoPE pairs (row 2u, row 2u + 1).
__host__ __device__ constexpr int rows_per_unit(int epi) {
    return (epi == EPI_SWIGLU || epi == EPI_QKV) ? 2 : 1;
}


// One wave computes R rows (a multiple of the unit size) of the matrix for M
// activation columns at a time; the four waves of a
// workgroup take consecutive units.  Each lane reads, per row, blocks lane,
// lane + 64, ... (U per step) with one 128-bit load each; all loads of a
// step are issued before the activations are staged, so they are in flight
// together.  The activations of the workgroup's columns sit in LDS (built
// there by the prologue, or copied from the Q8_0 input), and are read by
// every row.
// KLOOP: K may exceed 64 * U blocks (the weights are then loaded step by
// step); otherwise the whole row share is loaded at once.
// FMT: Q4_0 (fp16 scale per block), or row-scaled int4 / int2 (fp32 scale
// per row): their block sums are dx * isum, and the row's scale multiplies
// the row's total in the epilogue, once.
// Column of 16-byte chunk (or block) i of a pass whose columns hold `per`
// each (i < M * per): M - 1 compares instead of a division.
template <int M>
__device__ __forceinline__ uint32_t col_of(uint32_t i, uint32_t per) {
    uint32_t m = 0;
#pragma unroll
    for (int q = 1; q < M; ++q) m += i >= (uint32_t)q * per ? 1u : 0u;
    return m;
}

template <int FMT, int M, int R, int U, int EPI, int PRO, int KC, bool KLOOP>
__device__ __forceinline__ void gemv_body(const GemvArgs& a) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ double red[4];
    constexpr int RMAX = R;
    constexpr int P = rows_per_unit(EPI);
    static_assert(R % P == 0, "rows per wave must hold whole units");
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int g = blockIdx.y;
    constexpr int upw = R / P;               // units per wave
    // One-column kernels (decode): the kernel arguments that the set-up
    // below reads, fetched in one round.  The empty asm takes them all, so
    // the compiler issues their loads together instead of one wait per
    // branch that reads one.  (Not for several columns: there the asm turns
    // the grouped path's column-offset read into a vector load, which
    // measured slower on the MoE layer.)
    if constexpr (M == 1)
        asm volatile("" ::"s"(a.col_off), "s"(a.m), "s"(a.n), "s"(a.k), "s"(a.wq), "s"(a.wd),
                     "s"(a.ffn), "s"(PRO != PRO_NONE ? (const void*)a.xf : (const void*)a.xq));

    const int64_t nunits = (EPI == EPI_SWIGLU) ? a.ffn : (EPI == EPI_QKV ? a.n / 2 : a.n);
    const int64_t wg_unit0 = (int64_t)blockIdx.x * 4 * upw;
    const int64_t unit0 = wg_unit0 + (int64_t)wave * upw;

    int c0 = 0, nc = a.m;
    if (a.col_off) {   // uniform over the workgroup: keep them (and what they index) scalar
        c0 = __builtin_amdgcn_readfirstlane(a.col_off[g]);
        nc = __builtin_amdgcn_readfirstlane(a.col_off[g + 1]) - c0;
    }
    if (nc <= 0) return;   // uniform over the workgroup
    if (a.skip_cols_ge > 0 && nc >= a.skip_cols_ge) return;   // the grouped MFMA GEMM's share

    const int64_t k = a.k, nb = k / QBLK;
    constexpr uint32_t BB = FMT == FMT_Q2_ROW ? 8u : 16u;   // weight bytes per 32-block
    const uint32_t rowb = (uint32_t)nb * BB;
    const double* theta = a.rope_theta;   // read in place from the kernel arguments
    const uint8_t* __restrict__ wq = a.wq + (int64_t)g * a.wq_gstride;
    const uint16_t* __restrict__ wd = a.wd + (int64_t)g * a.wd_gstride;
    const float* __restrict__ wr = FMT != FMT_Q4_0 ? a.wr + (int64_t)g * a.wr_gstride : nullptr;

    // physical row of register row j (j = unit * P + part)
    const int64_t ffn = a.ffn;
    auto prow = [=](int j) -> int64_t {
        const int64_t unit = unit0 + j / P;
        const int p = j % P;
        return (EPI == EPI_SWIGLU) ? unit + p * ffn : (EPI == EPI_QKV ? 2 * unit + p : unit);
    };
    auto rvalid = [=](int j) -> bool { return unit0 + j / P < nunits; };

    // LDS: activation codes [M][k], scales [M][nb] (fp32), then the argmax
    // slots [M][4 RMAX]
    int8_t* lxq = reinterpret_cast<int8_t*>(smem);
    float* lxd = reinterpret_cast<float*>(smem + (size_t)M * k);
    double* ltail = reinterpret_cast<double*>(smem + (((size_t)M * k + (size_t)M * nb * 4 + 7) & ~(size_t)7));

    // Weight registers.  When the row share fits one step (!KLOOP) they are
    // loaded by the first column pass and kept for the others, so a group
    // with more columns than one pass takes reads its weights once (the
    // loads are non-temporal: a second pass would fetch them again).  The
    // first pass is a separate instantiation of the pass body, so that its
    // loads stay in one basic block and issue in the order written.
    uint4 w[RMAX][U];
    uint16_t dwh[RMAX][U];   // fp16 block scales (Q4_0), converted where used
    auto pass = [&](const int cc, auto first, auto mt) __attribute__((always_inline)) {
        constexpr int MM = decltype(mt)::value;   // columns of this pass
        constexpr int NN = RMAX * MM;             // sums per lane in the reduction
        constexpr bool load_now = decltype(first)::value || KLOOP;
        const int mc = nc - cc < MM ? nc - cc : MM;
        float drs[RMAX];     // row scales (row-scaled formats), loaded by every pass
        int xr[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int col = cc + m < nc ? cc + m : nc - 1;  // clamp: extra columns are discarded
            xr[m] = a.col_idx ? __builtin_amdgcn_readfirstlane(a.col_idx[c0 + col]) : c0 + col;
        }

        // 32-bit offsets from the (uniform) matrix base: one matrix is below
        // 4 GiB.  The loads are unconditional, so that all of a step's loads
        // issue before anything waits: a row past the matrix or a block past
        // the row reads row 0 / block 0 instead, and those values are never
        // used (the dot loop stops at the row's last block and rows past the
        // matrix are not stored).
        auto load_w = [&](int64_t b0) {
#pragma unroll
            for (int j = 0; j < RMAX; ++j) {
                const uint32_t row = rvalid(j) ? (uint32_t)prow(j) : 0u;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    uint32_t b = (uint32_t)b0 + u * WAVE + lane;
                    b = b < (uint32_t)nb ? b : 0u;
                    if (FMT == FMT_Q2_ROW) {
                        const uint2 v = load_stream8(wq + (row * rowb + b * BB));
                        w[j][u] = make_uint4(v.x, v.y, 0u, 0u);
                    } else {
                        w[j][u] = load_stream16(wq + (row * rowb + b * BB));
                    }
                    if (FMT == FMT_Q4_0)
                        dwh[j][u] = *reinterpret_cast<const uint16_t*>(
                            reinterpret_cast<const char*>(wd) + (row * (uint32_t)nb + b) * 2u);
                }
            }
        };
        auto load_rs = [&]() {
#pragma unroll
            for (int j = 0; j < RMAX; ++j) drs[j] = FMT != FMT_Q4_0 ? wr[rvalid(j) ? prow(j) : 0] : 0.0f;
        };

        // QKV epilogue inputs of the sum this lane will own (its column's
        // position and its RoPE pair's base frequency), read before the
        // activation row so that they arrive while the row is awaited rather
        // than after the reductions.  Lanes that own no sum read column c0 + cc
        // and pair 0 and discard them.
        int qpos = 0;
        double qtheta = 0.0;
        if constexpr (EPI == EPI_QKV) {
            constexpr int NVR = NN >= 4 ? NN / 4 : 1;
            const int rr = row_sums_base<NN>(lane) + (NVR > 1 ? (lane & 15) : 0);
            const bool ok = rr < NN && cc + rr / RMAX < nc;
            qpos = a.pos[c0 + cc + (ok ? rr / RMAX : 0)];
            const int64_t row0 = 2 * (unit0 + (ok ? rr % RMAX : 0) / 2);
            qtheta = theta[(row0 % a.hd) / 2];
        }
        // Likewise the residual that this lane adds in the store epilogue.
        // y may equal the residual: each element is read and then written by
        // the lane that owns its sum, and no two lanes own one.
        float rres = 0.0f;
        if (EPI == EPI_STORE && a.residual) {
            constexpr int NVR = NN >= 4 ? NN / 4 : 1;
            const int rr = row_sums_base<NN>(lane) + (NVR > 1 ? (lane & 15) : 0);
            const int rm = rr / RMAX, rj = rr % RMAX;
            const bool ok = rr < NN && rvalid(rj) && cc + rm < nc;
            rres = a.residual[(c0 + cc + (ok ? rm : 0)) * a.ldr + (ok ? prow(rj) : 0)];
        }
        if (cc > 0) lds_barrier();   // the previous pass finished reading LDS
        if (PRO != PRO_NONE) {
            RowRegs<KC> Rg;
            load_row<PRO, KC, (EPI == EPI_QKV || PRO == PRO_Q8)>(Rg, a.xf + (int64_t)xr[0] * k, a.gamma, k);
            if constexpr (load_now) load_w(0);
            stage_row<PRO, KC>(Rg, k, a.eps, red, lxq, lxd);
#pragma unroll
            for (int m = 1; m < MM; ++m) {
                if (m >= mc) break;       // uniform over the workgroup
                lds_barrier();            // `red` reused
                load_row<PRO, KC>(Rg, a.xf + (int64_t)xr[m] * k, a.gamma, k);
                stage_row<PRO, KC>(Rg, k, a.eps, red, lxq + (size_t)m * k, lxd + (size_t)m * nb);
            }
        } else {
            // copy the Q8_0 columns into LDS: the first XREG chunks per thread
            // are loaded before the weights, the rest after
            constexpr int XREG = MM == 1 ? 2 : (MM == 2 ? 3 : 6);   // up to K = 6144 staged early
            // 16-byte chunks per column, chunk counts of the pass (32-bit:
            // K and the column count are small)
            const uint32_t c16 = (uint32_t)k / 16u, unb = (uint32_t)nb;
            const uint32_t tot = (uint32_t)mc * c16, totd = (uint32_t)mc * unb;
            // activation row of pass column m (m < mc), looked up per use (the
            // lookups are unconditional, so they issue together)
            const int32_t* __restrict__ cidx = a.col_idx;
            auto col_row = [=](uint32_t m) -> int64_t {
                const int col = c0 + cc + (int)m;
                return cidx ? (int64_t)cidx[col] : (int64_t)col;
            };
            const uint32_t id = threadIdx.x < totd ? threadIdx.x : 0u;
            const uint32_t md = col_of<MM>(id, unb);
            uint16_t xdh;
            if constexpr (load_now && !KLOOP) {
            // (the loads are unconditional, so that none of them waits for
            // another: a thread past the end reloads chunk 0 and stores nothing)
            uint4 xs[XREG];
#pragma unroll
            for (int p = 0; p < XREG; ++p) {
                uint32_t i = threadIdx.x + (uint32_t)p * 256u;
                i = i < tot ? i : 0u;
                const uint32_t m = col_of<MM>(i, c16);
                xs[p] = *reinterpret_cast<const uint4*>(a.xq + col_row(m) * k + (i - m * c16) * 16u);
            }
            xdh = a.xd[col_row(md) * nb + (id - md * unb)];
            load_w(0);
            if (FMT != FMT_Q4_0) load_rs();
#pragma unroll
            for (int p = 0; p < XREG; ++p) {   // a thread past the end rewrites chunk 0 with itself
                uint32_t i = threadIdx.x + (uint32_t)p * 256u;
                i = i < tot ? i : 0u;
                const uint32_t m = col_of<MM>(i, c16);
                *reinterpret_cast<uint4*>(lxq + (size_t)m * k + (i - m * c16) * 16u) = xs[p];
            }
            for (uint32_t i = threadIdx.x + (uint32_t)XREG * 256u; i < tot; i += 256u) {
                const uint32_t m = col_of<MM>(i, c16);
                *reinterpret_cast<uint4*>(lxq + (size_t)m * k + (i - m * c16) * 16u) =
                    *reinterpret_cast<const uint4*>(a.xq + col_row(m) * k + (i - m * c16) * 16u);
            }
            } else {   // later passes (weights in registers already), or rows of several steps
            xdh = a.xd[col_row(md) * nb + (id - md * unb)];
            if constexpr (load_now) load_w(0);
            if (FMT != FMT_Q4_0) load_rs();
            for (uint32_t i = threadIdx.x; i < tot; i += 256u) {
                const uint32_t m = col_of<MM>(i, c16);
                *reinterpret_cast<uint4*>(lxq + (size_t)m * k + (i - m * c16) * 16u) =
                    *reinterpret_cast<const uint4*>(a.xq + col_row(m) * k + (i - m * c16) * 16u);
            }
            }
            lxd[id] = h2f(xdh);
            for (uint32_t i = threadIdx.x + 256u; i < totd; i += 256u) {
                const uint32_t m = col_of<MM>(i, unb);
                lxd[i] = h2f(a.xd[col_row(m) * nb + (i - m * unb)]);
            }
        }
        lds_barrier();

        double acc[RMAX][MM];
#pragma unroll
        for (int j = 0; j < RMAX; ++j)
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[j][m] = 0.0;

        for (int64_t b0 = 0; b0 < nb; b0 += (int64_t)WAVE * U) {
            if (KLOOP && b0 > 0) load_w(b0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t b = b0 + u * WAVE + lane;
                if (b >= nb) break;
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const int8_t* xp = lxq + (size_t)m * k + b * QBLK;
                    const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
                    const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 16);
                    const float dx = lxd[(size_t)m * nb + b];
                    const int s0 = (FMT == FMT_Q2_ROW ? -2 : -8) * byte_sum(x0, x1);
#pragma unroll
                    for (int j = 0; j < RMAX; ++j) {
                        if (FMT == FMT_Q4_0) {
                            // dw * dx is exact in fp32 (two fp16 values); times
                            // the int32 block dot it is exact in fp64
                            const int sdot = dot_block(w[j][u], x0, x1, s0);
                            acc[j][m] = fma((double)(h2f(dwh[j][u]) * dx), (double)sdot, acc[j][m]);
                        } else {
                            const int sdot = FMT == FMT_Q2_ROW ? dot_block2(w[j][u], x0, x1, s0)
                                                               : dot_block(w[j][u], x0, x1, s0);
                            acc[j][m] = fma((double)dx, (double)sdot, acc[j][m]);
                        }
                    }
                }
            }
            if (!KLOOP) break;
        }

        // all row/column sums of the wave at once; value index r = m * RMAX + j
        double v[NN];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int j = 0; j < RMAX; ++j) v[m * RMAX + j] = acc[j][m];
        const int base = row_sums<NN>(v, lane);
        // this lane's sum (index r) and, for two-row units, the unit's other
        // row (index r ^ 1: the same lane when a row holds several sums, else
        // the lane that differs in the last halving bit)
        constexpr int NV = NN >= 4 ? NN / 4 : 1;
        const int kk = NV > 1 ? (lane & 15) : 0;
        double s = v[0], s2 = 0.0;
#pragma unroll
        for (int q = 1; q < NV; ++q)
            if (kk == q) s = v[q];
        if (P == 2) {
            if (NV > 1) {
                s2 = v[0];
#pragma unroll
                for (int q = 1; q < NV; ++q)
                    if ((kk ^ 1) == q) s2 = v[q];
            } else {
                s2 = __shfl_xor(s, NN == 4 ? 16 : 32, WAVE);
            }
        }
        const int r = base + kk;
        const int m = r / RMAX, j = r % RMAX;
        if (FMT != FMT_Q4_0) {   // the row scales, applied once to the row totals
            float d1 = drs[0], d2 = drs[0];
#pragma unroll
            for (int q = 1; q < RMAX; ++q) {
                if (j == q) d1 = drs[q];
                if ((j ^ 1) == q) d2 = drs[q];
            }
            s *= (double)d1;
            if (P == 2) s2 *= (double)d2;
        }
        constexpr int OWN = NN >= 4 ? 16 : (NN == 2 ? 32 : 64);   // lanes sharing one row's sums
        const bool owner = (NV > 1 ? kk < NV : (lane & (OWN - 1)) == 0) && rvalid(j) && cc + m < nc;
        const int64_t row = prow(j);
        const int64_t ocol = c0 + cc + m;

        if (EPI == EPI_STORE) {
            if (owner) {
                float o = (float)s;
                if (a.residual) o = rres + o;   // read at the start of the pass
                a.y[ocol * a.ldy + row] = o;
            }
        } else if (EPI == EPI_SWIGLU || EPI == EPI_QKV) {
            if (owner && (j % 2) == 0) {
                const int64_t unit = unit0 + j / 2;
                if (EPI == EPI_SWIGLU) {
                    a.y[ocol * a.ldy + unit] = swiglu1((float)s, (float)s2);
                } else {
                    // RoPE angle of this pair in fp64, computed here where the
                    // weight registers are free
                    const int64_t row0 = 2 * unit;
                    const int p = qpos;   // a.pos[ocol], read at the start of the pass
                    double c = 1.0, sn = 0.0;
                    if (row0 < a.q_rows + a.kv_rows)
                        rope_sincos((double)p * qtheta, sn, c);
                    const double x1 = (double)(float)s, x2 = (double)(float)s2;
                    if (row0 < a.q_rows) {
                        a.q_out[ocol * a.q_rows + row0] = (float)(x1 * c - x2 * sn);
                        a.q_out[ocol * a.q_rows + row0 + 1] = (float)(x1 * sn + x2 * c);
                    } else if (p >= 0) {   // ring row p % cap
                        const bool is_k = row0 < a.q_rows + a.kv_rows;
                        const int64_t rr = row0 - a.q_rows - (is_k ? 0 : a.kv_rows);
                        const int64_t gh = rr / a.hd, d = rr % a.hd;
                        const int64_t dst = (((int64_t)a.seq[ocol] * a.n_kv + gh) * a.cap + p % a.cap) * a.hd + d;
                        uint16_t* cache = is_k ? a.kc : a.vc;
                        const float o1 = (float)(is_k ? x1 * c - x2 * sn : x1);
                        const float o2 = (float)(is_k ? x1 * sn + x2 * c : x2);
                        cache[dst] = f2h(o1);
                        cache[dst + 1] = f2h(o2);
                    }
                }
            }
        } else {  // EPI_ARGMAX: logits, then the workgroup's best (value, lowest row) per column
            constexpr int SLOTS = 4 * RMAX;
            float* bv = reinterpret_cast<float*>(ltail);
            int* bi = reinterpret_cast<int*>(bv + M * SLOTS);
            for (int i = threadIdx.x; i < M * SLOTS; i += 256) {
                bv[i] = -INFINITY;
                bi[i] = INT32_MAX;
            }
            lds_barrier();
            if (owner) {
                const float o = (float)s;
                a.y[ocol * a.ldy + row] = o;
                bv[m * SLOTS + wave * RMAX + j] = o;
                bi[m * SLOTS + wave * RMAX + j] = (int)row;
            }
            lds_barrier();
            if ((int)threadIdx.x < mc) {
                const int mm = threadIdx.x;
                float best = -INFINITY;
                int besti = INT32_MAX;
                for (int sl = 0; sl < SLOTS; ++sl) {
                    const float o = bv[mm * SLOTS + sl];
                    const int i = bi[mm * SLOTS + sl];
                    if (o > best || (o == best && i < besti)) {
                        best = o;
                        besti = i;
                    }
                }
                a.part_val[(int64_t)(cc + mm) * gridDim.x + blockIdx.x] = best;
                a.part_idx[(int64_t)(cc + mm) * gridDim.x + blockIdx.x] = besti;
            }
        }
    };
    using MFull = std::integral_constant<int, M>;
    if constexpr (KLOOP || PRO != PRO_NONE) {
        // (fused-prologue kernels keep loading per pass: their own row
        // staging must come first, and their passes are rare)
        for (int cc = 0; cc < nc; cc += M) pass(cc, std::true_type{}, MFull{});
    } else {
        // A two-column kernel runs a pass with one column left (an expert
        // with an odd token count) as a one-column body: the dots and the
        // scaling of a padding column are not done.
        auto run = [&](const int cc, auto first) __attribute__((always_inline)) {
            if constexpr (M == 2) {
                if (nc - cc == 1) {   // uniform over the workgroup
                    pass(cc, first, std::integral_constant<int, 1>{});
                    return;
                }
            }
            pass(cc, first, MFull{});
        };
        run(0, std::true_type{});
        for (int cc = M; cc < nc; cc += M) run(cc, std::false_type{});
    }
}

template <int M, int R, int U, int EPI, int PRO, int KC, bool KLOOP>
__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a) {
    gemv_body<FMT_Q4_0, M, R, U, EPI, PRO, KC, KLOOP>(a);
}

// Row-scaled int4 / int2 weights: no prologue, store or SwiGLU epilogue.
template <int FMT, int M, int R, int U, int EPI, bool KLOOP>
__global__ __launch_bounds__(256) void k_gemv_rowq(const GemvArgs a) {
    gemv_body<FMT, M, R, U, EPI, PRO_NONE, 1, KLOOP>(a);
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
    // eight partials per thread per round, their loads issued together
    // (indexes clamped into the column; the extra ones are not compared)
    for (int64_t i0 = 0; i0 < nparts; i0 += 8 * 256) {
        float v[8];
        int j[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + u * 256 + threadIdx.x;
            const int64_t ic = i < nparts ? i : 0;
            v[u] = pv[c * nparts + ic];
            j[u] = pi[c * nparts + ic];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (i0 + u * 256 + threadIdx.x < nparts && (v[u] > bv || (v[u] == bv && j[u] < bi))) {
                bv = v[u];
                bi = j[u];
            }
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

int pick_m(int64_t cols) { return cols <= 1 ? 1 : (cols <= 2 ? 2 : (cols <= 4 ? 4 : 8)); }

size_t stage_bytes(int M, int64_t k) {
    return (((size_t)M * k + (size_t)M * (k / QBLK) * 4) + 7) & ~(size_t)7;
}

// Physical rows per wave, at most four (two for 4 or 8 columns per pass, or
// for Q4_0 rows longer than 64 blocks behind a fused prologue: four rows
// measured slower for the decode down projection, while the grouped SwiGLU
// GEMV of the MoE layer, without a prologue, gained 5% from them).
// Kernels that stage their activations with a fused prologue (RMSNorm or
// Q8_0 of an fp32 row) take the most rows allowed, so that fewer workgroups
// repeat the prologue: on the 22-layer decode step this measured 5% faster
// than one unit per wave for the QKV and down projections, and eight rows
// per wave measured slower again.  The others run one unit per wave until
// the launch has more than 8192 units, then two, then four: small per-wave
// work and many waves keep the most loads in flight per CU.
int pick_rows(int epi, int pro, int M, int64_t k, int64_t units, int fmt = FMT_Q4_0) {
    const int P = rows_per_unit(epi);
    const int cap = (M <= 2 && (k / QBLK <= WAVE || fmt != FMT_Q4_0 || pro == PRO_NONE)) ? 4 : 2;
    int upw = units > 2 * 8192 ? 4 : (units > 8192 ? 2 : 1);
    if (pro != PRO_NONE) upw = 4;
    while (upw * P > cap) upw /= 2;
    return std::max(1, upw) * P;
}

size_t lds_bytes(int epi, int M, int64_t k, int rows) {
    size_t b = stage_bytes(M, k);
    if (epi == EPI_ARGMAX) b += (size_t)M * 4 * rows * 8;
    return b;
}

constexpr size_t LDS_LIMIT = 64 * 1024;

int64_t units_of(const GemvArgs& a, int epi) {
    return epi == EPI_SWIGLU ? a.ffn : (epi == EPI_QKV ? a.n / 2 : a.n);
}

// columns per pass: what the groups need on average, capped by LDS
int pick_cols(const GemvArgs& a, int epi) {
    int M = pick_m(a.max_cols);
    while (M > 1 && lds_bytes(epi, M, a.k, 4) > LDS_LIMIT) M /= 2;
    return M;
}

template <int FMT, int M, int R, int U, int EPI, int PRO, int KC, bool KLOOP>
void launch_cfg(const GemvArgs& a, hipStream_t s) {
    const int64_t units = units_of(a, EPI);
    const int64_t per_wg = 4 * (int64_t)(R / rows_per_unit(EPI));
    dim3 grid((unsigned)((units + per_wg - 1) / per_wg), (unsigned)a.groups);
    if constexpr (FMT == FMT_Q4_0) {
        hipLaunchKernelGGL((k_gemv<M, R, U, EPI, PRO, KC, KLOOP>), grid, dim3(256),
                           lds_bytes(EPI, M, a.k, R), s, a);
    } else {
        static_assert(PRO == PRO_NONE && (EPI == EPI_STORE || EPI == EPI_SWIGLU),
                      "row-scaled weights: no prologue, store or SwiGLU epilogue");
        hipLaunchKernelGGL((k_gemv_rowq<FMT, M, R, U, EPI, KLOOP>), grid, dim3(256),
                           lds_bytes(EPI, M, a.k, R), s, a);
    }
}

template <int FMT, int M, int U, int EPI, int PRO, int KC, bool KLOOP>
void launch_r(const GemvArgs& a, hipStream_t s) {
    constexpr int P = rows_per_unit(EPI);
    const int R = pick_rows(EPI, PRO, M, a.k, units_of(a, EPI) * a.groups, FMT);
    if constexpr (M <= 2) {
        if (R >= 4) { launch_cfg<FMT, M, 4, U, EPI, PRO, KC, KLOOP>(a, s); return; }
    }
    if constexpr (P == 1) {
        if (R == 1) { launch_cfg<FMT, M, 1, U, EPI, PRO, KC, KLOOP>(a, s); return; }
    }
    launch_cfg<FMT, M, 2, U, EPI, PRO, KC, KLOOP>(a, s);
}

// Prologue chunks (2048 values each) held in registers: one for K <= 2048.
template <int FMT, int M, int U, int EPI, int PRO, bool KLOOP>
void launch_kc(const GemvArgs& a, hipStream_t s) {
    if constexpr (PRO == PRO_NONE) {
        launch_r<FMT, M, U, EPI, PRO, 1, KLOOP>(a, s);
    } else {
        if (a.k <= 2048) launch_r<FMT, M, U, EPI, PRO, 1, KLOOP>(a, s);
        else launch_r<FMT, M, U, EPI, PRO, PRO_CHUNKS, KLOOP>(a, s);
    }
}

// Blocks per lane per step: one for K <= 2048, three up to K = 6144 (one
// step either way); longer rows (no prologue) loop over steps of three.
template <int FMT, int M, int EPI, int PRO>
void launch_u(const GemvArgs& a, hipStream_t s) {
    const int64_t nb = a.k / QBLK;
    if (nb <= WAVE) {
        launch_kc<FMT, M, 1, EPI, PRO, false>(a, s);
    } else if (nb <= 3 * WAVE) {
        launch_kc<FMT, M, 3, EPI, PRO, false>(a, s);
    } else {
        if constexpr (PRO == PRO_NONE && (EPI == EPI_STORE || EPI == EPI_SWIGLU))
            launch_kc<FMT, M, 3, EPI, PRO, true>(a, s);
    }
}

template <int EPI, int PRO, int FMT = FMT_Q4_0>
void launch_m(const GemvArgs& a, hipStream_t s) {
    switch (pick_cols(a, EPI)) {
        case 1: launch_u<FMT, 1, EPI, PRO>(a, s); break;
        case 2: launch_u<FMT, 2, EPI, PRO>(a, s); break;
        case 4: launch_u<FMT, 4, EPI, PRO>(a, s); break;
        default: launch_u<FMT, 8, EPI, PRO>(a, s); break;
    }
}

}  // namespace

bool gemv_fits(int64_t k) { return lds_bytes(EPI_ARGMAX, 1, k, 2) <= LDS_LIMIT; }

bool gemv_prologue_fits(int64_t k, int64_t max_cols) {
    (void)max_cols;
    return k <= (int64_t)PRO_CHUNKS * 2048 && gemv_fits(k);
}

int64_t gemv_argmax_parts(int64_t n, int64_t k, int64_t max_cols) {
    GemvArgs a{};
    a.n = n; a.k = k; a.max_cols = (int32_t)max_cols; a.groups = 1;
    const int M = pick_cols(a, EPI_ARGMAX);
    const int R = pick_rows(EPI_ARGMAX, PRO_RMSNORM, M, k, n);
    const int64_t per_wg = 4 * (int64_t)(M <= 2 ? R : std::min(R, 2));
    return (n + per_wg - 1) / per_wg;
}

int launch_gemv(const GemvArgs& a, int epi, hipStream_t s, int pro) {
    if (!gemv_fits(a.k)) return QK_ESHAPE;
    // one matrix below 4 GiB of nibbles (32-bit offsets in the kernel)
    if ((uint64_t)a.n * (uint64_t)(a.k / 2) >= (1ull << 32)) return QK_ESHAPE;
    if (a.k / QBLK > 3 * WAVE && (pro != PRO_NONE || (epi != EPI_STORE && epi != EPI_SWIGLU)))
        return QK_ESHAPE;
    if (pro != PRO_NONE && !gemv_prologue_fits(a.k, a.max_cols)) return QK_ESHAPE;
    if (epi == EPI_QKV && (a.hd % 2 || a.q_rows % 2 || a.kv_rows % 2)) return QK_ESHAPE;
    if (a.fmt != FMT_Q4_0) {
        if (pro != PRO_NONE || (epi != EPI_STORE && epi != EPI_SWIGLU)) return QK_ESHAPE;
        if (a.fmt == FMT_Q4_ROW) {
            if (epi == EPI_SWIGLU) launch_m<EPI_SWIGLU, PRO_NONE, FMT_Q4_ROW>(a, s);
            else launch_m<EPI_STORE, PRO_NONE, FMT_Q4_ROW>(a, s);
        } else if (a.fmt == FMT_Q2_ROW) {
            if (epi == EPI_SWIGLU) launch_m<EPI_SWIGLU, PRO_NONE, FMT_Q2_ROW>(a, s);
            else launch_m<EPI_STORE, PRO_NONE, FMT_Q2_ROW>(a, s);
        } else {
            return QK_EINVAL;
        }
        return qk_launch_status();
    }
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
    if (m > 8 || !gemv_fits(k)) return launch_gemm(a, EPI_STORE, (hipStream_t)stream);
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
    if (m > 8 || !gemv_fits(k)) return launch_gemm(a, EPI_SWIGLU, (hipStream_t)stream);
    return launch_gemv(a, EPI_SWIGLU, (hipStream_t)stream);
}
