// Grouped Q4_0 x Q8_0 expert GEMV of the MoE layer: every selected expert's
// weight matrix times the few activation columns (tokens) routed to it.
//
// The product is the block form of kenji.blog's llama.cpp guide, section 2.2
// (per 32-block: delta_w * delta_x * the exact int32 dot of the codes),
// applied per expert as in Colibri's token flow (step 5: each selected
// expert's FFN on the tokens routed to it).
//
// Design.  An expert's weights are read once and serve a handful of columns,
// so the work is a stream of weight bytes with little arithmetic per byte and
// what bounds it is how many of those bytes each CU keeps in flight.  A
// workgroup takes one expert (grid y) and a strided share of its row groups
// (grid x).  It stages the expert's activation columns in LDS once: the
// codes, and per block the fp32 scale and -8 * (sum of the codes), which
// applies the nibble offset to the integer dot.  It then walks its row
// groups with two register sets of weights: the next group's loads are issued
// before the current group's dots, so a wave has loads in flight across its
// whole share rather than only until its first group arrives.  Within a row
// group the arithmetic is that of the decode GEMV: lane i takes blocks
// i, i + 64, i + 128 of each row, a block's sum is scaled in fp64 as
// fma(dw * dx, isum, acc) (dw * dx is exact in fp32 and the product exact in
// fp64, so each block adds with one rounding), columns go two at a time (a
// last odd column alone) and the wave's row sums are reduced together.
//
// Row-scaled int4 / int2 experts (the row-scaled codec) take the same path:
// no per-block weight scale (a block sum is dx * isum, in fp64), and the
// row's fp32 scale multiplies the row's total once, after the reduction;
// int2 blocks are 8 bytes with the -2 offset.
#include "internal.h"
#include "qdot.h"

#include <type_traits>

namespace qk {

namespace {

// Workgroups per expert (grid x): on the 64-token, 256-expert layer (about
// 223 experts with tokens) 32 measured faster than 16 (8 % of the layer) and
// 64 (3 %), 8 slower by 11 %.
constexpr int XWG = 32;
constexpr size_t XLDS = 40 * 1024;    // LDS budget of the staged columns per workgroup

// EPI_SWIGLU: units are (gate row f, up row ffn + f), output y[col][f];
// EPI_STORE: units are rows, output y[col][row].  U blocks per lane and row
// (K <= 64 U blocks), UPW units per wave and row group.  FMT: FMT_Q4_0
// (fp16 scale per block) or FMT_Q4_ROW / FMT_Q2_ROW (fp32 scale per row).
// Register budget: two workgroups per CU; the one-block down rows (128
// VGPRs) four.
template <int FMT, int EPI, int U, int UPW>
__global__ __launch_bounds__(256, (U == 1 && EPI == EPI_STORE) ? 4 : 2) void k_expert_gemv(const GemvArgs a,
                                                                                            int mcols) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int P = EPI == EPI_SWIGLU ? 2 : 1;
    constexpr int R = UPW * P;   // rows per wave and row group
    static_assert(R == 2 || R == 4 || R == 8, "two to eight rows per wave");
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int g = blockIdx.y;
    // the expert's columns, uniform over the workgroup
    const int c0 = __builtin_amdgcn_readfirstlane(a.col_off[g]);
    const int nc = __builtin_amdgcn_readfirstlane(a.col_off[g + 1]) - c0;
    if (nc <= 0) return;
    if (a.skip_cols_ge > 0 && nc >= a.skip_cols_ge) return;   // the grouped MFMA GEMM's share
    const int64_t units = EPI == EPI_SWIGLU ? a.ffn : a.n;
    constexpr int PER_IT = 4 * UPW;   // units per workgroup and row group
    const int n_it = (int)((units + PER_IT - 1) / PER_IT);
    if ((int)blockIdx.x >= n_it) return;

    constexpr uint32_t BB = FMT == FMT_Q2_ROW ? 8u : 16u;   // weight bytes per block
    constexpr int OFF = FMT == FMT_Q2_ROW ? -2 : -8;          // code offset of the weights
    const uint32_t k = (uint32_t)a.k, nb = k / QBLK, rowb = nb * BB;
    const uint8_t* __restrict__ wq = a.wq + (int64_t)g * a.wq_gstride;
    const uint16_t* __restrict__ wd = FMT == FMT_Q4_0 ? a.wd + (int64_t)g * a.wd_gstride : nullptr;
    const float* __restrict__ wr = FMT != FMT_Q4_0 ? a.wr + (int64_t)g * a.wr_gstride : nullptr;
    // LDS: codes [mcols][k], then per (column, block) the fp32 scale's bits
    // and OFF * the block's code sum
    int8_t* lxq = reinterpret_cast<int8_t*>(smem);
    int2* lsx = reinterpret_cast<int2*>(smem + (size_t)mcols * k);
    const int64_t ffn = a.ffn;

    // physical row of register row j in row group it, or -1 past the matrix
    auto prow = [&](int it, int j) -> int64_t {
        const int64_t unit = (int64_t)it * PER_IT + wave * UPW + j / P;
        if (unit >= units) return -1;
        return EPI == EPI_SWIGLU ? unit + (j % P) * ffn : unit;
    };
    // 32-bit offsets from the expert's matrix (below 4 GiB).  Unconditional,
    // so that a group's loads all issue before anything waits: rows past the
    // matrix and blocks past the row read row 0 / block 0, never used.
    // A block's fp16 scale is read as the aligned 32-bit word that holds it
    // (its half picked where it is used): 16-bit loads let the compiler pack
    // two scales into one register as they arrive, which waits on them, and
    // so on every load before them, in the middle of the next group's loads.
    // Row-scaled weights keep the row's fp32 scale in d[j][0].
    auto load = [&](uint4 (&w)[R][U], uint32_t (&d)[R][U], int it) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t pr = prow(it, j);
            const uint32_t row = pr >= 0 ? (uint32_t)pr : 0u;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t b = (uint32_t)(u * WAVE + lane);
                b = b < nb ? b : 0u;
                if (FMT == FMT_Q2_ROW) {
                    const uint2 v = load_stream8(wq + (row * rowb + b * BB));
                    w[j][u] = make_uint4(v.x, v.y, 0u, 0u);
                } else {
                    w[j][u] = load_stream16(wq + (row * rowb + b * BB));
                }
                if (FMT == FMT_Q4_0)
                    d[j][u] = *reinterpret_cast<const uint32_t*>(
                        reinterpret_cast<const char*>(wd) + (((row * nb + b) * 2u) & ~3u));
                else if (u == 0)
                    d[j][0] = __builtin_bit_cast(uint32_t, wr[row]);
            }
        }
    };
    // the scale of register row j's block u from its 32-bit word
    auto scale = [&](const uint32_t (&d)[R][U], int it, int j, int u) -> float {
        const int64_t pr = prow(it, j);
        const uint32_t row = pr >= 0 ? (uint32_t)pr : 0u;
        const uint32_t b = (uint32_t)(u * WAVE + lane);
        return h2f((uint16_t)(d[j][u] >> (((row * nb + b) & 1u) * 16u)));
    };
    // columns [cs, cs + ncs) of the expert into LDS
    auto stage = [&](int cs, int ncs) {
        const uint32_t tot = (uint32_t)ncs * nb;
        for (uint32_t i = threadIdx.x; i < tot; i += 256u) {
            const uint32_t m = i / nb, b = i - m * nb;
            const int col = c0 + cs + (int)m;
            const int64_t row = a.col_idx ? (int64_t)a.col_idx[col] : (int64_t)col;
            const int8_t* src = a.xq + row * (int64_t)k + b * QBLK;
            const uint4 x0 = *reinterpret_cast<const uint4*>(src);
            const uint4 x1 = *reinterpret_cast<const uint4*>(src + 16);
            const float dx = h2f(a.xd[row * (int64_t)nb + b]);
            *reinterpret_cast<uint4*>(lxq + (size_t)m * k + b * QBLK) = x0;
            *reinterpret_cast<uint4*>(lxq + (size_t)m * k + b * QBLK + 16) = x1;
            lsx[(size_t)m * nb + b] = make_int2(__builtin_bit_cast(int, dx), OFF * byte_sum(x0, x1));
        }
    };

    // Dots, reduction and epilogue of row group `it` for staged columns
    // m0 .. m0 + MM - 1 (MM = 2, or 1 for a last odd column).
    auto cols = [&](const uint4 (&w)[R][U], const uint32_t (&d)[R][U], int it, int cs, int m0,
                    auto mt) __attribute__((always_inline)) {
        constexpr int MM = decltype(mt)::value;
        constexpr int NN = R * MM;   // sums per lane; index r = m * R + j
        double acc[R][MM];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[j][m] = 0.0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t b = (uint32_t)(u * WAVE + lane);
            if (b >= nb) break;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int8_t* xp = lxq + (size_t)(m0 + m) * k + b * QBLK;
                const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
                const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 16);
                const int2 sx = lsx[(size_t)(m0 + m) * nb + b];
                const float dx = __builtin_bit_cast(float, sx.x);
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    if (FMT == FMT_Q4_0) {
                        const int sdot = dot_block(w[j][u], x0, x1, sx.y);
                        acc[j][m] = fma((double)(scale(d, it, j, u) * dx), (double)sdot, acc[j][m]);
                    } else {
                        const int sdot = FMT == FMT_Q2_ROW ? dot_block2(w[j][u], x0, x1, sx.y)
                                                           : dot_block(w[j][u], x0, x1, sx.y);
                        acc[j][m] = fma((double)dx, (double)sdot, acc[j][m]);
                    }
                }
            }
        }
        double v[NN];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int j = 0; j < R; ++j) v[m * R + j] = acc[j][m];
        const int base = row_sums<NN>(v, lane);
        // this lane's sum (index base + kk) and, for SwiGLU, its unit's up
        // row (index ^ 1: the same lane when a row of lanes holds several
        // sums, else the lane 16 or 32 away)
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
        const int m = r / R, j = r % R;
        if (FMT != FMT_Q4_0) {   // the row scales, applied once to the row totals
            float d1 = __builtin_bit_cast(float, d[0][0]), d2 = d1;
#pragma unroll
            for (int q = 1; q < R; ++q) {
                if (j == q) d1 = __builtin_bit_cast(float, d[q][0]);
                if ((j ^ 1) == q) d2 = __builtin_bit_cast(float, d[q][0]);
            }
            s *= (double)d1;
            if (P == 2) s2 *= (double)d2;
        }
        const int64_t pr = prow(it, j);
        constexpr int OWN = NN >= 4 ? 16 : 32;   // lanes holding one sum
        const bool owner = (NV > 1 ? kk < NV : (lane & (OWN - 1)) == 0) && pr >= 0;
        const int64_t ocol = c0 + cs + m0 + m;
        if (EPI == EPI_STORE) {
            if (owner) a.y[ocol * a.ldy + pr] = (float)s;
        } else if (owner && (j % 2) == 0) {
            a.y[ocol * a.ldy + pr] = swiglu1((float)s, (float)s2);   // pr: the gate row = unit
        }
    };
    auto compute = [&](const uint4 (&w)[R][U], const uint32_t (&d)[R][U], int it, int cs,
                       int ncs) __attribute__((always_inline)) {
        for (int m0 = 0; m0 < ncs; m0 += 2) {
            if (ncs - m0 == 1) cols(w, d, it, cs, m0, std::integral_constant<int, 1>{});
            else cols(w, d, it, cs, m0, std::integral_constant<int, 2>{});
        }
    };

    uint4 wA[R][U], wB[R][U];
    uint32_t dA[R][U], dB[R][U];
    const int it0 = blockIdx.x, step = gridDim.x;
    const int nmy = (n_it - it0 + step - 1) / step;   // row groups of this workgroup (>= 1)
    auto IT = [&](int i) { return it0 + i * step; };
    for (int cs = 0; cs < nc; cs += mcols) {   // one stage unless the expert has > mcols columns
        const int ncs = nc - cs < mcols ? nc - cs : mcols;
        if (cs > 0) __syncthreads();   // the previous stage's columns are no longer read
        // the first group's weights go out first: the staging then waits for
        // them and its own loads together, and the dots start right after
        load(wA, dA, IT(0));
        stage(cs, ncs);
        __syncthreads();
        // pairs of groups with no branch around a load, so that the waits
        // before each group's dots leave the other group's loads in flight;
        // then the last one or two groups
        int i = 0;
        for (; i + 2 < nmy; i += 2) {
            load(wB, dB, IT(i + 1));
            compute(wA, dA, IT(i), cs, ncs);
            load(wA, dA, IT(i + 2));
            compute(wB, dB, IT(i + 1), cs, ncs);
        }
        if (nmy - i == 2) {
            load(wB, dB, IT(i + 1));
            compute(wA, dA, IT(i), cs, ncs);
            compute(wB, dB, IT(i + 1), cs, ncs);
        } else {
            compute(wA, dA, IT(i), cs, ncs);
        }
    }
}

template <int FMT, int EPI, int U, int UPW>
void launch_x(const GemvArgs& a, int mcols, size_t lds, hipStream_t s) {
    const int64_t units = EPI == EPI_SWIGLU ? a.ffn : a.n;
    const int64_t n_it = (units + 4 * UPW - 1) / (4 * UPW);
    dim3 grid((unsigned)std::min<int64_t>(n_it, XWG), (unsigned)a.groups);
    hipLaunchKernelGGL((k_expert_gemv<FMT, EPI, U, UPW>), grid, dim3(256), lds, s, a, mcols);
}

template <int FMT>
void launch_f(const GemvArgs& a, int epi, int64_t nb, int mcols, size_t lds, hipStream_t s) {
    if (epi == EPI_SWIGLU) {
        if (nb <= WAVE) launch_x<FMT, EPI_SWIGLU, 1, 2>(a, mcols, lds, s);
        else launch_x<FMT, EPI_SWIGLU, 3, 1>(a, mcols, lds, s);
    } else {
        if (nb <= WAVE) launch_x<FMT, EPI_STORE, 1, 4>(a, mcols, lds, s);
        else launch_x<FMT, EPI_STORE, 3, 2>(a, mcols, lds, s);
    }
}

}  // namespace

// Q4_0 scales are read as aligned 32-bit words: the array must be 4-byte
// aligned, each expert's scales must start on a word (even stride) and their
// count (n rows of nb blocks) be even, so that the word holding an expert's
// last scale lies inside the expert's scales.
bool expert_gemv_fits(const GemvArgs& a) {
    const int64_t nb = a.k / QBLK;
    const bool scales = a.fmt == FMT_Q4_0 ? (a.wd && QK_ALIGNED(a.wd, 4) && a.wd_gstride % 2 == 0 &&
                                             (a.n * nb) % 2 == 0)
                                          : (a.fmt == FMT_Q4_ROW || a.fmt == FMT_Q2_ROW) && a.wr &&
                                                QK_ALIGNED(a.wr, 4);
    return scales && a.col_off && !a.residual && a.k % QBLK == 0 && nb >= 1 && nb <= 3 * WAVE &&
           QK_ALIGNED(a.xq, 16) && QK_ALIGNED(a.wq, a.fmt == FMT_Q2_ROW ? 8 : 16);
}

int launch_expert_gemv(const GemvArgs& a, int epi, hipStream_t s) {
    if (!expert_gemv_fits(a) || (epi != EPI_SWIGLU && epi != EPI_STORE)) return QK_ESHAPE;
    // one expert's matrix below 4 GiB of weight bytes (32-bit offsets in the kernel)
    const uint64_t rows = epi == EPI_SWIGLU ? 2 * (uint64_t)a.ffn : (uint64_t)a.n;
    if (rows * (uint64_t)(a.k / 2) >= (1ull << 32)) return QK_ESHAPE;
    if (a.groups <= 0) return QK_OK;
    const int64_t nb = a.k / QBLK;
    const size_t per_col = (size_t)a.k + (size_t)nb * 8;
    const int mcols = (int)std::min<size_t>(16, XLDS / per_col);
    if (mcols < 1) return QK_ESHAPE;
    const size_t lds = (size_t)mcols * per_col;
    if (a.fmt == FMT_Q4_0) launch_f<FMT_Q4_0>(a, epi, nb, mcols, lds, s);
    else if (a.fmt == FMT_Q4_ROW) launch_f<FMT_Q4_ROW>(a, epi, nb, mcols, lds, s);
    else launch_f<FMT_Q2_ROW>(a, epi, nb, mcols, lds, s);
    return qk_launch_status();
}

}  // namespace qk
