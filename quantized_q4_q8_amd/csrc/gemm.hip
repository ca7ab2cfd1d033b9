// Q4_0 x Q8_0 matmul for many activation columns (prefill), on the int8
// matrix cores (v_mfma_i32_32x32x32_i8, gfx950).
//
// The product is the block form of kenji.blog's llama.cpp guide, section 2.2:
// every 32-element block contributes delta_w * delta_x * (exact int32 dot).
// One MFMA with K = 32 covers exactly one block, so its int32 result is the
// block dot of a 32 x 32 tile of (token, weight row) pairs; the two scales
// are applied right after it and the scaled block dots are summed in fp64.
//
// Tile: a workgroup (4 waves) computes 64 tokens x 128 weight rows; each
// wave 32 tokens x 64 rows as two MFMA tiles (two workgroups share a CU).
// A store-epilogue launch whose grid of such tiles would end on a round of
// the 512 resident slots that is at most half full (the 4 x 512 prefill's
// QKV matmul: 640 workgroups) takes 64-row tiles instead, one MFMA tile per
// wave and three workgroups per CU: prefill 141.2 K -> 142.3 K tokens/s.
// Activations are the MFMA's A operand (rows = tokens) and weights the B
// operand (columns = weight rows), so in the 32 x 32 accumulator a lane owns
// one weight row and 16 tokens and the stores of a register are 32
// consecutive floats of one output row.
// KB = 4 blocks (K = 128) are staged in LDS per step, double-buffered so the
// global loads of step s + 1 are in flight during the MFMAs of step s.  The
// weight nibbles become signed int8 codes once, while they are staged
// ((c + 0x78) ^ 0x80 maps c in [0, 15] to c - 8 with no carry between
// bytes), so every wave reads ready MFMA operands.  The activation scales
// are staged as fp64, which makes each scaled block sum
// fma(isum * dx, dw, acc): isum * dx is exact in fp64 (15 + 11 bits) and the
// fma rounds the exact triple product once.
//
// Grouped (the MoE layer's experts): grid z runs over the groups (or over a
// list of them made on the device), each with its own weights, its columns
// gathered from the sorted (token, expert) pairs and its outputs in the
// pairs' order; groups below a column count are left to the grouped GEMV.
#include "internal.h"

namespace qk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BT = 64;   // tokens per workgroup
constexpr int KB = 4;    // blocks per LDS stage
constexpr int NT = 256;  // threads per workgroup: 4 waves, 2 (tokens) x 2 (rows)
constexpr int STRIDE = KB * QBLK + 16;   // bytes per token / weight row in LDS (padded)
constexpr int A_PER = BT * KB * 2 / NT;  // 16-byte activation chunks per thread and step
static_assert(BT * KB == NT, "one activation scale per thread and step");

template <int BR>
struct __align__(16) Stage {
    int8_t a[BT * STRIDE];      // activation codes
    int8_t b[BR * STRIDE];      // weight codes (signed int8)
    double da[KB][BT];          // activation scales
    float db[KB][BR];           // weight scales
};

// swish(g) * u of fp32 matmul outputs, in fp64, rounded once
__device__ __forceinline__ float swiglu1(float g, float u) {
    const double gd = (double)g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}

__device__ __forceinline__ uint4 nib_codes(const uint4 v, int sh) {
    const uint32_t m4 = 0x0F0F0F0Fu;
    return make_uint4((((v.x >> sh) & m4) + 0x78787878u) ^ 0x80808080u,
                      (((v.y >> sh) & m4) + 0x78787878u) ^ 0x80808080u,
                      (((v.z >> sh) & m4) + 0x78787878u) ^ 0x80808080u,
                      (((v.w >> sh) & m4) + 0x78787878u) ^ 0x80808080u);
}

}  // namespace

template <int EPI, int WR>
__global__ __launch_bounds__(NT, WR == 2 ? 2 : 3) void k_gemm_mfma(const GemvArgs a) {
    static_assert(WR == 2 || (WR == 1 && EPI == EPI_STORE), "SwiGLU tiles hold gate and up rows");
    constexpr int BR = 64 * WR;          // weight rows per workgroup (physical)
    constexpr int B_PER = BR * KB / NT;  // 16-byte weight chunks per thread and step
    constexpr int DB_PER = BR * KB / NT; // weight scales per thread and step
    __shared__ Stage<BR> st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wt = wave >> 1;   // token half of the workgroup tile
    const int wc = wave & 1;    // column half
    const int h = lane >> 5;    // lane half: K bytes [16h, 16h + 16) of a block
    const int j = lane & 31;

    const int64_t k = a.k, nb = k / QBLK, kh = k / 2;
    // grouped: group g = blockIdx.z holds columns cg .. cg + m - 1 (output
    // rows), gathered from activation rows col_idx[c] (or c); its weights
    // sit at g * wq_gstride / g * wd_gstride
    int g = blockIdx.z;
    if (a.group_list) {   // grid z indexes the list of groups to take
        if (g >= __builtin_amdgcn_readfirstlane(a.group_list[0])) return;
        g = __builtin_amdgcn_readfirstlane(a.group_list[1 + g]);
    }
    int64_t cg = 0, m = a.m;
    if (a.col_off) {   // uniform over the workgroup
        cg = __builtin_amdgcn_readfirstlane(a.col_off[g]);
        m = __builtin_amdgcn_readfirstlane(a.col_off[g + 1]) - cg;
        if (m < a.min_cols) return;
    }
    const int64_t t0 = (int64_t)blockIdx.y * BT;
    if (t0 >= m) return;
    const uint8_t* __restrict__ wq = a.wq + (int64_t)g * a.wq_gstride;
    const uint16_t* __restrict__ wd = a.wd + (int64_t)g * a.wd_gstride;
    // activation row of local column t (t < m)
    auto act_row = [&](int64_t t) -> int64_t { return a.col_idx ? (int64_t)a.col_idx[cg + t] : cg + t; };
    // physical weight row of LDS row pr
    const int64_t c0 = (int64_t)blockIdx.x * (EPI == EPI_SWIGLU ? BR / 2 : BR);
    const int64_t nphys = (EPI == EPI_SWIGLU) ? 2 * a.ffn : a.n;
    auto prow_of = [&](int pr) -> int64_t {
        if (EPI == EPI_SWIGLU) return pr < BR / 2 ? c0 + pr : a.ffn + c0 + (pr - BR / 2);
        return c0 + pr;
    };
    auto prow_valid = [&](int pr) -> bool {
        if (EPI == EPI_SWIGLU) return c0 + (pr % (BR / 2)) < a.ffn;
        return c0 + pr < nphys;
    };

    // ---- global -> register staging (per thread and step: A_PER activation
    // chunks, B_PER weight chunks, one activation scale, DB_PER weight scales)
    // The fp16 scales are loaded from clamped indexes with no branch and kept
    // as raw bits plus a validity flag until sstore: a conversion here would
    // make the wave wait for every load of the stage before the MFMAs of the
    // current one could start.
    uint4 ra[A_PER], rb[B_PER];
    uint16_t rdah, rdbh[DB_PER];
    bool rda_ok, rdb_ok[DB_PER];
    // the activation rows this thread stages, looked up once
    int64_t arow[A_PER], srow;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int64_t t = t0 + ((tid + NT * i) >> 3);
        arow[i] = t < m ? act_row(t) : -1;
    }
    {
        const int64_t t = t0 + tid % BT;
        srow = t < m ? act_row(t) : -1;
    }
    auto gload = [&](int64_t kb0) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int idx = tid + NT * i;          // chunks of 16 B: [token][KB*2]
            const int part = idx & 7;
            const int64_t b = kb0 + (part >> 1);
            if (arow[i] >= 0 && b < nb)
                ra[i] = *reinterpret_cast<const uint4*>(a.xq + arow[i] * k + b * QBLK + (part & 1) * 16);
            else
                ra[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int idx = tid + NT * i;          // chunks of 16 B: [row][KB]
            const int pr = idx >> 2, bb = idx & 3;
            const int64_t b = kb0 + bb;
            if (prow_valid(pr) && b < nb)
                rb[i] = *reinterpret_cast<const uint4*>(wq + prow_of(pr) * kh + b * 16);
            else
                rb[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        }
        {
            const int bb = tid / BT;   // activation scales [KB][BT]
            const int64_t b = kb0 + bb;
            rda_ok = srow >= 0 && b < nb;
            rdah = a.xd[rda_ok ? srow * nb + b : 0];
        }
#pragma unroll
        for (int i = 0; i < DB_PER; ++i) {
            const int idx = tid + NT * i;            // weight scales [KB][BR]
            const int bb = idx / BR, r = idx % BR;
            const int64_t b = kb0 + bb;
            rdb_ok[i] = prow_valid(r) && b < nb;
            rdbh[i] = wd[rdb_ok[i] ? prow_of(r) * nb + b : 0];
        }
    };
    auto sstore = [&](Stage<BR>& s) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int idx = tid + NT * i;
            const int tr = idx >> 3, part = idx & 7;
            *reinterpret_cast<uint4*>(s.a + tr * STRIDE + part * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            // block bb of row pr: elements 0..15 from the low nibbles, 16..31
            // from the high ones
            const int idx = tid + NT * i;
            const int pr = idx >> 2, bb = idx & 3;
            *reinterpret_cast<uint4*>(s.b + pr * STRIDE + bb * QBLK) = nib_codes(rb[i], 0);
            *reinterpret_cast<uint4*>(s.b + pr * STRIDE + bb * QBLK + 16) = nib_codes(rb[i], 4);
        }
        s.da[tid / BT][tid % BT] = rda_ok ? (double)h2f(rdah) : 0.0;
#pragma unroll
        for (int i = 0; i < DB_PER; ++i) {
            const int idx = tid + NT * i;
            s.db[idx / BR][idx % BR] = rdb_ok[i] ? h2f(rdbh[i]) : 0.0f;
        }
    };

    double acc[WR][16];
#pragma unroll
    for (int cb = 0; cb < WR; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.0;

    // LDS row (weights) of column tile cb for this wave
    auto lds_col = [&](int cb) -> int {
        if (EPI == EPI_SWIGLU) return cb * (BR / 2) + wc * 32 + j;  // cb 0: gate, 1: up
        return wc * 32 * WR + cb * 32 + j;
    };
    const int tra = wt * 32 + j;   // activation row (token) of this lane's A operand

    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const int64_t nsteps = (nb + KB - 1) / KB;
    gload(0);
    sstore(st[0]);
    __syncthreads();
    for (int64_t s = 0; s < nsteps; ++s) {
        Stage<BR>& cur = st[s & 1];
        if (s + 1 < nsteps) gload((s + 1) * KB);
        // two blocks per iteration: the second one's LDS addresses become
        // immediate offsets (1.9 % on the 4 x 512 prefill; a full unroll of
        // the four spills)
#pragma unroll 2
        for (int bb = 0; bb < KB; ++bb) {
            const uint4 av = *reinterpret_cast<const uint4*>(cur.a + tra * STRIDE + bb * QBLK + h * 16);
            const v4i xa = v4i{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
            v16i isum[WR];
            double dw[WR];
#pragma unroll
            for (int cb = 0; cb < WR; ++cb) {
                const uint4 bv = *reinterpret_cast<const uint4*>(cur.b + lds_col(cb) * STRIDE + bb * QBLK + h * 16);
                isum[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa, v4i{(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w},
                                                                 zero, 0, 0, 0);
                dw[cb] = (double)cur.db[bb][lds_col(cb)];
            }
            // register v is token row 8 (v / 4) + 4 h + (v % 4) of the wave's 32
            double dx[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double2 d0 = *reinterpret_cast<const double2*>(&cur.da[bb][wt * 32 + 8 * q + 4 * h]);
                const double2 d1 = *reinterpret_cast<const double2*>(&cur.da[bb][wt * 32 + 8 * q + 4 * h + 2]);
                dx[4 * q] = d0.x; dx[4 * q + 1] = d0.y; dx[4 * q + 2] = d1.x; dx[4 * q + 3] = d1.y;
            }
#pragma unroll
            for (int cb = 0; cb < WR; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[cb][v] = fma((double)isum[cb][v] * dx[v], dw[cb], acc[cb][v]);
        }
        if (s + 1 < nsteps) sstore(st[(s + 1) & 1]);
        __syncthreads();
    }

    // ---- epilogue: lane j owns weight column lds_col(cb); register v is
    // token row 8 * (v / 4) + 4 * h + (v % 4) of the wave's 32-token tile.
    // The residual values are all read (from clamped indexes) before the
    // first store: y may equal residual, so the compiler could not move a
    // load above an earlier store, and each load would wait on its own.
    // Every element is read and then written by the same lane.
    float rv[WR][16];
    if (EPI == EPI_STORE && a.residual) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t t = t0 + wt * 32 + 8 * (v / 4) + 4 * h + (v % 4);
            const int64_t tc = cg + (t < m ? t : m - 1);
#pragma unroll
            for (int cb = 0; cb < WR; ++cb) {
                const int pr = lds_col(cb);
                const int64_t r = prow_valid(pr) ? prow_of(pr) : 0;
                rv[cb][v] = a.residual[tc * a.ldr + r];
            }
        }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + wt * 32 + 8 * (v / 4) + 4 * h + (v % 4);
        if (t >= m) continue;
        if (EPI == EPI_STORE) {
#pragma unroll
            for (int cb = 0; cb < WR; ++cb) {
                const int pr = lds_col(cb);
                if (!prow_valid(pr)) continue;
                const int64_t r = prow_of(pr);
                float val = (float)acc[cb][v];
                if (a.residual) val = rv[cb][v] + val;
                a.y[(cg + t) * a.ldy + r] = val;
            }
        } else {
            const int64_t f = c0 + wc * 32 + j;
            if (f < a.ffn) a.y[(cg + t) * a.ldy + f] = swiglu1((float)acc[0][v], (float)acc[1][v]);
        }
    }
}

int launch_gemm(const GemvArgs& a, int epi, hipStream_t s, int64_t max_group_cols,
                int64_t max_groups) {
    const int64_t cols = a.col_off ? max_group_cols : (int64_t)a.m;
    const unsigned gt = (unsigned)((cols + BT - 1) / BT);
    const unsigned gz = !a.col_off ? 1u : (a.group_list ? (unsigned)max_groups : (unsigned)a.groups);
    if (gt == 0 || gz == 0) return QK_OK;
    if (epi == EPI_SWIGLU) {
        constexpr int BR = 128;
        dim3 grid((unsigned)((a.ffn + BR / 2 - 1) / (BR / 2)), gt, gz);
        hipLaunchKernelGGL((k_gemm_mfma<EPI_SWIGLU, 2>), grid, dim3(NT), 0, s, a);
    } else {
        // 128-row tiles, unless their grid would end on a round of the 512
        // resident slots (two per CU) that is at most half full
        const int64_t wg2 = (a.n + 127) / 128 * (int64_t)gt * gz;
        const int64_t tail = wg2 % 512;
        if (tail > 0 && tail <= 256) {
            dim3 grid((unsigned)((a.n + 63) / 64), gt, gz);
            hipLaunchKernelGGL((k_gemm_mfma<EPI_STORE, 1>), grid, dim3(NT), 0, s, a);
        } else {
            dim3 grid((unsigned)((a.n + 127) / 128), gt, gz);
            hipLaunchKernelGGL((k_gemm_mfma<EPI_STORE, 2>), grid, dim3(NT), 0, s, a);
        }
    }
    return qk_launch_status();
}

}  // namespace qk
