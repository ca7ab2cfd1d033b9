// Q4_0 x Q8_0 matmul for many activation columns (prefill), on the int8
// matrix cores (v_mfma_i32_32x32x32_i8, gfx950).
//
// The product is the block form of kenji.blog's llama.cpp guide, section 2.2:
// every 32-element block contributes delta_w * delta_x * (exact int32 dot).
// One MFMA with K = 32 covers exactly one block, so its int32 result is the
// block dot of a 32 x 32 tile of (token, weight row) pairs; the two scales
// are applied right after it and the scaled block dots are summed in fp64.
//
// Tile: a workgroup (4 waves) computes 128 tokens x 128 weight rows; each
// wave 64 x 64 as 2 x 2 MFMA tiles.  Activations are the MFMA's A operand
// (rows = tokens) and weights the B operand (columns = weight rows), so in
// the 32 x 32 accumulator a lane owns one weight row and 16 tokens and the
// stores of a register are 32 consecutive floats of one output row.
// KB = 4 blocks (K = 128) are staged in LDS per step, double-buffered so the
// global loads of step s + 1 are in flight during the MFMAs of step s.
// Nibbles become signed int8 codes in registers: (c + 0x78) ^ 0x80 maps
// c in [0, 15] to c - 8 in two's complement with no carry between bytes.
#include "internal.h"

namespace qk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BT = 128;  // tokens per workgroup
constexpr int BR = 128;  // weight rows per workgroup (physical)
constexpr int KB = 4;    // blocks per LDS stage
constexpr int A_STRIDE = KB * QBLK + 16;   // bytes per token row in LDS (padded)
constexpr int B_STRIDE = KB * 16 + 16;     // bytes per weight row in LDS (padded)

struct __align__(16) Stage {
    uint8_t a[BT * A_STRIDE];   // activation codes
    uint8_t b[BR * B_STRIDE];   // weight nibbles
    float da[KB][BT];           // activation scales
    float db[KB][BR];           // weight scales
};

// swish(g) * u of fp32 matmul outputs, in fp64, rounded once
__device__ __forceinline__ float swiglu1(float g, float u) {
    const double gd = (double)g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}

}  // namespace

template <int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(const GemvArgs a) {
    __shared__ Stage st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wt = wave >> 1;   // token half of the workgroup tile
    const int wc = wave & 1;    // column half
    const int h = lane >> 5;    // lane half: K bytes [16h, 16h + 16) of a block
    const int j = lane & 31;

    const int64_t k = a.k, nb = k / QBLK, kh = k / 2;
    const int64_t m = a.m;
    const int64_t t0 = (int64_t)blockIdx.y * BT;
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

    // ---- global -> register staging (per thread: 4 A chunks, 2 B chunks, 2+2 scales)
    uint4 ra[4], rb[2];
    float rda[2], rdb[2];
    auto gload = [&](int64_t kb0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i;         // 1024 chunks of 16 B: [token][KB*2]
            const int tr = idx >> 3, part = idx & 7;
            const int64_t t = t0 + tr;
            const int64_t b = kb0 + (part >> 1);
            if (t < m && b < nb)
                ra[i] = *reinterpret_cast<const uint4*>(a.xq + t * k + b * QBLK + (part & 1) * 16);
            else
                ra[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;         // 512 chunks: [row][KB]
            const int pr = idx >> 2, bb = idx & 3;
            const int64_t b = kb0 + bb;
            if (prow_valid(pr) && b < nb)
                rb[i] = *reinterpret_cast<const uint4*>(a.wq + prow_of(pr) * kh + b * 16);
            else
                rb[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;         // 512 scales: [KB][128]
            const int bb = idx >> 7, r = idx & 127;
            const int64_t b = kb0 + bb;
            const int64_t t = t0 + r;
            rda[i] = (t < m && b < nb) ? h2f(a.xd[t * nb + b]) : 0.0f;
            rdb[i] = (prow_valid(r) && b < nb) ? h2f(a.wd[prow_of(r) * nb + b]) : 0.0f;
        }
    };
    auto sstore = [&](Stage& s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i;
            const int tr = idx >> 3, part = idx & 7;
            *reinterpret_cast<uint4*>(s.a + tr * A_STRIDE + part * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            const int pr = idx >> 2, bb = idx & 3;
            *reinterpret_cast<uint4*>(s.b + pr * B_STRIDE + bb * 16) = rb[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            const int bb = idx >> 7, r = idx & 127;
            s.da[bb][r] = rda[i];
            s.db[bb][r] = rdb[i];
        }
    };

    double acc[2][2][16];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0;

    // LDS row (weights) of column tile cb for this wave
    auto lds_col = [&](int cb) -> int {
        if (EPI == EPI_SWIGLU) return cb * (BR / 2) + wc * 32 + j;  // cb 0: gate, 1: up
        return wc * 64 + cb * 32 + j;
    };

    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const int64_t nsteps = (nb + KB - 1) / KB;
    gload(0);
    sstore(st[0]);
    __syncthreads();
    for (int64_t s = 0; s < nsteps; ++s) {
        Stage& cur = st[s & 1];
        if (s + 1 < nsteps) gload((s + 1) * KB);
#pragma unroll 1
        for (int bb = 0; bb < KB; ++bb) {
            v4i xa[2], wb[2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const int tr = wt * 64 + ta * 32 + j;
                const uint4 v = *reinterpret_cast<const uint4*>(cur.a + tr * A_STRIDE + bb * QBLK + h * 16);
                xa[ta] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const uint4 v = *reinterpret_cast<const uint4*>(cur.b + lds_col(cb) * B_STRIDE + bb * 16);
                const uint32_t m4 = 0x0F0F0F0Fu;
                const int sh = 4 * h;  // lane half 0: elements 0..15 (low nibbles), 1: 16..31
                uint32_t c[4] = {(v.x >> sh) & m4, (v.y >> sh) & m4, (v.z >> sh) & m4, (v.w >> sh) & m4};
#pragma unroll
                for (int q = 0; q < 4; ++q) c[q] = (c[q] + 0x78787878u) ^ 0x80808080u;
                wb[cb] = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
            }
            float dwl[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) dwl[cb] = cur.db[bb][lds_col(cb)];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                float dxa[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 d4 = *reinterpret_cast<const float4*>(
                        &cur.da[bb][wt * 64 + ta * 32 + 8 * q + 4 * h]);
                    dxa[4 * q] = d4.x; dxa[4 * q + 1] = d4.y; dxa[4 * q + 2] = d4.z; dxa[4 * q + 3] = d4.w;
                }
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const v16i isum = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa[ta], wb[cb], zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 16; ++v)   // scale product exact in fp32, term exact in fp64
                        acc[ta][cb][v] = fma((double)(dxa[v] * dwl[cb]), (double)isum[v], acc[ta][cb][v]);
                }
            }
        }
        if (s + 1 < nsteps) {
            sstore(st[(s + 1) & 1]);
        }
        __syncthreads();
    }

    // ---- epilogue: lane j owns weight column lds_col(cb); register v is token
    // row 8 * (v / 4) + 4 * h + (v % 4) of the 32-token tile.
#pragma unroll
    for (int ta = 0; ta < 2; ++ta) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t t = t0 + wt * 64 + ta * 32 + 8 * (v / 4) + 4 * h + (v % 4);
            if (t >= m) continue;
            if (EPI == EPI_STORE) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const int pr = lds_col(cb);
                    if (!prow_valid(pr)) continue;
                    const int64_t r = prow_of(pr);
                    float val = (float)acc[ta][cb][v];
                    if (a.residual) val = a.residual[t * a.ldr + r] + val;
                    a.y[t * a.ldy + r] = val;
                }
            } else {
                const int64_t f = c0 + wc * 32 + j;
                if (f < a.ffn) a.y[t * a.ldy + f] = swiglu1((float)acc[ta][0][v], (float)acc[ta][1][v]);
            }
        }
    }
}

int launch_gemm(const GemvArgs& a, int epi, hipStream_t s) {
    const unsigned gt = (unsigned)((a.m + BT - 1) / BT);
    if (epi == EPI_SWIGLU) {
        dim3 grid((unsigned)((a.ffn + BR / 2 - 1) / (BR / 2)), gt);
        hipLaunchKernelGGL(k_gemm_mfma<EPI_SWIGLU>, grid, dim3(256), 0, s, a);
    } else {
        dim3 grid((unsigned)((a.n + BR - 1) / BR), gt);
        hipLaunchKernelGGL(k_gemm_mfma<EPI_STORE>, grid, dim3(256), 0, s, a);
    }
    return qk_launch_status();
}

}  // namespace qk
