// RMSNorm (optionally fused with Q8_0 of its output), interleaved RoPE with
// the KV store, SwiGLU, embedding lookup and greedy argmax.
#include "internal.h"

namespace qk {

// ---------------------------------------------------------------- RMSNorm
// kenji.blog TinyLLaMA-in-C++ guide, section 4.1: y = x / sqrt(mean(x^2) +
// eps) * gamma.  One workgroup per row.  Pass 1 sums squares (fp64, wave
// butterflies then LDS across waves); pass 2 writes y and, when asked,
// quantizes it to Q8_0 with the same arithmetic as quantize_q8_0 (each lane
// holds 8 consecutive outputs, four lanes a block).
__global__ __launch_bounds__(256) void k_rmsnorm_q8(const float* __restrict__ x,
                                                    const float* __restrict__ gamma, int64_t dim,
                                                    float eps, float* __restrict__ y,
                                                    int8_t* __restrict__ xq,
                                                    uint16_t* __restrict__ xd) {
    __shared__ double red[4];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * dim;
    double ss = 0.0;
    for (int64_t i = threadIdx.x * 4; i < dim; i += 256 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(xr + i);
        ss = fma((double)v.x, (double)v.x, ss);
        ss = fma((double)v.y, (double)v.y, ss);
        ss = fma((double)v.z, (double)v.z, ss);
        ss = fma((double)v.w, (double)v.w, ss);
    }
    ss = group_sum<WAVE>(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double total = red[0] + red[1] + red[2] + red[3];
    const double denom = sqrt(total / (double)dim + (double)eps);
    // pass 2: 8 values per lane; the loop bound keeps whole quads together
    for (int64_t i0 = 0; i0 < dim; i0 += 256 * 8) {
        const int64_t i = i0 + threadIdx.x * 8;
        const bool live = i < dim;
        float v[8];
        if (live) {
            const float4 a = *reinterpret_cast<const float4*>(xr + i);
            const float4 b = *reinterpret_cast<const float4*>(xr + i + 4);
            const float4 ga = *reinterpret_cast<const float4*>(gamma + i);
            const float4 gb = *reinterpret_cast<const float4*>(gamma + i + 4);
            const float xs[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            const float gs[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (float)((double)xs[e] / denom * (double)gs[e]);
            if (y) {
                *reinterpret_cast<float4*>(y + row * dim + i) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4*>(y + row * dim + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = 0.0f;
        }
        if (xq) {
            uint32_t lo, hi;
            float d;
            q8_quad(v, lo, hi, d);
            if (live) {
                *reinterpret_cast<uint2*>(xq + row * dim + i) = make_uint2(lo, hi);
                if ((threadIdx.x & 3) == 0) xd[row * (dim / QBLK) + i / QBLK] = f2h(d);
            }
        }
    }
}

// Rows up to KC * 2048 values: each lane takes 8 consecutive values of every
// 2048-value chunk, and the row and gamma are loaded once, all at once
// (unconditional loads, indexes clamped into the row), into registers; the
// sum of squares, the normalization and the Q8_0 codes come from there.
// The lane mapping and the order of the fp64 sums are those of the GEMV's
// fused prologue, so both give the same sum of squares for a row.
template <int KC>
__global__ __launch_bounds__(256) void k_rmsnorm_q8_reg(const float* __restrict__ x,
                                                        const float* __restrict__ gamma,
                                                        int64_t dim, float eps,
                                                        float* __restrict__ y,
                                                        int8_t* __restrict__ xq,
                                                        uint16_t* __restrict__ xd) {
    __shared__ double red[4];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * dim;
    float xv[KC][8], gv[KC][8];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        int64_t i = (int64_t)c * 2048 + threadIdx.x * 8;
        i = i < dim ? i : 0;
        const float4 a = *reinterpret_cast<const float4*>(xr + i);
        const float4 b = *reinterpret_cast<const float4*>(xr + i + 4);
        const float4 ga = *reinterpret_cast<const float4*>(gamma + i);
        const float4 gb = *reinterpret_cast<const float4*>(gamma + i + 4);
        xv[c][0] = a.x; xv[c][1] = a.y; xv[c][2] = a.z; xv[c][3] = a.w;
        xv[c][4] = b.x; xv[c][5] = b.y; xv[c][6] = b.z; xv[c][7] = b.w;
        gv[c][0] = ga.x; gv[c][1] = ga.y; gv[c][2] = ga.z; gv[c][3] = ga.w;
        gv[c][4] = gb.x; gv[c][5] = gb.y; gv[c][6] = gb.z; gv[c][7] = gb.w;
    }
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        const bool in = (int64_t)c * 2048 + threadIdx.x * 8 < dim;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double v = in ? (double)xv[c][e] : 0.0;
            ss = fma(v, v, ss);
        }
    }
    ss = group_sum<WAVE>(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double total = red[0] + red[1] + red[2] + red[3];
    const double denom = sqrt(total / (double)dim + (double)eps);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        if ((int64_t)c * 2048 >= dim) break;   // uniform over the workgroup
        const int64_t i = (int64_t)c * 2048 + threadIdx.x * 8;
        const bool live = i < dim;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = live ? (float)((double)xv[c][e] / denom * (double)gv[c][e]) : 0.0f;
        if (y && live) {
            *reinterpret_cast<float4*>(y + row * dim + i) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(y + row * dim + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
        if (xq) {
            uint32_t lo, hi;
            float d;
            q8_quad(v, lo, hi, d);
            if (live) {
                *reinterpret_cast<uint2*>(xq + row * dim + i) = make_uint2(lo, hi);
                if ((threadIdx.x & 3) == 0) xd[row * (dim / QBLK) + i / QBLK] = f2h(d);
            }
        }
    }
}

int launch_rmsnorm_q8(const float* x, const float* gamma, int64_t rows, int64_t dim, float eps,
                      float* y, int8_t* xq, uint16_t* xd, hipStream_t s) {
    if (rows == 0) return QK_OK;
    const dim3 grid((unsigned)rows), block(256);
    if (dim <= 2048)
        hipLaunchKernelGGL(k_rmsnorm_q8_reg<1>, grid, block, 0, s, x, gamma, dim, eps, y, xq, xd);
    else if (dim <= 4096)
        hipLaunchKernelGGL(k_rmsnorm_q8_reg<2>, grid, block, 0, s, x, gamma, dim, eps, y, xq, xd);
    else if (dim <= 6144)
        hipLaunchKernelGGL(k_rmsnorm_q8_reg<3>, grid, block, 0, s, x, gamma, dim, eps, y, xq, xd);
    else
        hipLaunchKernelGGL(k_rmsnorm_q8, grid, block, 0, s, x, gamma, dim, eps, y, xq, xd);
    return qk_launch_status();
}

// ------------------------------------------------------------------- RoPE
// kenji.blog TinyLLaMA-in-C++ guide, section 4.2: the adjacent pair
// (x[2i], x[2i+1]) turns by m * theta_i, m the absolute position.  theta_i =
// base^(-2i/hd); the angle, cos/sin and the rotation are taken in fp64 per
// (token, pair) and the result rounded once to fp32.
// One workgroup per token; q heads then k heads are rotated in place, after
// which (when caches are given) k and v rows are stored to the fp16 KV cache
// at ring row pos % cap of the token's sequence (TinyLLaMA-in-C++ guide,
// section 7; the ring buffer of the inference-engine article, section 8).
__global__ __launch_bounds__(256) void k_rope_kv(float* __restrict__ base, int64_t tok_stride,
                                                 int64_t q_off, int64_t nq, int64_t k_off,
                                                 int64_t v_off, int64_t nkv, int64_t hd,
                                                 const int32_t* __restrict__ pos,
                                                 const int32_t* __restrict__ seq, float rbase,
                                                 uint16_t* __restrict__ kc,
                                                 uint16_t* __restrict__ vc, int64_t cap) {
    __shared__ double cs[2][256];
    const int64_t t = blockIdx.x;
    const int64_t half = hd / 2;
    const int p = pos[t];
    for (int64_t i = threadIdx.x; i < half; i += 256) {
        const double theta = pow((double)rbase, -2.0 * (double)i / (double)hd);
        double sn, cn;
        sincos((double)p * theta, &sn, &cn);
        cs[0][i] = cn;
        cs[1][i] = sn;
    }
    __syncthreads();
    float* row = base + t * tok_stride;
    const int64_t pairs = (nq + nkv) * half;
    for (int64_t idx = threadIdx.x; idx < pairs; idx += 256) {
        const int64_t hh = idx / half, i = idx % half;
        float* xp = hh < nq ? row + q_off + hh * hd + 2 * i : row + k_off + (hh - nq) * hd + 2 * i;
        const float2 v = *reinterpret_cast<float2*>(xp);
        const double c = cs[0][i], sn = cs[1][i];
        const double x1 = v.x, x2 = v.y;
        const float2 o = make_float2((float)(x1 * c - x2 * sn), (float)(x1 * sn + x2 * c));
        *reinterpret_cast<float2*>(xp) = o;
        if (kc && hh >= nq && p >= 0) {
            const int64_t g = hh - nq;
            const int64_t dst = (((int64_t)seq[t] * nkv + g) * cap + p % cap) * hd + 2 * i;
            kc[dst] = f2h(o.x);
            kc[dst + 1] = f2h(o.y);
        }
    }
    if (vc && p >= 0) {
        for (int64_t idx = threadIdx.x; idx < nkv * hd; idx += 256) {
            const int64_t g = idx / hd, d = idx % hd;
            const int64_t dst = (((int64_t)seq[t] * nkv + g) * cap + p % cap) * hd + d;
            vc[dst] = f2h(row[v_off + g * hd + d]);
        }
    }
}

int launch_rope_kv(float* base, int64_t tokens, int64_t tok_stride, int64_t q_off, int64_t nq,
                   int64_t k_off, int64_t v_off, int64_t nkv, int64_t hd, const int32_t* pos,
                   const int32_t* seq, float rope_base, uint16_t* k_cache, uint16_t* v_cache,
                   int64_t cap, hipStream_t s) {
    if (tokens == 0) return QK_OK;
    hipLaunchKernelGGL(k_rope_kv, dim3((unsigned)tokens), dim3(256), 0, s, base, tok_stride, q_off,
                       nq, k_off, v_off, nkv, hd, pos, seq, rope_base, k_cache, v_cache, cap);
    return qk_launch_status();
}

// ------------------------------------------------------------- KV append
__global__ __launch_bounds__(256) void k_kv_append(const float* __restrict__ k,
                                                   const float* __restrict__ v, int64_t tokens,
                                                   int64_t nkv, int64_t hd,
                                                   const int32_t* __restrict__ pos,
                                                   const int32_t* __restrict__ seq,
                                                   uint16_t* __restrict__ kc,
                                                   uint16_t* __restrict__ vc, int64_t cap) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= tokens * nkv * hd) return;
    const int64_t d = i % hd, g = (i / hd) % nkv, t = i / (hd * nkv);
    if (pos[t] < 0) return;  // negative positions are not written
    const int64_t dst = (((int64_t)seq[t] * nkv + g) * cap + pos[t] % cap) * hd + d;
    kc[dst] = f2h(k[i]);
    vc[dst] = f2h(v[i]);
}

// ----------------------------------------------------------------- SwiGLU
// kenji.blog TinyLLaMA-in-C++ guide, section 4.4.
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ g,
                                                const float* __restrict__ u, int64_t n,
                                                float* __restrict__ h) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double z = g[i];
    h[i] = (float)(z / (1.0 + exp(-z)) * (double)u[i]);
}

// -------------------------------------------------------------- embedding
__global__ __launch_bounds__(256) void k_embed(const float* __restrict__ table, int64_t vocab,
                                               int64_t hidden, const int32_t* __restrict__ ids,
                                               float* __restrict__ x) {
    const int64_t r = blockIdx.x;
    const int id = ids[r];
    const bool ok = id >= 0 && id < vocab;  // an out-of-range id gives a zero row
    const float* src = table + (int64_t)(ok ? id : 0) * hidden;
    for (int64_t i = threadIdx.x; i < hidden; i += 256) x[r * hidden + i] = ok ? src[i] : 0.0f;
}

// The same for 16-byte aligned rows of a multiple of 4 values: each thread
// issues its (up to) four 128-bit loads together, with indexes clamped into
// the row, before storing any, so a row up to 4096 values costs one memory
// round trip after the id.
__global__ __launch_bounds__(256) void k_embed4(const float4* __restrict__ table, int64_t vocab,
                                                int64_t h4, const int32_t* __restrict__ ids,
                                                float4* __restrict__ x) {
    const int64_t r = blockIdx.x;
    const int id = ids[r];
    const bool ok = id >= 0 && id < vocab;
    const float4* src = table + (int64_t)(ok ? id : 0) * h4;
    for (int64_t i0 = 0; i0 < h4; i0 += 4 * 256) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * 256 + threadIdx.x;
            v[u] = src[i < h4 ? i : 0];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * 256 + threadIdx.x;
            if (i < h4) x[r * h4 + i] = ok ? v[u] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
}

// ----------------------------------------------------------------- argmax
// One workgroup per row; (value, index) pairs reduce with ties to the lower
// index, NaN never wins.
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

__global__ __launch_bounds__(256) void k_argmax(const float* __restrict__ logits, int64_t vocab,
                                                int32_t* __restrict__ idx) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int64_t r = blockIdx.x;
    const float* l = logits + r * vocab;
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int64_t i = threadIdx.x; i < vocab; i += 256) better(bv, bi, l[i], (int)i);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, WAVE);
        const int oi = __shfl_xor(bi, o, WAVE);
        better(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = bv;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) better(bv, bi, sv[w], si[w]);
        if (bi == INT32_MAX) bi = 0;  // all NaN: fall back to index 0
        idx[r] = bi;
    }
}

}  // namespace qk

using namespace qk;

extern "C" int rmsnorm(const float* x, const float* gamma, int64_t rows, int64_t dim, float eps,
                       float* y, void* stream) {
    QK_REQUIRE(rows >= 0 && dim > 0, QK_EINVAL);
    QK_REQUIRE(dim % 8 == 0, QK_ESHAPE);
    if (rows == 0) return QK_OK;
    QK_REQUIRE(x && gamma && y, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(x, 16) && QK_ALIGNED(gamma, 16) && QK_ALIGNED(y, 16), QK_EALIGN);
    return launch_rmsnorm_q8(x, gamma, rows, dim, eps, y, nullptr, nullptr, (hipStream_t)stream);
}

extern "C" int rope(float* x, int64_t tokens, int64_t heads, int64_t head_dim,
                    const int32_t* pos, float base, void* stream) {
    QK_REQUIRE(tokens >= 0 && heads >= 0 && head_dim > 0, QK_EINVAL);
    QK_REQUIRE(head_dim % 2 == 0 && head_dim <= 512, QK_ESHAPE);
    if (tokens == 0 || heads == 0) return QK_OK;
    QK_REQUIRE(x && pos, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(x, 8), QK_EALIGN);
    return launch_rope_kv(x, tokens, heads * head_dim, 0, heads, 0, 0, 0, head_dim, pos, nullptr,
                          base, nullptr, nullptr, 0, (hipStream_t)stream);
}

extern "C" int swiglu(const float* gate, const float* up, int64_t n, float* h, void* stream) {
    QK_REQUIRE(n >= 0, QK_EINVAL);
    if (n == 0) return QK_OK;
    QK_REQUIRE(gate && up && h, QK_EINVAL);
    hipLaunchKernelGGL(k_swiglu, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, gate, up, n, h);
    return qk_launch_status();
}

extern "C" int qk_kv_append(const float* k, const float* v, int64_t tokens, int64_t n_kv,
                            int64_t hd, const int32_t* pos, const int32_t* seq, uint16_t* k_cache,
                            uint16_t* v_cache, int64_t cap, void* stream) {
    QK_REQUIRE(tokens >= 0 && n_kv > 0 && hd > 0 && cap > 0, QK_EINVAL);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(k && v && pos && seq && k_cache && v_cache, QK_EINVAL);
    const int64_t total = tokens * n_kv * hd;
    hipLaunchKernelGGL(k_kv_append, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, k, v, tokens, n_kv, hd, pos, seq, k_cache, v_cache,
                       cap);
    return qk_launch_status();
}

extern "C" int qk_embed_lookup(const float* table, int64_t vocab, int64_t hidden,
                               const int32_t* ids, int64_t n, float* x, void* stream) {
    QK_REQUIRE(vocab > 0 && hidden > 0 && n >= 0, QK_EINVAL);
    if (n == 0) return QK_OK;
    QK_REQUIRE(table && ids && x, QK_EINVAL);
    if (hidden % 4 == 0 && QK_ALIGNED(table, 16) && QK_ALIGNED(x, 16))
        hipLaunchKernelGGL(k_embed4, dim3((unsigned)n), dim3(256), 0, (hipStream_t)stream,
                           reinterpret_cast<const float4*>(table), vocab, hidden / 4, ids,
                           reinterpret_cast<float4*>(x));
    else
        hipLaunchKernelGGL(k_embed, dim3((unsigned)n), dim3(256), 0, (hipStream_t)stream, table,
                           vocab, hidden, ids, x);
    return qk_launch_status();
}

extern "C" int qk_argmax(const float* logits, int64_t rows, int64_t vocab, int32_t* idx,
                         void* stream) {
    QK_REQUIRE(rows >= 0 && vocab > 0 && vocab <= INT32_MAX, QK_EINVAL);
    if (rows == 0) return QK_OK;
    QK_REQUIRE(logits && idx, QK_EINVAL);
    hipLaunchKernelGGL(k_argmax, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, logits,
                       vocab, idx);
    return qk_launch_status();
}
