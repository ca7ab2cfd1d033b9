// Grouped-query attention over the fp16 KV cache.
//
// kenji.blog "No Python needed" engine, section 8 (softmax(Q K^T / sqrt(d))
// V with a KV cache), TinyLLaMA-in-C++ guide 4.3 (several query heads share
// one KV head) and 7 (attend over cache rows 0..N).
//
// Split over the context: workgroup (chunk c, KV head g, token t) handles
// cache rows [64c, 64c + 64) intersected with [0, pos[t]] for all query heads
// of group g, so each K/V row is read once for the whole group.  It writes
// the chunk's running max, exp-sum and un-normalized output; a second kernel
// merges the chunks of a (token, head) by log-sum-exp rescaling.  Scores and
// softmax are fp32 (accurate expf); K/V rows are widened from fp16 in LDS.
#include "internal.h"

namespace qk {

constexpr int ACH = 64;  // cache rows per chunk

size_t attention_ws_bytes(int64_t tokens, int64_t nq, int64_t hd, int64_t cap) {
    const int64_t nch = (cap + ACH - 1) / ACH;
    return (size_t)(tokens * nq * nch * (hd + 2)) * sizeof(float);
}

template <int HD>
__global__ __launch_bounds__(256) void k_attn_chunk(const float* __restrict__ q, int64_t q_ts,
                                                    int64_t nq, int64_t nkv,
                                                    const uint16_t* __restrict__ kc,
                                                    const uint16_t* __restrict__ vc, int64_t cap,
                                                    const int32_t* __restrict__ pos,
                                                    const int32_t* __restrict__ seq,
                                                    float* __restrict__ part, int64_t nch) {
    constexpr int MAXG = 512 / HD;
    __shared__ float qs[MAXG][HD];
    __shared__ float ks[ACH][HD + 1];
    __shared__ float vs[ACH][HD];
    __shared__ float ps[MAXG][ACH];

    const int64_t c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int p = pos[t];
    const int64_t r0 = c * ACH;
    if (p < 0 || p >= cap || r0 > p) return;  // out-of-range positions read nothing
    const int rows = (int)min((int64_t)ACH, (int64_t)p + 1 - r0);
    const int G = (int)(nq / nkv);
    const int tid = threadIdx.x;
    const float scale = 1.0f / sqrtf((float)HD);

    for (int i = tid; i < G * HD; i += 256) {
        const int hh = i / HD, d = i % HD;
        qs[hh][d] = q[t * q_ts + (g * G + hh) * HD + d] * scale;
    }
    const int64_t cbase = (((int64_t)seq[t] * nkv + g) * cap + r0) * HD;
    for (int i = tid; i < ACH * HD / 8; i += 256) {
        const int r = (i * 8) / HD, d = (i * 8) % HD;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (r < rows) {
            kv = *reinterpret_cast<const uint4*>(kc + cbase + (int64_t)r * HD + d);
            vv = *reinterpret_cast<const uint4*>(vc + cbase + (int64_t)r * HD + d);
        }
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ks[r][d + 2 * e] = h2f((uint16_t)(kw[e] & 0xFFFF));
            ks[r][d + 2 * e + 1] = h2f((uint16_t)(kw[e] >> 16));
            vs[r][d + 2 * e] = h2f((uint16_t)(vw[e] & 0xFFFF));
            vs[r][d + 2 * e + 1] = h2f((uint16_t)(vw[e] >> 16));
        }
    }
    __syncthreads();

    for (int i = tid; i < G * ACH; i += 256) {
        const int hh = i / ACH, r = i % ACH;
        float s = -INFINITY;
        if (r < rows) {
            s = 0.0f;
#pragma unroll 16
            for (int d = 0; d < HD; ++d) s = fmaf(qs[hh][d], ks[r][d], s);
        }
        ps[hh][r] = s;
    }
    __syncthreads();

    // softmax pieces: one wave per head, lane = row
    const int lane = tid & 63, wave = tid >> 6;
    for (int hh = wave; hh < G; hh += 4) {
        const float s = ps[hh][lane];
        const float mx = group_max<WAVE>(s);
        const float e = lane < rows ? expf(s - mx) : 0.0f;
        const float l = group_sum<WAVE>(e);
        ps[hh][lane] = e;
        if (lane == 0) {
            float* o = part + (((t * nq) + g * G + hh) * nch + c) * (HD + 2);
            o[0] = mx;
            o[1] = l;
        }
    }
    __syncthreads();

    for (int i = tid; i < G * HD; i += 256) {
        const int hh = i / HD, d = i % HD;
        float o = 0.0f;
        for (int r = 0; r < rows; ++r) o = fmaf(ps[hh][r], vs[r][d], o);
        part[(((t * nq) + g * G + hh) * nch + c) * (HD + 2) + 2 + d] = o;
    }
}

// Merge the chunks of one (token, head): M = max m_c,
// out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part, int64_t nq,
                                                    int64_t hd, int64_t nch, int64_t cap,
                                                    const int32_t* __restrict__ pos,
                                                    float* __restrict__ out, int64_t o_ts) {
    const int64_t h = blockIdx.x, t = blockIdx.y;
    if (pos[t] < 0 || pos[t] >= cap) {  // out-of-range position: zeros, no reads
        for (int64_t d = threadIdx.x; d < hd; d += blockDim.x) out[t * o_ts + h * hd + d] = 0.0f;
        return;
    }
    const int64_t used = pos[t] / ACH + 1;
    const float* pc = part + (t * nq + h) * nch * (hd + 2);
    float mx = -INFINITY;
    for (int64_t c = 0; c < used; ++c) mx = fmaxf(mx, pc[c * (hd + 2)]);
    float l = 0.0f;
    for (int64_t c = 0; c < used; ++c) l += expf(pc[c * (hd + 2)] - mx) * pc[c * (hd + 2) + 1];
    const float inv = 1.0f / l;
    for (int64_t d = threadIdx.x; d < hd; d += blockDim.x) {
        float o = 0.0f;
        for (int64_t c = 0; c < used; ++c) o += expf(pc[c * (hd + 2)] - mx) * pc[c * (hd + 2) + 2 + d];
        out[t * o_ts + h * hd + d] = o * inv;
    }
}

int launch_attention(const float* q, int64_t q_ts, int64_t tokens, int64_t nq, int64_t nkv,
                     int64_t hd, const uint16_t* kc, const uint16_t* vc, int64_t cap,
                     const int32_t* pos, const int32_t* seq, float* out, int64_t o_ts, void* ws,
                     size_t ws_bytes, hipStream_t s) {
    if (tokens == 0) return QK_OK;
    if (ws_bytes < attention_ws_bytes(tokens, nq, hd, cap) || !ws) return QK_EWORKSPACE;
    const int64_t nch = (cap + ACH - 1) / ACH;
    float* part = static_cast<float*>(ws);
    dim3 grid((unsigned)nch, (unsigned)nkv, (unsigned)tokens);
    switch (hd) {
        case 32: hipLaunchKernelGGL(k_attn_chunk<32>, grid, dim3(256), 0, s, q, q_ts, nq, nkv, kc, vc, cap, pos, seq, part, nch); break;
        case 64: hipLaunchKernelGGL(k_attn_chunk<64>, grid, dim3(256), 0, s, q, q_ts, nq, nkv, kc, vc, cap, pos, seq, part, nch); break;
        default: return QK_ESHAPE;
    }
    hipLaunchKernelGGL(k_attn_merge, dim3((unsigned)nq, (unsigned)tokens), dim3(64), 0, s, part,
                       nq, hd, nch, cap, pos, out, o_ts);
    return qk_launch_status();
}

}  // namespace qk

using namespace qk;

extern "C" size_t qk_gqa_attention_workspace(int64_t tokens, int64_t n_q_heads, int64_t head_dim,
                                             int64_t cap) {
    if (tokens < 0 || n_q_heads <= 0 || head_dim <= 0 || cap <= 0) return 0;
    return attention_ws_bytes(tokens, n_q_heads, head_dim, cap);
}

extern "C" int gqa_attention(const float* q, int64_t tokens, int64_t n_q_heads,
                             int64_t n_kv_heads, int64_t head_dim, const uint16_t* k_cache,
                             const uint16_t* v_cache, int64_t cap, const int32_t* pos,
                             const int32_t* seq, float* out, void* ws, size_t ws_bytes,
                             void* stream) {
    QK_REQUIRE(tokens >= 0 && n_q_heads > 0 && n_kv_heads > 0 && cap > 0, QK_EINVAL);
    QK_REQUIRE(n_q_heads % n_kv_heads == 0, QK_ESHAPE);
    QK_REQUIRE(head_dim == 32 || head_dim == 64, QK_ESHAPE);
    QK_REQUIRE((n_q_heads / n_kv_heads) * head_dim <= 512, QK_ESHAPE);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(q && k_cache && v_cache && pos && seq && out, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(k_cache, 16) && QK_ALIGNED(v_cache, 16), QK_EALIGN);
    QK_REQUIRE(ws && ws_bytes >= attention_ws_bytes(tokens, n_q_heads, head_dim, cap),
               QK_EWORKSPACE);
    return launch_attention(q, n_q_heads * head_dim, tokens, n_q_heads, n_kv_heads, head_dim,
                            k_cache, v_cache, cap, pos, seq, out, n_q_heads * head_dim, ws,
                            ws_bytes, (hipStream_t)stream);
}
