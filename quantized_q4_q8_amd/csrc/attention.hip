// Grouped-query attention over the fp16 KV cache.
//
// kenji.blog "No Python needed" engine, section 8 (softmax(Q K^T / sqrt(d))
// V with a KV cache), TinyLLaMA-in-C++ guide 4.3 (several query heads share
// one KV head) and 7 (attend over cache rows 0..N).
//
// Split over the context: workgroup (chunk c, KV head g, token t) handles
// cache rows [ACH c, ACH c + ACH) intersected with [0, pos[t]] for all query
// heads of group g, so each K/V row is read once for the whole group, and
// writes the chunk's record per head: running max m, exp-sum l and the
// un-normalized output o.  A second kernel, one workgroup per (head, token),
// merges the records by log-sum-exp rescaling (every thread issues its loads
// in one round) and writes the fp32 output and/or its Q8_0 quantization.
// Cross-workgroup merging inside one kernel would need device-scope release
// fences, which on this multi-die part write back the whole L2; the kernel
// boundary is cheaper.  Scores, softmax and the weighted sums are fp64 (K/V
// rows are widened from fp16 in LDS) and the output is rounded once to fp32.
#include "internal.h"

namespace qk {

namespace {

constexpr int MAX_MERGE_CHUNKS = 128;

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int pick_chunk(int64_t tokens, int64_t nkv, int64_t cap) {
    const int64_t wgs64 = tokens * nkv * ((cap + 63) / 64);
    return (wgs64 < 512 && (cap + 31) / 32 <= MAX_MERGE_CHUNKS) ? 32 : 64;
}

}  // namespace

int64_t attention_counter_words(int64_t tokens, int64_t nkv) {
    (void)tokens;
    (void)nkv;
    return 0;
}

namespace {
size_t ws_bytes_for(int64_t tokens, int64_t nq, int64_t hd, int64_t nch) {
    return (size_t)(tokens * nq * nch * (hd + 2)) * sizeof(double);
}
}  // namespace

size_t attention_ws_bytes(int64_t tokens, int64_t nq, int64_t nkv, int64_t hd, int64_t cap) {
    const int ach = pick_chunk(tokens, nkv, cap);
    return ws_bytes_for(tokens, nq, hd, (cap + ach - 1) / ach);
}

template <int HD, int ACH>
__global__ __launch_bounds__(256) void k_attn_chunk(
    const float* __restrict__ q, int64_t q_ts, int64_t nq, int64_t nkv,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int64_t cap,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, double* __restrict__ part,
    int64_t nch) {
    constexpr int MAXG = 512 / HD;
    __shared__ float qs[MAXG][HD];
    __shared__ __align__(16) float ks[ACH][HD + 1];
    __shared__ __align__(16) float vs[ACH][HD];
    __shared__ double ps[MAXG][ACH];

    const int64_t c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int p = pos[t];
    const int64_t r0 = c * ACH;
    if (p < 0 || p >= cap || r0 > p) return;  // out-of-range positions read nothing
    const int rows = (int)min((int64_t)ACH, (int64_t)p + 1 - r0);
    const int G = (int)(nq / nkv);
    const int tid = threadIdx.x;
    const double rscale = sqrt((double)HD);

    for (int i = tid; i < G * HD; i += 256) {
        const int hh = i / HD, d = i % HD;
        qs[hh][d] = q[t * q_ts + (g * G + hh) * HD + d];
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
        double s = -INFINITY;
        if (r < rows) {
            double dot = 0.0;
#pragma unroll 16
            for (int d = 0; d < HD; ++d) dot = fma((double)qs[hh][d], (double)ks[r][d], dot);
            s = dot / rscale;
        }
        ps[hh][r] = s;
    }
    __syncthreads();

    // softmax pieces of the chunk: one wave per head, lane = row
    const int lane = tid & 63, wave = tid >> 6;
    for (int hh = wave; hh < G; hh += 4) {
        const double s = lane < ACH ? ps[hh][lane] : -INFINITY;
        const double mx = group_max<WAVE>(s);
        const double e = lane < rows ? exp(s - mx) : 0.0;
        const double l = group_sum<WAVE>(e);
        if (lane < ACH) ps[hh][lane] = e;
        if (lane == 0) {
            double* o = part + (((t * nq) + g * G + hh) * nch + c) * (HD + 2);
            o[0] = mx;
            o[1] = l;
        }
    }
    __syncthreads();

    for (int i = tid; i < G * HD; i += 256) {
        const int hh = i / HD, d = i % HD;
        double o = 0.0;
        for (int r = 0; r < rows; ++r) o = fma(ps[hh][r], (double)vs[r][d], o);
        part[(((t * nq) + g * G + hh) * nch + c) * (HD + 2) + 2 + d] = o;
    }

}

// Merge the chunk records of head h of token t: M = max m_c, w_c = e^(m_c - M),
// out = sum_c w_c o_c / sum_c w_c l_c.  256 threads = (HD / 2 output pairs) x
// (slices of the chunks); slice partial sums are added in LDS in slice order.
template <int HD, int ACH>
__global__ __launch_bounds__(256) void k_attn_merge(const double* __restrict__ part, int64_t nq,
                                                    int64_t nch, int64_t cap,
                                                    const int32_t* __restrict__ pos,
                                                    float* __restrict__ out, int64_t o_ts,
                                                    int8_t* __restrict__ oq,
                                                    uint16_t* __restrict__ od) {
    constexpr int PAIRS = HD / 2;
    constexpr int SLICES = 256 / PAIRS;
    constexpr int PER = (MAX_MERGE_CHUNKS + SLICES - 1) / SLICES;
    __shared__ double w[MAX_MERGE_CHUNKS];
    __shared__ double red[4];
    __shared__ double2 acc_s[SLICES][PAIRS];
    __shared__ double res[HD];
    const int64_t h = blockIdx.x, t = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    const int64_t col = h * HD;
    if (p < 0 || p >= cap) {   // out-of-range position: zeros, no reads
        for (int d = tid; d < HD; d += 256) {
            if (out) out[t * o_ts + col + d] = 0.0f;
            if (oq) oq[t * o_ts + col + d] = 0;
        }
        if (oq && tid < HD / QBLK) od[(t * o_ts + col) / QBLK + tid] = 0;
        return;
    }
    const int64_t used = p / ACH + 1;
    const double* rec = part + (t * nq + h) * nch * (HD + 2);
    // chunk weights
    const double m = tid < used ? rec[tid * (HD + 2)] : -INFINITY;
    const double l = tid < used ? rec[tid * (HD + 2) + 1] : 0.0;
    double mx = group_max<WAVE>(m);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    const double wc = tid < used ? exp(m - mx) : 0.0;
    if (tid < MAX_MERGE_CHUNKS) w[tid] = wc;
    double ls = group_sum<WAVE>(wc * l);
    __syncthreads();   // everyone has read red[]
    if (lane == 0) red[wave] = ls;
    __syncthreads();
    const double lsum = (red[0] + red[1]) + (red[2] + red[3]);
    // weighted outputs: thread (pair, slice) over chunks slice, slice + SLICES, ...
    const int pr = tid % PAIRS, sl = tid / PAIRS;
    double2 xv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int64_t cc = sl + (int64_t)e * SLICES;
        xv[e] = cc < used ? *reinterpret_cast<const double2*>(rec + cc * (HD + 2) + 2 + 2 * pr)
                          : make_double2(0.0, 0.0);
    }
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int64_t cc = sl + (int64_t)e * SLICES;
        const double ww = cc < used ? w[cc] : 0.0;
        a0 = fma(ww, xv[e].x, a0);
        a1 = fma(ww, xv[e].y, a1);
    }
    acc_s[sl][pr] = make_double2(a0, a1);
    __syncthreads();
    if (tid < PAIRS) {
        double s0 = 0.0, s1 = 0.0;
        for (int q = 0; q < SLICES; ++q) {
            s0 += acc_s[q][tid].x;
            s1 += acc_s[q][tid].y;
        }
        res[2 * tid] = s0 / lsum;
        res[2 * tid + 1] = s1 / lsum;
    }
    __syncthreads();
    if (tid < HD / 8) {   // four lanes per Q8_0 block
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)res[8 * tid + e];
        if (out) {
#pragma unroll
            for (int e = 0; e < 8; ++e) out[t * o_ts + col + 8 * tid + e] = v[e];
        }
        if (oq) {
            uint32_t lo, hi;
            float dd;
            q8_quad(v, lo, hi, dd);
            *reinterpret_cast<uint2*>(oq + t * o_ts + col + 8 * tid) = make_uint2(lo, hi);
            if ((tid & 3) == 0) od[(t * o_ts + col + 8 * tid) / QBLK] = f2h(dd);
        }
    }
}

int launch_attention(const float* q, int64_t q_ts, int64_t tokens, int64_t nq, int64_t nkv,
                     int64_t hd, const uint16_t* kc, const uint16_t* vc, int64_t cap,
                     const int32_t* pos, const int32_t* seq, float* out, int64_t o_ts,
                     int8_t* oq, uint16_t* od, void* ws, size_t ws_bytes, bool counters_zeroed,
                     hipStream_t s) {
    (void)counters_zeroed;
    if (tokens == 0) return QK_OK;
    if (!ws || ws_bytes < attention_ws_bytes(tokens, nq, nkv, hd, cap)) return QK_EWORKSPACE;
    const int ach = pick_chunk(tokens, nkv, cap);
    const int64_t nch = (cap + ach - 1) / ach;
    if (nch > MAX_MERGE_CHUNKS) return QK_ESHAPE;
    double* part = static_cast<double*>(ws);
    dim3 grid((unsigned)nch, (unsigned)nkv, (unsigned)tokens);
    dim3 mgrid((unsigned)nq, (unsigned)tokens);
#define QK_ATT(HD_, ACH_)                                                                          \
    do {                                                                                           \
        hipLaunchKernelGGL((k_attn_chunk<HD_, ACH_>), grid, dim3(256), 0, s, q, q_ts, nq, nkv, kc, \
                           vc, cap, pos, seq, part, nch);                                          \
        hipLaunchKernelGGL((k_attn_merge<HD_, ACH_>), mgrid, dim3(256), 0, s, part, nq, nch, cap,  \
                           pos, out, o_ts, oq, od);                                                \
    } while (0)
    if (hd == 32 && ach == 32) QK_ATT(32, 32);
    else if (hd == 32) QK_ATT(32, 64);
    else if (hd == 64 && ach == 32) QK_ATT(64, 32);
    else if (hd == 64) QK_ATT(64, 64);
    else return QK_ESHAPE;
#undef QK_ATT
    return qk_launch_status();
}

}  // namespace qk

using namespace qk;

extern "C" size_t qk_gqa_attention_workspace(int64_t tokens, int64_t n_q_heads, int64_t head_dim,
                                             int64_t cap) {
    if (tokens < 0 || n_q_heads <= 0 || head_dim <= 0 || cap <= 0) return 0;
    // an upper bound over every KV-head count: records for the 32-row chunk
    return ws_bytes_for(tokens, n_q_heads, head_dim, (cap + 31) / 32);
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
    QK_REQUIRE(cap <= (int64_t)MAX_MERGE_CHUNKS * 64, QK_ESHAPE);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(q && k_cache && v_cache && pos && seq && out, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(k_cache, 16) && QK_ALIGNED(v_cache, 16) && QK_ALIGNED(q, 4) &&
                   QK_ALIGNED(out, 4),
               QK_EALIGN);
    QK_REQUIRE(ws && ws_bytes >= attention_ws_bytes(tokens, n_q_heads, n_kv_heads, head_dim, cap),
               QK_EWORKSPACE);
    return launch_attention(q, n_q_heads * head_dim, tokens, n_q_heads, n_kv_heads, head_dim,
                            k_cache, v_cache, cap, pos, seq, out, n_q_heads * head_dim, nullptr,
                            nullptr, ws, ws_bytes, false, (hipStream_t)stream);
}
