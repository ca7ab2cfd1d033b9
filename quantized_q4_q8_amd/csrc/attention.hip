// Grouped-query attention over the fp16 KV cache.
//
// kenji.blog "No Python needed" engine, section 8 (softmax(Q K^T / sqrt(d))
// V with a KV cache), TinyLLaMA-in-C++ guide 4.3 (several query heads share
// one KV head) and 7 (attend over cache rows 0..N).
//
// Split over the context in two passes.  The chunk pass reads each 64-row
// chunk of a KV head once for all query heads of its group and writes one
// record per (head, chunk); the merge pass combines a head's records by
// log-sum-exp rescaling.  The kernel boundary between them is the cheapest
// way to make the records of every die visible to the merging workgroup.
// Scores, softmax and the weighted sums are fp64 and the output is rounded
// once to fp32.
#include "internal.h"

namespace qk {

namespace {

constexpr int ACH = 64;            // cache rows per chunk: one per lane
constexpr int MAX_CHUNKS = 128;    // chunks per head (cap <= 8192)
constexpr int64_t FLASH_MIN_TOKENS = 8;   // more tokens than this: the tiled pass

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t attention_ws_bytes(int64_t tokens, int64_t nq, int64_t nkv, int64_t hd, int64_t cap) {
    (void)nkv;
    const int64_t nch = (cap + ACH - 1) / ACH;
    return align256((size_t)(tokens * nq * nch * (hd + 2)) * sizeof(double));
}

// Chunk pass.  Workgroup (chunk c, KV head g, token t) reads cache rows
// [64 c, 64 c + 64) intersected with [0, pos[t]] of its sequence once for all
// query heads of group g; wave w takes query heads w, w + 8, ...  For its head
// a wave writes the chunk's record: running max m, exp-sum l and the
// un-normalized output o[hd] (fp64).  Lane = cache row for the scores and the
// softmax, lane = output dimension for the weighted sum.  q is staged in LDS
// as fp64, K and V rows as fp32 (exact widenings of fp16), read 128 bits at a
// time.
template <int HD>
__global__ __launch_bounds__(512) void k_attn_chunk(
    const float* __restrict__ q, int64_t q_ts, int64_t nq, int64_t nkv,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int64_t cap,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, double* __restrict__ rec,
    int64_t nch) {
    constexpr int MAXG = 512 / HD;
    constexpr int KS = HD + 4;          // K row stride in floats: 16-byte rows, spread over banks
    constexpr int NW = 8;               // waves per workgroup
    __shared__ __align__(16) double qs[MAXG][HD];
    __shared__ __align__(16) float ks[ACH][KS];
    __shared__ __align__(16) float vs[ACH][HD];
    __shared__ __align__(16) double es[NW][ACH];

    const int64_t c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int G = (int)(nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    if (p < 0) return;   // negative positions read nothing
    const int64_t pe = min((int64_t)p, cap - 1);   // last ring row attended
    const int64_t r0 = c * ACH;
    if (r0 > pe) return;
    const int rows = (int)min((int64_t)ACH, pe + 1 - r0);
    const double rscale = sqrt((double)HD);

    for (int i = tid; i < G * HD; i += 512)
        qs[i / HD][i % HD] = (double)q[t * q_ts + (g * G) * HD + i];
    const int64_t cbase = (((int64_t)seq[t] * nkv + g) * cap + r0) * HD;
    for (int i = tid; i < ACH * HD / 8; i += 512) {
        const int r = (i * 8) / HD, d = (i * 8) % HD;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (r < rows) {
            kv = *reinterpret_cast<const uint4*>(kc + cbase + (int64_t)r * HD + d);
            vv = *reinterpret_cast<const uint4*>(vc + cbase + (int64_t)r * HD + d);
        }
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
        float4 k0, k1, v0, v1;
        k0.x = h2f((uint16_t)(kw[0] & 0xFFFF)); k0.y = h2f((uint16_t)(kw[0] >> 16));
        k0.z = h2f((uint16_t)(kw[1] & 0xFFFF)); k0.w = h2f((uint16_t)(kw[1] >> 16));
        k1.x = h2f((uint16_t)(kw[2] & 0xFFFF)); k1.y = h2f((uint16_t)(kw[2] >> 16));
        k1.z = h2f((uint16_t)(kw[3] & 0xFFFF)); k1.w = h2f((uint16_t)(kw[3] >> 16));
        v0.x = h2f((uint16_t)(vw[0] & 0xFFFF)); v0.y = h2f((uint16_t)(vw[0] >> 16));
        v0.z = h2f((uint16_t)(vw[1] & 0xFFFF)); v0.w = h2f((uint16_t)(vw[1] >> 16));
        v1.x = h2f((uint16_t)(vw[2] & 0xFFFF)); v1.y = h2f((uint16_t)(vw[2] >> 16));
        v1.z = h2f((uint16_t)(vw[3] & 0xFFFF)); v1.w = h2f((uint16_t)(vw[3] >> 16));
        *reinterpret_cast<float4*>(&ks[r][d]) = k0;
        *reinterpret_cast<float4*>(&ks[r][d + 4]) = k1;
        *reinterpret_cast<float4*>(&vs[r][d]) = v0;
        *reinterpret_cast<float4*>(&vs[r][d + 4]) = v1;
    }
    __syncthreads();

    for (int hh = wave; hh < G; hh += NW) {
        double* rp = rec + ((t * nq + g * G + hh) * nch + c) * (HD + 2);
        double s = -INFINITY;
        if (lane < rows) {   // score of row `lane`
            double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
#pragma unroll
            for (int d = 0; d < HD; d += 4) {
                const float4 kk = *reinterpret_cast<const float4*>(&ks[lane][d]);
                const double2 qa = *reinterpret_cast<const double2*>(&qs[hh][d]);
                const double2 qb = *reinterpret_cast<const double2*>(&qs[hh][d + 2]);
                d0 = fma(qa.x, (double)kk.x, d0);
                d1 = fma(qa.y, (double)kk.y, d1);
                d2 = fma(qb.x, (double)kk.z, d2);
                d3 = fma(qb.y, (double)kk.w, d3);
            }
            s = ((d0 + d1) + (d2 + d3)) / rscale;
        }
        const double m = group_max<WAVE>(s);
        const double e = lane < rows ? exp(s - m) : 0.0;
        const double l = group_sum<WAVE>(e);
        es[wave][lane] = e;
        __builtin_amdgcn_wave_barrier();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane < HD) {   // weighted values, lane = dimension
            double o0 = 0.0, o1 = 0.0, o2 = 0.0, o3 = 0.0;
            if (rows == ACH) {   // full chunk: unrolled, LDS reads run ahead
#pragma unroll
                for (int r = 0; r < ACH; r += 4) {
                    const double2 ea = *reinterpret_cast<const double2*>(&es[wave][r]);
                    const double2 eb = *reinterpret_cast<const double2*>(&es[wave][r + 2]);
                    o0 = fma(ea.x, (double)vs[r][lane], o0);
                    o1 = fma(ea.y, (double)vs[r + 1][lane], o1);
                    o2 = fma(eb.x, (double)vs[r + 2][lane], o2);
                    o3 = fma(eb.y, (double)vs[r + 3][lane], o3);
                }
            } else {
                int r = 0;
                for (; r + 1 < rows; r += 2) {
                    const double2 ee = *reinterpret_cast<const double2*>(&es[wave][r]);
                    o0 = fma(ee.x, (double)vs[r][lane], o0);
                    o1 = fma(ee.y, (double)vs[r + 1][lane], o1);
                }
                if (r < rows) o0 = fma(es[wave][r], (double)vs[r][lane], o0);
            }
            rp[2 + lane] = (o0 + o1) + (o2 + o3);
        }
        if (lane == 0) {
            rp[0] = m;
            rp[1] = l;
        }
        __builtin_amdgcn_wave_barrier();   // es is rewritten for the next head
    }
}

// Merge pass: workgroup (head h, token t) combines the head's chunk records
// by log-sum-exp rescaling, out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Thread (pair i, slice s) owns output dimensions 2i, 2i + 1 over chunks
// s, s + SLICES, ...; thread c also loads chunk c's (m, l).  Every load is
// issued before anything waits; the chunk weights are then formed one per
// thread.  Slice sums are added in slice order, so the result does not
// depend on timing.  Writes the fp32 output and/or its Q8_0 codes (four
// lanes per block).
template <int HD>
__global__ __launch_bounds__(256) void k_attn_merge(const double* __restrict__ rec, int64_t nq,
                                                    int64_t nch, int64_t cap,
                                                    const int32_t* __restrict__ pos,
                                                    float* __restrict__ out, int64_t o_ts,
                                                    int8_t* __restrict__ oq,
                                                    uint16_t* __restrict__ od) {
    constexpr int PAIRS = HD / 2;
    constexpr int SLICES = 256 / PAIRS;
    constexpr int PER = (MAX_CHUNKS + SLICES - 1) / SLICES;
    __shared__ double wsh[MAX_CHUNKS];
    __shared__ double red[4];
    __shared__ double2 acc_s[SLICES][PAIRS];
    __shared__ double res[HD];
    const int64_t h = blockIdx.x, t = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    const int64_t col = h * HD;
    const bool valid = p >= 0;   // negative position: zeros, no reads
    const int used = valid ? (int)(min((int64_t)p, cap - 1) / ACH) + 1 : 0;
    const double* hr = rec + (t * nq + h) * nch * (HD + 2);
    const int pr = tid % PAIRS, sl = tid / PAIRS;

    // all loads first: chunk tid's (m, l) and this thread's output pairs
    const double2 ml = tid < used ? *reinterpret_cast<const double2*>(hr + tid * (HD + 2))
                                  : make_double2(-INFINITY, 0.0);
    double2 xv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int cc = sl + e * SLICES;
        xv[e] = cc < used ? *reinterpret_cast<const double2*>(hr + cc * (HD + 2) + 2 + 2 * pr)
                          : make_double2(0.0, 0.0);
    }
    double mx = group_max<WAVE>(ml.x);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    const double wc = tid < used ? exp(ml.x - mx) : 0.0;
    if (tid < MAX_CHUNKS) wsh[tid] = wc;
    const double ls = group_sum<WAVE>(wc * ml.y);
    __syncthreads();   // everyone has read red[]; wsh is complete
    if (lane == 0) red[wave] = ls;
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int cc = sl + e * SLICES;
        if (cc < used) {
            a0 = fma(wsh[cc], xv[e].x, a0);
            a1 = fma(wsh[cc], xv[e].y, a1);
        }
    }
    acc_s[sl][pr] = make_double2(a0, a1);
    __syncthreads();
    if (tid < PAIRS) {
        const double lsum = (red[0] + red[1]) + (red[2] + red[3]);
        double s0 = 0.0, s1 = 0.0;
        for (int q = 0; q < SLICES; ++q) {
            s0 += acc_s[q][tid].x;
            s1 += acc_s[q][tid].y;
        }
        res[2 * tid] = valid ? s0 / lsum : 0.0;
        res[2 * tid + 1] = valid ? s1 / lsum : 0.0;
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

// Many-token pass (prefill): workgroup (tile of TQ consecutive tokens, KV
// head g) walks the KV chunks once for all tokens and all query heads of
// the group, keeping a running (max, sum, output) per (token, head) row and
// rescaling it as each chunk's scores arrive (the online form of the
// max-subtracted softmax); nothing is written between chunks.  A tile is
// processed in runs of consecutive tokens of the same sequence.  Wave w
// takes query heads w, w + 8; lane = key for the scores, lane = output
// dimension for the weighted sum.  fp64 throughout, K/V widened in LDS.
template <int HD>
__global__ __launch_bounds__(512) void k_attn_flash(
    const float* __restrict__ q, int64_t q_ts, int64_t tokens, int64_t nq, int64_t nkv,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int64_t cap,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, float* __restrict__ out,
    int64_t o_ts, int8_t* __restrict__ oq, uint16_t* __restrict__ od) {
    constexpr int TQ = 8;               // tokens per tile
    constexpr int NW = 8;               // waves per workgroup
    constexpr int MAXG = 512 / HD;      // query heads per group at most
    constexpr int HPW = MAXG / NW;      // query heads per wave at most
    __shared__ __align__(16) double qs[TQ][MAXG * HD];
    __shared__ float ks[ACH][HD + 1];
    __shared__ __align__(16) float vs[ACH][HD];
    __shared__ __align__(16) double ps[NW][TQ][ACH];

    const int64_t g = blockIdx.y, t0 = (int64_t)blockIdx.x * TQ;
    const int G = (int)(nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntile = (int)min((int64_t)TQ, tokens - t0);
    const double rscale = sqrt((double)HD);

    for (int i0 = 0; i0 < ntile;) {   // runs of one sequence (uniform)
        const int s0 = seq[t0 + i0];
        int i1 = i0 + 1;
        while (i1 < ntile && seq[t0 + i1] == s0) ++i1;
        const int nrun = i1 - i0;
        int pi[TQ];
        int kmax = -1;
#pragma unroll
        for (int i = 0; i < TQ; ++i) {
            pi[i] = -1;
            if (i < nrun) {
                const int p = pos[t0 + i0 + i];
                if (p >= 0) {   // negative positions attend to nothing
                    pi[i] = (int)min((int64_t)p, cap - 1);   // last ring row attended
                    kmax = max(kmax, pi[i]);
                }
            }
        }
        __syncthreads();   // the previous run is done with qs
        for (int idx = tid; idx < nrun * G * HD; idx += 512) {
            const int i = idx / (G * HD), r = idx % (G * HD);
            qs[i][r] = (double)q[(t0 + i0 + i) * q_ts + g * G * HD + r];
        }

        double m[HPW][TQ], l[HPW][TQ], o[HPW][TQ];
#pragma unroll
        for (int hp = 0; hp < HPW; ++hp)
#pragma unroll
            for (int i = 0; i < TQ; ++i) {
                m[hp][i] = -INFINITY;
                l[hp][i] = 0.0;
                o[hp][i] = 0.0;
            }

        const int64_t cbase = (((int64_t)s0 * nkv + g) * cap) * HD;
        for (int c = 0; c * ACH <= kmax; ++c) {
            const int64_t r0 = (int64_t)c * ACH;
            __syncthreads();   // ks/vs (and qs, first time) ready for rewriting / reading
            for (int i = tid; i < ACH * HD / 8; i += 512) {
                const int r = (i * 8) / HD, d = (i * 8) % HD;
                uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
                if (r0 + r <= kmax) {
                    kv = *reinterpret_cast<const uint4*>(kc + cbase + (r0 + r) * HD + d);
                    vv = *reinterpret_cast<const uint4*>(vc + cbase + (r0 + r) * HD + d);
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
#pragma unroll
            for (int hp = 0; hp < HPW; ++hp) {
                const int hh = wave + hp * NW;
                if (hh >= G) break;   // uniform over the wave
                // scores of key r0 + lane for the run's tokens
                double sc[TQ];
#pragma unroll
                for (int i = 0; i < TQ; ++i) sc[i] = 0.0;
#pragma unroll 4
                for (int d = 0; d < HD; d += 2) {
                    const double k0 = (double)ks[lane][d], k1 = (double)ks[lane][d + 1];
#pragma unroll
                    for (int i = 0; i < TQ; ++i) {
                        const double2 qq = *reinterpret_cast<const double2*>(&qs[i][hh * HD + d]);
                        sc[i] = fma(qq.x, k0, sc[i]);
                        sc[i] = fma(qq.y, k1, sc[i]);
                    }
                }
                const int key = (int)r0 + lane;
#pragma unroll
                for (int i = 0; i < TQ; ++i) {
                    const bool ok = key <= pi[i];   // pi = -1 for absent or out-of-range tokens
                    const double s = ok ? sc[i] / rscale : -INFINITY;
                    const double cm = group_max<WAVE>(s);
                    double pv = 0.0;
                    if (cm != -INFINITY) {   // uniform over the wave
                        const double mn = fmax(m[hp][i], cm);
                        const double f = exp(m[hp][i] - mn);   // 0 when m was -inf
                        pv = ok ? exp(s - mn) : 0.0;
                        l[hp][i] = fma(l[hp][i], f, group_sum<WAVE>(pv));
                        o[hp][i] *= f;
                        m[hp][i] = mn;
                    }
                    ps[wave][i][lane] = pv;
                }
                __builtin_amdgcn_wave_barrier();
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (lane < HD) {   // weighted values, lane = dimension
#pragma unroll 4
                    for (int j = 0; j < ACH; j += 2) {
                        const double v0 = (double)vs[j][lane], v1 = (double)vs[j + 1][lane];
#pragma unroll
                        for (int i = 0; i < TQ; ++i) {
                            const double2 pp = *reinterpret_cast<const double2*>(&ps[wave][i][j]);
                            o[hp][i] = fma(pp.x, v0, o[hp][i]);
                            o[hp][i] = fma(pp.y, v1, o[hp][i]);
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();   // ps is rewritten next
            }
        }

        // outputs of the run: fp32 and/or Q8_0 (one 32-lane group per block)
#pragma unroll
        for (int hp = 0; hp < HPW; ++hp) {
            const int hh = wave + hp * NW;
            if (hh >= G) break;
#pragma unroll
            for (int i = 0; i < TQ; ++i) {
                if (i >= nrun) break;
                const float v = l[hp][i] > 0.0 ? (float)(o[hp][i] / l[hp][i]) : 0.0f;
                const int64_t col = (t0 + i0 + i) * o_ts + (g * G + hh) * HD;
                if (lane < HD) {
                    if (out) out[col + lane] = v;
                    if (oq) {
                        const float amax = group_max<QBLK>(fabsf(v));
                        const float d = amax / 127.0f;
                        int qv = 0;
                        if (d != 0.0f) qv = (int)fminf(127.0f, fmaxf(-127.0f, roundf(v / d)));
                        oq[col + lane] = (int8_t)qv;
                        if ((lane & (QBLK - 1)) == 0) od[(col + lane) / QBLK] = f2h(d);
                    }
                }
            }
        }
        i0 = i1;
    }
}

int launch_attention(const float* q, int64_t q_ts, int64_t tokens, int64_t nq, int64_t nkv,
                     int64_t hd, const uint16_t* kc, const uint16_t* vc, int64_t cap,
                     const int32_t* pos, const int32_t* seq, float* out, int64_t o_ts,
                     int8_t* oq, uint16_t* od, void* ws, size_t ws_bytes, hipStream_t s) {
    if (tokens == 0) return QK_OK;
    if (!ws || ws_bytes < attention_ws_bytes(tokens, nq, nkv, hd, cap)) return QK_EWORKSPACE;
    const int64_t nch = (cap + ACH - 1) / ACH;
    if (nch > MAX_CHUNKS || (nq / nkv) * hd > 512) return QK_ESHAPE;
    if (tokens > FLASH_MIN_TOKENS) {
        dim3 fgrid((unsigned)((tokens + 7) / 8), (unsigned)nkv);
        if (hd == 32)
            hipLaunchKernelGGL(k_attn_flash<32>, fgrid, dim3(512), 0, s, q, q_ts, tokens, nq, nkv, kc,
                               vc, cap, pos, seq, out, o_ts, oq, od);
        else if (hd == 64)
            hipLaunchKernelGGL(k_attn_flash<64>, fgrid, dim3(512), 0, s, q, q_ts, tokens, nq, nkv, kc,
                               vc, cap, pos, seq, out, o_ts, oq, od);
        else
            return QK_ESHAPE;
        return qk_launch_status();
    }
    double* rec = static_cast<double*>(ws);
    dim3 grid((unsigned)nch, (unsigned)nkv, (unsigned)tokens);
    dim3 mgrid((unsigned)nq, (unsigned)tokens);
    if (hd == 32) {
        hipLaunchKernelGGL(k_attn_chunk<32>, grid, dim3(512), 0, s, q, q_ts, nq, nkv, kc, vc, cap,
                           pos, seq, rec, nch);
        hipLaunchKernelGGL(k_attn_merge<32>, mgrid, dim3(256), 0, s, rec, nq, nch, cap, pos, out,
                           o_ts, oq, od);
    } else if (hd == 64) {
        hipLaunchKernelGGL(k_attn_chunk<64>, grid, dim3(512), 0, s, q, q_ts, nq, nkv, kc, vc, cap,
                           pos, seq, rec, nch);
        hipLaunchKernelGGL(k_attn_merge<64>, mgrid, dim3(256), 0, s, rec, nq, nch, cap, pos, out,
                           o_ts, oq, od);
    } else {
        return QK_ESHAPE;
    }
    return qk_launch_status();
}

}  // namespace qk

using namespace qk;

extern "C" size_t qk_gqa_attention_workspace(int64_t tokens, int64_t n_q_heads, int64_t head_dim,
                                             int64_t cap) {
    if (tokens < 0 || n_q_heads <= 0 || head_dim <= 0 || cap <= 0) return 0;
    return attention_ws_bytes(tokens, n_q_heads, n_q_heads, head_dim, cap);
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
    QK_REQUIRE(cap <= (int64_t)MAX_CHUNKS * ACH, QK_ESHAPE);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(q && k_cache && v_cache && pos && seq && out, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(k_cache, 16) && QK_ALIGNED(v_cache, 16) && QK_ALIGNED(q, 4) &&
                   QK_ALIGNED(out, 4),
               QK_EALIGN);
    QK_REQUIRE(ws && ws_bytes >= attention_ws_bytes(tokens, n_q_heads, n_kv_heads, head_dim, cap),
               QK_EWORKSPACE);
    return launch_attention(q, n_q_heads * head_dim, tokens, n_q_heads, n_kv_heads, head_dim,
                            k_cache, v_cache, cap, pos, seq, out, n_q_heads * head_dim, nullptr,
                            nullptr, ws, ws_bytes, (hipStream_t)stream);
}
