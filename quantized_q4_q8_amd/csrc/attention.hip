// Grouped-query attention over the fp16 KV cache.
//
// kenji.blog "No Python needed" engine, section 8 (softmax(Q K^T / sqrt(d))
// V with a KV cache), TinyLLaMA-in-C++ guide 4.3 (several query heads share
// one KV head) and 7 (attend over cache rows 0..N).
//
// Few tokens (decode): split over the context in two passes.  The chunk
// pass reads each 64-row chunk of a KV head once for all query heads of its
// group and writes one record per (head, chunk); the merge pass combines a
// head's records by log-sum-exp rescaling, up to 512 chunks per head (cap up
// to 32768 rows).  The kernel boundary between them is the cheapest way
// measured to make the records of every die visible to the merging
// workgroup: merging inside the chunk pass (the last workgroup of a KV head
// to finish, found with a device-scope counter, merges its heads) was slower
// on the TinyLLaMA-shape decode, its record stores, counter and record loads
// being three dependent device-scope round trips.  Many tokens (prefill): one pass over the chunks with
// an online softmax, its two products on the fp64 matrix cores.
// Scores, softmax and the weighted sums are fp64 and the output is rounded
// once to fp32.
#include "internal.h"

#include <type_traits>

namespace qk {

namespace {

constexpr int ACH = 64;            // cache rows per chunk: one per lane
constexpr int MAX_CHUNKS = 512;    // chunks per head (cap <= 32768)
constexpr int64_t FLASH_MIN_TOKENS = 8;   // more tokens than this: the tiled pass
constexpr int MERGE_W_CHUNKS = 64;         // records per head up to which the merge is one wave

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t attention_ws_bytes(int64_t tokens, int64_t nq, int64_t nkv, int64_t hd, int64_t cap) {
    (void)nkv;
    const int64_t nch = (cap + ACH - 1) / ACH;
    return align256((size_t)(tokens * nq * nch * (hd + 2)) * sizeof(double));
}

// One thread's 8-value piece of a K and a V row (fp16 bits) into the
// chunk's LDS rows as fp32 (exact widenings).
template <int HD>
__device__ __forceinline__ void stage_kv_piece(const uint4 kv, const uint4 vv, int r, int d,
                                               float (*ks)[HD + 4], float (*vs)[HD]) {
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

// One query head against the chunk's first `rows` LDS rows (one wave): the
// chunk max m, the exp-sum l and, in lanes < HD, the un-normalized output of
// dimension `lane`.  esw is the wave's row of exp weights.
template <int HD>
__device__ __forceinline__ void head_chunk(const double* qh, const float (*ks)[HD + 4],
                                           const float (*vs)[HD], double* esw, int lane, int rows,
                                           double& m, double& l, double& oc) {
    const double rscale = sqrt((double)HD);
    double s = -INFINITY;
    if (lane < rows) {   // score of row `lane`
        double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
#pragma unroll
        for (int d = 0; d < HD; d += 4) {
            const float4 kk = *reinterpret_cast<const float4*>(&ks[lane][d]);
            const double2 qa = *reinterpret_cast<const double2*>(&qh[d]);
            const double2 qb = *reinterpret_cast<const double2*>(&qh[d + 2]);
            d0 = fma(qa.x, (double)kk.x, d0);
            d1 = fma(qa.y, (double)kk.y, d1);
            d2 = fma(qb.x, (double)kk.z, d2);
            d3 = fma(qb.y, (double)kk.w, d3);
        }
        s = ((d0 + d1) + (d2 + d3)) / rscale;
    }
    m = group_max<WAVE>(s);
    const double e = lane < rows ? exp(s - m) : 0.0;
    l = group_sum<WAVE>(e);
    esw[lane] = e;
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    oc = 0.0;
    if (lane < HD) {   // weighted values, lane = dimension
        double o0 = 0.0, o1 = 0.0, o2 = 0.0, o3 = 0.0;
        if (rows == ACH) {   // full chunk: unrolled, LDS reads run ahead
#pragma unroll
            for (int r = 0; r < ACH; r += 4) {
                const double2 ea = *reinterpret_cast<const double2*>(&esw[r]);
                const double2 eb = *reinterpret_cast<const double2*>(&esw[r + 2]);
                o0 = fma(ea.x, (double)vs[r][lane], o0);
                o1 = fma(ea.y, (double)vs[r + 1][lane], o1);
                o2 = fma(eb.x, (double)vs[r + 2][lane], o2);
                o3 = fma(eb.y, (double)vs[r + 3][lane], o3);
            }
        } else {
            int r = 0;
            for (; r + 1 < rows; r += 2) {
                const double2 ee = *reinterpret_cast<const double2*>(&esw[r]);
                o0 = fma(ee.x, (double)vs[r][lane], o0);
                o1 = fma(ee.y, (double)vs[r + 1][lane], o1);
            }
            if (r < rows) o0 = fma(esw[r], (double)vs[r][lane], o0);
        }
        oc = (o0 + o1) + (o2 + o3);
    }
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
    // position and sequence read together, before the early exits, so that
    // the two small loads cost one round trip (the empty asm takes both
    // values, which keeps the compiler from moving the second load past the
    // exits)
    const int p = pos[t];
    const int sq = seq[t];
    asm volatile("" ::"s"(p), "s"(sq));
    if (p < 0) return;   // negative positions read nothing
    const int64_t pe = min((int64_t)p, cap - 1);   // last ring row attended
    const int64_t r0 = c * ACH;
    if (r0 > pe) return;
    const int rows = (int)min((int64_t)ACH, pe + 1 - r0);
    const double rscale = sqrt((double)HD);

    // One q value and one 8-value piece of a K and a V row per thread
    // (G * HD <= 512 and ACH * HD / 8 <= 512).  The three loads are
    // unconditional, with indexes clamped into the chunk, so that they are
    // all in flight before anything waits; rows past the last attended one
    // are staged but never read.
    static_assert(ACH * HD / 8 <= 512, "one K/V piece per thread");
    const int iq = tid < G * HD ? tid : 0;
    const float qv = q[t * q_ts + (g * G) * HD + iq];
    const int64_t cbase = (((int64_t)sq * nkv + g) * cap + r0) * HD;
    const int i = tid < ACH * HD / 8 ? tid : 0;
    const int r = (i * 8) / HD, d = (i * 8) % HD;
    const int64_t roff = (int64_t)(r < rows ? r : 0) * HD + d;
    const uint4 kv = *reinterpret_cast<const uint4*>(kc + cbase + roff);
    const uint4 vv = *reinterpret_cast<const uint4*>(vc + cbase + roff);
    if (tid < G * HD) qs[tid / HD][tid % HD] = (double)qv;
    if (tid < ACH * HD / 8) {
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

// Chunk pass for long caches: workgroup (record x, KV head g, token t) walks
// the LCPW chunks from chunk LCPW x on, with the next chunk's rows loaded
// while the current one is used, and folds them into one record per head by
// the merge pass's log-sum-exp rescaling (both sides scaled to the larger
// max, in fp64).  A workgroup then streams its rows instead of loading one
// chunk and stopping, and the merge reads LCPW times fewer records.  (At
// 8192 rows and fewer the one-chunk pass is faster: its workgroups already
// fit the chip in one round.)
constexpr int LCPW = 4;

template <int HD>
__global__ __launch_bounds__(512) void k_attn_chunk_long(
    const float* __restrict__ q, int64_t q_ts, int64_t nq, int64_t nkv,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int64_t cap,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, double* __restrict__ rec,
    int64_t nrec) {
    constexpr int MAXG = 512 / HD;
    constexpr int KS = HD + 4;
    constexpr int NW = 8;
    constexpr int HPW = (MAXG + NW - 1) / NW;   // query heads per wave, at most
    __shared__ __align__(16) double qs[MAXG][HD];
    __shared__ __align__(16) float ks[ACH][KS];
    __shared__ __align__(16) float vs[ACH][HD];
    __shared__ __align__(16) double es[NW][ACH];

    const int64_t x = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int G = (int)(nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    const int sq = seq[t];
    asm volatile("" ::"s"(p), "s"(sq));
    if (p < 0) return;
    const int64_t pe = min((int64_t)p, cap - 1);
    const int64_t c0 = x * LCPW;
    if (c0 * ACH > pe) return;
    const int nc = (int)min((int64_t)LCPW, pe / ACH - c0 + 1);   // chunks with rows

    static_assert(ACH * HD / 8 <= 512, "one K/V piece per thread");
    const int iq = tid < G * HD ? tid : 0;
    const float qv = q[t * q_ts + (g * G) * HD + iq];
    const int64_t hbase = ((int64_t)sq * nkv + g) * cap * HD;
    const int i = tid < ACH * HD / 8 ? tid : 0;
    const int r = (i * 8) / HD, d = (i * 8) % HD;
    uint4 kv, vv;
    auto load_kv = [&](int64_t c) {   // clamped into the chunk's rows
        const int rows = (int)min((int64_t)ACH, pe + 1 - c * ACH);
        const int64_t roff = (c * ACH + (r < rows ? r : 0)) * HD + d;
        kv = *reinterpret_cast<const uint4*>(kc + hbase + roff);
        vv = *reinterpret_cast<const uint4*>(vc + hbase + roff);
    };
    load_kv(c0);
    if (tid < G * HD) qs[tid / HD][tid % HD] = (double)qv;

    double rm[HPW], rl[HPW], ro[HPW];
    for (int j = 0; j < nc; ++j) {
        const int64_t c = c0 + j;
        const int rows = (int)min((int64_t)ACH, pe + 1 - c * ACH);
        if (j > 0) __syncthreads();   // every wave is done with the previous chunk's rows
        if (tid < ACH * HD / 8) stage_kv_piece<HD>(kv, vv, r, d, ks, vs);
        __syncthreads();
        if (j + 1 < nc) load_kv(c + 1);
#pragma unroll
        for (int hi = 0; hi < HPW; ++hi) {
            const int hh = wave + hi * NW;
            if (hh >= G) break;
            double m, l, oc;
            head_chunk<HD>(qs[hh], ks, vs, es[wave], lane, rows, m, l, oc);
            if (j == 0) {
                rm[hi] = m;
                rl[hi] = l;
                ro[hi] = oc;
            } else {
                const double mn = fmax(rm[hi], m);
                const double a = exp(rm[hi] - mn), b = exp(m - mn);
                rl[hi] = rl[hi] * a + l * b;
                ro[hi] = ro[hi] * a + oc * b;
                rm[hi] = mn;
            }
            __builtin_amdgcn_wave_barrier();   // es is rewritten for the next head
        }
    }
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi) {
        const int hh = wave + hi * NW;
        if (hh >= G) break;
        double* rp = rec + ((t * nq + g * G + hh) * nrec + x) * (HD + 2);
        if (lane < HD) rp[2 + lane] = ro[hi];
        if (lane == 0) {
            rp[0] = rm[hi];
            rp[1] = rl[hi];
        }
    }
}

// Merge pass: workgroup (head h, token t) combines the head's nch records
// (one per 2^CPW_LOG2 chunks) by log-sum-exp rescaling,
// out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Thread (pair i, slice s) owns output dimensions 2i, 2i + 1 over chunks
// s, s + SLICES, ...; threads c and c + 256 load chunk c's and chunk
// c + 256's (m, l).  The (m, l) loads and a thread's first PB output pairs
// are issued before anything waits; the chunk weights are then formed one
// per chunk, and longer contexts load their further pairs PB at a time.  A
// thread adds its chunks in order and the slice sums are added in slice
// order, so the result does not depend on timing.  Writes the fp32 output
// and/or its Q8_0 codes (four lanes per block).  SPLIT > 1 (long contexts):
// the head's dims are split over SPLIT workgroups (grid z), each a whole
// number of Q8_0 blocks; every split forms the same chunk weights.
template <int HD, int SPLIT, int CPW_LOG2 = 0>
__global__ __launch_bounds__(256) void k_attn_merge(const double* __restrict__ rec, int64_t nq,
                                                    int64_t nch, int64_t cap,
                                                    const int32_t* __restrict__ pos,
                                                    float* __restrict__ out, int64_t o_ts,
                                                    int8_t* __restrict__ oq,
                                                    uint16_t* __restrict__ od) {
    constexpr int DH = HD / SPLIT;   // dims of this workgroup
    constexpr int PAIRS = DH / 2;
    constexpr int SLICES = 256 / PAIRS;
    constexpr int PB = 16;   // output pairs per thread per round of loads
    static_assert(MAX_CHUNKS == 512, "(m, l) of two chunks per thread");
    static_assert(DH % QBLK == 0, "whole Q8_0 blocks per workgroup");
    __shared__ double wsh[MAX_CHUNKS];
    __shared__ double red[4];
    __shared__ double2 acc_s[SLICES][PAIRS];
    __shared__ double res[DH];
    const int64_t h = blockIdx.x, t = blockIdx.y;
    const int d0 = (int)blockIdx.z * DH;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    const int64_t col = h * HD + d0;
    const bool valid = p >= 0;   // negative position: zeros, no reads
    const int used = valid ? (int)((min((int64_t)p, cap - 1) / ACH) >> CPW_LOG2) + 1 : 0;   // records with rows
    const double* hr = rec + (t * nq + h) * nch * (HD + 2);
    const int pr = tid % PAIRS, sl = tid / PAIRS;

    const double2 ml0 = tid < used ? *reinterpret_cast<const double2*>(hr + tid * (HD + 2))
                                   : make_double2(-INFINITY, 0.0);
    const double2 ml1 = tid + 256 < used ? *reinterpret_cast<const double2*>(hr + (tid + 256) * (HD + 2))
                                         : make_double2(-INFINITY, 0.0);
    double2 xv[PB];
    auto load_pairs = [&](int e0) {
#pragma unroll
        for (int e = 0; e < PB; ++e) {
            const int cc = sl + (e0 + e) * SLICES;
            xv[e] = cc < used ? *reinterpret_cast<const double2*>(hr + cc * (HD + 2) + 2 + d0 + 2 * pr)
                              : make_double2(0.0, 0.0);
        }
    };
    load_pairs(0);
    double mx = group_max<WAVE>(fmax(ml0.x, ml1.x));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    const double wc0 = tid < used ? exp(ml0.x - mx) : 0.0;
    const double wc1 = tid + 256 < used ? exp(ml1.x - mx) : 0.0;
    wsh[tid] = wc0;
    wsh[tid + 256] = wc1;
    const double ls = group_sum<WAVE>(wc0 * ml0.y + wc1 * ml1.y);
    __syncthreads();   // everyone has read red[]; wsh is complete
    if (lane == 0) red[wave] = ls;
    double a0 = 0.0, a1 = 0.0;
    for (int e0 = 0; sl + e0 * SLICES < used; e0 += PB) {
        if (e0 > 0) load_pairs(e0);
#pragma unroll
        for (int e = 0; e < PB; ++e) {
            const int cc = sl + (e0 + e) * SLICES;
            if (cc < used) {
                a0 = fma(wsh[cc], xv[e].x, a0);
                a1 = fma(wsh[cc], xv[e].y, a1);
            }
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
    if (tid < DH / 8) {   // four lanes per Q8_0 block
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

// Merge pass in one wave per (head, token), for at most 64 records per head
// (each of 2^CPW_LOG2 chunks): the same log-sum-exp combination as
// k_attn_merge with no workgroup barrier.  Lane c loads record c's (m, l)
// and lane d dim d of every record (record indexes clamped to record 0; the
// weight of a record without rows is 0), the max, the record weights and
// their l-weighted sum are wave reductions, the weights pass through LDS
// within the wave, and each lane adds its dim's weighted values in record
// order, so the result does not depend on timing.  Head dim 32: lanes
// 32..63 repeat lanes 0..31 and store nothing.  The Q8_0 output goes
// through LDS to eight values per lane, as in k_attn_merge.
template <int HD, int CPW_LOG2>
__global__ __launch_bounds__(64) void k_attn_merge_w(const double* __restrict__ rec, int64_t nq,
                                                     int64_t nch, int64_t cap,
                                                     const int32_t* __restrict__ pos,
                                                     float* __restrict__ out, int64_t o_ts,
                                                     int8_t* __restrict__ oq,
                                                     uint16_t* __restrict__ od) {
    static_assert(HD == 32 || HD == 64, "a dim per lane");
    static_assert(MERGE_W_CHUNKS == WAVE, "a record per lane");
    __shared__ __align__(16) double ws[WAVE];
    __shared__ __align__(16) float res[HD];
    const int64_t h = blockIdx.x, t = blockIdx.y;
    const int lane = threadIdx.x, d = lane & (HD - 1);
    const int p = pos[t];
    const bool valid = p >= 0;   // negative position: zeros (its records are not read as results)
    const int used = valid ? (int)((min((int64_t)p, cap - 1) / ACH) >> CPW_LOG2) + 1 : 0;   // records with rows
    const double* hr = rec + (t * nq + h) * nch * (HD + 2);
    // every load is issued before the first wait (one round trip)
    const double2 ml = *reinterpret_cast<const double2*>(hr + (lane < used ? lane : 0) * (HD + 2));
    double ov[WAVE];
#pragma unroll
    for (int c = 0; c < WAVE; ++c) ov[c] = hr[(c < used ? c : 0) * (HD + 2) + 2 + d];
    const double mx = group_max<WAVE>(lane < used ? ml.x : -INFINITY);
    const double w = lane < used ? exp(ml.x - mx) : 0.0;
    const double ls = group_sum<WAVE>(w * ml.y);
    ws[lane] = w;
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < WAVE; c += 2) {
        const double2 wc = *reinterpret_cast<const double2*>(&ws[c]);
        acc = fma(wc.x, ov[c], acc);
        acc = fma(wc.y, ov[c + 1], acc);
    }
    const float v = valid ? (float)(acc / ls) : 0.0f;
    const int64_t col = t * o_ts + h * HD;
    if (out && lane < HD) out[col + lane] = v;
    if (oq) {
        if (lane < HD) res[lane] = v;
        __builtin_amdgcn_wave_barrier();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float vv[8];
        const int i8 = (lane % (HD / 8)) * 8;   // lanes < HD / 8 hold values 8 lane .. 8 lane + 7
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = res[i8 + e];
        uint32_t lo, hi;
        float dd;
        q8_quad(vv, lo, hi, dd);   // four lanes per Q8_0 block
        if (lane < HD / 8) {
            *reinterpret_cast<uint2*>(oq + col + 8 * lane) = make_uint2(lo, hi);
            if ((lane & 3) == 0) od[(col + 8 * lane) / QBLK] = f2h(dd);
        }
    }
}

// Merge pass for 65..128 records per head, head dim 64: two waves per
// (head, token), wave z taking dims 32 z .. 32 z + 31, with no workgroup
// barrier.  Lane c loads the (m, l) of records c and c + 64; lane (half hh,
// dim d) the values of dim 32 z + d in records 64 hh .. 64 hh + 63.  The
// max, the record weights and their l-weighted sum are wave reductions; the
// weights pass through LDS within the wave; each lane adds its 64 records in
// order and the half holding records 64..127 is added to the other.
template <int CPW_LOG2>
__global__ __launch_bounds__(64) void k_attn_merge_w2(const double* __restrict__ rec, int64_t nq,
                                                      int64_t nch, int64_t cap,
                                                      const int32_t* __restrict__ pos,
                                                      float* __restrict__ out, int64_t o_ts,
                                                      int8_t* __restrict__ oq,
                                                      uint16_t* __restrict__ od) {
    constexpr int HD = 64, DH = 32;
    __shared__ __align__(16) double ws[2 * WAVE];
    __shared__ __align__(16) float res[DH];
    const int64_t h = blockIdx.x, t = blockIdx.y;
    const int z = blockIdx.z;
    const int lane = threadIdx.x, hh = lane >> 5, d = lane & 31;
    const int p = pos[t];
    const bool valid = p >= 0;
    const int used = valid ? (int)((min((int64_t)p, cap - 1) / ACH) >> CPW_LOG2) + 1 : 0;   // records with rows
    const double* hr = rec + (t * nq + h) * nch * (HD + 2);
    const double2 ml0 = *reinterpret_cast<const double2*>(hr + (lane < used ? lane : 0) * (HD + 2));
    const double2 ml1 = *reinterpret_cast<const double2*>(hr + (lane + WAVE < used ? lane + WAVE : 0) * (HD + 2));
    double ov[WAVE];
#pragma unroll
    for (int c = 0; c < WAVE; ++c) {
        const int r = hh * WAVE + c;
        ov[c] = hr[(r < used ? r : 0) * (HD + 2) + 2 + z * DH + d];
    }
    double m = lane < used ? ml0.x : -INFINITY;
    if (lane + WAVE < used) m = fmax(m, ml1.x);
    const double mx = group_max<WAVE>(m);
    const double w0 = lane < used ? exp(ml0.x - mx) : 0.0;
    const double w1 = lane + WAVE < used ? exp(ml1.x - mx) : 0.0;
    const double ls = group_sum<WAVE>(fma(w1, ml1.y, w0 * ml0.y));
    ws[lane] = w0;
    ws[lane + WAVE] = w1;
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < WAVE; c += 2) {
        const double2 wc = *reinterpret_cast<const double2*>(&ws[hh * WAVE + c]);
        acc = fma(wc.x, ov[c], acc);
        acc = fma(wc.y, ov[c + 1], acc);
    }
    const double other = __shfl_xor(acc, 32, WAVE);
    const double tot = hh == 0 ? acc + other : other + acc;   // records 0..63, then 64..127
    const float v = valid ? (float)(tot / ls) : 0.0f;
    const int64_t col = t * o_ts + h * HD + z * DH;
    if (out && lane < DH) out[col + lane] = v;
    if (oq) {
        if (lane < DH) res[lane] = v;
        __builtin_amdgcn_wave_barrier();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float vv[8];
        const int i8 = (lane & 3) * 8;   // lanes 0..3: the block's four quarters
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = res[i8 + e];
        uint32_t lo, hi;
        float dd;
        q8_quad(vv, lo, hi, dd);
        if (lane < DH / 8) {
            *reinterpret_cast<uint2*>(oq + col + 8 * lane) = make_uint2(lo, hi);
            if (lane == 0) od[col / QBLK] = f2h(dd);
        }
    }
}

// Longest-first order of the tiled pass's token tiles (TQ tokens each): a
// tile's cost is the number of 64-row chunks its furthest position attends,
// and order[] lists the tiles by cost, largest first (a counting sort; the
// order within a cost does not matter, every tile's result is its own).
// Dispatched in token order, the costliest tiles of a causal prefill (the
// last tokens of each sequence) started last and left most of the chip idle
// in the kernel's tail.
__global__ __launch_bounds__(1024) void k_tile_order(const int32_t* __restrict__ pos, int64_t tokens,
                                                     int tq, int64_t cap, int nch, int ntiles,
                                                     int32_t* __restrict__ order) {
    constexpr int KEEP = 4;   // tiles per thread whose cost is kept in registers
    __shared__ int cnt[MAX_CHUNKS + 1];
    __shared__ int base[MAX_CHUNKS + 1];
    const int tid = threadIdx.x;
    for (int i = tid; i <= nch; i += 1024) cnt[i] = 0;
    // a tile's positions are read eight at a time from clamped indexes, so
    // that their loads are in flight together
    auto cost = [&](int tile) {
        int kmax = -1;
        for (int j0 = 0; j0 < tq; j0 += 8) {
            int p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t t = (int64_t)tile * tq + j0 + j;
                p[j] = (j0 + j < tq && t < tokens) ? pos[t] : -1;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (p[j] >= 0) kmax = max(kmax, (int)min((int64_t)p[j], cap - 1));
        }
        return kmax >= 0 ? kmax / ACH + 1 : 0;   // <= MAX_CHUNKS
    };
    int kept[KEEP];
#pragma unroll
    for (int i = 0; i < KEEP; ++i) {
        const int tile = tid + 1024 * i;
        kept[i] = tile < ntiles ? cost(tile) : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KEEP; ++i)
        if (tid + 1024 * i < ntiles) atomicAdd(&cnt[kept[i]], 1);
    for (int tile = tid + 1024 * KEEP; tile < ntiles; tile += 1024) atomicAdd(&cnt[cost(tile)], 1);
    __syncthreads();
    if (tid == 0) {   // base[c]: the tiles that cost more than c (costs are at most nch)
        int run = 0;
        for (int c = nch; c >= 0; --c) {
            base[c] = run;
            run += cnt[c];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KEEP; ++i) {
        const int tile = tid + 1024 * i;
        if (tile < ntiles) order[atomicAdd(&base[kept[i]], 1)] = tile;
    }
    for (int tile = tid + 1024 * KEEP; tile < ntiles; tile += 1024) order[atomicAdd(&base[cost(tile)], 1)] = tile;
}

typedef double v4d __attribute__((ext_vector_type(4)));

// Attention for many tokens on the fp64 matrix cores (v_mfma_f64_16x16x4f64).
// Same result as the online softmax above: per (token, head) row the scores
// of each 64-key chunk are s = q.k / sqrt(hd) in fp64, the running max,
// sum and output are rescaled by exp(m_old - m_new), and the output is
// o / l rounded once.  Layout of one 16x16x4 product (wave64): A[i][k] in
// lane i + 16k, B[k][j] in lane j + 16k, C[i][j] in lane j + 16 (i % 4),
// register i / 4.
// A workgroup (4 waves) takes 64 query rows = (64 / G) tokens x the G query
// heads of one KV head; wave w owns rows 16w .. 16w + 15, and lane l works on
// row 16w + l % 16.  The scores are formed transposed, S^T = K Q^T (A = K
// from LDS, B = Q^T from registers), so that each lane's C registers are
// exactly the B operand of O^T = V^T P^T (register v of key tile kt is key
// step 4 kt + v): the probabilities never leave registers.  K and V are
// staged in LDS as fp32 (exact widenings of fp16), double-buffered: the
// next chunk's rows are loaded into registers while the current one is
// multiplied.  Within a row the values are permuted so that each lane's
// operands are contiguous: K element d sits at (d % 4) HD/4 + d / 4 (a
// lane reads the k-steps of its k index with 128-bit reads) and V element d
// at (d % 16) HD/16 + d / 16 (one read gives a lane its value of every
// output dim tile).  Row stride HD + 4 keeps both reads free of bank
// conflicts on 32 banks.
template <int HD>
__global__ __launch_bounds__(256, 2) void k_attn_flash_mfma(
    const float* __restrict__ q, int64_t q_ts, int64_t tokens, int64_t nq, int64_t nkv,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int64_t cap,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, float* __restrict__ out,
    int64_t o_ts, int8_t* __restrict__ oq, uint16_t* __restrict__ od,
    const int32_t* __restrict__ order) {
    constexpr int NS = HD / 4;     // k-steps of the score product (dims)
    constexpr int NDT = HD / 16;   // dim tiles of the output
    constexpr int KS = HD + 4, VS = HD + 4;
    constexpr int KQ = HD / 4, VQ = HD / 16;   // permuted row: K by k index, V by dim tile
    constexpr int KVPER = ACH * HD / 8 / 256;   // 8-value chunks of K (and of V) per thread
    __shared__ __align__(16) float ks[2][ACH][KS];
    __shared__ __align__(16) float vs[2][ACH][VS];

    const int G = (int)(nq / nkv);
    const int TQ = 64 / G;   // tokens per workgroup
    // workgroup rank * nkv + KV head: the tile of that rank in the
    // longest-first order, every KV head of a tile one after another, so
    // that the tiles that walk the most chunks start first
    const int64_t g = blockIdx.x % nkv;
    const int64_t t0 = (int64_t)__builtin_amdgcn_readfirstlane(order[blockIdx.x / nkv]) * TQ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntile = (int)min((int64_t)TQ, tokens - t0);
    const int qr = 16 * wave + (lane & 15);            // this lane's query row
    const int qi = qr / G, qh = qr % G;                // its token and head
    const bool qvalid = qr < TQ * G && qi < ntile;
    const int kq = lane >> 4;                          // lane's k index (0..3)
    const double rscale = sqrt((double)HD);

    // The tile's sequence ids and positions, read once into LDS: the scans
    // below would otherwise wait for one load after another.
    __shared__ int tseq[64], tpos[64];
    if (tid < ntile) {
        tseq[tid] = seq[t0 + tid];
        tpos[tid] = pos[t0 + tid];
    }
    __syncthreads();

    for (int i0 = 0; i0 < ntile;) {   // runs of one sequence (uniform)
        const int s0 = tseq[i0];
        int i1 = i0 + 1;
        while (i1 < ntile && tseq[i1] == s0) ++i1;
        // row limits: the last ring row attended (-1: nothing)
        int kmax = -1;
        for (int i = i0; i < i1; ++i) {
            const int p = tpos[i];
            if (p >= 0) kmax = max(kmax, (int)min((int64_t)p, cap - 1));
        }
        const bool mine = qvalid && qi >= i0 && qi < i1;
        int pl = -1;
        if (mine) {
            const int p = tpos[qi];
            pl = p >= 0 ? (int)min((int64_t)p, cap - 1) : -1;
        }
        // q loads from a clamped index (row t0, head g G when the lane has no
        // query row), all issued before any of them is used
        const int64_t qoff = mine ? (t0 + qi) * q_ts + (g * G + qh) * HD : t0 * q_ts + g * G * HD;
        double qT[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const float qv = q[qoff + 4 * st + kq];
            qT[st] = mine ? (double)qv : 0.0;
        }

        double m = -INFINITY, lsum = 0.0;
        v4d o[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = v4d{0.0, 0.0, 0.0, 0.0};

        const int64_t cbase = (((int64_t)s0 * nkv + g) * cap) * HD;
        uint4 pk[KVPER], pv[KVPER];   // rows of the next chunk, in flight
        auto gload_kv = [&](int r0) {
#pragma unroll
            for (int e = 0; e < KVPER; ++e) {
                const int i = tid + 256 * e;
                const int r = (i * 8) / HD, d = (i * 8) % HD;
                pk[e] = make_uint4(0, 0, 0, 0);
                pv[e] = make_uint4(0, 0, 0, 0);
                if (r0 + r <= kmax) {
                    pk[e] = *reinterpret_cast<const uint4*>(kc + cbase + (int64_t)(r0 + r) * HD + d);
                    pv[e] = *reinterpret_cast<const uint4*>(vc + cbase + (int64_t)(r0 + r) * HD + d);
                }
            }
        };
        auto sstore_kv = [&](int buf) {
#pragma unroll
            for (int e = 0; e < KVPER; ++e) {
                const int i = tid + 256 * e;
                const int r = (i * 8) / HD, d = (i * 8) % HD;
                const uint32_t kw[4] = {pk[e].x, pk[e].y, pk[e].z, pk[e].w};
                const uint32_t vw[4] = {pv[e].x, pv[e].y, pv[e].z, pv[e].w};
                float kf[8], vf[8];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    kf[2 * f] = h2f((uint16_t)(kw[f] & 0xFFFF));
                    kf[2 * f + 1] = h2f((uint16_t)(kw[f] >> 16));
                    vf[2 * f] = h2f((uint16_t)(vw[f] & 0xFFFF));
                    vf[2 * f + 1] = h2f((uint16_t)(vw[f] >> 16));
                }
                // K: dims d + j (d % 8 == 0) go to (j % 4) KQ + d / 4 + j / 4
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    *reinterpret_cast<float2*>(&ks[buf][r][f * KQ + d / 4]) = make_float2(kf[f], kf[f + 4]);
                // V: dims d + j go to ((d + j) % 16) VQ + d / 16
#pragma unroll
                for (int j = 0; j < 8; ++j) vs[buf][r][((d + j) % 16) * VQ + d / 16] = vf[j];
            }
        };
        if (kmax >= 0) {
            __syncthreads();   // the previous run is done with both buffers
            gload_kv(0);
            sstore_kv(0);
            __syncthreads();
        }
        for (int c = 0; c * ACH <= kmax; ++c) {
            const int r0 = c * ACH;
            const int cur = c & 1;
            const bool more = (c + 1) * ACH <= kmax;   // uniform
            if (more) gload_kv(r0 + ACH);

            // S^T for 4 key tiles: C[key][row], key = 16 kt + 4 v + kq
            v4d sc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sc[kt] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s4 = 0; s4 < NS; s4 += 4) {   // four k-steps per 128-bit read
                float4 kv[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    kv[kt] = *reinterpret_cast<const float4*>(&ks[cur][16 * kt + (lane & 15)][kq * KQ + s4]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) {
                        const float a = i == 0 ? kv[kt].x : (i == 1 ? kv[kt].y : (i == 2 ? kv[kt].z : kv[kt].w));
                        sc[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a, qT[s4 + i], sc[kt], 0, 0, 0);
                    }
            }
            // mask, scale and the chunk's row max (the row's 64 keys sit in
            // this lane's 16 registers and lanes l ^ 16, l ^ 32, l ^ 48)
            double cm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int key = r0 + 16 * kt + 4 * v + kq;
                    const double sv = key <= pl ? sc[kt][v] / rscale : -INFINITY;
                    sc[kt][v] = sv;
                    cm = fmax(cm, sv);
                }
            cm = fmax(cm, __shfl_xor(cm, 16, WAVE));
            cm = fmax(cm, __shfl_xor(cm, 32, WAVE));
            const bool live = cm != -INFINITY;
            const double mn = live ? fmax(m, cm) : m;
            const double f = live ? exp(m - mn) : 1.0;   // 0 when m was -inf
            double rs = 0.0;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const double pv = sc[kt][v] != -INFINITY ? exp(sc[kt][v] - mn) : 0.0;
                    sc[kt][v] = pv;
                    rs += pv;
                }
            rs += __shfl_xor(rs, 16, WAVE);
            rs += __shfl_xor(rs, 32, WAVE);
            if (live) {
                lsum = fma(lsum, f, rs);
                m = mn;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) o[dt] *= f;
            }
            // O^T += V^T P^T: key step 4 kt + v takes register v of tile kt
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    // this lane's value of every dim tile: one read (NDT = 4
                    // or 2 contiguous floats)
                    const float* vr = &vs[cur][16 * kt + 4 * v + kq][(lane & 15) * VQ];
                    float va[NDT];
                    if constexpr (NDT == 4) {
                        const float4 t = *reinterpret_cast<const float4*>(vr);
                        va[0] = t.x; va[1] = t.y; va[2] = t.z; va[3] = t.w;
                    } else {
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) va[dt] = vr[dt];
                    }
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
                        o[dt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)va[dt], sc[kt][v], o[dt], 0, 0, 0);
                }
            if (more) sstore_kv(cur ^ 1);   // read two chunks ago, past the last barrier
            __syncthreads();
        }

        // outputs of the run: this lane holds dims 16 dt + 4 v + kq of its row
        float ov[NDT][4];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) ov[dt][v] = lsum > 0.0 ? (float)(o[dt][v] / lsum) : 0.0f;
        const int64_t col = (t0 + qi) * o_ts + (g * G + qh) * HD;
        if (out && mine) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int v = 0; v < 4; ++v) out[col + 16 * dt + 4 * v + kq] = ov[dt][v];
        }
        if (oq) {
            // Q8_0 block b of the row: dim tiles 2b, 2b + 1 over the four
            // lanes of the row
#pragma unroll
            for (int b = 0; b < HD / QBLK; ++b) {
                float amax = 0.0f;
#pragma unroll
                for (int dt = 2 * b; dt < 2 * b + 2; ++dt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(ov[dt][v]));
                amax = fmaxf(amax, __shfl_xor(amax, 16, WAVE));
                amax = fmaxf(amax, __shfl_xor(amax, 32, WAVE));
                const float d = amax / 127.0f;
                if (mine) {
#pragma unroll
                    for (int dt = 2 * b; dt < 2 * b + 2; ++dt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            int qv = 0;
                            if (d != 0.0f) qv = (int)fminf(127.0f, fmaxf(-127.0f, roundf(ov[dt][v] / d)));
                            oq[col + 16 * dt + 4 * v + kq] = (int8_t)qv;
                        }
                    if (kq == 0) od[(col + b * QBLK) / QBLK] = f2h(d);
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
        if (hd != 32 && hd != 64) return QK_ESHAPE;
        const int64_t tq = 64 / (nq / nkv);   // tokens per workgroup of the matrix-core pass
        const int64_t ntiles = (tokens + tq - 1) / tq;
        if (ntiles * nkv > INT32_MAX) return QK_ESHAPE;
        // the tile order sits at the start of the workspace (the chunk
        // records of the few-token pass are not used here; they take at
        // least 34 bytes per token, the order 4 per tile)
        int32_t* order = static_cast<int32_t*>(ws);
        hipLaunchKernelGGL(k_tile_order, dim3(1), dim3(1024), 0, s, pos, tokens, (int)tq, cap, (int)nch,
                           (int)ntiles, order);
        dim3 fgrid((unsigned)(nkv * ntiles));
        if (hd == 32)
            hipLaunchKernelGGL(k_attn_flash_mfma<32>, fgrid, dim3(256), 0, s, q, q_ts, tokens, nq, nkv,
                               kc, vc, cap, pos, seq, out, o_ts, oq, od, order);
        else
            hipLaunchKernelGGL(k_attn_flash_mfma<64>, fgrid, dim3(256), 0, s, q, q_ts, tokens, nq, nkv,
                               kc, vc, cap, pos, seq, out, o_ts, oq, od, order);
        return qk_launch_status();
    }
    double* rec = static_cast<double*>(ws);
    // caches of 256 chunks or more (16384 rows): LCPW chunks per chunk-pass
    // workgroup, one record for them
    static_assert(LCPW == 4, "the merge's CPW_LOG2 below");
    const bool lng = nch >= 256;
    const int64_t nrec = lng ? (nch + LCPW - 1) / LCPW : nch;   // records per head
    dim3 grid((unsigned)nrec, (unsigned)nkv, (unsigned)tokens);
    dim3 mgrid((unsigned)nq, (unsigned)tokens);
    dim3 mgrid2((unsigned)nq, (unsigned)tokens, 2u);
    // the merge: one wave per head for up to 64 records per head (4096 rows,
    // or 16384 with the long pass); head dim 64 with up to 128 records (the
    // 8192- and 32768-row rings): two waves per head, 32 dims each; more
    // records, or head dim 32 past 64: k_attn_merge (a one-wave form with
    // two records per lane measured slower at 8192 and 32768 rows)
    auto merge = [&](auto hdc, auto cpw) {
        constexpr int HD = decltype(hdc)::value, CPW = decltype(cpw)::value;
        if (nrec <= MERGE_W_CHUNKS) {
            hipLaunchKernelGGL((k_attn_merge_w<HD, CPW>), mgrid, dim3(64), 0, s, rec, nq, nrec, cap, pos,
                               out, o_ts, oq, od);
        } else if constexpr (HD == 64) {   // two waves per head, 32 dims each
            if (nrec <= 2 * MERGE_W_CHUNKS)
                hipLaunchKernelGGL((k_attn_merge_w2<CPW>), mgrid2, dim3(64), 0, s, rec, nq, nrec, cap, pos,
                                   out, o_ts, oq, od);
            else
                hipLaunchKernelGGL((k_attn_merge<HD, 2, CPW>), mgrid2, dim3(256), 0, s, rec, nq, nrec, cap, pos,
                                   out, o_ts, oq, od);
        } else {
            hipLaunchKernelGGL((k_attn_merge<HD, 1, CPW>), mgrid, dim3(256), 0, s, rec, nq, nrec, cap, pos,
                               out, o_ts, oq, od);
        }
    };
    using C0 = std::integral_constant<int, 0>;
    using C2 = std::integral_constant<int, 2>;
    if (hd == 32) {
        using H = std::integral_constant<int, 32>;
        if (lng) {
            hipLaunchKernelGGL(k_attn_chunk_long<32>, grid, dim3(512), 0, s, q, q_ts, nq, nkv, kc, vc,
                               cap, pos, seq, rec, nrec);
            merge(H{}, C2{});
        } else {
            hipLaunchKernelGGL(k_attn_chunk<32>, grid, dim3(512), 0, s, q, q_ts, nq, nkv, kc, vc, cap,
                               pos, seq, rec, nch);
            merge(H{}, C0{});
        }
    } else if (hd == 64) {
        using H = std::integral_constant<int, 64>;
        if (lng) {
            hipLaunchKernelGGL(k_attn_chunk_long<64>, grid, dim3(512), 0, s, q, q_ts, nq, nkv, kc, vc,
                               cap, pos, seq, rec, nrec);
            merge(H{}, C2{});
        } else {
            hipLaunchKernelGGL(k_attn_chunk<64>, grid, dim3(512), 0, s, q, q_ts, nq, nkv, kc, vc, cap,
                               pos, seq, rec, nch);
            merge(H{}, C0{});
        }
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
