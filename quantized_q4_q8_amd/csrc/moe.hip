// Routed mixture-of-experts layer with every expert resident in HBM.
//
// kerneldigest.dev, "Colibri: running 744B MoE models on consumer hardware
// by streaming experts": a sigmoid router of the DeepSeek-V3 kind picks the
// experts (System architecture; token flow step 2), the experts run int8
// activation x int4 weight kernels (step 5) and their results are combined
// into the token (step 6).  Each expert is a SwiGLU FFN (kenji.blog
// TinyLLaMA-in-C++ guide, section 4.4).
//
// Pipeline (all on the caller's stream, deterministic, no float atomics):
//  1. router logits r = x . W_r in fp64, H split into slices whose partial
//     sums are added in a fixed order, rounded to fp32;
//  2. per token: top-k on r (ties to the lower expert), sigmoid scores,
//     weights normalized over the selection;
//  3. stable counting sort of the (token, rank) pairs by expert -> per-expert
//     column ranges, the token of every sorted column, and each pair's slot;
//  4. Q8_0 of x; grouped gate/up matmul with the SwiGLU epilogue over the
//     sorted columns; Q8_0 of h; grouped down matmul.  In calls averaging
//     at least 16 tokens per expert (Q4_0 experts), an expert with at least
//     16 tokens runs on the int8 matrix cores (grouped MFMA GEMM) and the
//     others on the grouped GEMV; otherwise the GEMV takes them all;
//  5. per token, sum over ranks 0..k-1 of weight * expert output, in order.
#include "internal.h"

namespace qk {

namespace {

constexpr int RT = 4;        // tokens per router workgroup
constexpr int RSLICE = 128;  // hidden elements per router slice: all its loads issue together
constexpr int MFMA_MIN_COLS = 16;   // tokens from which an expert takes the grouped MFMA GEMM
constexpr int MFMA_MIN_AVG = 16;    // ... when the call averages this many tokens per expert

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct MoeWs {
    double* rpart;      // [slices][T][E]
    int32_t* off;       // [E + 1]
    int32_t* col_tok;   // [P] token of each sorted column
    int32_t* slot;      // [P] sorted column of pair p = t * k + rank
    int32_t* big;       // [1 + E]: the count, then the experts of at least MFMA_MIN_COLS tokens
    int8_t* xq;         // [T][H]
    uint16_t* xd;       // [T][H/32]
    float* h;           // [P][F]
    int8_t* hq;         // [P][F]
    uint16_t* hd;       // [P][F/32]
    float* ys;          // [P][H]
    size_t total;
};

MoeWs moe_layout(void* base, int64_t T, int64_t H, int64_t E, int64_t k, int64_t F) {
    const int64_t P = T * k;
    const int64_t slices = (H + RSLICE - 1) / RSLICE;
    MoeWs w{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return base ? static_cast<char*>(base) + at : nullptr;
    };
    w.rpart = reinterpret_cast<double*>(take(sizeof(double) * slices * T * E));
    w.off = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
    w.col_tok = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * P));
    w.slot = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * P));
    w.big = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
    w.xq = reinterpret_cast<int8_t*>(take((size_t)(T * H)));
    w.xd = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * T * (H / QBLK)));
    w.h = reinterpret_cast<float*>(take(sizeof(float) * P * F));
    w.hq = reinterpret_cast<int8_t*>(take((size_t)(P * F)));
    w.hd = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * P * (F / QBLK)));
    w.ys = reinterpret_cast<float*>(take(sizeof(float) * P * H));
    w.total = o;
    return w;
}

}  // namespace

// rpart[s][t][e] = sum over h in slice s of x[t][h] * W_r[h][e]; thread = expert.
__global__ __launch_bounds__(256) void k_router(const float* __restrict__ x, int64_t T, int64_t H,
                                                const float* __restrict__ wr, int64_t E,
                                                double* __restrict__ rpart) {
    __shared__ float xs[RT][RSLICE];
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * RT;
    const int64_t s = blockIdx.z;
    const int64_t h0 = s * RSLICE;
    const int64_t hn = min((int64_t)RSLICE, H - h0);
    for (int64_t i = threadIdx.x; i < RT * RSLICE; i += 256) {
        const int64_t tt = i / RSLICE, hh = i % RSLICE;
        xs[tt][hh] = (t0 + tt < T && hh < hn) ? x[(t0 + tt) * H + h0 + hh] : 0.0f;
    }
    __syncthreads();
    if (e >= E) return;
    double acc[RT];
#pragma unroll
    for (int tt = 0; tt < RT; ++tt) acc[tt] = 0.0;
    const float* __restrict__ wcol = wr + h0 * E + e;
    if (hn == RSLICE) {
        // every load of the slice first (unconditional), so one memory
        // latency covers the slice
        float w[RSLICE];
#pragma unroll
        for (int q = 0; q < RSLICE; ++q) w[q] = wcol[(int64_t)q * E];
#pragma unroll
        for (int q = 0; q < RSLICE; ++q)
#pragma unroll
            for (int tt = 0; tt < RT; ++tt) acc[tt] = fma((double)xs[tt][q], (double)w[q], acc[tt]);
    } else {   // ragged last slice
        for (int h1 = 0; h1 < (int)hn; ++h1) {
            const double w = wcol[(int64_t)h1 * E];
#pragma unroll
            for (int tt = 0; tt < RT; ++tt) acc[tt] = fma((double)xs[tt][h1], w, acc[tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < RT; ++tt)
        if (t0 + tt < T) rpart[(s * T + t0 + tt) * E + e] = acc[tt];
}

// One workgroup (1024 threads) per token: r[e] from the slice partials,
// then the top k in one pass: expert e's rank is the number of experts that
// come before it in the order (value descending, lower index first among
// equal values, NaN after every number and among NaNs by index), which is
// the order of repeated maxima over the experts not yet taken; the expert
// with rank < k goes to slot `rank`.  Sigmoid weights are normalized over
// the choice (the sum in rank order).
//
// Thread (g, e) of G groups sums slices g, g + G, ... for expert e, and then
// counts the experts j of its quarter (g-th G-th) of the index range that
// come before e; both are added over the groups in group order.  Values are
// compared as order-preserving integer keys: NaN is 0, below every number,
// and -0 and +0 share a key.
__device__ __forceinline__ uint32_t route_key(float v) {
    if (v != v) return 0u;
    const uint32_t b = __float_as_uint(v + 0.0f);   // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ rpart, int64_t slices,
                                               int64_t T, int64_t E, int32_t k,
                                               int32_t* __restrict__ sel_idx,
                                               float* __restrict__ sel_w) {
    __shared__ float rv[1024];
    __shared__ __align__(16) uint32_t key[1024];
    __shared__ double part[1024];
    __shared__ int prank[1024];
    __shared__ int chosen[32];
    __shared__ double sg[32];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int ep = (int)((E + WAVE - 1) / WAVE) * WAVE;   // experts rounded to waves
    const int G = 1024 / ep;
    const int g = tid / ep, e = tid % ep;
    const bool act = g < G && e < E;
    if (act) {   // eight loads in flight at a time
        double r = 0.0;
        int64_t s = g;
        for (; s + 7 * G < slices; s += 8 * G) {
            double v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = rpart[((s + i * G) * T + t) * E + e];
#pragma unroll
            for (int i = 0; i < 8; ++i) r += v[i];
        }
        for (; s < slices; s += G) r += rpart[(s * T + t) * E + e];
        part[g * ep + e] = r;
    }
    __syncthreads();
    if (tid < E) {
        double r = 0.0;
        for (int q = 0; q < G; ++q) r += part[q * ep + tid];
        rv[tid] = (float)r;
        key[tid] = route_key((float)r);
    }
    __syncthreads();
    if (act) {
        const uint32_t ke = key[e];
        const int per = ((ep + G - 1) / G + 3) & ~3;   // this group's index range, a multiple of 4
        const int j0 = g * per, j1 = min((int)E, j0 + per);
        int rank = 0;
        for (int j4 = j0; j4 < j1; j4 += 4) {   // four keys per read (j1 <= E <= 1024)
            const uint4 q = *reinterpret_cast<const uint4*>(&key[j4]);
            const uint32_t kq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = j4 + i;
                rank += (j < j1 && (kq[i] > ke || (kq[i] == ke && j < e))) ? 1 : 0;
            }
        }
        prank[g * ep + e] = rank;
    }
    __syncthreads();
    if (tid < E) {
        int rank = 0;
        for (int q = 0; q < G; ++q) rank += prank[q * ep + tid];
        if (rank < k) chosen[rank] = tid;
    }
    __syncthreads();
    if (tid < k) sg[tid] = 1.0 / (1.0 + exp(-(double)rv[chosen[tid]]));
    __syncthreads();
    if (tid == 0) {
        double ssum = 0.0;
        for (int kk = 0; kk < k; ++kk) ssum += sg[kk];
        for (int kk = 0; kk < k; ++kk) {
            sel_idx[t * k + kk] = chosen[kk];
            sel_w[t * k + kk] = (float)(sg[kk] / ssum);
        }
    }
}

// Stable counting sort of the P = T * k pairs by expert (one workgroup of
// 1024 threads).  Counts by LDS atomics; the expert offsets by a workgroup
// scan (thread e owns expert e).  Pairs are then taken in chunks of 1024 in
// pair order; a pair's column is off[e] + (pairs of e in earlier chunks) +
// (pairs of e earlier in its chunk), so columns of an expert follow
// (token, rank) order.
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ sel_idx, int64_t P,
                                                int32_t k, int64_t E, int32_t* __restrict__ off,
                                                int32_t* __restrict__ col_tok,
                                                int32_t* __restrict__ slot, int32_t* __restrict__ big,
                                                int min_cols) {
    __shared__ int cnt[1024];
    __shared__ int base[1024];
    __shared__ __align__(16) int chunk_e[1024];
    __shared__ int wsum[16];
    __shared__ int nbig;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < E) cnt[tid] = 0;
    if (tid == 0) nbig = 0;
    __syncthreads();
    for (int64_t p = tid; p < P; p += 1024) atomicAdd(&cnt[sel_idx[p]], 1);
    __syncthreads();
    // the experts with at least min_cols tokens, in any order (each one's
    // result does not depend on the others)
    if (tid < E && cnt[tid] >= min_cols) big[1 + atomicAdd(&nbig, 1)] = tid;
    // exclusive scan of the counts: inclusive within each wave, then the
    // totals of the waves before
    const int c = tid < E ? cnt[tid] : 0;
    int inc = c;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (lane == WAVE - 1) wsum[wave] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + inc - c;
    if (tid < E) {
        off[tid] = excl;
        base[tid] = excl;
        if (tid == E - 1) off[E] = excl + c;
    }
    __syncthreads();
    if (tid == 0) big[0] = nbig;
    for (int64_t c0 = 0; c0 < P; c0 += 1024) {
        const int64_t p = c0 + tid;
        const int n = (int)min((int64_t)1024, P - c0);
        const int e = p < P ? sel_idx[p] : -1;
        chunk_e[tid] = e;
        __syncthreads();
        if (p < P) {
            int rank = 0;
            int q = 0;
            for (; q + 4 <= tid; q += 4) {   // four entries per read
                const int4 v = *reinterpret_cast<const int4*>(&chunk_e[q]);
                rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
            }
            for (; q < tid; ++q) rank += chunk_e[q] == e;
            const int col = base[e] + rank;
            col_tok[col] = (int32_t)(p / k);
            slot[p] = col;
        }
        __syncthreads();   // every pair of the chunk has read base
        if (tid < n) atomicAdd(&base[e], 1);
        __syncthreads();
    }
}

// out[t][i] = sum_{r < k} sel_w[t][r] * ys[slot[t k + r]][i], ranks in order.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ys, int64_t H, int32_t k,
                                                 const int32_t* __restrict__ slot,
                                                 const float* __restrict__ sel_w,
                                                 float* __restrict__ out) {
    const int64_t t = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= H) return;
    double acc = 0.0;
    for (int r = 0; r < k; ++r)
        acc = fma((double)sel_w[t * k + r], (double)ys[(int64_t)slot[t * k + r] * H + i], acc);
    out[t * H + i] = (float)acc;
}

}  // namespace qk

using namespace qk;

extern "C" size_t qk_moe_workspace(int64_t tokens, int64_t hidden, int64_t n_experts,
                                   int32_t top_k, int64_t ffn) {
    if (tokens < 0 || hidden <= 0 || n_experts <= 0 || top_k <= 0 || ffn <= 0) return 0;
    return moe_layout(nullptr, tokens, hidden, n_experts, top_k, ffn).total;
}

namespace {

// Expert weights of one format, stacked over the experts.
struct ExpertWeights {
    int fmt;                   // FMT_Q4_0, FMT_Q4_ROW or FMT_Q2_ROW
    const uint8_t* gu_q;       // [E][2F] rows of H weights
    const void* gu_s;          // Q4_0: fp16 [E][2F][H/32]; row-scaled: fp32 [E][2F]
    const uint8_t* dn_q;       // [E][H] rows of F weights
    const void* dn_s;          // Q4_0: fp16 [E][H][F/32]; row-scaled: fp32 [E][H]
};

int moe_apply(const float* x, int64_t tokens, int64_t hidden, const float* w_router,
              int64_t n_experts, int32_t top_k, const ExpertWeights& ew, int64_t ffn, float* y,
              int32_t* sel_idx, float* sel_w, void* ws, size_t ws_bytes, hipStream_t s) {
    QK_REQUIRE(tokens >= 0 && hidden > 0 && ffn > 0, QK_EINVAL);
    QK_REQUIRE(n_experts > 0 && n_experts <= 1024 && top_k > 0 && top_k <= 32 &&
                   top_k <= n_experts,
               QK_EINVAL);
    QK_REQUIRE(hidden % QBLK == 0 && ffn % QBLK == 0, QK_ESHAPE);
    QK_REQUIRE(tokens * top_k <= INT32_MAX, QK_EINVAL);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(x && w_router && ew.gu_q && ew.gu_s && ew.dn_q && ew.dn_s && y && sel_idx && sel_w,
               QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(x, 16) && QK_ALIGNED(y, 16) && QK_ALIGNED(ew.gu_q, 16) &&
                   QK_ALIGNED(ew.dn_q, 16) && QK_ALIGNED(ew.gu_s, ew.fmt == FMT_Q4_0 ? 2 : 4) &&
                   QK_ALIGNED(ew.dn_s, ew.fmt == FMT_Q4_0 ? 2 : 4),
               QK_EALIGN);
    const MoeWs w = moe_layout(ws, tokens, hidden, n_experts, top_k, ffn);
    QK_REQUIRE(ws && ws_bytes >= w.total, QK_EWORKSPACE);
    const int64_t T = tokens, H = hidden, E = n_experts, F = ffn, P = T * top_k;
    const int64_t slices = (H + RSLICE - 1) / RSLICE;
    const int64_t bpb = ew.fmt == FMT_Q2_ROW ? 8 : 16;   // weight bytes per 32-block

    hipLaunchKernelGGL(k_router, dim3((unsigned)((E + 255) / 256), (unsigned)((T + RT - 1) / RT),
                                      (unsigned)slices),
                       dim3(256), 0, s, x, T, H, w_router, E, w.rpart);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)T), dim3(1024), 0, s, w.rpart, slices, T, E, top_k,
                       sel_idx, sel_w);
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, sel_idx, P, top_k, E, w.off, w.col_tok,
                       w.slot, w.big, MFMA_MIN_COLS);
    int rc = launch_quantize_q8(x, T, H, w.xq, w.xd, s);
    if (rc) return rc;

    GemvArgs g{};
    g.fmt = ew.fmt; g.wq = ew.gu_q; g.n = 2 * F; g.k = H;
    g.wq_gstride = 2 * F * (H / QBLK) * bpb;
    if (ew.fmt == FMT_Q4_0) {
        g.wd = static_cast<const uint16_t*>(ew.gu_s); g.wd_gstride = 2 * F * (H / QBLK);
    } else {
        g.wr = static_cast<const float*>(ew.gu_s); g.wr_gstride = 2 * F;
    }
    g.xq = w.xq; g.xd = w.xd; g.col_off = w.off; g.col_idx = w.col_tok;
    g.m = 0; g.groups = (int32_t)E; g.y = w.h; g.ldy = F; g.residual = nullptr; g.ldr = 0;
    g.ffn = F; g.max_cols = (int32_t)std::min<int64_t>(8, (P + E - 1) / E);
    // Experts with at least MFMA_MIN_COLS tokens run on the int8 matrix
    // cores (grouped GEMM), the others on the grouped GEMV; the split is read
    // from the grouping on the device, so both launches go out and each
    // skips the other's experts.  An expert has at most T tokens.
    // The GEMM's grid covers the list of such experts that the grouping
    // writes: at most P / MFMA_MIN_COLS of them.  Below an average of
    // MFMA_MIN_AVG tokens per expert few experts are that large, and the two
    // launches cost more than they save (1.5 % of a 64-token, 256-expert
    // layer that has none, 1.2 % at 256 tokens): the GEMV takes every expert.
    const bool mfma = ew.fmt == FMT_Q4_0 && T >= MFMA_MIN_COLS && P >= (int64_t)MFMA_MIN_AVG * E;
    const int64_t max_big = std::min<int64_t>(E, P / MFMA_MIN_COLS);
    g.skip_cols_ge = mfma ? MFMA_MIN_COLS : 0;
    g.min_cols = MFMA_MIN_COLS;
    g.group_list = w.big;
    rc = expert_gemv_fits(g) ? launch_expert_gemv(g, EPI_SWIGLU, s) : launch_gemv(g, EPI_SWIGLU, s);
    if (rc) return rc;
    if (mfma && (rc = launch_gemm(g, EPI_SWIGLU, s, T, max_big))) return rc;
    rc = launch_quantize_q8(w.h, P, F, w.hq, w.hd, s);
    if (rc) return rc;

    GemvArgs d{};
    d.fmt = ew.fmt; d.wq = ew.dn_q; d.n = H; d.k = F;
    d.wq_gstride = H * (F / QBLK) * bpb;
    if (ew.fmt == FMT_Q4_0) {
        d.wd = static_cast<const uint16_t*>(ew.dn_s); d.wd_gstride = H * (F / QBLK);
    } else {
        d.wr = static_cast<const float*>(ew.dn_s); d.wr_gstride = H;
    }
    d.xq = w.hq; d.xd = w.hd; d.col_off = w.off; d.col_idx = nullptr;
    d.m = 0; d.groups = (int32_t)E; d.y = w.ys; d.ldy = H; d.residual = nullptr; d.ldr = 0;
    d.ffn = 0; d.max_cols = g.max_cols;
    d.skip_cols_ge = g.skip_cols_ge;
    d.min_cols = MFMA_MIN_COLS;
    d.group_list = w.big;
    rc = expert_gemv_fits(d) ? launch_expert_gemv(d, EPI_STORE, s) : launch_gemv(d, EPI_STORE, s);
    if (rc) return rc;
    if (mfma && (rc = launch_gemm(d, EPI_STORE, s, T, max_big))) return rc;

    hipLaunchKernelGGL(k_combine, dim3((unsigned)((H + 255) / 256), (unsigned)T), dim3(256), 0, s,
                       w.ys, H, top_k, w.slot, sel_w, y);
    return qk_launch_status();
}

}  // namespace

extern "C" int moe_route_and_apply(const float* x, int64_t tokens, int64_t hidden,
                                   const float* w_router, int64_t n_experts, int32_t top_k,
                                   const uint8_t* gate_up_q, const uint16_t* gate_up_d,
                                   const uint8_t* down_q, const uint16_t* down_d, int64_t ffn,
                                   float* y, int32_t* sel_idx, float* sel_w, void* ws,
                                   size_t ws_bytes, void* stream) {
    const ExpertWeights ew{FMT_Q4_0, gate_up_q, gate_up_d, down_q, down_d};
    return moe_apply(x, tokens, hidden, w_router, n_experts, top_k, ew, ffn, y, sel_idx, sel_w, ws,
                     ws_bytes, (hipStream_t)stream);
}

extern "C" int qk_moe_route_and_apply_rowq(int32_t bits, const float* x, int64_t tokens,
                                           int64_t hidden, const float* w_router,
                                           int64_t n_experts, int32_t top_k,
                                           const uint8_t* gate_up_q, const float* gate_up_r,
                                           const uint8_t* down_q, const float* down_r,
                                           int64_t ffn, float* y, int32_t* sel_idx, float* sel_w,
                                           void* ws, size_t ws_bytes, void* stream) {
    QK_REQUIRE(bits == 4 || bits == 2, QK_EINVAL);
    const ExpertWeights ew{bits == 4 ? FMT_Q4_ROW : FMT_Q2_ROW, gate_up_q, gate_up_r, down_q, down_r};
    return moe_apply(x, tokens, hidden, w_router, n_experts, top_k, ew, ffn, y, sel_idx, sel_w, ws,
                     ws_bytes, (hipStream_t)stream);
}
