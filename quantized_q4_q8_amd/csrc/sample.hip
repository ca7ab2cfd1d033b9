// Sampler chain: from logits to the next token.
//
// kenji.blog TinyLLaMA-in-C++ guide, section 8 (the logits' probabilities are
// scaled by a temperature, Top-K or Top-P narrows the candidates, and a random
// number picks the token) and the llama.cpp guide, section 5.4 (the chain
// top-k, top-p keeping at least one, temperature, then a seeded draw).
//
// One workgroup of 1024 threads per row; each thread holds up to 32 of the
// row's logits in registers (one coalesced load round, 16-byte loads when the
// row allows).  The top_k set is found without sorting the row:
//  - a lower bound for the top_k-th largest logit.  For top_k <= 48 it is the
//    top_k-th largest of 64 group maxima (16 threads x 32 logits per group),
//    picked by wave 0; for larger top_k, each wave picks the
//    ceil(top_k / 16)-th largest of its 64 per-thread maxima and the bound is
//    the least of the 16.  Either way at least top_k distinct logits reach it;
//    the picks are bitwise selects with wave ballots;
//  - the logits at or above the bound (for spread logits about 1.5x top_k
//    when top_k <= 48, a few times top_k beyond) are gathered in LDS, one
//    atomic per wave, and each is ranked by counting the ones before it
//    (logit descending, then id ascending);
//  - when more than 1024 logits reach the bound (heavy ties), an exact radix
//    select over all keys (8-bit passes, LDS histograms) gives the top_k-th
//    largest key, and a second one over the ids of the keys equal to it how
//    far the lowest ids go; exactly top_k keys are then gathered and ranked.
// The weights of the ranked candidates are formed in parallel, then wave 0
// holds four ranks per lane and takes the sums and running sums of the chain
// in fp64 with DPP scans.
#include "internal.h"

namespace qk {

namespace {

constexpr int MAXK = 256;
constexpr int NT = 1024;
constexpr int KPT = 32;                 // keys per thread: vocab <= 32768
constexpr int CR = 1024;                // candidate capacity of the fast path
constexpr int NWV = NT / WAVE;          // waves per workgroup
constexpr int GROUP_K = 48;             // largest top_k bounded by group maxima
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_WAVE_SHR1 = 0x138, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;
static_assert(CR == NT, "one candidate slot per thread");

// Monotone map of float bits to unsigned order (finite values).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t b = __builtin_bit_cast(uint32_t, f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t t = __shfl_up(v, off, WAVE);
        if (lane >= off) v += t;
    }
    return v;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_rows(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_rows<CTRL, ROWS>((uint32_t)b), hi = dpp_rows<CTRL, ROWS>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the wave with DPP: shifts of 1, 2, 4, 8 inside
// each row of 16 lanes (lanes past the row start add zero), then the row
// totals carried forward by the broadcasts of lanes 15 and 31.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    v += dpp_rows<DPP_ROW_SHR1, 0xF>(v);
    v += dpp_rows<DPP_ROW_SHR2, 0xF>(v);
    v += dpp_rows<DPP_ROW_SHR4, 0xF>(v);
    v += dpp_rows<DPP_ROW_SHR8, 0xF>(v);
    v += dpp_rows<DPP_ROW_BCAST15, 0xA>(v);
    v += dpp_rows<DPP_ROW_BCAST31, 0xC>(v);
    return v;
}

// The value of the previous lane (zero in lane 0).
__device__ __forceinline__ double wave_prev(double v) { return dpp_rows<DPP_WAVE_SHR1, 0xF>(v); }

__device__ __forceinline__ int wave_min(int v) { return -group_max<WAVE>(-v); }

// The m-th largest of the wave's 64 lane values (1 <= m <= 64), bit by bit
// from the top with ballots; uniform across the wave.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, uint32_t m) {
    uint64_t live = ~0ull;
    uint32_t val = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint64_t ones = __ballot((v >> bit) & 1u) & live;
        const uint32_t c = (uint32_t)__popcll(ones);
        if (c >= m) {
            live = ones;
            val |= 1u << bit;
        } else {
            m -= c;
            live &= ~ones;
        }
    }
    return val;
}

// Radix select step over 8 bits, run by wave 0: the bin holding the need-th
// value in selection order (largest bin first when from_top) and the rank
// left inside it.  Lane L scans positions 4L .. 4L + 3.
__device__ __forceinline__ void pick_bin(const uint32_t* hist, uint32_t need, bool from_top,
                                         int lane, uint32_t prefix, int shift, uint32_t* s_a,
                                         uint32_t* s_b) {
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int pos = 4 * lane + q;
        c[q] = hist[from_top ? 255 - pos : pos];
        tot += c[q];
    }
    uint32_t run = wave_scan(tot, lane) - tot;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int pos = 4 * lane + q;
        if (run < need && run + c[q] >= need) {
            *s_a = prefix | ((uint32_t)(from_top ? 255 - pos : pos) << shift);
            *s_b = need - run;
        }
        run += c[q];
    }
}

// Radix select over the workgroup's values get(j), j < N, those whose bit j
// of vmask is set: the need-th largest (TOP) or smallest value of width
// nbytes bytes.  rem receives the rank left among the values equal to it.
template <int N, bool TOP, class Get>
__device__ __forceinline__ uint32_t radix_kth(Get get, uint32_t vmask, uint32_t need, int nbytes,
                                              uint32_t* hist, uint32_t* s_a, uint32_t* s_b,
                                              uint32_t& rem) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    for (int pass = 0; pass < nbytes; ++pass) {
        const int shift = 8 * (nbytes - 1 - pass);
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const uint32_t v = get(j);
            if (((vmask >> j) & 1u) && (v & mask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < WAVE) pick_bin(hist, need, TOP, tid, prefix, shift, s_a, s_b);
        __syncthreads();
        prefix = *s_a;
        need = *s_b;
        mask |= 255u << shift;
        // the next pass writes s_a only after two more barriers
    }
    rem = need;
    return prefix;
}

// Key of a logit, with -0 taken as +0 (the two compare equal).
__device__ __forceinline__ uint32_t logit_key(float f) { return order_key(f + 0.0f); }

__device__ __forceinline__ float key_logit(uint32_t k) {
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Slot s of thread tid holds logit id_of(s): with vec, the thread reads
// float4 number tid + (s / 4) * NT, otherwise logit tid + s * NT.
__global__ __launch_bounds__(NT) void k_sample(const float* __restrict__ logits, int64_t vocab,
                                               int32_t top_k, float top_p, float temperature,
                                               const double* __restrict__ u,
                                               int32_t* __restrict__ out, int vec) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_a, s_b, s_n;
    __shared__ uint32_t s_wave[NWV], s_lo;
    __shared__ float s_group[NT / 16];
    __shared__ __align__(16) uint64_t cand[CR];   // (key << 32) | ~id: larger ranks earlier
    __shared__ int32_t sid[MAXK];
    __shared__ double sl[MAXK], e1[MAXK], ew[MAXK];
    const int64_t r = blockIdx.x;
    const float* __restrict__ l = logits + r * vocab;
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int k = (int)min((int64_t)top_k, vocab);
    auto id_of = [&](int s) -> uint32_t {
        return vec ? (uint32_t)(4 * (tid + (s >> 2) * NT) + (s & 3)) : (uint32_t)(tid + s * NT);
    };
    const double ur = tid < WAVE ? u[r] : 0.0;

    float x[KPT];
    uint32_t own = 0;   // bit s: slot s holds a logit
    if (vec) {
        const float4* __restrict__ l4 = reinterpret_cast<const float4*>(l);
        const int64_t n4 = vocab >> 2;
#pragma unroll
        for (int j = 0; j < KPT / 4; ++j) {
            const int64_t i = tid + (int64_t)j * NT;
            const bool ok = i < n4;
            const float4 f = ok ? l4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            x[4 * j] = f.x;
            x[4 * j + 1] = f.y;
            x[4 * j + 2] = f.z;
            x[4 * j + 3] = f.w;
            own |= ok ? (0xFu << (4 * j)) : 0u;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int64_t i = tid + (int64_t)j * NT;
            const bool ok = i < vocab;
            x[j] = ok ? l[i] : -INFINITY;
            own |= ok ? (1u << j) : 0u;
        }
    }
    cand[tid] = 0;   // NT == CR: every slot starts below any candidate
    if (tid == 0) s_n = 0;

    uint32_t c;
    if (vocab <= CR) {
        // every logit is a candidate: thread tid holds logit tid
        if (own & 1u) cand[tid] = ((uint64_t)logit_key(x[0]) << 32) | (uint32_t)~(uint32_t)tid;
        c = (uint32_t)vocab;
        __syncthreads();
    } else {
        // 1. a lower bound for the k-th largest key (every thread holds a
        //    logit here)
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < KPT; ++j) mx = fmaxf(mx, x[j]);
        if (k <= GROUP_K) {
            const float gm = group_max<16>(mx);
            if ((lane & 15) == 0) s_group[tid / 16] = gm;
            __syncthreads();
            if (tid < WAVE) {
                const uint32_t lo = wave_kth_largest(logit_key(s_group[lane]), (uint32_t)k);
                if (lane == 0) s_lo = lo;
            }
        } else {
            const uint32_t wk = wave_kth_largest(logit_key(mx), (uint32_t)(k + NWV - 1) / NWV);
            if (lane == 0) s_wave[tid / WAVE] = wk;
            __syncthreads();
            if (tid == 0) {
                uint32_t lo = s_wave[0];
                for (int w = 1; w < NWV; ++w) lo = min(lo, s_wave[w]);
                s_lo = lo;
            }
        }
        __syncthreads();
        const float lof = key_logit(s_lo);

        // 2. gather the logits at or above it (the keys at or above the
        //    bound's key): a DPP prefix sum of the per-thread counts and one
        //    LDS atomic per wave place them
        uint32_t sel = 0;
        if (mx >= lof) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) sel |= (uint32_t)(x[j] >= lof) << j;
            sel &= own;
        }
        const uint32_t cnt = (uint32_t)__popc(sel);
        const uint32_t incl = wave_incl_scan(cnt);
        uint32_t base = 0;
        if (lane == WAVE - 1) base = atomicAdd(&s_n, incl);
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, WAVE - 1);
        if (sel) {
            uint32_t pos = base + incl - cnt;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                if ((sel >> j) & 1u) {
                    if (pos < (uint32_t)CR) cand[pos] = ((uint64_t)logit_key(x[j]) << 32) | (uint32_t)~id_of(j);
                    ++pos;
                }
            }
        }
        __syncthreads();
        c = s_n;
        if (c > (uint32_t)CR) {
            // Too many logits at the bound (heavy ties): exact radix select
            // of the k-th largest key, then of the last id taken among the
            // keys equal to it; exactly k keys are then gathered.
            cand[tid] = 0;
            uint32_t rem;
            const uint32_t kth = radix_kth<KPT, true>([&](int j) { return logit_key(x[j]); }, own,
                                                      (uint32_t)k, 4, hist, &s_a, &s_b, rem);
            uint32_t eq = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) eq |= (logit_key(x[j]) == kth) ? (1u << j) : 0u;
            eq &= own;
            uint32_t rem2;
            const uint32_t idlim = radix_kth<KPT, false>(id_of, eq, rem, 2, hist, &s_a, &s_b, rem2);
            if (tid == 0) s_n = 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint32_t key = logit_key(x[j]);
                if (((own >> j) & 1u) && (key > kth || (key == kth && id_of(j) <= idlim))) {
                    const uint32_t slot = atomicAdd(&s_n, 1u);
                    cand[slot] = ((uint64_t)key << 32) | (uint32_t)~id_of(j);
                }
            }
            __syncthreads();
            c = (uint32_t)k;
        }
    }

    // 3. rank of each candidate: how many candidates precede it (the slots
    //    past c hold zero, below every candidate)
    if (tid < (int)c) {
        const uint64_t me = cand[tid];
        const ulonglong2* __restrict__ c2 = reinterpret_cast<const ulonglong2*>(cand);
        int rank = 0;
        for (int j = 0; j < (int)(c + 15) / 16; ++j) {
            ulonglong2 p[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) p[q] = c2[8 * j + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) rank += (p[q].x > me) + (p[q].y > me);
        }
        if (rank < k) {
            sid[rank] = (int32_t)~(uint32_t)me;
            sl[rank] = (double)key_logit((uint32_t)(me >> 32));
        }
    }
    __syncthreads();
    if (temperature <= 0.0f) {   // greedy
        if (tid == 0) out[r] = sid[0];
        return;
    }

    // 4. weights in parallel (exp(l - l_max) for the probabilities, and at
    //    the temperature for the draw)
    if (tid < k) {
        const double d = sl[tid] - sl[0];
        e1[tid] = exp(d);
        ew[tid] = exp(d / (double)temperature);
    }
    __syncthreads();
    if (tid < WAVE) {
        // wave 0, ranks 4 * lane + q
        double e[4], w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * lane + q;
            e[q] = i < k ? e1[i] : 0.0;
            w[q] = i < k ? ew[i] : 0.0;
        }
        const double s1 = group_sum<WAVE>((e[0] + e[1]) + (e[2] + e[3]));
        // top-p: keep ranks up to the first whose running probability
        // reaches top_p (all k if none does)
        double pr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) pr[q] = e[q] / s1;
        double run = wave_prev(wave_incl_scan((pr[0] + pr[1]) + (pr[2] + pr[3])));
        int first = k;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            run += pr[q];
            if (4 * lane + q < k && run >= (double)top_p) first = min(first, 4 * lane + q);
        }
        const int keep = min(wave_min(first) + 1, k);
        // the draw: the first kept rank whose running weight exceeds u * sum
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = 4 * lane + q < keep ? w[q] : 0.0;
        const double lw = (w[0] + w[1]) + (w[2] + w[3]);
        const double target = ur * group_sum<WAVE>(lw);
        double cw = wave_prev(wave_incl_scan(lw));
        int pick = keep - 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cw += w[q];
            if (4 * lane + q < keep && cw > target) pick = min(pick, 4 * lane + q);
        }
        pick = wave_min(pick);
        if (lane == 0) out[r] = sid[pick];
    }
}

}  // namespace

}  // namespace qk

using namespace qk;

extern "C" int qk_sample(const float* logits, int64_t rows, int64_t vocab, int32_t top_k,
                         float top_p, float temperature, const double* u, int32_t* ids,
                         void* stream) {
    QK_REQUIRE(rows >= 0 && vocab > 0, QK_EINVAL);
    QK_REQUIRE(top_k >= 1 && top_k <= MAXK, QK_EINVAL);
    QK_REQUIRE(vocab <= (int64_t)NT * KPT, QK_ESHAPE);
    if (rows == 0) return QK_OK;
    QK_REQUIRE(logits && u && ids, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(logits, 4) && QK_ALIGNED(u, 8) && QK_ALIGNED(ids, 4), QK_EALIGN);
    const int vec = (vocab % 4 == 0 && vocab >= 4 * NT && QK_ALIGNED(logits, 16)) ? 1 : 0;
    hipLaunchKernelGGL(k_sample, dim3((unsigned)rows), dim3(NT), 0, (hipStream_t)stream, logits,
                       vocab, top_k, top_p, temperature, u, ids, vec);
    return qk_launch_status();
}
