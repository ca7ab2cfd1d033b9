// Greedy decode of a whole LLaMA-shaped model in one persistent kernel.
//
// What is computed is the pipeline of kenji.blog's TinyLLaMA-in-C++ guide,
// section 2 (embedding, the decoder layers, final RMSNorm, LM head, greedy
// choice), each layer as in section 5.2 (norm, Q/K/V projections, RoPE, KV
// store, attention over cache rows 0..p, output projection, residual) and
// section 4.4 (RMSNorm, SwiGLU feed-forward, residual), every matmul the
// Q4_0 x Q8_0 block product of the llama.cpp guide, section 2.2.  The
// arithmetic is that of the per-layer kernels (fp64 reductions rounded once,
// the same Q8_0 and RoPE code), so the two paths agree to rounding order.
//
// Design (gfx950).  One workgroup of 16 waves per CU, all resident at once.
// A token runs 6 phases per layer (QKV, attention chunks, attention merge,
// output projection, gate/up, down) and one LM-head phase.  Phases hand their
// results to the next through exchange buffers of 64-bit words that carry a
// 32-bit payload and a 32-bit tag naming the phase that wrote them: a reader
// polls the words it needs until every one carries the tag it expects, so
// there is no grid barrier, and each word is waited for only until its own
// writer has stored it.  Stores and polls are agent-scope (they bypass the
// non-coherent per-XCD L2); measured on MI355X, one store-to-poll round trip
// between CUs is about 0.85 us, while a flag barrier over 256 workgroups cost
// about 3 us.
//
// Within a workgroup, waves 12..15 gather the next phase's inputs (they poll,
// and stage them in LDS) while waves 0..11 compute the current phase; the
// weights of a phase are loaded into the compute waves' registers one or two
// phases ahead, so the HBM stream runs under the dependent chain instead of
// after it.  The gathering waves issue no weight loads: a wave's loads
// complete in order, so a poll issued behind a weight load would wait for it.
// For the same reason the kernel must not spill: a reload from scratch is a
// load too, and waiting for it would wait for every prefetch in flight.
// Every wait is bounded: a wave that polls past the limit, or sees another
// workgroup's error flag, makes its workgroup record the error and return, so
// every wave ends.
#include "internal.h"
#include "qdot.h"

namespace qk {

namespace {

constexpr int DT = 1024;              // threads per workgroup
constexpr int DWV = DT / WAVE;        // 16 waves
constexpr int NIO = 4;                // gathering waves
constexpr int CWV = DWV - NIO;        // compute waves 0..11
constexpr int CWT = CWV * WAVE;       // compute threads
constexpr int IOP = NIO * WAVE;       // gathering lanes: word pairs per round and k
constexpr int MAXH = 2048;            // hidden, and q heads x head_dim
constexpr int MAXF = 6144;            // FFN width
constexpr int MAXG = 8;               // query heads per KV head
constexpr int MAXHD = 64;
constexpr int CH_ROWS = 64;           // cache rows per attention pass (one per lane)
constexpr int CH_PASSES = 2;          // passes per chunk: at most 128 rows
constexpr int MAXCPH = 64;            // attention chunks per KV head
constexpr int LM_UPW = 4;             // LM-head rows per compute wave and pass
constexpr int MAXDS = 8;              // head dims per merge workgroup
constexpr int MAXWG = 512;            // workgroups (one per CU)
constexpr int MAXL = 64;              // layers
// 16-byte pieces of the chunk's K rows (and as many of its V rows) per
// compute thread
constexpr int KVH = (CH_PASSES * CH_ROWS * (MAXHD / 8) + CWT - 1) / CWT;

#if defined(__HIP_DEVICE_COMPILE__)
#define GLB __attribute__((address_space(1)))
#define CONSTAS __attribute__((address_space(4)))
#define LDSAS __attribute__((address_space(3)))
#else
#define GLB
#define CONSTAS
#define LDSAS
#endif

struct DecodeArgs {
    const qk_layer* layers;       // device array [L]
    const float* embed;           // [V][H]
    const float* gamma_final;     // [H]
    const uint8_t* lm_q;          // [V][H/2]
    const uint16_t* lm_d;         // [V][H/32]
    uint16_t* kc;                 // [L][nkv][cap][hd]
    uint16_t* vc;
    const int32_t* first_id;
    const int32_t* forced;        // [n] or null
    int32_t* out_ids;             // [n]
    float* logits;                // [logits_rows][V] or null
    // exchange words (payload | tag << 32), offsets into xw in words:
    //  ox  [H]  layer input x (the down output of the layer before)
    //  ox1 [H]  x1 = x + attention (output projection + residual)
    //  oq  [nq * hd] rotated q;  okv [2 * nkv * hd] this position's K, then V
    //  oml [nq][cph][4] chunk max and sum, each fp64 as two words
    //  oor [nq][cph][hd][2] chunk outputs, fp64 as two words
    //  oo  [nq * hd] attention output;  oh [F] SwiGLU output
    //  olm [nwg][2] each workgroup's best logit and its row
    //  olf [MAXWG][2] each workgroup's completion flag of the latest phase
    //      (a 32-bit tag at the head of a 16-byte slot)
    uint64_t* xw;
    int32_t ox, ox1, oq, okv, oml, oor, oo, oh, olm, olf;
    int32_t* ctl;                 // [0]: error flag
    int64_t cap, logits_rows, pos0, vocab;
    int32_t L, H, nq, nkv, hd, F, n_tokens, cph, wph;
    uint32_t spin_limit;
    float eps;
    double theta[MAXHD / 2];      // RoPE base^(-2i/hd), fp64 from the host
};

// The kernel copies its arguments and the layer table into LDS once and reads
// them there.  Read from the argument segment or global memory instead, a
// read that the compiler places under divergent control flow becomes a
// vector load, and waiting for it (loads complete in order) would wait for
// every weight prefetch in flight.
typedef const LDSAS DecodeArgs KArgs;
typedef const LDSAS qk_layer KLayer;
typedef const CONSTAS DecodeArgs CArgs;

// ------------------------------------------------------------ memory access
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

// A pointer made provably uniform, so that buffer resources built from it
// stay in scalar registers.
template <typename T>
__device__ __forceinline__ T* uni(T* p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, 0x00020000);
}

// buffer load cache-policy bits: non-temporal (weights stream through once),
// and system-coherent (data other CUs wrote during this kernel)
constexpr int CP_NT = 2, CP_SC1 = 16;

__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off, int cp) {
    v4u_t v;
    if (cp == CP_NT) v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP_NT);
    else v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP_SC1);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t ld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// exchange words: agent-scope stores (they write through the per-XCD L2)
__device__ __forceinline__ void put(uint64_t* p, uint32_t v, uint32_t tag) {
    __hip_atomic_store((GLB uint64_t*)p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f64(uint64_t* p, double v, uint32_t tag) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    put(p, (uint32_t)(b >> 32), tag);
    put(p + 1, (uint32_t)b, tag);
}
__device__ __forceinline__ double f64_of(uint32_t hi, uint32_t lo) {
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ void set_error(KArgs& a) {
    __hip_atomic_store((GLB int32_t*)a.ctl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ctl_error(KArgs& a) {
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load((GLB int32_t*)a.ctl, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)) != 0;
}

// A gathering wave waits for K word pairs per lane: the 16 bytes at pair
// index pair_of(k) of the exchange words, both words tagged `tag`; they end
// in v[k] (x, z payloads; y, w tags).  pair_of must give a pair of the data
// being waited for even where the lane has nothing to read (the caller
// ignores those), so that every load is unconditional.  A pair is loaded
// again by the whole wave while any lane still waits for it (pairs already
// complete read the same words again: nothing rewrites them until this
// workgroup has moved on).  False when the wait gives up (the spin limit, or
// another workgroup's error flag).
template <int K, typename PairF>
__device__ __forceinline__ bool fetch(__amdgpu_buffer_rsrc_t r, PairF pair_of, uint32_t tag,
                                      uint4 (&v)[K], KArgs& a) {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = ld16(r, (uint32_t)pair_of(k) * 16u, CP_SC1);
    uint32_t spins = 0;
    for (;;) {
        bool stale = false;
#pragma unroll
        for (int k = 0; k < K; ++k) stale |= v[k].y != tag || v[k].w != tag;
        if (!__any(stale)) return true;
        if (++spins > a.spin_limit) return false;
        if ((spins & 15) == 0 && ctl_error(a)) return false;
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (__any(v[k].y != tag || v[k].w != tag)) v[k] = ld16(r, (uint32_t)pair_of(k) * 16u, CP_SC1);
    }
}

// LDS barrier that waits only for LDS traffic: global loads in flight (the
// prefetched weights) stay in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------ weight stages
// A compute wave's share of one GEMV phase: units u = gw, gw + nwc, ... (UPW
// of them), each of P rows (plain: row u; SwiGLU: rows u and u + F; QKV:
// RoPE pair rows 2u, 2u + 1), blocks lane + 64 i (i < BL) of each row.
// Slot (k * P + p) * BL + i holds one block: 16 nibble bytes and its scale.
enum { KIND_PLAIN = 0, KIND_SWIGLU = 1, KIND_QKV = 2 };

template <int S>
struct Stage {
    uint4 w[S];
    uint16_t d[S];
};

template <int UPW, int P, int BL, int KIND, int S>
__device__ __forceinline__ void issue(Stage<S>& st, const uint8_t* wq, const uint16_t* wd, int nb,
                                      int units, int ffn, int gw, int nwc, int lane) {
    static_assert(UPW * P * BL <= S, "stage too small");
    const __amdgpu_buffer_rsrc_t rq = rsrc(uni(wq)), rd = rsrc(uni(wd));
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
        const int u = gw + k * nwc;
        const bool ok = u < units;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            int row = KIND == KIND_SWIGLU ? u + p * ffn : (KIND == KIND_QKV ? 2 * u + p : u);
            row = ok ? row : 0;
#pragma unroll
            for (int i = 0; i < BL; ++i) {
                int b = lane + WAVE * i;
                b = b < nb ? b : 0;
                const int s = (k * P + p) * BL + i;
                const uint32_t blk = (uint32_t)row * (uint32_t)nb + (uint32_t)b;
                st.w[s] = ld16(rq, blk * 16u, CP_NT);
                st.d[s] = ld2(rd, blk * 2u);
            }
        }
    }
}

// Block-scaled sums of the stage's rows against the staged Q8_0 input (LDS);
// same per-block arithmetic as the GEMV.
template <int UPW, int P, int BL, int S>
__device__ __forceinline__ void dots(const Stage<S>& st, const int8_t* lxq, const float* lxd, int nb,
                                     int lane, double (&acc)[UPW * P]) {
#pragma unroll
    for (int r = 0; r < UPW * P; ++r) acc[r] = 0.0;
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int b = lane + WAVE * i;
        if (b < nb) {
            const uint4 x0 = *reinterpret_cast<const uint4*>(lxq + b * QBLK);
            const uint4 x1 = *reinterpret_cast<const uint4*>(lxq + b * QBLK + 16);
            const float dx = lxd[b];
            const int s0 = -8 * byte_sum(x0, x1);
#pragma unroll
            for (int r = 0; r < UPW * P; ++r) {
                const int s = r * BL + i;
                const int sdot = dot_block(st.w[s], x0, x1, s0);
                acc[r] = fma((double)(h2f(st.d[s]) * dx), (double)sdot, acc[r]);
            }
        }
    }
}

// After row_sums: whether this lane owns a row total, which one (r), its sum
// and, for two-row units, the unit's other row.
template <int N, int P>
__device__ __forceinline__ bool owned_sum(double (&v)[N], int lane, int& r, double& s, double& s2) {
    const int base = row_sums<N>(v, lane);
    constexpr int NV = N >= 4 ? N / 4 : 1;
    const int kk = NV > 1 ? (lane & 15) : 0;
    s = v[0];
#pragma unroll
    for (int q = 1; q < NV; ++q)
        if (kk == q) s = v[q];
    s2 = 0.0;
    if (P == 2) {
        if (NV > 1) {
            s2 = v[0];
#pragma unroll
            for (int q = 1; q < NV; ++q)
                if ((kk ^ 1) == q) s2 = v[q];
        } else {
            s2 = __shfl_xor(s, N == 4 ? 16 : 32, WAVE);
        }
    }
    r = base + kk;
    constexpr int OWN = N >= 4 ? 16 : (N == 2 ? 32 : 64);
    return NV > 1 ? kk < NV : (lane & (OWN - 1)) == 0;
}

struct Lds {
    float rawA[MAXH];               // layer input x (kept for the residual of the output projection)
    float rawE[MAXH];               // x1 (kept for the residual of the down projection)
    union {                         // gains of the current norm / merge inputs
        float gam[MAXH];
        struct {
            double m[MAXCPH];
            double l[MAXCPH];
            double o[MAXCPH][MAXDS];
        } mg;
    } u1;
    alignas(16) int8_t lxq[MAXF];   // staged Q8_0 codes of the GEMV input
    float lxd[MAXF / QBLK];         // their scales
    double qs[MAXG][MAXHD];         // q of the group's heads
    float ks[CH_PASSES * CH_ROWS][MAXHD + 4];
    union {
        float vs[CH_PASSES * CH_ROWS][MAXHD];
        float rawT[MAXF];           // phase inputs that need no keeping
    } u2;
    double es[MAXG][CH_ROWS];
    double ssp[NIO];                // sums of squares of the staged input, per gathering wave
    float lm_v[CWV];
    int lm_i[CWV];
    int lm_cnt;
    int arrive;                     // compute waves done with the current phase
    uint32_t ready;                 // tag whose completion flags the gathering waves have seen
    uint32_t flagged;               // tag of this workgroup's latest completion flag
    int fail;
    DecodeArgs args;                // the kernel's arguments
    qk_layer layers[MAXL];          // the layer table
};

// Layer l's entry of the table, addressed from the (per-phase laundered)
// argument pointer so that the compiler cannot hoist the reads and keep them
// live across phases.
__device__ __forceinline__ KLayer& layer_of(KArgs* pa, int l) {
    const LDSAS char* base = (const LDSAS char*)pa + (offsetof(Lds, layers) - offsetof(Lds, args));
    return ((KLayer*)base)[l];
}

// RMSNorm (optional) and Q8_0 of K staged values into lxq / lxd, by every
// thread: groups of 4 values, 8 threads per 32-block, with the arithmetic of
// the GEMV prologue (y = x * inv * gamma in fp64, rounded to fp32; d =
// max|y| / 127; codes round half away from zero, clamped to +-127).
__device__ __forceinline__ void stage_q8(Lds& S, const float* raw, int K, bool norm, float eps) {
    const int ng = K / 4;
    double inv = 1.0;
    if (norm) {
        const double ss = (S.ssp[0] + S.ssp[1]) + (S.ssp[2] + S.ssp[3]);
        inv = 1.0 / sqrt(ss / (double)K + (double)eps);
    }
    for (int gi = threadIdx.x; gi < ng; gi += DT) {
        const float4 xv = *reinterpret_cast<const float4*>(raw + 4 * gi);
        float v[4] = {xv.x, xv.y, xv.z, xv.w};
        if (norm) {
            const float4 gv = *reinterpret_cast<const float4*>(S.u1.gam + 4 * gi);
            const float g[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (float)((double)v[e] * inv * (double)g[e]);
        }
        float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        amax = group_max<8>(amax);
        const float d = amax / 127.0f;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int q = 0;
            if (d != 0.0f) q = (int)fminf(127.0f, fmaxf(-127.0f, roundf(v[e] / d)));
            packed |= (uint32_t)(q & 0xFF) << (8 * e);
        }
        *reinterpret_cast<uint32_t*>(S.lxq + 4 * gi) = packed;
        if ((gi & 7) == 0) S.lxd[gi / 8] = h2f(f2h(d));
    }
}

// best (value, lowest row) of two candidates
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// The position's attention chunk of workgroup chunk c: rows [r0, r0 + n) of
// the attended rows 0..min(p, cap - 1), cph chunks per KV head.
struct Chunk {
    int r0, n;
};
__device__ __forceinline__ Chunk chunk_of(KArgs& a, int64_t p, int c) {
    const int64_t pe = p < a.cap - 1 ? p : a.cap - 1;
    const int rows = (int)pe + 1;
    const int ch = (rows + a.cph - 1) / a.cph;
    Chunk k;
    k.r0 = c * ch;
    k.n = max(0, min(ch, rows - k.r0));
    return k;
}

// ---------------------------------------------------------------------------
// The gathering waves.  For each phase they wait for the phase's inputs,
// stage them in LDS (with the sums of squares where a norm follows), and
// meet the compute waves at the phase's two barriers.  Gathering wave io
// takes word pairs k * 256 + io * 64 + lane of a vector.
// ---------------------------------------------------------------------------
struct IoWave {
    KArgs* pa;
    Lds& S;
    int io, lane, wg;

    // Makes the values derived from the thread and the arguments new at each
    // phase, so that the compiler does not keep them live (or spill them)
    // across the whole persistent loop.
    __device__ __forceinline__ void launder() {
        pa = uni(pa);
        io = __builtin_amdgcn_readfirstlane(io);
        wg = __builtin_amdgcn_readfirstlane(wg);
        asm volatile("" : "+s"(pa), "+s"(io), "+v"(lane), "+s"(wg));
    }

    __device__ __forceinline__ void fail(bool ok) {
        if (!ok && lane == 0) S.fail = 1;
    }

    // Waits until every workgroup has flagged the phase `tag` done.  Each
    // workgroup's flag is a 32-bit word at the head of its own 16-byte slot
    // (eight workgroups share a 128-byte line: packing them tighter makes
    // the writers and the pollers of a line contend).  Gathering waves 0 and
    // 1 poll, all of a lane's loads in flight at once and wave 1's polls
    // half a round trip behind wave 0's, so that the last flag is seen soon
    // after it lands; the first of them to see every flag posts the tag in
    // LDS, where the other gathering waves wait.  Only then are the phase's
    // outputs read, once: polling the outputs themselves from every
    // workgroup would flood the memory side.  A flag can be seen before some
    // of its workgroup's outputs, whose tags catch that; a workgroup may
    // already have flagged a later phase (flags only grow within a launch),
    // hence "at least".
    __device__ __forceinline__ bool wait_flags(uint32_t tag) {
        KArgs& a = *pa;
        if (io < 2) {
            const __amdgpu_buffer_rsrc_t rf = rsrc(uni(a.xw + a.olf));
            const int nwg = (int)gridDim.x;
            if (io == 1) {
                __builtin_amdgcn_s_sleep(8);
                __builtin_amdgcn_s_sleep(8);
            }
            uint32_t v[MAXWG / WAVE];
#pragma unroll
            for (int k = 0; k < MAXWG / WAVE; ++k)
                if (k * WAVE < nwg) v[k] = ld16(rf, (uint32_t)(k * WAVE + lane) * 16u, CP_SC1).x;
            uint32_t spins = 0;
            for (;;) {
                bool stale = false;
#pragma unroll
                for (int k = 0; k < MAXWG / WAVE; ++k) stale |= k * WAVE + lane < nwg && v[k] < tag;
                if (!__any(stale)) break;
                if (__hip_atomic_load(&S.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= tag) return true;
                if (++spins > a.spin_limit) return false;
                if ((spins & 15) == 0 && ctl_error(a)) return false;
#pragma unroll
                for (int k = 0; k < MAXWG / WAVE; ++k)
                    if (k * WAVE < nwg && __any(k * WAVE + lane < nwg && v[k] < tag))
                        v[k] = ld16(rf, (uint32_t)(k * WAVE + lane) * 16u, CP_SC1).x;
            }
            if (lane == 0) __hip_atomic_fetch_max(&S.ready, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return true;
        }
        uint32_t spins = 0;
        while (__hip_atomic_load(&S.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < tag) {
            if (__hip_atomic_load(&S.fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
            if (++spins > a.spin_limit) return false;
            __builtin_amdgcn_s_sleep(1);
        }
        return true;
    }

    // a vector of K words (K even) at word offset off, tagged `tag`, into
    // raw; with `ss` also this wave's sum of squares into S.ssp[io]
    template <int KV>
    __device__ __forceinline__ bool vec(float* raw, int off, int K, uint32_t tag, bool ss) {
        KArgs& a = *pa;
        const __amdgpu_buffer_rsrc_t rw = rsrc(uni(a.xw));
        double acc = 0.0;
        const int np = K / 2, p0 = off / 2;
        for (int base = 0; base < np; base += KV * IOP) {
            uint4 v[KV];
            auto pair = [&](int k) {
                const int q = base + k * IOP + io * WAVE + lane;
                return q < np ? p0 + q : p0;
            };
            if (!fetch<KV>(rw, pair, tag, v, a)) return false;
#pragma unroll
            for (int k = 0; k < KV; ++k) {
                const int q = base + k * IOP + io * WAVE + lane;
                if (q < np) {
                    const float f0 = bitsf(v[k].x), f1 = bitsf(v[k].z);
                    *reinterpret_cast<float2*>(raw + 2 * q) = make_float2(f0, f1);
                    acc = fma((double)f0, (double)f0, acc);
                    acc = fma((double)f1, (double)f1, acc);
                }
            }
        }
        if (ss) {
            acc = group_sum<WAVE>(acc);
            if (lane == 0) S.ssp[io] = acc;
        }
        return true;
    }

    // this wave's quarter of a norm's gains into LDS
    __device__ __forceinline__ void gamma(const float* g, int K) {
        const GLB float* gg = (const GLB float*)uni(g);
        for (int i = (io * WAVE + lane) * 4; i < K; i += IOP * 4)
            *reinterpret_cast<float4*>(S.u1.gam + i) = *reinterpret_cast<const GLB float4*>(gg + i);
    }

    // (wave io = 0) argmax over the workgroups' LM-head partials of one token
    __device__ __forceinline__ bool argmax(uint32_t tag, int& id) {
        KArgs& a = *pa;
        const __amdgpu_buffer_rsrc_t rw = rsrc(uni(a.xw));
        const int nwg = (int)gridDim.x;
        float bv = -INFINITY;
        int bi = INT32_MAX;
        for (int base = 0; base < nwg; base += 4 * WAVE) {
            uint4 v[4];
            auto pair = [&](int k) {
                const int w = base + k * WAVE + lane;
                return a.olm / 2 + (w < nwg ? w : 0);
            };
            if (!fetch<4>(rw, pair, tag, v, a)) return false;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (base + k * WAVE + lane < nwg) better(bv, bi, bitsf(v[k].x), (int)v[k].z);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, WAVE);
            const int oi = __shfl_xor(bi, o, WAVE);
            better(bv, bi, ov, oi);
        }
        id = bi == INT32_MAX ? 0 : bi;
        return true;
    }

    // A: the layer input (at layer 0 the embedding row of this token's id,
    // fetched by wave 0) and gamma_attn
    __device__ __forceinline__ void A(int j, int l, uint32_t tbase) {
        KArgs& a = *pa;
        KLayer& lw = layer_of(pa, l);
        const int H = a.H;
        gamma(lw.gamma_attn, H);
        if (l > 0) {
            const uint32_t t = tbase + 6 * l - 1;
            fail(wait_flags(t) && vec<MAXH / 2 / IOP>(S.rawA, a.ox, H, t, true));
            return;
        }
        if (io != 0) {
            if (lane == 0) S.ssp[io] = 0.0;
            return;
        }
        // this token's id: forced, the first id, or the greedy choice of the
        // previous token (workgroup 0 records that choice)
        bool ok = true;
        int id = 0;
        if (j > 0 && (!a.forced || wg == 0)) {
            ok = argmax(tbase - 1, id);
            if (ok && wg == 0 && lane == 0) ((GLB int32_t*)a.out_ids)[j - 1] = id;
        }
        if (a.forced) id = ((const GLB int32_t*)a.forced)[j];
        else if (j == 0) id = ((const GLB int32_t*)a.first_id)[0];
        id = __builtin_amdgcn_readfirstlane(id);
        id = id < 0 ? 0 : (id >= a.vocab ? (int)a.vocab - 1 : id);
        if (ok) {
            const GLB float* e = (const GLB float*)a.embed + (size_t)id * H;
            double acc = 0.0;
            for (int i = lane * 4; i < H; i += WAVE * 4) {
                const float4 v = *reinterpret_cast<const GLB float4*>(e + i);
                *reinterpret_cast<float4*>(S.rawA + i) = v;
                acc = fma((double)v.x, (double)v.x, acc);
                acc = fma((double)v.y, (double)v.y, acc);
                acc = fma((double)v.z, (double)v.z, acc);
                acc = fma((double)v.w, (double)v.w, acc);
            }
            acc = group_sum<WAVE>(acc);
            if (lane == 0) S.ssp[0] = acc;
        }
        fail(ok);
    }

    // B: q of the chunk's head group (all gathering waves); this position's
    // K/V row when it falls in the chunk (wave 3; the compute waves staged
    // the chunk's other rows)
    __device__ __forceinline__ void B(int64_t p, uint32_t tA) {
        KArgs& a = *pa;
        const __amdgpu_buffer_rsrc_t rw = rsrc(uni(a.xw));
        const int hd = a.hd, G = a.nq / a.nkv, Nkv = a.nkv * hd;
        if (wg >= a.nkv * a.cph) return;
        const int g = wg / a.cph, c = wg % a.cph;
        bool ok = true;
        {
            const int np = G * hd / 2;   // <= 256 pairs
            const int q0 = (a.oq + g * G * hd) / 2;
            uint4 v[1];
            auto pair = [&](int) {
                const int q = io * WAVE + lane;
                return q0 + (q < np ? q : 0);
            };
            ok = fetch<1>(rw, pair, tA, v, a);
            const int i = 2 * (io * WAVE + lane);
            if (ok && i < 2 * np) {
                S.qs[i / hd][i % hd] = (double)bitsf(v[0].x);
                S.qs[i / hd][i % hd + 1] = (double)bitsf(v[0].z);
            }
        }
        const Chunk ck = chunk_of(a, p, c);
        const int rn = (int)(p % a.cap);
        if (ok && io == NIO - 1 && rn >= ck.r0 && rn < ck.r0 + ck.n) {
            // lanes 0..hd/2-1: K dims 2l, 2l+1; lanes hd/2..hd-1: V dims
            uint4 v[1];
            const int hp = hd / 2;
            auto pair = [&](int) {
                if (lane < hp) return (a.okv + g * hd) / 2 + lane;
                if (lane < hd) return (a.okv + Nkv + g * hd) / 2 + (lane - hp);
                return (a.okv + g * hd) / 2;
            };
            ok = fetch<1>(rw, pair, tA, v, a);
            if (ok && lane < hd) {
                const int d = 2 * (lane < hp ? lane : lane - hp);
                float* row = lane < hp ? &S.ks[rn - ck.r0][0] : &S.u2.vs[rn - ck.r0][0];
                row[d] = bitsf(v[0].x);
                row[d + 1] = bitsf(v[0].z);
            }
        }
        fail(ok);
    }

    // C: (max, sum) of every chunk of this workgroup's head and the chunks'
    // outputs for its slice of dims; each fp64 is one word pair (hi, lo)
    __device__ __forceinline__ void C(uint32_t tB) {
        KArgs& a = *pa;
        const __amdgpu_buffer_rsrc_t rw = rsrc(uni(a.xw));
        const int cph = a.cph, hd = a.hd, ds = hd / a.wph;
        if (!wait_flags(tB)) {
            fail(false);
            return;
        }
        if (wg >= a.nq * a.wph) return;
        const int h = wg / a.wph, sl = wg % a.wph;
        const int npairs = 2 * cph + cph * ds;   // <= 128 + 512
        // (ds, hd and cph are powers of two: shifts, not divisions)
        const int dsh = __builtin_ctz(ds);
        const int ml0 = a.oml / 2 + h * cph * 2, or0 = a.oor / 2 + h * cph * hd + sl * ds;
        bool ok = true;
        for (int base = 0; base < npairs && ok; base += 3 * IOP) {
            uint4 v[3];
            auto pair = [&](int k) {
                const int q = base + k * IOP + io * WAVE + lane;
                if (q >= npairs) return ml0;
                if (q < 2 * cph) return ml0 + q;   // pair 2c: m of chunk c, 2c + 1: l
                const int q2 = q - 2 * cph;
                return or0 + (q2 >> dsh) * hd + (q2 & (ds - 1));
            };
            ok = fetch<3>(rw, pair, tB, v, a);
            if (ok) {
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const int q = base + k * IOP + io * WAVE + lane;
                    if (q < npairs) {
                        const double x = f64_of(v[k].x, v[k].z);
                        if (q < 2 * cph) {
                            if (q & 1) S.u1.mg.l[q / 2] = x;
                            else S.u1.mg.m[q / 2] = x;
                        } else {
                            const int q2 = q - 2 * cph;
                            S.u1.mg.o[q2 >> dsh][q2 & (ds - 1)] = x;
                        }
                    }
                }
            }
        }
        fail(ok);
    }

    __device__ __forceinline__ void run() {
        KArgs& a0 = *pa;
        const int L = a0.L, ntok = a0.n_tokens;
        const uint32_t per_tok = (uint32_t)(6 * L + 1);
        lds_sync();
        for (int j = 0; j < ntok; ++j) {
            const uint32_t tbase = 1u + (uint32_t)j * per_tok;
            for (int l = 0; l < L; ++l) {
                const uint32_t tA = tbase + 6 * l;
                launder();
                A(j, l, tbase);                                            // A
                lds_sync();
                if (S.fail) return;
                stage_q8(S, S.rawA, pa->H, true, pa->eps);
                lds_sync();
                launder();
                B(pa->pos0 + j, tA);                                        // B
                lds_sync();
                if (S.fail) return;
                lds_sync();
                launder();
                C(tA + 1);                                                  // C
                lds_sync();
                if (S.fail) return;
                lds_sync();
                launder();
                fail(wait_flags(tA + 2) &&                                      // D
                     vec<MAXH / 2 / IOP>(S.u2.rawT, pa->oo, pa->nq * pa->hd, tA + 2, false));
                lds_sync();
                if (S.fail) return;
                stage_q8(S, S.u2.rawT, pa->nq * pa->hd, false, 0.0f);
                lds_sync();
                launder();
                gamma(layer_of(pa, l).gamma_ffn, pa->H);                    // E
                fail(wait_flags(tA + 3) && vec<MAXH / 2 / IOP>(S.rawE, pa->ox1, pa->H, tA + 3, true));
                lds_sync();
                if (S.fail) return;
                stage_q8(S, S.rawE, pa->H, true, pa->eps);
                lds_sync();
                launder();
                fail(wait_flags(tA + 4) &&                                      // F
                     vec<MAXF / 2 / IOP>(S.u2.rawT, pa->oh, pa->F, tA + 4, false));
                lds_sync();
                if (S.fail) return;
                stage_q8(S, S.u2.rawT, pa->F, false, 0.0f);
                lds_sync();
            }
            launder();
            gamma(pa->gamma_final, pa->H);                                  // G
            fail(wait_flags(tbase + 6 * L - 1) &&
                 vec<MAXH / 2 / IOP>(S.u2.rawT, pa->ox, pa->H, tbase + 6 * L - 1, true));
            lds_sync();
            if (S.fail) return;
            stage_q8(S, S.u2.rawT, pa->H, true, pa->eps);
            lds_sync();
        }
        // the last token's greedy id
        launder();
        if (io == 0 && wg == 0 && ntok > 0) {
            int id = 0;
            if (argmax(1u + (uint32_t)(ntok - 1) * per_tok + 6 * L, id)) {
                if (lane == 0) ((GLB int32_t*)pa->out_ids)[ntok - 1] = id;
            } else if (lane == 0) {
                set_error(*pa);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// The compute waves: the phases' matmuls, attention and merge, from the
// staged inputs and the weights prefetched into registers.
// ---------------------------------------------------------------------------
struct Compute {
    KArgs* pa;
    Lds& S;
    int tid, lane, wave, wg, gw, nwc;
    Stage<4> s0;           // QKV, gate/up
    Stage<3> s1;           // output projection, down
    Stage<LM_UPW> slm;     // LM head
    uint4 kvk[KVH], kvv[KVH];   // the chunk's cache rows for the next attention phase

    // as in IoWave
    __device__ __forceinline__ void launder() {
        pa = uni(pa);
        wave = __builtin_amdgcn_readfirstlane(wave);
        wg = __builtin_amdgcn_readfirstlane(wg);
        gw = __builtin_amdgcn_readfirstlane(gw);
        nwc = __builtin_amdgcn_readfirstlane(nwc);
        asm volatile("" : "+s"(pa), "+v"(tid), "+v"(lane), "+s"(wave), "+s"(wg), "+s"(gw), "+s"(nwc));
    }

    __device__ __forceinline__ void issue_qkv(int l) {
        KArgs& a = *pa;
        KLayer& w = layer_of(pa, l);
        issue<1, 2, 1, KIND_QKV>(s0, w.w_qkv_q, w.w_qkv_d, a.H / QBLK,
                                 (a.nq + 2 * a.nkv) * a.hd / 2, 0, gw, nwc, lane);
    }
    __device__ __forceinline__ void issue_o(int l) {
        KArgs& a = *pa;
        KLayer& w = layer_of(pa, l);
        issue<1, 1, 1, KIND_PLAIN>(s1, w.w_o_q, w.w_o_d, a.nq * a.hd / QBLK, a.H, 0, gw, nwc, lane);
    }
    __device__ __forceinline__ void issue_gu(int l) {
        KArgs& a = *pa;
        KLayer& w = layer_of(pa, l);
        issue<2, 2, 1, KIND_SWIGLU>(s0, w.w_gate_up_q, w.w_gate_up_d, a.H / QBLK, a.F, a.F, gw, nwc, lane);
    }
    __device__ __forceinline__ void issue_dn(int l) {
        KArgs& a = *pa;
        KLayer& w = layer_of(pa, l);
        issue<1, 1, 3, KIND_PLAIN>(s1, w.w_down_q, w.w_down_d, a.F / QBLK, a.H, 0, gw, nwc, lane);
    }
    __device__ __forceinline__ void issue_lm(int pass) {
        KArgs& a = *pa;
        issue<LM_UPW, 1, 1, KIND_PLAIN>(slm, a.lm_q, a.lm_d, a.H / QBLK, (int)a.vocab, 0,
                                        gw + pass * LM_UPW * nwc, nwc, lane);
    }

    // piece e of this thread among the chunk's K (or V) rows: row in the
    // chunk (up to two passes of 64) and 8-value part
    __device__ __forceinline__ void kv_piece(int e, int& row, int& part) const {
        const int pr = pa->hd / 8;
        const int i = tid + e * CWT;
        row = i / pr;
        part = i % pr;
    }
    // the cache rows of this workgroup's chunk at position p (layer l), all
    // but the row the position writes, read coherently
    __device__ __forceinline__ void issue_kv(int l, int64_t p) {
        KArgs& a = *pa;
        const int hd = a.hd, g = wg / a.cph, c = wg % a.cph;
        const bool on = wg < a.nkv * a.cph;
        const Chunk ck = chunk_of(a, p, c);
        const int rn = (int)(p % a.cap);
        const size_t lstride = (size_t)a.nkv * (size_t)a.cap * (size_t)hd;
        const __amdgpu_buffer_rsrc_t rk = rsrc(uni(a.kc + (size_t)l * lstride));
        const __amdgpu_buffer_rsrc_t rv = rsrc(uni(a.vc + (size_t)l * lstride));
#pragma unroll
        for (int e = 0; e < KVH; ++e) {
            int row, part;
            kv_piece(e, row, part);
            const bool ok = on && row < ck.n && ck.r0 + row != rn;
            const uint32_t off = ok ? (uint32_t)((((size_t)g * a.cap + ck.r0 + row) * hd + part * 8) * 2) : 0u;
            kvk[e] = ld16(rk, off, CP_SC1);
            kvv[e] = ld16(rv, off, CP_SC1);
        }
    }
    __device__ __forceinline__ void kv_to_lds(int64_t p) {
        KArgs& a = *pa;
        const int c = wg % a.cph;
        const bool on = wg < a.nkv * a.cph;
        const Chunk ck = chunk_of(a, p, c);
        const int rn = (int)(p % a.cap);
#pragma unroll
        for (int e = 0; e < KVH; ++e) {
            int row, part;
            kv_piece(e, row, part);
            if (on && row < ck.n && ck.r0 + row != rn) {
                const uint32_t wk[4] = {kvk[e].x, kvk[e].y, kvk[e].z, kvk[e].w};
                const uint32_t wv[4] = {kvv[e].x, kvv[e].y, kvv[e].z, kvv[e].w};
                float* dk = &S.ks[row][part * 8];
                float* dv = &S.u2.vs[row][part * 8];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    dk[2 * f] = h2f((uint16_t)(wk[f] & 0xFFFF));
                    dk[2 * f + 1] = h2f((uint16_t)(wk[f] >> 16));
                    dv[2 * f] = h2f((uint16_t)(wv[f] & 0xFFFF));
                    dv[2 * f + 1] = h2f((uint16_t)(wv[f] >> 16));
                }
            }
        }
    }

    // This wave is done with phase `tag`; the last of the workgroup's compute
    // waves to get here raises the workgroup's completion flag, and every
    // compute wave waits for that before it goes on to issue the next weight
    // prefetch.  A CU's memory requests leave in issue order, so outputs or a
    // flag issued behind another wave's prefetch (tens of KB per CU) would
    // wait for it, and so would every workgroup that polls them.
    __device__ __forceinline__ void arrive(uint32_t tag) {
        KArgs& a = *pa;
        if (lane == 0) {
            if (atomicAdd(&S.arrive, 1) == CWV - 1) {
                S.arrive = 0;
                __hip_atomic_store((GLB uint32_t*)(a.xw + a.olf + 2 * wg), tag, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&S.flagged, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        // (the last arriver is a wave of this workgroup that waits on nothing
        // global before it gets here; the bound is a guard)
        uint32_t spins = 0;
        while (__hip_atomic_load(&S.flagged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < tag &&
               ++spins <= a.spin_limit)
            __builtin_amdgcn_s_sleep(1);
    }

    // A: QKV rows, RoPE, q out, K/V to the cache and the exchange
    __device__ __forceinline__ void A(int l, int64_t p, uint32_t tA) {
        KArgs& a = *pa;
        const int hd = a.hd, Nq = a.nq * hd, Nkv = a.nkv * hd, Nqkv = Nq + 2 * Nkv;
        double acc[2];
        dots<1, 2, 1>(s0, S.lxq, S.lxd, a.H / QBLK, lane, acc);
        int r;
        double s, s2;
        const bool own = owned_sum<2, 2>(acc, lane, r, s, s2);
        const int u = gw;
        if (own && r == 0 && u < Nqkv / 2) {
            const int row0 = 2 * u;
            const double x1 = (double)(float)s, x2 = (double)(float)s2;
            double c = 1.0, sn = 0.0;
            if (row0 < Nq + Nkv) rope_sincos((double)p * a.theta[(row0 % hd) / 2], sn, c);
            if (row0 < Nq) {
                put(a.xw + a.oq + row0, fbits((float)(x1 * c - x2 * sn)), tA);
                put(a.xw + a.oq + row0 + 1, fbits((float)(x1 * sn + x2 * c)), tA);
            } else {
                const bool is_k = row0 < Nq + Nkv;
                const int rr = row0 - Nq - (is_k ? 0 : Nkv);
                const int gh = rr / hd, d = rr % hd;
                const float o1 = (float)(is_k ? x1 * c - x2 * sn : x1);
                const float o2 = (float)(is_k ? x1 * sn + x2 * c : x2);
                const uint16_t h1 = f2h(o1), h2 = f2h(o2);
                const size_t lstride = (size_t)a.nkv * (size_t)a.cap * (size_t)hd;
                uint16_t* cache = (is_k ? a.kc : a.vc) + (size_t)l * lstride +
                                  ((size_t)gh * a.cap + (size_t)(p % a.cap)) * hd + d;
                __hip_atomic_store((GLB uint32_t*)cache, (uint32_t)h1 | ((uint32_t)h2 << 16),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                uint64_t* kv = a.xw + a.okv + (is_k ? 0 : Nkv) + gh * hd + d;
                put(kv, fbits(h2f(h1)), tA);
                put(kv + 1, fbits(h2f(h2)), tA);
            }
        }
    }

    // B: scores, softmax and weighted values of the group's heads over the
    // chunk (online across its passes), one record per head
    __device__ __forceinline__ void B(int64_t p, uint32_t tB) {
        KArgs& a = *pa;
        const int hd = a.hd, G = a.nq / a.nkv, cph = a.cph;
        if (wg >= a.nkv * cph || wave >= G) return;
        const int g = wg / cph, c = wg % cph;
        const int hh = g * G + wave;
        const Chunk ck = chunk_of(a, p, c);
        const double rscale = sqrt((double)hd);
        double m_run = -INFINITY, l_run = 0.0, o_run = 0.0;
        for (int pass = 0; pass * CH_ROWS < ck.n; ++pass) {
            const int rb = pass * CH_ROWS;
            const int prow = ck.n - rb < CH_ROWS ? ck.n - rb : CH_ROWS;
            double sc = -INFINITY;
            if (lane < prow) {
                double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
                for (int d = 0; d < hd; d += 4) {
                    const float4 kk = *reinterpret_cast<const float4*>(&S.ks[rb + lane][d]);
                    d0 = fma(S.qs[wave][d], (double)kk.x, d0);
                    d1 = fma(S.qs[wave][d + 1], (double)kk.y, d1);
                    d2 = fma(S.qs[wave][d + 2], (double)kk.z, d2);
                    d3 = fma(S.qs[wave][d + 3], (double)kk.w, d3);
                }
                sc = ((d0 + d1) + (d2 + d3)) / rscale;
            }
            const double mp = group_max<WAVE>(sc);
            const double mn = fmax(m_run, mp);
            const double e = lane < prow ? exp(sc - mn) : 0.0;
            const double lp = group_sum<WAVE>(e);
            const double f = m_run == -INFINITY ? 0.0 : exp(m_run - mn);
            S.es[wave][lane] = e;
            __builtin_amdgcn_wave_barrier();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane < hd) {
                double o0 = 0.0, o1 = 0.0, o2 = 0.0, o3 = 0.0;
                if (prow == CH_ROWS) {
#pragma unroll
                    for (int r = 0; r < CH_ROWS; r += 4) {
                        o0 = fma(S.es[wave][r], (double)S.u2.vs[rb + r][lane], o0);
                        o1 = fma(S.es[wave][r + 1], (double)S.u2.vs[rb + r + 1][lane], o1);
                        o2 = fma(S.es[wave][r + 2], (double)S.u2.vs[rb + r + 2][lane], o2);
                        o3 = fma(S.es[wave][r + 3], (double)S.u2.vs[rb + r + 3][lane], o3);
                    }
                } else {
                    int r = 0;
                    for (; r + 1 < prow; r += 2) {
                        o0 = fma(S.es[wave][r], (double)S.u2.vs[rb + r][lane], o0);
                        o1 = fma(S.es[wave][r + 1], (double)S.u2.vs[rb + r + 1][lane], o1);
                    }
                    if (r < prow) o0 = fma(S.es[wave][r], (double)S.u2.vs[rb + r][lane], o0);
                }
                o_run = o_run * f + ((o0 + o1) + (o2 + o3));
            }
            l_run = l_run * f + lp;
            m_run = mn;
            __builtin_amdgcn_wave_barrier();   // es is rewritten by the next pass
        }
        const int rec = hh * cph + c;
        if (lane == 0) {
            put_f64(a.xw + a.oml + rec * 4, m_run, tB);
            put_f64(a.xw + a.oml + rec * 4 + 2, l_run, tB);
        }
        if (lane < hd) put_f64(a.xw + a.oor + (rec * hd + lane) * 2, o_run, tB);
    }

    // C: out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c, one dim per wave
    __device__ __forceinline__ void C(uint32_t tC) {
        KArgs& a = *pa;
        const int hd = a.hd, cph = a.cph, ds = hd / a.wph;
        if (wg >= a.nq * a.wph || wave >= ds) return;
        const int h = wg / a.wph, sl = wg % a.wph;
        const double mc = lane < cph ? S.u1.mg.m[lane] : -INFINITY;
        const double M = group_max<WAVE>(mc);
        const double wc = (lane < cph && mc != -INFINITY) ? exp(mc - M) : 0.0;
        const double Ls = group_sum<WAVE>(lane < cph ? wc * S.u1.mg.l[lane] : 0.0);
        const double O = group_sum<WAVE>(lane < cph ? wc * S.u1.mg.o[lane][wave] : 0.0);
        if (lane == 0) put(a.xw + a.oo + h * hd + sl * ds + wave, fbits((float)(O / Ls)), tC);
    }

    // D: output projection + residual
    __device__ __forceinline__ void D(uint32_t tD) {
        KArgs& a = *pa;
        double acc[1];
        dots<1, 1, 1>(s1, S.lxq, S.lxd, a.nq * a.hd / QBLK, lane, acc);
        int r;
        double s, s2;
        const bool own = owned_sum<1, 1>(acc, lane, r, s, s2);
        if (own && gw < a.H) put(a.xw + a.ox1 + gw, fbits(S.rawA[gw] + (float)s), tD);
    }

    // E: gate/up + SwiGLU
    __device__ __forceinline__ void E(uint32_t tE) {
        KArgs& a = *pa;
        double acc[4];
        dots<2, 2, 1>(s0, S.lxq, S.lxd, a.H / QBLK, lane, acc);
        int r;
        double s, s2;
        const bool own = owned_sum<4, 2>(acc, lane, r, s, s2);
        const int u = gw + (r / 2) * nwc;
        if (own && (r % 2) == 0 && u < a.F) put(a.xw + a.oh + u, fbits(swiglu1((float)s, (float)s2)), tE);
    }

    // F: down projection + residual
    __device__ __forceinline__ void Fd(uint32_t tF) {
        KArgs& a = *pa;
        double acc[1];
        dots<1, 1, 3>(s1, S.lxq, S.lxd, a.F / QBLK, lane, acc);
        int r;
        double s, s2;
        const bool own = owned_sum<1, 1>(acc, lane, r, s, s2);
        if (own && gw < a.H) put(a.xw + a.ox + gw, fbits(S.rawE[gw] + (float)s), tF);
    }

    // G: LM head, logits and this workgroup's best
    __device__ __forceinline__ void G(int j, uint32_t tG) {
        KArgs& a = *pa;
        float bv = -INFINITY;
        int bi = INT32_MAX;
        const int upw_all = ((int)a.vocab + nwc - 1) / nwc;   // rows per compute wave
        for (int pass = 0; pass * LM_UPW < upw_all; ++pass) {
            if (pass > 0) issue_lm(pass);
            double acc[LM_UPW];
            dots<LM_UPW, 1, 1>(slm, S.lxq, S.lxd, a.H / QBLK, lane, acc);
            int r;
            double s, s2;
            const bool own = owned_sum<LM_UPW, 1>(acc, lane, r, s, s2);
            const int row = gw + (pass * LM_UPW + r) * nwc;
            if (own && row < a.vocab) {
                const float o = (float)s;
                if (a.logits) ((GLB float*)a.logits)[(size_t)(j % a.logits_rows) * a.vocab + row] = o;
                better(bv, bi, o, row);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, WAVE);
            const int oi = __shfl_xor(bi, o, WAVE);
            better(bv, bi, ov, oi);
        }
        // the last compute wave to finish combines the waves' bests
        int last = 0;
        if (lane == 0) {
            S.lm_v[wave] = bv;
            S.lm_i[wave] = bi;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            last = atomicAdd(&S.lm_cnt, 1) == CWV - 1;
        }
        last = __shfl(last, 0, WAVE);
        if (last && lane == 0) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            float cv = -INFINITY;
            int ci = INT32_MAX;
            for (int w = 0; w < CWV; ++w) better(cv, ci, S.lm_v[w], S.lm_i[w]);
            S.lm_cnt = 0;
            put(a.xw + a.olm + 2 * wg, fbits(cv), tG);
            put(a.xw + a.olm + 2 * wg + 1, (uint32_t)ci, tG);
        }
    }

    __device__ __forceinline__ void run() {
        KArgs& a0 = *pa;
        const int L = a0.L, ntok = a0.n_tokens;
        const uint32_t per_tok = (uint32_t)(6 * L + 1);
        lds_sync();
        // everything held before the first phase
        launder();
        issue_qkv(0);
        issue_o(0);
        issue_kv(0, pa->pos0);
        for (int j = 0; j < ntok; ++j) {
            const uint32_t tbase = 1u + (uint32_t)j * per_tok;
            for (int l = 0; l < L; ++l) {
                const uint32_t tA = tbase + 6 * l;
                lds_sync();                                   // A
                if (S.fail) return;
                launder();
                stage_q8(S, S.rawA, pa->H, true, pa->eps);
                lds_sync();
                A(l, pa->pos0 + j, tA);
                arrive(tA);
                issue_gu(l);
                kv_to_lds(pa->pos0 + j);
                lds_sync();                                   // B
                if (S.fail) return;
                lds_sync();
                launder();
                B(pa->pos0 + j, tA + 1);
                arrive(tA + 1);
                lds_sync();                                   // C
                if (S.fail) return;
                lds_sync();
                launder();
                C(tA + 2);
                arrive(tA + 2);
                lds_sync();                                   // D
                if (S.fail) return;
                launder();
                stage_q8(S, S.u2.rawT, pa->nq * pa->hd, false, 0.0f);
                lds_sync();
                D(tA + 3);
                arrive(tA + 3);
                issue_dn(l);
                lds_sync();                                   // E
                if (S.fail) return;
                launder();
                stage_q8(S, S.rawE, pa->H, true, pa->eps);
                lds_sync();
                E(tA + 4);
                arrive(tA + 4);
                issue_qkv(l + 1 < L ? l + 1 : 0);
                lds_sync();                                   // F
                if (S.fail) return;
                launder();
                stage_q8(S, S.u2.rawT, pa->F, false, 0.0f);
                lds_sync();
                Fd(tA + 5);
                arrive(tA + 5);
                if (l + 1 < L) {
                    issue_o(l + 1);
                    issue_kv(l + 1, pa->pos0 + j);
                } else {
                    issue_lm(0);
                }
            }
            lds_sync();                                       // G
            if (S.fail) return;
            launder();
            stage_q8(S, S.u2.rawT, pa->H, true, pa->eps);
            lds_sync();
            G(j, tbase + 6 * L);
            if (j + 1 < ntok) {
                issue_o(0);
                issue_kv(0, pa->pos0 + j + 1);
            }
        }
    }
};

}  // namespace

// The whole decode.  Grid: one workgroup per CU (all resident).
__global__ __launch_bounds__(DT) void k_decode(const DecodeArgs args) {
    (void)args;   // read through the kernel-argument segment below
    const CArgs* kp = (const CArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    __shared__ Lds S;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    static_assert(sizeof(DecodeArgs) % 4 == 0 && sizeof(qk_layer) % 4 == 0, "word copies");
    for (int i = tid; i < (int)(sizeof(DecodeArgs) / 4); i += DT)
        reinterpret_cast<uint32_t*>(&S.args)[i] = reinterpret_cast<const CONSTAS uint32_t*>(kp)[i];
    {
        const GLB uint32_t* src = (const GLB uint32_t*)kp->layers;
        const int nw = kp->L * (int)(sizeof(qk_layer) / 4);
        for (int i = tid; i < nw; i += DT) reinterpret_cast<uint32_t*>(&S.layers[0])[i] = src[i];
    }
    __syncthreads();
    KArgs* pa = (KArgs*)&S.args;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wg = blockIdx.x, nwg = (int)gridDim.x;
    if (tid == 0) {
        S.fail = 0;
        S.lm_cnt = 0;
        S.arrive = 0;
        S.ready = 0;
        S.flagged = 0;
    }
    if (wave >= CWV) {
        IoWave io{pa, S, wave - CWV, lane, wg};
        io.run();
    } else {
        Compute c{pa, S, tid, lane, wave, wg, wave * nwg + wg, CWV * nwg};
        c.run();
    }
    // a workgroup that stopped on an error records it for every workgroup
    if (tid == 0 && S.fail) set_error(*pa);
}

// Clears the exchange words and the error flag before a decode.
__global__ __launch_bounds__(256) void k_decode_clear(uint64_t* __restrict__ w, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        w[i] = 0;
}

namespace {

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecodeLayout {
    size_t x, x1, q, kv, ml, orr, o, h, lm, lf, ctl, total_words, bytes;
    int nwg, cph, wph;
};

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

DecodeLayout decode_layout(const qk_layer_cfg& c, int nwg) {
    DecodeLayout d{};
    d.nwg = nwg;
    d.cph = (int)std::min<int64_t>(MAXCPH, std::max<int64_t>(1, nwg / c.n_kv_heads));
    int w = 1;
    while (w * 2 <= c.head_dim && (int64_t)(w * 2) * c.n_q_heads <= nwg && w * 2 <= 8) w *= 2;
    d.wph = w;
    const size_t H = c.hidden, Nq = c.n_q_heads * c.head_dim, Nkv = c.n_kv_heads * c.head_dim;
    size_t o = 0;
    auto take = [&](size_t words) {
        size_t at = o;
        o += (words + 31) & ~(size_t)31;   // 256-byte aligned regions
        return at;
    };
    d.x = take(H);
    d.x1 = take(H);
    d.q = take(Nq);
    d.kv = take(2 * Nkv);
    d.ml = take((size_t)c.n_q_heads * d.cph * 4);
    d.orr = take((size_t)c.n_q_heads * d.cph * c.head_dim * 2);
    d.o = take(Nq);
    d.h = take(c.ffn);
    d.lm = take(2 * (size_t)nwg);
    d.lf = take(2 * (size_t)MAXWG);
    d.ctl = take(8);
    d.total_words = o;
    d.bytes = al256(o * 8);
    return d;
}

// Shapes the persistent kernel supports on a device of `nwg` CUs.
int decode_shape_ok(const qk_layer_cfg& c, int nwg, int64_t vocab) {
    const int64_t nwc = (int64_t)CWV * nwg;
    const int64_t H = c.hidden, Nq = c.n_q_heads * c.head_dim, F = c.ffn;
    const int64_t Nqkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
    if (nwg <= 0) return QK_EHIP;
    if (nwg > MAXWG) return QK_ESHAPE;
    if (c.head_dim != 32 && c.head_dim != 64) return QK_ESHAPE;
    if (c.n_q_heads % c.n_kv_heads || c.n_q_heads / c.n_kv_heads > MAXG) return QK_ESHAPE;
    if (H > MAXH || Nq > MAXH || F > MAXF || H % QBLK || F % QBLK || Nq % QBLK) return QK_ESHAPE;
    if (Nqkv / 2 > nwc || H > nwc || F > 2 * nwc) return QK_ESHAPE;
    if (c.n_q_heads > nwg || c.n_kv_heads > nwg) return QK_ESHAPE;
    const DecodeLayout d = decode_layout(c, nwg);
    if (c.head_dim / d.wph > MAXDS) return QK_ESHAPE;
    // rows per chunk at the largest context: at most CH_PASSES passes
    if ((c.cap + d.cph - 1) / d.cph > (int64_t)CH_PASSES * CH_ROWS) return QK_ESHAPE;
    if (vocab <= 0 || vocab > INT32_MAX / 2) return QK_EINVAL;
    return QK_OK;
}

}  // namespace

}  // namespace qk

using namespace qk;

extern "C" size_t qk_decode_workspace(const qk_layer_cfg* cfg) {
    if (!cfg || cfg->hidden <= 0 || cfg->n_q_heads <= 0 || cfg->n_kv_heads <= 0 ||
        cfg->head_dim <= 0 || cfg->ffn <= 0 || cfg->cap <= 0)
        return 0;
    const int nwg = device_cus();
    if (nwg <= 0) return 0;
    return decode_layout(*cfg, nwg).bytes;
}

extern "C" int qk_decode_greedy(const qk_decoder* m, const qk_layer_cfg* cfg,
                                const int32_t* first_id, const int32_t* forced, int64_t pos0,
                                int64_t n_tokens, int32_t* out_ids, float* logits,
                                int64_t logits_rows, uint32_t spin_limit, void* ws,
                                size_t ws_bytes, void* stream) {
    QK_REQUIRE(m && cfg, QK_EINVAL);
    QK_REQUIRE(cfg->hidden > 0 && cfg->n_q_heads > 0 && cfg->n_kv_heads > 0 && cfg->head_dim > 0 &&
                   cfg->ffn > 0 && cfg->cap > 0,
               QK_EINVAL);
    QK_REQUIRE(m->n_layers > 0 && m->vocab > 0, QK_EINVAL);
    if (m->n_layers > MAXL) return QK_ESHAPE;
    QK_REQUIRE(n_tokens >= 0 && pos0 >= 0 && pos0 + n_tokens <= INT32_MAX, QK_EINVAL);
    QK_REQUIRE((uint64_t)n_tokens * (uint64_t)(6 * m->n_layers + 1) < (1ull << 31), QK_EINVAL);
    if (n_tokens == 0) return QK_OK;
    QK_REQUIRE(m->layers && m->embed && m->gamma_final && m->lm_q && m->lm_d && m->k_cache &&
                   m->v_cache && out_ids && (first_id || forced),
               QK_EINVAL);
    QK_REQUIRE(!logits || logits_rows > 0, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(m->embed, 16) && QK_ALIGNED(m->gamma_final, 16) && QK_ALIGNED(m->lm_q, 16) &&
                   QK_ALIGNED(m->k_cache, 16) && QK_ALIGNED(m->v_cache, 16) && QK_ALIGNED(m->layers, 8),
               QK_EALIGN);
    const int nwg = device_cus();
    const int rc = decode_shape_ok(*cfg, nwg, m->vocab);
    if (rc) return rc;
    const DecodeLayout d = decode_layout(*cfg, nwg);
    QK_REQUIRE(ws && ws_bytes >= d.bytes && QK_ALIGNED(ws, 256), QK_EWORKSPACE);
    // every workgroup must be resident at once: one per CU
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_decode, DT, 0) != hipSuccess || occ < 1)
        return QK_EHIP;

    DecodeArgs a{};
    a.layers = m->layers;
    a.embed = m->embed;
    a.gamma_final = m->gamma_final;
    a.lm_q = m->lm_q;
    a.lm_d = m->lm_d;
    a.kc = m->k_cache;
    a.vc = m->v_cache;
    a.first_id = first_id;
    a.forced = forced;
    a.out_ids = out_ids;
    a.logits = logits;
    uint64_t* w = static_cast<uint64_t*>(ws);
    a.xw = w;
    a.ox = (int32_t)d.x;
    a.ox1 = (int32_t)d.x1;
    a.oq = (int32_t)d.q;
    a.okv = (int32_t)d.kv;
    a.oml = (int32_t)d.ml;
    a.oor = (int32_t)d.orr;
    a.oo = (int32_t)d.o;
    a.oh = (int32_t)d.h;
    a.olm = (int32_t)d.lm;
    a.olf = (int32_t)d.lf;
    a.ctl = reinterpret_cast<int32_t*>(w + d.ctl);
    a.cap = cfg->cap;
    a.logits_rows = logits ? logits_rows : 1;
    a.pos0 = pos0;
    a.vocab = m->vocab;
    a.L = (int32_t)m->n_layers;
    a.H = (int32_t)cfg->hidden;
    a.nq = (int32_t)cfg->n_q_heads;
    a.nkv = (int32_t)cfg->n_kv_heads;
    a.hd = (int32_t)cfg->head_dim;
    a.F = (int32_t)cfg->ffn;
    a.n_tokens = (int32_t)n_tokens;
    a.cph = d.cph;
    a.wph = d.wph;
    a.spin_limit = spin_limit ? spin_limit : (1u << 20);
    a.eps = cfg->eps;
    for (int i = 0; i < cfg->head_dim / 2; ++i)   // the RoPE frequencies, fp64 on the host
        a.theta[i] = std::pow((double)cfg->rope_base, -2.0 * (double)i / (double)cfg->head_dim);

    hipStream_t s = (hipStream_t)stream;
    const int64_t nclr = (int64_t)d.total_words;
    hipLaunchKernelGGL(k_decode_clear, dim3((unsigned)std::min<int64_t>(1024, (nclr + 255) / 256)),
                       dim3(256), 0, s, w, nclr);
    hipLaunchKernelGGL(k_decode, dim3((unsigned)nwg), dim3(DT), 0, s, a);
    return qk_launch_status();
}

extern "C" int qk_decode_error(const void* ws, const qk_layer_cfg* cfg, int32_t* flag) {
    QK_REQUIRE(ws && cfg && flag, QK_EINVAL);
    const int nwg = device_cus();
    if (nwg <= 0) return QK_EHIP;
    const DecodeLayout d = decode_layout(*cfg, nwg);
    const int32_t* ctl = reinterpret_cast<const int32_t*>(static_cast<const uint64_t*>(ws) + d.ctl);
    if (hipMemcpy(flag, ctl, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return QK_EHIP;
    return QK_OK;
}
