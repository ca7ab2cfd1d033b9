/*
 * CPU oracle for the Q4_0 x Q8_0 LLaMA decoder-layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library.
 * Only the tests, the smoke entry point and the benchmark's CPU-baseline leg
 * may load it; the GPU library shares no source, header, table or helper with
 * it, and neither one calls the other.
 *
 * It is plain, slow and written to be read against the pages:
 *  - integer steps (quantization codes, block dot products) are exact;
 *  - floating-point steps are computed in double and rounded once to the
 *    storage type that the interface fixes (fp32 activations and outputs,
 *    fp16 scales and KV rows);
 *  - the build uses -O2 -ffp-contract=off and no fast-math (the pages' build
 *    flags enable fast-math, which would break the half-away-from-zero
 *    rounding and IEEE division the quantizers rely on);
 *  - OpenMP only splits independent outputs, so results do not depend on the
 *    thread count.
 *
 * Sources, cited by page title and section:
 *  [GUIDE]    kenji.blog, "Guide to developing small-scale AI models (such as
 *             TinyLLaMA) with C++": section 2 (pipeline figure), 4.1 RMSNorm,
 *             4.2 RoPE, 4.3 GQA, 4.4 SwiGLU, 5.2 (per-step graph figure),
 *             6.1 block quantization, 7 KV cache.
 *  [LLAMACPP] kenji.blog, "Guide to using llama.cpp and customizing it with
 *             C++": section 2.1 (GEMV bottleneck), 2.2 (block quantization
 *             equations).
 *  [ENGINE]   kenji.blog, "No Python needed: an AI inference engine in C++
 *             only": section 6 (GEMM definition), 8 (attention and KV cache).
 *  [COLIBRI]  kerneldigest.dev, "Colibri: running 744B MoE models on consumer
 *             hardware by streaming experts": "System architecture" and the
 *             token-flow figure (sigmoid router, int8 activations, expert
 *             kernels, combine); the model-conversion flow and the layer
 *             table (int4 container with per-row scales, int4/int2 packing).
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * closed forms, invariants, numpy's IEEE binary16 conversion or fp64 brute
 * force.  Parity unpinned: none of the functions.  Greedy tokens where the
 * top-2 logit gap is within the logit tolerance are not pinned (either token
 * is a correct greedy choice there).
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <vector>

namespace {

constexpr int QBLK = 32;  // elements per quantization block [GUIDE 6.1]

// Status codes returned by the oracle (independent of the GPU library's).
constexpr int OK = 0;
constexpr int E_INVAL = -1;
constexpr int E_SHAPE = -2;

// ---------------------------------------------------------------------------
// IEEE binary16 <-> binary32.  Written from the format definition: 1 sign
// bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals have exponent
// field 0 and value frac * 2^-24.  float -> half rounds to nearest, ties to
// even, keeps subnormals, and overflows to infinity at 65520 and above.
// ---------------------------------------------------------------------------
float half_to_float(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1F;
    const int frac = h & 0x3FF;
    double v;
    if (expo == 0)
        v = std::ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = std::ldexp((double)(1024 + frac), expo - 25);
    return (float)(sign ? -v : v);
}

// Round a non-negative double to the nearest integer, ties to even.
double round_half_even(double v) {
    double f = std::floor(v);
    double r = v - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (std::fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

uint16_t float_to_half(float f) {
    const uint16_t sign = std::signbit(f) ? 0x8000 : 0;
    if (std::isnan(f)) return 0x7E00;
    double a = std::fabs((double)f);
    if (a >= 65520.0) return sign | 0x7C00;  // rounds to 2^16: overflow
    if (a == 0.0) return sign;
    // Quantum (spacing of binary16 values) around a.
    int e;
    std::frexp(a, &e);          // a = m * 2^e with m in [0.5, 1)
    int unbiased = e - 1;       // a in [2^unbiased, 2^(unbiased+1))
    if (unbiased < -14) unbiased = -14;  // subnormal range shares 2^-24 quantum
    const double quantum = std::ldexp(1.0, unbiased - 10);
    const double m = round_half_even(a / quantum);  // a/quantum is exact
    const double v = m * quantum;                   // the rounded value
    if (v < std::ldexp(1.0, -14))                   // subnormal (or zero)
        return sign | (uint16_t)m;
    int ev;
    std::frexp(v, &ev);
    const int ub = ev - 1;                          // v in [2^ub, 2^(ub+1))
    const double frac = v / std::ldexp(1.0, ub) - 1.0;  // in [0, 1)
    return sign | (uint16_t)((ub + 15) << 10) | (uint16_t)(frac * 1024.0);
}

inline double h2d(uint16_t h) { return (double)half_to_float(h); }

// ---------------------------------------------------------------------------
// Block quantizers.
// ---------------------------------------------------------------------------

// Q4_0 weight block [LLAMACPP 2.2; GUIDE 6.1]: delta = max|w| / 7 (fp32),
// q = round-half-away-from-zero(w / delta) clamped to [-8, 7], stored as the
// nibble q + 8; delta is stored as fp16.  A block of zeros stores nibbles of 8
// and delta 0.  Byte j of a block holds element j in its low nibble and
// element j + 16 in its high nibble.
void q4_0_block(const float* w, uint8_t* packed16, uint16_t* d) {
    float amax = 0.0f;
    for (int j = 0; j < QBLK; ++j) amax = std::max(amax, std::fabs(w[j]));
    const float delta = amax / 7.0f;
    uint8_t nib[QBLK];
    for (int j = 0; j < QBLK; ++j) {
        if (delta == 0.0f) {
            nib[j] = 8;
        } else {
            float q = std::roundf(w[j] / delta);
            q = std::min(7.0f, std::max(-8.0f, q));
            nib[j] = (uint8_t)((int)q + 8);
        }
    }
    for (int j = 0; j < 16; ++j) packed16[j] = (uint8_t)(nib[j] | (nib[j + 16] << 4));
    *d = float_to_half(delta);
}

// Q8_0 activation block [LLAMACPP 2.2: x is quantized like the weights, with
// its own scale; COLIBRI: int8 activations]: d = max|x| / 127 (fp32),
// q = round-half-away-from-zero(x / d) clamped to [-127, 127], d stored as
// fp16.  An all-zero block gives d = 0 and q = 0.
void q8_0_block(const float* x, int8_t* q, uint16_t* d) {
    float amax = 0.0f;
    for (int j = 0; j < QBLK; ++j) amax = std::max(amax, std::fabs(x[j]));
    const float dd = amax / 127.0f;
    for (int j = 0; j < QBLK; ++j) {
        if (dd == 0.0f) {
            q[j] = 0;
        } else {
            float v = std::roundf(x[j] / dd);
            v = std::min(127.0f, std::max(-127.0f, v));
            q[j] = (int8_t)(int)v;
        }
    }
    *d = float_to_half(dd);
}

inline int nibble(const uint8_t* row_q, int64_t i) {
    // element i of a Q4_0 row: block b = i / 32, j = i % 32
    const int64_t b = i / QBLK;
    const int j = (int)(i % QBLK);
    const uint8_t byte = row_q[b * 16 + (j & 15)];
    return (j < 16) ? (byte & 0x0F) : (byte >> 4);
}

// Exact integer block dot [LLAMACPP 2.2]: sum_j (nib_j - 8) * qx_j.
int32_t block_dot(const uint8_t* row_q, const int8_t* xq, int64_t b) {
    int32_t s = 0;
    for (int j = 0; j < QBLK; ++j)
        s += (nibble(row_q, b * QBLK + j) - 8) * (int32_t)xq[b * QBLK + j];
    return s;
}

// y[t][r] = sum_b dw[r][b] * dx[t][b] * isum[t][r][b], in double, rounded to
// fp32 [LLAMACPP 2.2: y ~ delta * delta_x * sum q * q_x, block by block;
// ENGINE 6: C = A B].
void qmatmul(const uint8_t* w_q, const uint16_t* w_d, int64_t n, int64_t k,
             const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y) {
    const int64_t nb = k / QBLK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < m; ++t) {
        for (int64_t r = 0; r < n; ++r) {
            const uint8_t* rq = w_q + r * (k / 2);
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const int32_t isum = block_dot(rq, x_q + t * k, b);
                acc += h2d(w_d[r * nb + b]) * h2d(x_d[t * nb + b]) * (double)isum;
            }
            y[t * n + r] = (float)acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Row-scaled int4 / int2 weights [COLIBRI "System architecture" and the
// model-conversion flow: the engine's int4 container carries one scale per
// row, and its integer kernels pack int4 and int2 codes].  For bits b:
//   delta = max|w_row| / (2^(b-1) - 1) in fp32 (/7 for int4, as for Q4_0;
//   /1 for int2), q = round-half-away-from-zero(w / delta) clamped to
//   [-2^(b-1), 2^(b-1) - 1], stored as q + 2^(b-1); delta stays fp32.
// A row of zeros stores delta 0 and q = 0.  Per 32-element group:
//   int4: 16 bytes, byte j holds element j (low nibble) and j + 16 (high);
//   int2: 8 bytes, byte j holds elements j, j + 8, j + 16, j + 24 in bits
//         0-1, 2-3, 4-5, 6-7.
// ---------------------------------------------------------------------------
void rowq_quantize_row(int bits, const float* w, int64_t k, uint8_t* packed, float* d) {
    float amax = 0.0f;
    for (int64_t i = 0; i < k; ++i) amax = std::max(amax, std::fabs(w[i]));
    const int hi = (1 << (bits - 1)) - 1, lo = -(1 << (bits - 1));
    const float delta = amax / (float)hi;
    const int64_t group_bytes = bits * QBLK / 8;
    std::memset(packed, 0, (size_t)(k / QBLK * group_bytes));
    for (int64_t i = 0; i < k; ++i) {
        int q = 0;
        if (delta != 0.0f) {
            float v = std::roundf(w[i] / delta);
            v = std::min((float)hi, std::max((float)lo, v));
            q = (int)v;
        }
        const uint8_t c = (uint8_t)(q - lo);
        const int64_t g = i / QBLK;
        const int j = (int)(i % QBLK);
        if (bits == 4)
            packed[g * group_bytes + (j & 15)] |= (uint8_t)(c << (j < 16 ? 0 : 4));
        else
            packed[g * group_bytes + (j & 7)] |= (uint8_t)(c << (2 * (j / 8)));
    }
    *d = delta;
}

// Signed code of element i of a row-scaled row.
inline int rowq_code(int bits, const uint8_t* row_q, int64_t i) {
    const int64_t g = i / QBLK;
    const int j = (int)(i % QBLK);
    if (bits == 4) {
        const uint8_t byte = row_q[g * 16 + (j & 15)];
        return ((j < 16) ? (byte & 0x0F) : (byte >> 4)) - 8;
    }
    const uint8_t byte = row_q[g * 8 + (j & 7)];
    return ((byte >> (2 * (j / 8))) & 3) - 2;
}

// y[t][r] = delta_r * sum_b dx[t][b] * isum[t][r][b], isum the exact integer
// dot of block b, in double, rounded to fp32 once.
void rowq_matmul(int bits, const uint8_t* w_q, const float* w_r, int64_t n, int64_t k,
                 const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y) {
    const int64_t nb = k / QBLK, row_bytes = k * bits / 8;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < m; ++t) {
        for (int64_t r = 0; r < n; ++r) {
            const uint8_t* rq = w_q + r * row_bytes;
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t isum = 0;
                for (int j = 0; j < QBLK; ++j)
                    isum += rowq_code(bits, rq, b * QBLK + j) * (int32_t)x_q[t * k + b * QBLK + j];
                acc += h2d(x_d[t * nb + b]) * (double)isum;
            }
            y[t * n + r] = (float)((double)w_r[r] * acc);
        }
    }
}

void quantize_q8(const float* x, int64_t rows, int64_t k, int8_t* x_q, uint16_t* x_d) {
    const int64_t nb = k / QBLK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            q8_0_block(x + r * k + b * QBLK, x_q + r * k + b * QBLK, x_d + r * nb + b);
}

// RMSNorm [GUIDE 4.1]: y = x / sqrt(mean(x^2) + eps) * gamma.
void rmsnorm(const float* x, const float* gamma, int64_t rows, int64_t dim, float eps, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * dim;
        double ss = 0.0;
        for (int64_t i = 0; i < dim; ++i) ss += (double)xr[i] * (double)xr[i];
        const double denom = std::sqrt(ss / (double)dim + (double)eps);
        for (int64_t i = 0; i < dim; ++i)
            y[r * dim + i] = (float)((double)xr[i] / denom * (double)gamma[i]);
    }
}

// RoPE [GUIDE 4.2]: the adjacent pair (x[2i], x[2i+1]) of every head turns by
// the angle m * theta_i, m = absolute position, theta_i = base^(-2i/hd).
void rope(float* x, int64_t tokens, int64_t heads, int64_t hd, const int32_t* pos, float base) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t i = 0; i < hd / 2; ++i) {
            const double theta = std::pow((double)base, -2.0 * (double)i / (double)hd);
            const double ang = (double)pos[t] * theta;
            const double c = std::cos(ang), s = std::sin(ang);
            for (int64_t h = 0; h < heads; ++h) {
                float* p = x + (t * heads + h) * hd + 2 * i;
                const double x1 = p[0], x2 = p[1];
                p[0] = (float)(x1 * c - x2 * s);
                p[1] = (float)(x1 * s + x2 * c);
            }
        }
    }
}

// KV store [GUIDE 7]: the step's K and V rows go to row pos of the
// preallocated fp16 cache of their sequence.  Cache layout
// [seqs][n_kv][cap][hd].
// The cache of a sequence is a ring of cap rows [ENGINE 8: sized once for the
// longest context and used as a ring buffer]: position p lives in row p % cap.
void kv_append(const float* k, const float* v, int64_t tokens, int64_t n_kv, int64_t hd,
               const int32_t* pos, const int32_t* seq, uint16_t* kc, uint16_t* vc, int64_t cap) {
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t g = 0; g < n_kv; ++g)
            for (int64_t d = 0; d < hd; ++d) {
                const int64_t dst = (((int64_t)seq[t] * n_kv + g) * cap + pos[t] % cap) * hd + d;
                kc[dst] = float_to_half(k[(t * n_kv + g) * hd + d]);
                vc[dst] = float_to_half(v[(t * n_kv + g) * hd + d]);
            }
}

// Scaled dot-product attention with GQA [ENGINE 8; GUIDE 4.3, 7]: query
// head h reads KV head g = h / (nq / nkv); token t at position p attends to
// positions max(0, p - cap + 1)..p of its sequence, which are cache rows
// 0..min(p, cap - 1) of the ring (their order does not matter to the sum);
// s_j = q.k_j / sqrt(hd); softmax with the maximum subtracted;
// o = sum_j p_j v_j.
void attention(const float* q, int64_t tokens, int64_t nq, int64_t nkv, int64_t hd,
               const uint16_t* kc, const uint16_t* vc, int64_t cap, const int32_t* pos,
               const int32_t* seq, float* out) {
    const int64_t group = nq / nkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t h = 0; h < nq; ++h) {
            const int64_t g = h / group;
            const int64_t n = std::min((int64_t)pos[t] + 1, cap);
            const uint16_t* K = kc + ((int64_t)seq[t] * nkv + g) * cap * hd;
            const uint16_t* V = vc + ((int64_t)seq[t] * nkv + g) * cap * hd;
            const float* qh = q + (t * nq + h) * hd;
            std::vector<double> s((size_t)n);
            double smax = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < hd; ++d) dot += (double)qh[d] * h2d(K[j * hd + d]);
                s[(size_t)j] = dot / std::sqrt((double)hd);
                smax = std::max(smax, s[(size_t)j]);
            }
            double sum = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                s[(size_t)j] = std::exp(s[(size_t)j] - smax);
                sum += s[(size_t)j];
            }
            for (int64_t d = 0; d < hd; ++d) {
                double o = 0.0;
                for (int64_t j = 0; j < n; ++j) o += s[(size_t)j] / sum * h2d(V[j * hd + d]);
                out[(t * nq + h) * hd + d] = (float)o;
            }
        }
    }
}

// SwiGLU [GUIDE 4.4]: h = swish(gate) * up, swish(z) = z / (1 + e^-z).
void swiglu(const float* gate, const float* up, int64_t n, float* h) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double g = gate[i];
        h[i] = (float)(g / (1.0 + std::exp(-g)) * (double)up[i]);
    }
}

// Positions are non-negative.  A call holding more than one token of a
// sequence keeps that sequence's positions below cap: past the wrap, a later
// token's row would overwrite a position an earlier token of the same call
// still attends to.
bool valid_pos_seq(const int32_t* pos, const int32_t* seq, int64_t tokens, int64_t cap) {
    std::map<int32_t, std::pair<int64_t, int32_t>> per_seq;   // seq -> (tokens, max pos)
    for (int64_t t = 0; t < tokens; ++t) {
        if (pos[t] < 0 || seq[t] < 0) return false;
        auto& e = per_seq[seq[t]];
        e.first += 1;
        e.second = std::max(e.second, pos[t]);
    }
    for (const auto& kv : per_seq)
        if (kv.second.first > 1 && kv.second.second >= cap) return false;
    return true;
}

}  // namespace

extern "C" {

// Layer weights: Q4_0 in the split layout (nibbles [rows][k/2], fp16 scales
// [rows][k/32]).  w_qkv stacks the Q rows (nq*hd), then K rows, then V rows;
// w_gate_up stacks the F gate rows, then the F up rows.
struct oracle_layer {
    const uint8_t* w_qkv_q;  const uint16_t* w_qkv_d;
    const uint8_t* w_o_q;    const uint16_t* w_o_d;
    const uint8_t* w_gu_q;   const uint16_t* w_gu_d;
    const uint8_t* w_down_q; const uint16_t* w_down_d;
    const float* gamma_attn;
    const float* gamma_ffn;
};

struct oracle_layer_cfg {
    int64_t hidden, n_q_heads, n_kv_heads, head_dim, ffn;
    float eps, rope_base;
    int64_t cap;
};

uint16_t oracle_f32_to_f16(float f) { return float_to_half(f); }
float oracle_f16_to_f32(uint16_t h) { return half_to_float(h); }

void oracle_f32_to_f16_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = float_to_half(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t* h, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = half_to_float(h[i]);
}

int oracle_quantize_q4_0(const float* w, int64_t n, int64_t k, uint8_t* w_q, uint16_t* w_d) {
    if (k <= 0 || k % QBLK || n < 0) return E_SHAPE;
    const int64_t nb = k / QBLK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b)
            q4_0_block(w + r * k + b * QBLK, w_q + r * (k / 2) + b * 16, w_d + r * nb + b);
    return OK;
}

int oracle_quantize_q8_0(const float* x, int64_t rows, int64_t k, int8_t* x_q, uint16_t* x_d) {
    if (k <= 0 || k % QBLK || rows < 0) return E_SHAPE;
    quantize_q8(x, rows, k, x_q, x_d);
    return OK;
}

// isum[t][r][b] for activation rows t < m.
int oracle_block_dots_q4_0_q8_0(const uint8_t* w_q, int64_t n, int64_t k, const int8_t* x_q,
                                int64_t m, int32_t* isum) {
    if (k <= 0 || k % QBLK || n < 0 || m < 0) return E_SHAPE;
    const int64_t nb = k / QBLK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < m; ++t)
        for (int64_t r = 0; r < n; ++r)
            for (int64_t b = 0; b < nb; ++b)
                isum[(t * n + r) * nb + b] = block_dot(w_q + r * (k / 2), x_q + t * k, b);
    return OK;
}

int oracle_qmatmul_q4_0_q8_0(const uint8_t* w_q, const uint16_t* w_d, int64_t n, int64_t k,
                             const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y) {
    if (k <= 0 || k % QBLK || n < 0 || m < 0) return E_SHAPE;
    qmatmul(w_q, w_d, n, k, x_q, x_d, m, y);
    return OK;
}

int oracle_quantize_rowq(int32_t bits, const float* w, int64_t n, int64_t k, uint8_t* w_q, float* w_r) {
    if ((bits != 4 && bits != 2) || k <= 0 || k % QBLK || n < 0) return E_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) rowq_quantize_row(bits, w + r * k, k, w_q + r * (k * bits / 8), w_r + r);
    return OK;
}

int oracle_qmatmul_rowq_q8_0(int32_t bits, const uint8_t* w_q, const float* w_r, int64_t n, int64_t k,
                             const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y) {
    if ((bits != 4 && bits != 2) || k <= 0 || k % QBLK || n < 0 || m < 0) return E_SHAPE;
    rowq_matmul(bits, w_q, w_r, n, k, x_q, x_d, m, y);
    return OK;
}

int oracle_rmsnorm(const float* x, const float* gamma, int64_t rows, int64_t dim, float eps, float* y) {
    if (dim <= 0 || rows < 0) return E_SHAPE;
    rmsnorm(x, gamma, rows, dim, eps, y);
    return OK;
}

int oracle_rope(float* x, int64_t tokens, int64_t heads, int64_t head_dim, const int32_t* pos, float base) {
    if (head_dim <= 0 || head_dim % 2 || tokens < 0 || heads < 0) return E_SHAPE;
    rope(x, tokens, heads, head_dim, pos, base);
    return OK;
}

int oracle_kv_append(const float* k, const float* v, int64_t tokens, int64_t n_kv, int64_t hd,
                     const int32_t* pos, const int32_t* seq, uint16_t* k_cache, uint16_t* v_cache,
                     int64_t cap) {
    if (!valid_pos_seq(pos, seq, tokens, cap)) return E_INVAL;
    kv_append(k, v, tokens, n_kv, hd, pos, seq, k_cache, v_cache, cap);
    return OK;
}

int oracle_gqa_attention(const float* q, int64_t tokens, int64_t n_q_heads, int64_t n_kv_heads,
                         int64_t head_dim, const uint16_t* k_cache, const uint16_t* v_cache,
                         int64_t cap, const int32_t* pos, const int32_t* seq, float* out) {
    if (n_kv_heads <= 0 || n_q_heads % n_kv_heads) return E_SHAPE;
    if (!valid_pos_seq(pos, seq, tokens, cap)) return E_INVAL;
    attention(q, tokens, n_q_heads, n_kv_heads, head_dim, k_cache, v_cache, cap, pos, seq, out);
    return OK;
}

int oracle_swiglu(const float* gate, const float* up, int64_t n, float* h) {
    if (n < 0) return E_SHAPE;
    swiglu(gate, up, n, h);
    return OK;
}

// Embedding lookup [GUIDE 2, pipeline figure]: x[i] = table[ids[i]].
int oracle_embed_lookup(const float* table, int64_t vocab, int64_t hidden, const int32_t* ids,
                        int64_t n, float* x) {
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= vocab) return E_INVAL;
    for (int64_t i = 0; i < n; ++i)
        std::memcpy(x + i * hidden, table + (int64_t)ids[i] * hidden, sizeof(float) * hidden);
    return OK;
}

// Greedy choice of the next token [GUIDE 2]: index of the largest logit,
// ties to the lowest index.
int oracle_argmax(const float* logits, int64_t rows, int64_t vocab, int32_t* idx) {
    if (vocab <= 0) return E_SHAPE;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t best = 0;
        for (int64_t i = 1; i < vocab; ++i)
            if (logits[r * vocab + i] > logits[r * vocab + best]) best = i;
        idx[r] = (int32_t)best;
    }
    return OK;
}

// Sampler chain [GUIDE 8: temperature scales the probabilities, Top-K or
// Top-P (nucleus) narrows the candidates, a random number picks the token;
// LLAMACPP 5.4: the chain top-k, top-p (keeping at least one), temperature,
// then a seeded draw].  Per row, with the caller's uniform u in [0, 1):
//  1. rank every id by logit, largest first, equal logits by lower id; keep
//     the first top_k;
//  2. p_i = exp(l_i - l_0) / sum_kept exp(l_j - l_0); keep the shortest rank
//     prefix whose running sum of p reaches top_p (at least one id);
//  3. w_i = exp((l_i - l_0) / temperature) over the kept ids;
//  4. the token is the first kept id (in rank order) whose running sum of w
//     exceeds u * sum w (the last kept id if rounding leaves none).
// temperature <= 0 is greedy: the rank-0 id.  Sums run in rank order in fp64.
int oracle_sample(const float* logits, int64_t rows, int64_t vocab, int32_t top_k, double top_p,
                  float temperature, const double* u, int32_t* out) {
    if (vocab <= 0 || top_k <= 0) return E_SHAPE;
    for (int64_t r = 0; r < rows; ++r) {
        const float* l = logits + r * vocab;
        std::vector<int32_t> ids((size_t)vocab);
        for (int64_t i = 0; i < vocab; ++i) ids[(size_t)i] = (int32_t)i;
        std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return l[a] > l[b]; });
        const int64_t k = std::min<int64_t>(top_k, vocab);
        if (temperature <= 0.0f) {
            out[r] = ids[0];
            continue;
        }
        const double l0 = (double)l[ids[0]];
        double s1 = 0.0;
        for (int64_t i = 0; i < k; ++i) s1 += std::exp((double)l[ids[(size_t)i]] - l0);
        int64_t keep = 0;
        double cum = 0.0;
        while (keep < k) {
            cum += std::exp((double)l[ids[(size_t)keep]] - l0) / s1;
            ++keep;
            if (cum >= top_p) break;
        }
        double wsum = 0.0;
        for (int64_t i = 0; i < keep; ++i) wsum += std::exp(((double)l[ids[(size_t)i]] - l0) / (double)temperature);
        const double target = u[r] * wsum;
        int32_t pick = ids[(size_t)(keep - 1)];
        double cw = 0.0;
        for (int64_t i = 0; i < keep; ++i) {
            cw += std::exp(((double)l[ids[(size_t)i]] - l0) / (double)temperature);
            if (cw > target) {
                pick = ids[(size_t)i];
                break;
            }
        }
        out[r] = pick;
    }
    return OK;
}

// One pre-norm LLaMA decoder layer [GUIDE 5.2 figure: norm -> Q/K/V -> RoPE
// -> KV store/load -> attention -> scale and softmax -> output projection ->
// residual; GUIDE 4.4 for the FFN half]:
//   x1 = x  + Wo   . Q8(attn(rope(Wqkv . Q8(rmsnorm(x, g_attn)))))
//   x2 = x1 + Wd   . Q8(swiglu(Wg . Q8(u), Wu . Q8(u))),  u = rmsnorm(x1, g_ffn)
// Every Q4_0 matmul input is Q8_0-quantized; the FFN input is quantized once
// for both gate and up.  x is updated in place; K/V rows go to the caches.
int oracle_layer_forward(const oracle_layer* w, const oracle_layer_cfg* c, float* x, int64_t tokens,
                         const int32_t* pos, const int32_t* seq, uint16_t* k_cache, uint16_t* v_cache) {
    const int64_t H = c->hidden, nq = c->n_q_heads, nkv = c->n_kv_heads, hd = c->head_dim, F = c->ffn;
    if (H % QBLK || F % QBLK || nkv <= 0 || nq % nkv || hd % 2 || (nq * hd) % QBLK) return E_SHAPE;
    if (!valid_pos_seq(pos, seq, tokens, c->cap)) return E_INVAL;
    const int64_t T = tokens, Nq = nq * hd, Nkv = nkv * hd, Nqkv = Nq + 2 * Nkv;

    std::vector<float> xn((size_t)(T * H)), qkv((size_t)(T * Nqkv));
    std::vector<int8_t> xq((size_t)(T * std::max(H, std::max(Nq, F))));
    std::vector<uint16_t> xd((size_t)(T * std::max(H, std::max(Nq, F)) / QBLK));

    // attention half
    rmsnorm(x, w->gamma_attn, T, H, c->eps, xn.data());
    quantize_q8(xn.data(), T, H, xq.data(), xd.data());
    qmatmul(w->w_qkv_q, w->w_qkv_d, Nqkv, H, xq.data(), xd.data(), T, qkv.data());
    std::vector<float> q((size_t)(T * Nq)), k((size_t)(T * Nkv)), v((size_t)(T * Nkv));
    for (int64_t t = 0; t < T; ++t) {
        std::memcpy(&q[(size_t)(t * Nq)], &qkv[(size_t)(t * Nqkv)], sizeof(float) * Nq);
        std::memcpy(&k[(size_t)(t * Nkv)], &qkv[(size_t)(t * Nqkv + Nq)], sizeof(float) * Nkv);
        std::memcpy(&v[(size_t)(t * Nkv)], &qkv[(size_t)(t * Nqkv + Nq + Nkv)], sizeof(float) * Nkv);
    }
    rope(q.data(), T, nq, hd, pos, c->rope_base);
    rope(k.data(), T, nkv, hd, pos, c->rope_base);
    kv_append(k.data(), v.data(), T, nkv, hd, pos, seq, k_cache, v_cache, c->cap);
    std::vector<float> o((size_t)(T * Nq));
    attention(q.data(), T, nq, nkv, hd, k_cache, v_cache, c->cap, pos, seq, o.data());
    quantize_q8(o.data(), T, Nq, xq.data(), xd.data());
    std::vector<float> y((size_t)(T * H));
    qmatmul(w->w_o_q, w->w_o_d, H, Nq, xq.data(), xd.data(), T, y.data());
    for (int64_t i = 0; i < T * H; ++i) x[i] = (float)((double)x[i] + (double)y[(size_t)i]);

    // FFN half
    rmsnorm(x, w->gamma_ffn, T, H, c->eps, xn.data());
    quantize_q8(xn.data(), T, H, xq.data(), xd.data());
    std::vector<float> gu((size_t)(T * 2 * F)), g((size_t)(T * F)), u((size_t)(T * F)), h((size_t)(T * F));
    qmatmul(w->w_gu_q, w->w_gu_d, 2 * F, H, xq.data(), xd.data(), T, gu.data());
    for (int64_t t = 0; t < T; ++t) {
        std::memcpy(&g[(size_t)(t * F)], &gu[(size_t)(t * 2 * F)], sizeof(float) * F);
        std::memcpy(&u[(size_t)(t * F)], &gu[(size_t)(t * 2 * F + F)], sizeof(float) * F);
    }
    swiglu(g.data(), u.data(), T * F, h.data());
    quantize_q8(h.data(), T, F, xq.data(), xd.data());
    qmatmul(w->w_down_q, w->w_down_d, H, F, xq.data(), xd.data(), T, y.data());
    for (int64_t i = 0; i < T * H; ++i) x[i] = (float)((double)x[i] + (double)y[(size_t)i]);
    return OK;
}

// Sigmoid router [COLIBRI, architecture: DeepSeek-V3-style sigmoid router;
// token flow step 2]: r = x . W_r (W_r is [hidden][E]), rounded to fp32;
// s = 1 / (1 + e^-r).  The top_k experts are the ones with the largest
// scores, ties to the lower expert index; since the sigmoid is strictly
// increasing they are ranked on the fp32 logit r itself.  Weights are the
// selected scores normalized to sum to 1.
int oracle_moe_route(const float* x, int64_t tokens, int64_t hidden, const float* w_router,
                     int64_t n_experts, int32_t top_k, int32_t* sel_idx, float* sel_w,
                     float* logits_out /* may be null: [tokens][E] */) {
    if (top_k <= 0 || top_k > n_experts) return E_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        std::vector<float> r((size_t)n_experts);
        for (int64_t e = 0; e < n_experts; ++e) {
            double acc = 0.0;
            for (int64_t i = 0; i < hidden; ++i)
                acc += (double)x[t * hidden + i] * (double)w_router[i * n_experts + e];
            r[(size_t)e] = (float)acc;
            if (logits_out) logits_out[t * n_experts + e] = (float)acc;
        }
        std::vector<char> taken((size_t)n_experts, 0);
        std::vector<double> s((size_t)top_k);
        double ssum = 0.0;
        for (int32_t kk = 0; kk < top_k; ++kk) {
            int64_t best = -1;
            for (int64_t e = 0; e < n_experts; ++e)
                if (!taken[(size_t)e] && (best < 0 || r[(size_t)e] > r[(size_t)best])) best = e;
            taken[(size_t)best] = 1;
            sel_idx[t * top_k + kk] = (int32_t)best;
            s[(size_t)kk] = 1.0 / (1.0 + std::exp(-(double)r[(size_t)best]));
            ssum += s[(size_t)kk];
        }
        for (int32_t kk = 0; kk < top_k; ++kk) sel_w[t * top_k + kk] = (float)(s[(size_t)kk] / ssum);
    }
    return OK;
}

// One expert's SwiGLU FFN on one token [COLIBRI token flow step 5; GUIDE
// 4.4]: y = Wd . Q8(swiglu(Wg . Q8(x), Wu . Q8(x))), no norm, no residual.
// gu_q/gu_d: [2F][hidden] Q4_0 (gate rows, then up rows); dn_q/dn_d:
// [hidden][F] Q4_0.
int oracle_moe_expert_ffn(const float* x, int64_t hidden, int64_t ffn, const uint8_t* gu_q,
                          const uint16_t* gu_d, const uint8_t* dn_q, const uint16_t* dn_d, float* y) {
    if (hidden % QBLK || ffn % QBLK) return E_SHAPE;
    std::vector<int8_t> xq((size_t)std::max(hidden, ffn));
    std::vector<uint16_t> xd((size_t)(std::max(hidden, ffn) / QBLK));
    std::vector<float> gu((size_t)(2 * ffn)), h((size_t)ffn);
    quantize_q8(x, 1, hidden, xq.data(), xd.data());
    qmatmul(gu_q, gu_d, 2 * ffn, hidden, xq.data(), xd.data(), 1, gu.data());
    swiglu(gu.data(), gu.data() + ffn, ffn, h.data());
    quantize_q8(h.data(), 1, ffn, xq.data(), xd.data());
    qmatmul(dn_q, dn_d, hidden, ffn, xq.data(), xd.data(), 1, y);
    return OK;
}

// Routed MoE layer [COLIBRI token flow steps 2, 5, 6]: route, run each
// selected expert on its token, and combine per token as
// out[t] = sum over ranks 0..top_k-1 of w * y_expert, in rank order.
// Experts are stacked: gu_q [E][2F][hidden/2], gu_d [E][2F][hidden/32],
// dn_q [E][hidden][F/2], dn_d [E][hidden][F/32].
int oracle_moe_route_and_apply(const float* x, int64_t tokens, int64_t hidden, const float* w_router,
                               int64_t n_experts, int32_t top_k, const uint8_t* gu_q,
                               const uint16_t* gu_d, const uint8_t* dn_q, const uint16_t* dn_d,
                               int64_t ffn, float* out, int32_t* sel_idx, float* sel_w) {
    int rc = oracle_moe_route(x, tokens, hidden, w_router, n_experts, top_k, sel_idx, sel_w, nullptr);
    if (rc) return rc;
    if (hidden % QBLK || ffn % QBLK) return E_SHAPE;
    const int64_t gu_rows = 2 * ffn;
    std::vector<float> ys((size_t)(tokens * top_k * hidden));
    for (int64_t t = 0; t < tokens; ++t)
        for (int32_t kk = 0; kk < top_k; ++kk) {
            const int64_t e = sel_idx[t * top_k + kk];
            oracle_moe_expert_ffn(x + t * hidden, hidden, ffn,
                                  gu_q + e * gu_rows * (hidden / 2), gu_d + e * gu_rows * (hidden / QBLK),
                                  dn_q + e * hidden * (ffn / 2), dn_d + e * hidden * (ffn / QBLK),
                                  &ys[(size_t)((t * top_k + kk) * hidden)]);
        }
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t i = 0; i < hidden; ++i) {
            double acc = 0.0;
            for (int32_t kk = 0; kk < top_k; ++kk)
                acc += (double)sel_w[t * top_k + kk] * (double)ys[(size_t)((t * top_k + kk) * hidden + i)];
            out[t * hidden + i] = (float)acc;
        }
    return OK;
}

// The routed MoE layer with row-scaled int4 or int2 experts: routing and
// combine as above; each expert's FFN with the row-scaled matmul.  Experts
// are stacked: gu_q [E][2F][hidden * bits / 8], gu_r [E][2F] (fp32),
// dn_q [E][hidden][F * bits / 8], dn_r [E][hidden].
int oracle_moe_route_and_apply_rowq(int32_t bits, const float* x, int64_t tokens, int64_t hidden,
                                    const float* w_router, int64_t n_experts, int32_t top_k,
                                    const uint8_t* gu_q, const float* gu_r, const uint8_t* dn_q,
                                    const float* dn_r, int64_t ffn, float* out, int32_t* sel_idx,
                                    float* sel_w) {
    if (bits != 4 && bits != 2) return E_SHAPE;
    int rc = oracle_moe_route(x, tokens, hidden, w_router, n_experts, top_k, sel_idx, sel_w, nullptr);
    if (rc) return rc;
    if (hidden % QBLK || ffn % QBLK) return E_SHAPE;
    const int64_t F = ffn, H = hidden;
    std::vector<float> ys((size_t)(tokens * top_k * H));
    std::vector<int8_t> xq((size_t)std::max(H, F));
    std::vector<uint16_t> xd((size_t)(std::max(H, F) / QBLK));
    std::vector<float> gu((size_t)(2 * F)), h((size_t)F);
    for (int64_t t = 0; t < tokens; ++t)
        for (int32_t kk = 0; kk < top_k; ++kk) {
            const int64_t e = sel_idx[t * top_k + kk];
            quantize_q8(x + t * H, 1, H, xq.data(), xd.data());
            rowq_matmul(bits, gu_q + e * 2 * F * (H * bits / 8), gu_r + e * 2 * F, 2 * F, H, xq.data(),
                        xd.data(), 1, gu.data());
            swiglu(gu.data(), gu.data() + F, F, h.data());
            quantize_q8(h.data(), 1, F, xq.data(), xd.data());
            rowq_matmul(bits, dn_q + e * H * (F * bits / 8), dn_r + e * H, H, F, xq.data(), xd.data(), 1,
                        &ys[(size_t)((t * top_k + kk) * H)]);
        }
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t i = 0; i < H; ++i) {
            double acc = 0.0;
            for (int32_t kk = 0; kk < top_k; ++kk)
                acc += (double)sel_w[t * top_k + kk] * (double)ys[(size_t)((t * top_k + kk) * H + i)];
            out[t * H + i] = (float)acc;
        }
    return OK;
}

}  // extern "C"
