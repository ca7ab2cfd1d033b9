// Launchers shared between the libqk translation units (host side).
#pragma once

#include "common.h"

namespace qk {

enum GemvEpilogue : int {
    EPI_STORE = 0,   // y = acc (+ residual)
    EPI_SWIGLU = 1,  // rows f and f + ffn are gate and up: y[f] = swish(gate) * up
    EPI_QKV = 2,     // RoPE on q and k row pairs; q -> q_out, k and v -> fp16 caches
    EPI_ARGMAX = 3,  // y = acc, plus each workgroup's (max, lowest index) per column
};

enum GemvPrologue : int {
    PRO_NONE = 0,     // activations read as Q8_0 (xq, xd) from global memory
    PRO_RMSNORM = 1,  // activations = Q8_0(rmsnorm(xf, gamma)), built in LDS per workgroup
    PRO_Q8 = 2,       // activations = Q8_0(xf), built in LDS per workgroup
};

// A (possibly grouped) Q4_0 x Q8_0 product.  Group g (blockIdx.y) uses the
// weight matrix at wq + g * wq_gstride (wd + g * wd_gstride) and the
// activation columns c in [col_off[g], col_off[g+1]) (all m columns when
// col_off is null).  Column c reads activation row col_idx[c] (c when col_idx
// is null) and writes output row c: y[c * ldy + row].  With a residual,
// y[c * ldy + row] = residual[c * ldr + row] + acc (y may equal residual).
// Weight formats of the GEMV: Q4_0 (fp16 scale per 32-block), row-scaled
// int4 and int2 (fp32 scale per row; int4 in the Q4_0 nibble order, int2 with
// elements j, j + 8, j + 16, j + 24 of a 32-block in byte j).
enum { FMT_Q4_0 = 0, FMT_Q4_ROW = 1, FMT_Q2_ROW = 2 };

struct GemvArgs {
    const uint8_t* wq;
    const uint16_t* wd;      // FMT_Q4_0 block scales
    const float* wr;         // row-scaled formats: scales [n] per group
    int32_t fmt;
    int64_t n, k;          // rows (physical) and K of one group's matrix
    int64_t wq_gstride, wd_gstride, wr_gstride;
    const int8_t* xq;
    const uint16_t* xd;
    const int32_t* col_off;  // [groups + 1] or null
    const int32_t* col_idx;  // gather list or null
    int32_t m;               // columns when col_off is null
    int32_t groups;
    float* y;
    int64_t ldy;
    const float* residual;
    int64_t ldr;
    int64_t ffn;             // EPI_SWIGLU: gate rows [0, ffn), up rows [ffn, 2 ffn)
    int32_t max_cols;        // typical columns per group (picks columns per pass)
    // prologue (PRO_RMSNORM / PRO_Q8): fp32 activations [rows][k], gain, eps
    const float* xf;
    const float* gamma;
    float eps;
    // EPI_QKV: rows [0, q_rows) are q, then kv_rows of k, then kv_rows of v;
    // head_dim hd, n_kv heads, caches [seqs][n_kv][cap][hd]; q_out [m][q_rows]
    int64_t q_rows, kv_rows, hd, n_kv, cap;
    float rope_base;
    double rope_theta[64];   // theta_i = rope_base^(-2i/hd) for i < hd/2 (hd <= 128), set by the host
    const int32_t* pos;
    const int32_t* seq;
    uint16_t* kc;
    uint16_t* vc;
    float* q_out;
    // EPI_ARGMAX: partials [column][workgroup]
    float* part_val;
    int32_t* part_idx;
    // grouped launches (col_off set): the GEMV leaves groups of at least
    // skip_cols_ge columns (0: none) to the grouped MFMA GEMM, which takes
    // only groups of at least min_cols columns
    int32_t skip_cols_ge;
    int32_t min_cols;
    // grouped MFMA GEMM: [0] = n, [1 .. n] = the groups to take (grid z
    // indexes this list; null: grid z is the group)
    const int32_t* group_list;
};

// Launch the GEMV with the given epilogue and prologue; returns QK_ESHAPE when
// the prologue's LDS staging would not fit (the caller then stages itself).
int launch_gemv(const GemvArgs& a, int epi, hipStream_t s, int pro = PRO_NONE);
bool gemv_prologue_fits(int64_t k, int64_t max_cols);
// Whether one activation column of length k fits the GEMV's LDS staging.
bool gemv_fits(int64_t k);

// Final step of EPI_ARGMAX: idx[c] = index of the best partial of column c.
int launch_argmax_partials(const float* part_val, const int32_t* part_idx, int64_t nparts,
                           int64_t cols, int32_t* idx, hipStream_t s);
int64_t gemv_argmax_parts(int64_t n, int64_t k, int64_t max_cols);

// Q8_0 of [rows][k] fp32 (k % 32 == 0).
int launch_quantize_q8(const float* x, int64_t rows, int64_t k, int8_t* xq, uint16_t* xd,
                       hipStream_t s);

// Grouped expert GEMV of the MoE layer (Q4_0 or row-scaled int4 / int2,
// col_off set, no residual, K <= 6144, EPI_SWIGLU or EPI_STORE): each
// workgroup stages one group's
// columns once and walks a share of its rows with the next rows' weight
// loads in flight.  Returns QK_ESHAPE for arguments outside that
// (expert_gemv_fits tells beforehand).
bool expert_gemv_fits(const GemvArgs& a);
int launch_expert_gemv(const GemvArgs& a, int epi, hipStream_t s);

// MFMA GEMM for many columns (prefill).  Same argument meaning as GemvArgs.
// Q4_0 weights only.  Grouped (col_off set, `groups` groups): group g's
// columns are col_off[g] .. col_off[g + 1] - 1, its activation rows
// col_idx[c] (or c), its output rows c, its weights at g * wq_gstride /
// g * wd_gstride; groups of fewer than min_cols columns are skipped, and
// max_group_cols bounds every group's column count, and with group_list
// max_groups bounds its length (they size the grid).
int launch_gemm(const GemvArgs& a, int epi, hipStream_t s, int64_t max_group_cols = 0,
                int64_t max_groups = 0);

// y = rmsnorm(x) rows; optional Q8_0 of y into (xq, xd); y may be null.
int launch_rmsnorm_q8(const float* x, const float* gamma, int64_t rows, int64_t dim, float eps,
                      float* y, int8_t* xq, uint16_t* xd, hipStream_t s);

// Rotate q (heads_q) and k (heads_k) of every token in place, then store k
// and v rows into the caches.  Token t's q head h starts at
// base + t * tok_stride + q_off + h * hd, etc.
int launch_rope_kv(float* base, int64_t tokens, int64_t tok_stride, int64_t q_off, int64_t nq,
                   int64_t k_off, int64_t v_off, int64_t nkv, int64_t hd, const int32_t* pos,
                   const int32_t* seq, float rope_base, uint16_t* k_cache, uint16_t* v_cache,
                   int64_t cap, hipStream_t s);

// Attention with explicit q/out token strides (elements): a chunk kernel and a
// merge kernel.  The merge writes fp32 `out` (when non-null) and/or the Q8_0
// of the output row (oq, od; when non-null, with out_tok_stride also the Q8_0
// row length).
int launch_attention(const float* q, int64_t q_tok_stride, int64_t tokens, int64_t nq,
                     int64_t nkv, int64_t hd, const uint16_t* kc, const uint16_t* vc, int64_t cap,
                     const int32_t* pos, const int32_t* seq, float* out, int64_t out_tok_stride,
                     int8_t* oq, uint16_t* od, void* ws, size_t ws_bytes, hipStream_t s);
size_t attention_ws_bytes(int64_t tokens, int64_t nq, int64_t nkv, int64_t hd, int64_t cap);

}  // namespace qk
