/*
 * qk.h - C interface of libqk, the MI355X (gfx950) library for the forward
 * pass of a LLaMA-architecture decoder layer over 4-bit block-quantized
 * weights (Q4_0) and 8-bit block-quantized activations (Q8_0).
 *
 * Sources, cited by page title and section:
 *  [GUIDE]    kenji.blog, "Guide to developing small-scale AI models (such as
 *             TinyLLaMA) with C++": 2 pipeline figure, 4.1 RMSNorm, 4.2 RoPE,
 *             4.3 GQA, 4.4 SwiGLU, 5.1 arena allocation, 5.2 per-step graph
 *             figure, 6.1 block quantization, 7 KV cache.
 *  [LLAMACPP] kenji.blog, "Guide to using llama.cpp and customizing it with
 *             C++": 2.1 (decode is a GEMV), 2.2 block quantization equations.
 *  [ENGINE]   kenji.blog, "No Python needed: an AI inference engine in C++
 *             only": 6 GEMM, 7.1 backend interface, 8 attention and KV cache.
 *  [COLIBRI]  kerneldigest.dev, "Colibri: running 744B MoE models on consumer
 *             hardware by streaming experts": System architecture, token flow,
 *             model-conversion flow and layer table (per-row int4 container,
 *             int4/int2 packing).
 *
 * Conventions (all entry points):
 *  - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *    the comment says "host".  Outputs are caller-allocated
 *    (out-parameter style, as in the backend interface of [ENGINE 7.1]).
 *  - Calls enqueue work on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and return without synchronizing.  Buffers must stay
 *    alive until the stream has finished.  No call allocates or frees device
 *    memory: scratch space is a caller workspace `ws` of `ws_bytes` bytes
 *    whose size the matching qk_*_workspace() query returns (the arena
 *    principle of [GUIDE 5.1]: nothing is allocated inside the loop).
 *  - Return value: QK_OK (0) on success, a negative QK_E* code otherwise.
 *    Arguments are validated on the host before anything is enqueued; on a
 *    validation error nothing is enqueued and outputs are untouched.
 *    QK_EHIP reports a launch failure from the HIP runtime.
 *  - Layouts are row-major.  fp16 values travel as uint16_t bit patterns
 *    (IEEE binary16).
 *  - Q4_0 weights [n][k] (k % 32 == 0) are stored split:
 *      w_q : uint8 [n][k/2], 16 bytes per 32-element block; byte j of a block
 *            holds element j in its low nibble and element j+16 in its high
 *            nibble; a nibble c encodes the integer c - 8 (c in [0, 15]);
 *      w_d : fp16 [n][k/32], the block scales.
 *    Weight value = w_d * (c - 8) [LLAMACPP 2.2; GUIDE 6.1].  w_q must be
 *    16-byte aligned.
 *  - Q8_0 activations [m][k] are stored split: x_q int8 [m][k] (16-byte
 *    aligned), x_d fp16 [m][k/32].  Value = x_d * x_q.
 *  - float arrays must be 16-byte aligned.
 *  - Calls on different streams that touch disjoint buffers may run
 *    concurrently; calls that share a workspace must be ordered.
 */
#ifndef QK_H
#define QK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QK_OK 0
#define QK_EINVAL (-1)     /* null pointer or out-of-range value */
#define QK_ESHAPE (-2)     /* k % 32 != 0, nq % nkv != 0, odd head_dim, ... */
#define QK_EALIGN (-3)     /* a pointer is not aligned as documented */
#define QK_EWORKSPACE (-4) /* workspace missing or smaller than required */
#define QK_EHIP (-5)       /* the HIP runtime reported an error */

/* Text for a status code (static storage, never NULL).  [LLAMACPP 5.2-5.4:
 * the library's C calls report failure through their return value (a null
 * model, a negative token count, a non-zero decode result); here every call
 * returns one of the codes above and this call names it.]  Unknown codes
 * give a generic text. */
const char* qk_strerror(int status);

/* ---------------------------------------------------------------------- */
/* Quantization                                                           */
/* ---------------------------------------------------------------------- */

/* Q8_0 quantization of activations [LLAMACPP 2.2: the input vector is
 * block-quantized like the weights; COLIBRI: int8 activations].  For each
 * block of 32 values of each row: d = max|x| / 127 in fp32 (IEEE division),
 * q = round-half-away-from-zero(x / d) clamped to [-127, 127] (q = 0 when
 * d == 0), and d is stored as fp16 (round to nearest even).
 * x [rows][k] fp32 -> x_q int8 [rows][k], x_d fp16 [rows][k/32].
 * Requires k % 32 == 0.  Bit-exact by contract. */
int quantize_q8_0(const float* x, int64_t rows, int64_t k, int8_t* x_q, uint16_t* x_d,
                  void* stream);

/* Q4_0 quantization of weights [LLAMACPP 2.2: delta = max|w| / 7, codes in
 * [-8, 7]; GUIDE 6.1: 32 values per block, fp16 scale].  Per block:
 * delta = max|w| / 7 in fp32, c = round-half-away-from-zero(w / delta)
 * clamped to [-8, 7], nibble = c + 8 (8 for an all-zero block), delta stored
 * as fp16.  w [n][k] fp32 -> w_q [n][k/2], w_d [n][k/32].  Bit-exact. */
int qk_quantize_q4_0(const float* w, int64_t n, int64_t k, uint8_t* w_q, uint16_t* w_d,
                     void* stream);

/* Host helper: convert Q4_0 from interleaved 18-byte blocks to the split
 * layout [GUIDE 6.1: a Q4_0 block is 32 weights, one fp16 scale (2 bytes)
 * and 32 4-bit codes (16 bytes), 18 bytes in all].  aos18 holds [n][k/32]
 * blocks, each the fp16 scale followed by the 16 code bytes (byte j: code j
 * in the low nibble, code j + 16 in the high one), in host memory; w_q and
 * w_d are host memory too and owned by the caller.  Copies only, no
 * rounding.  Returns QK_EINVAL for n < 0, k <= 0 or (when n > 0) a null
 * pointer, and QK_ESHAPE when k % 32 != 0. */
int qk_q4_0_from_blocks(const void* aos18, int64_t n, int64_t k, uint8_t* w_q, uint16_t* w_d);

/* ---------------------------------------------------------------------- */
/* The quantized matmul                                                   */
/* ---------------------------------------------------------------------- */

/* y[t][r] = sum_b fp(w_d[r][b]) * fp(x_d[t][b]) * isum[t][r][b], with the
 * exact int32 block dot isum = sum_{j<32} (c_{r,32b+j} - 8) * x_q[t][32b+j]
 * [LLAMACPP 2.2: y ~ delta * delta_x * sum q q_x, the integer part being pure
 * integer arithmetic; ENGINE 6: C = A B].  W [n][k] Q4_0, x [m][k] Q8_0,
 * y [m][n] fp32 (accumulated in fp64 and rounded once).  m <= 8 runs the decode GEMV, larger
 * m the int8 MFMA GEMM. */
int qmatmul_q4_0_q8_0(const uint8_t* w_q, const uint16_t* w_d, int64_t n, int64_t k,
                      const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y,
                      void* stream);

/* Gate/up projection fused with SwiGLU [GUIDE 4.4: SwiGLU(x) = swish(x W_gate)
 * * (x W_up), built from silu and mul on the two matmul outputs]: W [2 ffn][k]
 * Q4_0 holds the ffn gate rows, then the ffn up rows; for every token t and
 * f < ffn, h[t][f] = swish(g) * u with g, u the quantized matmul outputs of
 * rows f and ffn + f (as in qmatmul_q4_0_q8_0).  h [m][ffn] fp32. */
int qk_gate_up_swiglu(const uint8_t* w_q, const uint16_t* w_d, int64_t ffn, int64_t k,
                      const int8_t* x_q, const uint16_t* x_d, int64_t m, float* h, void* stream);

/* The per-block int32 dot products themselves, for bit-exact checking
 * [LLAMACPP 2.2: within a block the product of the weight and input codes is
 * pure integer arithmetic; COLIBRI, System architecture: int8 activations
 * times int4 weights in integer kernels]: isum[t][r][b] =
 * sum_{j<32} (c_{r,32b+j} - 8) * x_q[t][32b+j] for t < m, r < n, b < k/32,
 * int32 [m][n][k/32] (|isum| <= 32 * 8 * 127 = 32512, exact).  The scales
 * play no part, so none are passed.  Device pointers; k % 32 == 0. */
int qk_block_dots_q4_0_q8_0(const uint8_t* w_q, int64_t n, int64_t k, const int8_t* x_q,
                            int64_t m, int32_t* isum, void* stream);

/* ---------------------------------------------------------------------- */
/* Element-wise and normalization ops                                     */
/* ---------------------------------------------------------------------- */

/* RMSNorm [GUIDE 4.1]: y = x / sqrt(mean(x^2) + eps) * gamma, row by row.
 * x, y [rows][dim] fp32 (y may equal x), gamma [dim]. */
int rmsnorm(const float* x, const float* gamma, int64_t rows, int64_t dim, float eps, float* y,
            void* stream);

/* Interleaved RoPE [GUIDE 4.2], in place: for token t at absolute position
 * m = pos[t], pair i = (x[2i], x[2i+1]) of every head turns by the angle
 * m * base^(-2i/head_dim).  x [tokens][heads][head_dim] fp32, pos int32
 * [tokens] (device).  Requires even head_dim. */
int rope(float* x, int64_t tokens, int64_t heads, int64_t head_dim, const int32_t* pos,
         float base, void* stream);

/* SwiGLU [GUIDE 4.4]: h = swish(gate) * up, swish(z) = z / (1 + e^-z).
 * gate, up, h: n fp32 each. */
int swiglu(const float* gate, const float* up, int64_t n, float* h, void* stream);

/* KV store [GUIDE 7; ENGINE 8, the cache as a ring buffer]:
 * k_cache[seq[t]][g][pos[t] % cap][:] = fp16(k[t][g][:]) and likewise for v.
 * k, v [tokens][n_kv][hd] fp32; caches fp16 [seqs][n_kv][cap][hd]; pos, seq
 * int32 [tokens] (device).  pos >= 0 (negative rows are skipped); past cap
 * the row of position pos - cap is overwritten.  seq must name an existing
 * sequence (not checked on the device: the caller owns the cache bounds). */
int qk_kv_append(const float* k, const float* v, int64_t tokens, int64_t n_kv, int64_t hd,
                 const int32_t* pos, const int32_t* seq, uint16_t* k_cache, uint16_t* v_cache,
                 int64_t cap, void* stream);

/* Embedding lookup [GUIDE 2 figure]: x[i][:] = table[ids[i]][:].
 * table [vocab][hidden] fp32, ids int32 [n] (device, each in [0, vocab)). */
int qk_embed_lookup(const float* table, int64_t vocab, int64_t hidden, const int32_t* ids,
                    int64_t n, float* x, void* stream);

/* Greedy next token [GUIDE 2 figure]: idx[r] = argmax_i logits[r][i], ties
 * to the lowest index.  logits [rows][vocab] fp32, idx int32 [rows]. */
int qk_argmax(const float* logits, int64_t rows, int64_t vocab, int32_t* idx, void* stream);

/* ---------------------------------------------------------------------- */
/* Sampling                                                               */
/* ---------------------------------------------------------------------- */

/* Sampler chain [TinyLLaMA-in-C++ guide 8: temperature, Top-K or Top-P,
 * then a random number picks the token; llama.cpp guide 5.4: the chain
 * top-k, top-p keeping at least one, temperature, seeded draw].  Per row of
 * logits [rows][vocab] (fp32, finite):
 *  1. rank the ids by logit, largest first, equal logits by lower id, and keep
 *     the first top_k (1 <= top_k <= 256);
 *  2. p_i = exp(l_i - l_0) / sum over the kept exp(l_j - l_0) (fp64); keep the
 *     shortest rank prefix whose running sum of p reaches top_p (at least one);
 *  3. w_i = exp((l_i - l_0) / temperature) over the kept ids;
 *  4. ids[row] = the first kept id, in rank order, whose running sum of w
 *     exceeds u[row] * sum w, with the caller's uniform u[row] in [0, 1) (fp64,
 *     device); the last kept id if rounding leaves none.
 * temperature <= 0 gives the rank-0 id (greedy).  The sums are fp64 but
 * taken as a tree, so a u within about 1e-12 of a boundary of the running
 * sums (or a top_p that close to a running probability) may fall either way.
 * logits and ids are device memory, top_p is used at float precision.  No
 * workspace.  Returns QK_EINVAL for top_k outside [1, 256], QK_ESHAPE for
 * vocab > 32768. */
int qk_sample(const float* logits, int64_t rows, int64_t vocab, int32_t top_k, float top_p,
              float temperature, const double* u, int32_t* ids, void* stream);

/* ---------------------------------------------------------------------- */
/* Attention                                                              */
/* ---------------------------------------------------------------------- */

/* Grouped-query attention over an fp16 KV cache [ENGINE 8; GUIDE 4.3, 7].
 * Query head h of token t reads KV head g = h / (n_q_heads / n_kv_heads) of
 * sequence seq[t] and attends to positions max(0, pos - cap + 1)..pos
 * (inclusive), i.e. ring rows 0..min(pos[t], cap - 1):
 * s_j = q . k_j / sqrt(head_dim), p = softmax(s), out = sum_j p_j v_j.
 * q, out [tokens][n_q_heads][head_dim] fp32; caches fp16
 * [seqs][n_kv_heads][cap][head_dim]; pos, seq int32 [tokens] (device,
 * pos >= 0; a negative position gives zeros).  head_dim must be 32 or 64,
 * n_q_heads / n_kv_heads at most 512 / head_dim and cap at most 32768.  ws:
 * qk_gqa_attention_workspace() bytes. */
int gqa_attention(const float* q, int64_t tokens, int64_t n_q_heads, int64_t n_kv_heads,
                  int64_t head_dim, const uint16_t* k_cache, const uint16_t* v_cache,
                  int64_t cap, const int32_t* pos, const int32_t* seq, float* out, void* ws,
                  size_t ws_bytes, void* stream);

size_t qk_gqa_attention_workspace(int64_t tokens, int64_t n_q_heads, int64_t head_dim,
                                  int64_t cap);

/* ---------------------------------------------------------------------- */
/* The decoder layer                                                      */
/* ---------------------------------------------------------------------- */

typedef struct qk_layer {
    /* Q4_0 weights, split layout.  w_qkv [(nq + 2 nkv) hd][hidden]: Q rows,
     * then K rows, then V rows.  w_o [hidden][nq hd].  w_gate_up
     * [2 ffn][hidden]: the ffn gate rows, then the ffn up rows.
     * w_down [hidden][ffn]. */
    const uint8_t* w_qkv_q;
    const uint16_t* w_qkv_d;
    const uint8_t* w_o_q;
    const uint16_t* w_o_d;
    const uint8_t* w_gate_up_q;
    const uint16_t* w_gate_up_d;
    const uint8_t* w_down_q;
    const uint16_t* w_down_d;
    const float* gamma_attn; /* [hidden] */
    const float* gamma_ffn;  /* [hidden] */
} qk_layer;

typedef struct qk_layer_cfg {
    int64_t hidden, n_q_heads, n_kv_heads, head_dim;
    int64_t ffn; /* multiple of 32 (pad with zero rows/columns) */
    float eps, rope_base;
    int64_t cap; /* KV cache rows per sequence */
} qk_layer_cfg;

/* One pre-norm LLaMA decoder layer [GUIDE 5.2 figure; GUIDE 4.1-4.4]:
 *   u  = rmsnorm(x, gamma_attn); [q|k|v] = w_qkv . Q8_0(u)
 *   q, k = rope(q, k, pos); k, v -> cache rows pos % cap of seq
 *   x1 = x + w_o . Q8_0(gqa_attention(q, cache))
 *   u1 = rmsnorm(x1, gamma_ffn); [g|up] = w_gate_up . Q8_0(u1)
 *   x2 = x1 + w_down . Q8_0(swiglu(g, up))
 * x [tokens][hidden] fp32 is updated in place to x2.  Tokens may belong to
 * different sequences; each token attends causally to positions
 * max(0, pos - cap + 1)..pos[t] of its sequence, which includes the rows this
 * call writes.  The cache is a ring [ENGINE 8]: position p lives in row
 * p % cap.  A sequence with more than one token in the call must keep its
 * positions below cap (its later rows would overwrite positions its earlier
 * tokens attend to); a sequence with one token may be at any position.
 * cap <= 32768.
 * ws: qk_layer_workspace(cfg, tokens) bytes. */
int layer_forward(const qk_layer* w, const qk_layer_cfg* cfg, float* x, int64_t tokens,
                  const int32_t* pos, const int32_t* seq, uint16_t* k_cache, uint16_t* v_cache,
                  void* ws, size_t ws_bytes, void* stream);

size_t qk_layer_workspace(const qk_layer_cfg* cfg, int64_t tokens);

/* layer_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and errors as layer_forward, without the
 * caller workspace.  The workspace is a device array of QK_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends; the call
 * allocates nothing.  A call whose qk_layer_workspace(cfg, tokens) exceeds
 * QK_SCRATCH_BYTES returns QK_EWORKSPACE with nothing enqueued (the
 * TinyLLaMA-1.1B shape fits for up to 8 tokens at cap 2176 and up to 3
 * tokens at cap 8192).  Returns QK_EHIP when the array's device address
 * cannot be obtained.  Every call on a GPU shares that GPU's array: calls
 * that overlap in time on one GPU (different streams, not ordered) race. */
#define QK_SCRATCH_BYTES (8u << 20)
int qk_layer_forward_scratch(const qk_layer* w, const qk_layer_cfg* cfg, float* x, int64_t tokens,
                             const int32_t* pos, const int32_t* seq, uint16_t* k_cache,
                             uint16_t* v_cache, void* stream);

/* ---------------------------------------------------------------------- */
/* Whole-model greedy decode in one persistent kernel                     */
/* ---------------------------------------------------------------------- */

/* A LLaMA-shaped decoder held on the device for qk_decode_greedy. */
typedef struct qk_decoder {
    const qk_layer* layers;    /* DEVICE array [n_layers] of layer weight pointers */
    int64_t n_layers;
    const float* embed;        /* [vocab][hidden] fp32 */
    const float* gamma_final;  /* [hidden] */
    const uint8_t* lm_q;       /* LM head Q4_0 [vocab][hidden] */
    const uint16_t* lm_d;
    int64_t vocab;
    uint16_t* k_cache;         /* fp16 [n_layers][n_kv_heads][cap][head_dim], one sequence */
    uint16_t* v_cache;
} qk_decoder;

/* n_tokens greedy decode steps of one sequence [GUIDE 2 pipeline figure:
 * embedding, the decoder layers, final RMSNorm, LM head, argmax; each layer
 * as layer_forward computes it for one token], all in one launch.
 * Step j runs at position pos0 + j (ring row (pos0 + j) % cap of every
 * layer's cache, attending to rows 0..min(pos0 + j, cap - 1)); its input
 * token is forced[j] when `forced` is non-NULL (teacher forcing), else
 * first_id[0] for j = 0 and the greedy token of step j - 1 after that.
 * out_ids[j] (device, [n_tokens]) receives step j's greedy token (largest
 * logit, lowest id on ties); when `logits` is non-NULL, step j's logits go
 * to row j % logits_rows of logits [logits_rows][vocab].
 * The kernel keeps one workgroup on every CU of the device, resident for the
 * whole call, so no other work may run on the device meanwhile.  Its
 * workgroups hand results to each other through `ws` (qk_decode_workspace
 * bytes, 256-byte aligned; the call clears what it needs, so no
 * initialization is required).  Every wait inside the kernel is bounded by
 * spin_limit polls (0: 2^20, about a second): a wait that gives up ends the
 * kernel early with wrong outputs and sets the flag that qk_decode_error
 * reads.
 * Shapes: head_dim 32 or 64; n_q_heads / n_kv_heads <= 8; hidden and
 * n_q_heads * head_dim <= 2048; ffn <= 6144 (multiples of 32); cap at most
 * 128 rows per attention chunk (8192 for the TinyLLaMA-1.1B shape on 256
 * CUs); otherwise QK_ESHAPE.  Weight and gain pointers inside `layers` must
 * be 16-byte aligned (they cannot be checked on the host). */
size_t qk_decode_workspace(const qk_layer_cfg* cfg);
int qk_decode_greedy(const qk_decoder* m, const qk_layer_cfg* cfg, const int32_t* first_id,
                     const int32_t* forced, int64_t pos0, int64_t n_tokens, int32_t* out_ids,
                     float* logits, int64_t logits_rows, uint32_t spin_limit, void* ws,
                     size_t ws_bytes, void* stream);
/* Synchronous: *flag (host) = nonzero when a wait of the last qk_decode_greedy
 * on `ws` gave up.  Waits for the copy (not a call for the decode loop). */
int qk_decode_error(const void* ws, const qk_layer_cfg* cfg, int32_t* flag);

/* First half of the feed-forward block [GUIDE 4.1, 4.4]:
 * h = SwiGLU(W_gate . Q8_0(u), W_up . Q8_0(u)), u = rmsnorm(x, gamma), with
 * W [2 ffn][hidden] Q4_0 (gate rows, then up rows).  x [tokens][hidden],
 * gamma [hidden], h [tokens][ffn] fp32.  ws: qk_ffn_up_workspace() bytes
 * (unused, and may be NULL, for tokens <= 8). */
int qk_ffn_up(const float* x, const float* gamma, float eps, const uint8_t* w_q,
              const uint16_t* w_d, int64_t ffn, int64_t hidden, int64_t tokens, float* h,
              void* ws, size_t ws_bytes, void* stream);

size_t qk_ffn_up_workspace(int64_t hidden, int64_t tokens);

/* Model head [GUIDE 2 figure: final RMSNorm, LM head, logits, greedy next
 * token]: logits = W . Q8_0(rmsnorm(x, gamma)) with W [vocab][hidden] Q4_0,
 * next[t] = argmax_i logits[t][i] (ties to the lowest index).
 * x [tokens][hidden], gamma [hidden], logits [tokens][vocab] fp32, next int32
 * [tokens].  ws: qk_lm_head_workspace() bytes. */
int qk_lm_head(const float* x, const float* gamma, float eps, const uint8_t* w_q,
               const uint16_t* w_d, int64_t vocab, int64_t hidden, int64_t tokens, float* logits,
               int32_t* next, void* ws, size_t ws_bytes, void* stream);

size_t qk_lm_head_workspace(int64_t vocab, int64_t hidden, int64_t tokens);

/* ---------------------------------------------------------------------- */
/* Mixture of experts                                                     */
/* ---------------------------------------------------------------------- */

/* Routed MoE layer [COLIBRI: sigmoid router of the DeepSeek-V3 kind, int8
 * activation x int4 expert kernels, results combined per token]:
 *   r = x . w_router (fp32), s = sigmoid(r);
 *   the top_k experts by s (ties to the lower index; ranked on r itself,
 *   which orders the same way) with weights s / sum(selected s);
 *   y_e = down_e . Q8_0(swiglu(gate_e . Q8_0(x), up_e . Q8_0(x)));
 *   y[t] = sum over ranks 0..top_k-1 of weight * y_e, in rank order.
 * x [tokens][hidden] fp32; w_router [hidden][n_experts] fp32;
 * experts stacked: gate_up_q [E][2 ffn][hidden/2], gate_up_d
 * [E][2 ffn][hidden/32] (gate rows then up rows), down_q [E][hidden][ffn/2],
 * down_d [E][hidden][ffn/32]; y [tokens][hidden]; sel_idx int32 and sel_w
 * fp32 [tokens][top_k].  Deterministic: no floating-point atomics.
 * n_experts <= 1024, top_k <= 32.  ws: qk_moe_workspace() bytes. */
int moe_route_and_apply(const float* x, int64_t tokens, int64_t hidden, const float* w_router,
                        int64_t n_experts, int32_t top_k, const uint8_t* gate_up_q,
                        const uint16_t* gate_up_d, const uint8_t* down_q,
                        const uint16_t* down_d, int64_t ffn, float* y, int32_t* sel_idx,
                        float* sel_w, void* ws, size_t ws_bytes, void* stream);

size_t qk_moe_workspace(int64_t tokens, int64_t hidden, int64_t n_experts, int32_t top_k,
                        int64_t ffn);

/* ---------------------------------------------------------------------- */
/* Row-scaled int4 / int2 weights                                          */
/* ---------------------------------------------------------------------- */

/* Row-scaled quantization [COLIBRI: the engine's int4 container with one
 * scale per row (model-conversion flow); int4/int2 packing (layer table)].
 * bits 4 or 2.  Per row: delta = max|w| / (2^(bits-1) - 1) in fp32 (/7 or
 * /1), code = round-half-away-from-zero(w / delta) clamped to
 * [-2^(bits-1), 2^(bits-1) - 1], stored as code + 2^(bits-1); a zero row
 * stores delta 0 and code 0.  Per 32-element group of a row, int4 takes 16
 * bytes (byte j: element j in the low nibble, j + 16 in the high one, as
 * Q4_0) and int2 takes 8 bytes (byte j: elements j, j + 8, j + 16, j + 24 in
 * bits 0-1, 2-3, 4-5, 6-7).  w fp32 [n][k] (16-byte aligned), w_q uint8
 * [n][k * bits / 8] (16-byte aligned), w_r fp32 [n]; device memory; k % 32
 * == 0.  QK_EINVAL for other bits. */
int qk_quantize_rowq(int32_t bits, const float* w, int64_t n, int64_t k, uint8_t* w_q, float* w_r,
                     void* stream);

/* y[t][r] = w_r[r] * sum_b dx[t][b] * isum[t][r][b] with isum the exact int32
 * dot of row r's block b codes with x_q (fp64 accumulation, one rounding to
 * fp32).  Same layouts as qk_quantize_rowq; x_q, x_d as qmatmul_q4_0_q8_0.
 * Any m (passes of up to 8 columns); k up to 58176. */
int qk_qmatmul_rowq_q8_0(int32_t bits, const uint8_t* w_q, const float* w_r, int64_t n, int64_t k,
                         const int8_t* x_q, const uint16_t* x_d, int64_t m, float* y,
                         void* stream);

/* moe_route_and_apply with row-scaled int4 (bits 4) or int2 (bits 2) experts:
 * gate_up_q [E][2 ffn][hidden * bits / 8], gate_up_r fp32 [E][2 ffn], down_q
 * [E][hidden][ffn * bits / 8], down_r fp32 [E][hidden].  Routing, SwiGLU,
 * Q8_0 of the expert inputs and the combine are those of
 * moe_route_and_apply; ws: qk_moe_workspace() bytes. */
int qk_moe_route_and_apply_rowq(int32_t bits, const float* x, int64_t tokens, int64_t hidden,
                                const float* w_router, int64_t n_experts, int32_t top_k,
                                const uint8_t* gate_up_q, const float* gate_up_r,
                                const uint8_t* down_q, const float* down_r, int64_t ffn, float* y,
                                int32_t* sel_idx, float* sel_w, void* ws, size_t ws_bytes,
                                void* stream);

/* ---------------------------------------------------------------------- */
/* Measurement                                                            */
/* ---------------------------------------------------------------------- */

/* Achievable read rate, for the rooflines of the streaming kernels (not an
 * operation of the method): reads `bytes` (a multiple of 16) of device
 * memory at `buf` (16-byte aligned) with 128-bit non-temporal loads in a
 * grid-stride loop over `blocks` workgroups of 256 threads (1..65536), and
 * writes the XOR of the words each workgroup read to out[blocks] (device,
 * uint32).  The caller times it.  QK_EINVAL / QK_ESHAPE / QK_EALIGN for bad
 * arguments; bytes == 0 still launches and writes zeros. */
int qk_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QK_H */
