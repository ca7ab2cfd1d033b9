// The pre-norm decoder layer, its workspace, and status strings.
//
// Order of operations: kenji.blog TinyLLaMA-in-C++ guide, section 5.2 (per-
// step graph: norm, Q/K/V projections, RoPE, KV store and load, attention,
// scale and softmax, output projection, residual add) and section 4.4 for the
// SwiGLU feed-forward half, which repeats the norm -> projection -> residual
// pattern with its own gain.  Every Q4_0 matmul reads Q8_0 activations
// (llama.cpp guide 2.2); the FFN input is quantized once for gate and up.
#include <cmath>
#include <mutex>

#include "internal.h"

namespace qk {

namespace {

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct LayerWs {
    int8_t* xq;       // [T][max(H, Nq, F)]
    uint16_t* xd;     // [T][max/32]
    float* qkv;       // [T][Nqkv] (prefill path; the decode path keeps q only)
    float* h;         // [T][F]
    void* att_ws;     // attention chunk records
    size_t att_bytes;
    size_t total;
};

LayerWs layer_layout(void* base, const qk_layer_cfg& c, int64_t T) {
    const int64_t H = c.hidden, Nq = c.n_q_heads * c.head_dim;
    const int64_t Nqkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, F = c.ffn;
    const int64_t KX = std::max(H, std::max(Nq, F));
    LayerWs w{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return base ? static_cast<char*>(base) + at : nullptr;
    };
    w.xq = reinterpret_cast<int8_t*>(take((size_t)(T * KX)));
    w.xd = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * T * (KX / QBLK)));
    w.qkv = reinterpret_cast<float*>(take(sizeof(float) * T * Nqkv));
    w.h = reinterpret_cast<float*>(take(sizeof(float) * T * F));
    w.att_bytes = attention_ws_bytes(T, c.n_q_heads, c.n_kv_heads, c.head_dim, c.cap);
    w.att_ws = take(w.att_bytes);
    w.total = o;
    return w;
}

int check_cfg(const qk_layer_cfg* c) {
    if (!c) return QK_EINVAL;
    if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
        c->ffn <= 0 || c->cap <= 0)
        return QK_EINVAL;
    if (c->hidden % QBLK || c->ffn % QBLK || (c->n_q_heads * c->head_dim) % QBLK) return QK_ESHAPE;
    if (c->n_q_heads % c->n_kv_heads) return QK_ESHAPE;
    if (c->head_dim != 32 && c->head_dim != 64) return QK_ESHAPE;
    if ((c->n_q_heads / c->n_kv_heads) * c->head_dim > 512) return QK_ESHAPE;
    if (c->cap > 32768) return QK_ESHAPE;   // chunk-merge limit of the attention kernels
    return QK_OK;
}

GemvArgs plain(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, int64_t m) {
    GemvArgs a{};
    a.wq = wq; a.wd = wd; a.n = n; a.k = k;
    a.m = (int32_t)m; a.groups = 1; a.ldy = n; a.ldr = n; a.max_cols = (int32_t)m;
    return a;
}

int matmul(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, const int8_t* xq,
           const uint16_t* xd, int64_t m, float* y, const float* residual, int epi, int64_t ffn,
           hipStream_t s) {
    GemvArgs a = plain(wq, wd, n, k, m);
    a.xq = xq; a.xd = xd;
    a.y = y; a.ldy = (epi == EPI_SWIGLU) ? ffn : n;
    a.residual = residual; a.ffn = ffn;
    return m > 8 ? launch_gemm(a, epi, s) : launch_gemv(a, epi, s);
}

// Few tokens: five kernels, each Q4_0 matmul with its producer fused in.
//  1. QKV GEMV, prologue RMSNorm + Q8_0 of x, epilogue RoPE + KV store
//  2. attention (chunks, then the merge, which writes the Q8_0 of the output)
//  3. output projection GEMV + residual
//  4. gate/up GEMV, prologue RMSNorm + Q8_0, epilogue SwiGLU
//  5. down GEMV, prologue Q8_0 of h, + residual
int layer_decode(const qk_layer* w, const qk_layer_cfg& c, float* x, int64_t T,
                 const int32_t* pos, const int32_t* seq, uint16_t* kc, uint16_t* vc,
                 const LayerWs& L, hipStream_t s) {
    const int64_t H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, hd = c.head_dim;
    const int64_t Nq = nq * hd, Nkv = nkv * hd, Nqkv = Nq + 2 * Nkv, F = c.ffn;
    int rc;
    GemvArgs a = plain(w->w_qkv_q, w->w_qkv_d, Nqkv, H, T);
    a.xf = x; a.gamma = w->gamma_attn; a.eps = c.eps;
    a.q_rows = Nq; a.kv_rows = Nkv; a.hd = hd; a.n_kv = nkv; a.cap = c.cap;
    a.rope_base = c.rope_base; a.pos = pos; a.seq = seq; a.kc = kc; a.vc = vc; a.q_out = L.qkv;
    for (int64_t i = 0; i < hd / 2; ++i)   // the RoPE frequencies, in fp64 on the host
        a.rope_theta[i] = std::pow((double)c.rope_base, -2.0 * (double)i / (double)hd);
    if ((rc = launch_gemv(a, EPI_QKV, s, PRO_RMSNORM))) return rc;
    if ((rc = launch_attention(L.qkv, Nq, T, nq, nkv, hd, kc, vc, c.cap, pos, seq, nullptr, Nq,
                               L.xq, L.xd, L.att_ws, L.att_bytes, s)))
        return rc;
    GemvArgs o = plain(w->w_o_q, w->w_o_d, H, Nq, T);
    o.xq = L.xq; o.xd = L.xd; o.y = x; o.residual = x;
    if ((rc = launch_gemv(o, EPI_STORE, s, PRO_NONE))) return rc;
    GemvArgs gu = plain(w->w_gate_up_q, w->w_gate_up_d, 2 * F, H, T);
    gu.xf = x; gu.gamma = w->gamma_ffn; gu.eps = c.eps; gu.y = L.h; gu.ldy = F; gu.ffn = F;
    if ((rc = launch_gemv(gu, EPI_SWIGLU, s, PRO_RMSNORM))) return rc;
    GemvArgs dn = plain(w->w_down_q, w->w_down_d, H, F, T);
    dn.xf = L.h; dn.y = x; dn.residual = x;
    return launch_gemv(dn, EPI_STORE, s, PRO_Q8);
}

// Many tokens: MFMA GEMMs with separate norm/quantize kernels.
int layer_prefill(const qk_layer* w, const qk_layer_cfg& c, float* x, int64_t T,
                  const int32_t* pos, const int32_t* seq, uint16_t* kc, uint16_t* vc,
                  const LayerWs& L, hipStream_t s) {
    const int64_t H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, hd = c.head_dim;
    const int64_t Nq = nq * hd, Nkv = nkv * hd, Nqkv = Nq + 2 * Nkv, F = c.ffn;
    int rc;
    if ((rc = launch_rmsnorm_q8(x, w->gamma_attn, T, H, c.eps, nullptr, L.xq, L.xd, s))) return rc;
    if ((rc = matmul(w->w_qkv_q, w->w_qkv_d, Nqkv, H, L.xq, L.xd, T, L.qkv, nullptr, EPI_STORE, 0, s)))
        return rc;
    if ((rc = launch_rope_kv(L.qkv, T, Nqkv, 0, nq, Nq, Nq + Nkv, nkv, hd, pos, seq, c.rope_base,
                             kc, vc, c.cap, s)))
        return rc;
    if ((rc = launch_attention(L.qkv, Nqkv, T, nq, nkv, hd, kc, vc, c.cap, pos, seq, nullptr, Nq,
                               L.xq, L.xd, L.att_ws, L.att_bytes, s)))
        return rc;
    if ((rc = matmul(w->w_o_q, w->w_o_d, H, Nq, L.xq, L.xd, T, x, x, EPI_STORE, 0, s))) return rc;
    if ((rc = launch_rmsnorm_q8(x, w->gamma_ffn, T, H, c.eps, nullptr, L.xq, L.xd, s))) return rc;
    if ((rc = matmul(w->w_gate_up_q, w->w_gate_up_d, 2 * F, H, L.xq, L.xd, T, L.h, nullptr,
                     EPI_SWIGLU, F, s)))
        return rc;
    if ((rc = launch_quantize_q8(L.h, T, F, L.xq, L.xd, s))) return rc;
    return matmul(w->w_down_q, w->w_down_d, H, F, L.xq, L.xd, T, x, x, EPI_STORE, 0, s);
}

}  // namespace

}  // namespace qk

using namespace qk;

extern "C" size_t qk_layer_workspace(const qk_layer_cfg* cfg, int64_t tokens) {
    if (check_cfg(cfg) != QK_OK || tokens < 0) return 0;
    return layer_layout(nullptr, *cfg, tokens).total;
}

extern "C" int layer_forward(const qk_layer* w, const qk_layer_cfg* cfg, float* x, int64_t tokens,
                             const int32_t* pos, const int32_t* seq, uint16_t* k_cache,
                             uint16_t* v_cache, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    QK_REQUIRE(tokens >= 0 && tokens <= INT32_MAX, QK_EINVAL);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(w && x && pos && seq && k_cache && v_cache, QK_EINVAL);
    QK_REQUIRE(w->w_qkv_q && w->w_qkv_d && w->w_o_q && w->w_o_d && w->w_gate_up_q &&
                   w->w_gate_up_d && w->w_down_q && w->w_down_d && w->gamma_attn && w->gamma_ffn,
               QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(w->w_qkv_q, 16) && QK_ALIGNED(w->w_o_q, 16) &&
                   QK_ALIGNED(w->w_gate_up_q, 16) && QK_ALIGNED(w->w_down_q, 16) &&
                   QK_ALIGNED(x, 16) && QK_ALIGNED(w->gamma_attn, 16) &&
                   QK_ALIGNED(w->gamma_ffn, 16) && QK_ALIGNED(k_cache, 16) &&
                   QK_ALIGNED(v_cache, 16),
               QK_EALIGN);
    const qk_layer_cfg& c = *cfg;
    const LayerWs L = layer_layout(ws, c, tokens);
    QK_REQUIRE(ws && ws_bytes >= L.total, QK_EWORKSPACE);

    hipStream_t s = (hipStream_t)stream;
    const bool few = tokens <= 8 && gemv_prologue_fits(c.hidden, tokens) &&
                     gemv_prologue_fits(c.ffn, tokens);
    if (few) return layer_decode(w, c, x, tokens, pos, seq, k_cache, v_cache, L, s);
    return layer_prefill(w, c, x, tokens, pos, seq, k_cache, v_cache, L, s);
}

// ------------------------------------------------ layer without a workspace
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the layer's workspace lives in a file-scope device array instead of
// a caller buffer.  Each GPU holds its own copy of the array, whose device
// address is looked up once per device (with that device current) on the
// first call there; the kernels then receive that address like any
// workspace.  Nothing in the workspace has to start at zero (every byte a
// call reads was written earlier in the same call), and the array keeps the
// last call's contents.  Calls that overlap on one GPU share the array and
// race: they must be ordered (one stream, or synchronized streams).

namespace {

static __device__ __align__(256) unsigned char scratch[QK_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];

// Device address of this device's copy of `scratch` (null on failure).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" int qk_layer_forward_scratch(const qk_layer* w, const qk_layer_cfg* cfg, float* x,
                                        int64_t tokens, const int32_t* pos, const int32_t* seq,
                                        uint16_t* k_cache, uint16_t* v_cache, void* stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    QK_REQUIRE(tokens >= 0 && tokens <= INT32_MAX, QK_EINVAL);
    const size_t need = layer_layout(nullptr, *cfg, tokens).total;
    QK_REQUIRE(need <= (size_t)QK_SCRATCH_BYTES, QK_EWORKSPACE);
    if (tokens == 0) return QK_OK;
    void* ws = scratch_for_current_device();
    if (!ws) return QK_EHIP;
    return layer_forward(w, cfg, x, tokens, pos, seq, k_cache, v_cache, ws, need, stream);
}

// ------------------------------------------------------------- FFN first half
// kenji.blog TinyLLaMA-in-C++ guide, sections 4.1 and 4.4: h = SwiGLU of the
// gate and up projections of the RMSNorm'd input, each projection reading the
// Q8_0 of that input.

extern "C" size_t qk_ffn_up_workspace(int64_t hidden, int64_t tokens) {
    if (hidden <= 0 || tokens < 0) return 0;
    return align256((size_t)(tokens * hidden)) + align256(sizeof(uint16_t) * tokens * (hidden / QBLK));
}

extern "C" int qk_ffn_up(const float* x, const float* gamma, float eps, const uint8_t* w_q,
                         const uint16_t* w_d, int64_t ffn, int64_t hidden, int64_t tokens,
                         float* h, void* ws, size_t ws_bytes, void* stream) {
    QK_REQUIRE(ffn > 0 && hidden > 0 && tokens >= 0 && tokens <= INT32_MAX, QK_EINVAL);
    QK_REQUIRE(hidden % QBLK == 0 && ffn % QBLK == 0, QK_ESHAPE);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(x && gamma && w_q && w_d && h, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(x, 16) && QK_ALIGNED(gamma, 16) && QK_ALIGNED(w_q, 16) &&
                   QK_ALIGNED(h, 4),
               QK_EALIGN);
    hipStream_t s = (hipStream_t)stream;
    if (tokens <= 8 && gemv_prologue_fits(hidden, tokens)) {
        GemvArgs a = plain(w_q, w_d, 2 * ffn, hidden, tokens);
        a.xf = x; a.gamma = gamma; a.eps = eps; a.y = h; a.ldy = ffn; a.ffn = ffn;
        return launch_gemv(a, EPI_SWIGLU, s, PRO_RMSNORM);
    }
    QK_REQUIRE(ws && ws_bytes >= qk_ffn_up_workspace(hidden, tokens), QK_EWORKSPACE);
    int8_t* xq = static_cast<int8_t*>(ws);
    uint16_t* xd = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + align256((size_t)(tokens * hidden)));
    int rc = launch_rmsnorm_q8(x, gamma, tokens, hidden, eps, nullptr, xq, xd, s);
    if (rc) return rc;
    return matmul(w_q, w_d, 2 * ffn, hidden, xq, xd, tokens, h, nullptr, EPI_SWIGLU, ffn, s);
}

// ---------------------------------------------------------------- LM head
// kenji.blog TinyLLaMA-in-C++ guide, section 2 (pipeline figure): the last
// hidden state goes through RMSNorm and the LM head to the logits, and the
// greedy choice takes the largest one.

namespace {

struct HeadWs {
    float* pval;
    int32_t* pidx;
    int8_t* xq;
    uint16_t* xd;
    size_t total;
};

HeadWs head_layout(void* base, int64_t vocab, int64_t hidden, int64_t tokens) {
    const int64_t parts = gemv_argmax_parts(vocab, hidden, tokens);
    HeadWs w{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return base ? static_cast<char*>(base) + at : nullptr;
    };
    w.pval = reinterpret_cast<float*>(take(sizeof(float) * tokens * parts));
    w.pidx = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * tokens * parts));
    w.xq = reinterpret_cast<int8_t*>(take((size_t)(tokens * hidden)));
    w.xd = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * tokens * (hidden / QBLK)));
    w.total = o;
    return w;
}

}  // namespace

extern "C" size_t qk_lm_head_workspace(int64_t vocab, int64_t hidden, int64_t tokens) {
    if (vocab <= 0 || hidden <= 0 || tokens < 0) return 0;
    return head_layout(nullptr, vocab, hidden, tokens).total;
}

extern "C" int qk_lm_head(const float* x, const float* gamma, float eps, const uint8_t* w_q,
                          const uint16_t* w_d, int64_t vocab, int64_t hidden, int64_t tokens,
                          float* logits, int32_t* next, void* ws, size_t ws_bytes, void* stream) {
    QK_REQUIRE(vocab > 0 && vocab <= INT32_MAX && hidden > 0 && tokens >= 0 &&
                   tokens <= INT32_MAX,
               QK_EINVAL);
    QK_REQUIRE(hidden % QBLK == 0, QK_ESHAPE);
    if (tokens == 0) return QK_OK;
    QK_REQUIRE(x && gamma && w_q && w_d && logits && next, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(x, 16) && QK_ALIGNED(gamma, 16) && QK_ALIGNED(w_q, 16) &&
                   QK_ALIGNED(logits, 4),
               QK_EALIGN);
    const HeadWs H = head_layout(ws, vocab, hidden, tokens);
    QK_REQUIRE(ws && ws_bytes >= H.total, QK_EWORKSPACE);
    hipStream_t s = (hipStream_t)stream;
    int rc;
    if (tokens <= 8 && gemv_prologue_fits(hidden, tokens)) {
        GemvArgs a = plain(w_q, w_d, vocab, hidden, tokens);
        a.xf = x; a.gamma = gamma; a.eps = eps; a.y = logits; a.ldy = vocab;
        a.part_val = H.pval; a.part_idx = H.pidx;
        if ((rc = launch_gemv(a, EPI_ARGMAX, s, PRO_RMSNORM))) return rc;
        return launch_argmax_partials(H.pval, H.pidx, gemv_argmax_parts(vocab, hidden, tokens),
                                      tokens, next, s);
    }
    if ((rc = launch_rmsnorm_q8(x, gamma, tokens, hidden, eps, nullptr, H.xq, H.xd, s))) return rc;
    if ((rc = matmul(w_q, w_d, vocab, hidden, H.xq, H.xd, tokens, logits, nullptr, EPI_STORE, 0, s)))
        return rc;
    return qk_argmax(logits, tokens, vocab, next, stream);
}

extern "C" const char* qk_strerror(int status) {
    switch (status) {
        case QK_OK: return "success";
        case QK_EINVAL: return "invalid argument (null pointer or out-of-range value)";
        case QK_ESHAPE: return "unsupported shape (k % 32, heads, head_dim or ffn constraint)";
        case QK_EALIGN: return "misaligned pointer";
        case QK_EWORKSPACE: return "workspace missing or too small";
        case QK_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}
