// The pre-norm decoder layer, its workspace, and status strings.
//
// Order of operations: kenji.blog TinyLLaMA-in-C++ guide, section 5.2 (per-
// step graph: norm, Q/K/V projections, RoPE, KV store and load, attention,
// scale and softmax, output projection, residual add) and section 4.4 for the
// SwiGLU feed-forward half, which repeats the norm -> projection -> residual
// pattern with its own gain.  Every Q4_0 matmul reads Q8_0 activations
// (llama.cpp guide 2.2); the FFN input is quantized once for gate and up.
#include "internal.h"

namespace qk {

namespace {

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct LayerWs {
    int8_t* xq;       // [T][max(H, Nq, F)]
    uint16_t* xd;     // [T][max/32]
    float* qkv;       // [T][Nqkv]
    float* attn;      // [T][Nq]
    float* h;         // [T][F]
    void* att_ws;     // attention partials
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
    w.attn = reinterpret_cast<float*>(take(sizeof(float) * T * Nq));
    w.h = reinterpret_cast<float*>(take(sizeof(float) * T * F));
    w.att_bytes = attention_ws_bytes(T, c.n_q_heads, c.head_dim, c.cap);
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
    return QK_OK;
}

int matmul(const uint8_t* wq, const uint16_t* wd, int64_t n, int64_t k, const int8_t* xq,
           const uint16_t* xd, int64_t m, float* y, const float* residual, int epi, int64_t ffn,
           hipStream_t s) {
    GemvArgs a{};
    a.wq = wq; a.wd = wd; a.n = n; a.k = k;
    a.xq = xq; a.xd = xd; a.m = (int32_t)m; a.groups = 1;
    a.y = y; a.ldy = (epi == EPI_SWIGLU) ? ffn : n;
    a.residual = residual; a.ldr = n; a.ffn = ffn; a.max_cols = (int32_t)m;
    return m > 8 ? launch_gemm(a, epi, s) : launch_gemv(a, epi, s);
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
    const int64_t T = tokens, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, hd = c.head_dim;
    const int64_t Nq = nq * hd, Nkv = nkv * hd, Nqkv = Nq + 2 * Nkv, F = c.ffn;

    // attention half
    if ((rc = launch_rmsnorm_q8(x, w->gamma_attn, T, H, c.eps, nullptr, L.xq, L.xd, s))) return rc;
    if ((rc = matmul(w->w_qkv_q, w->w_qkv_d, Nqkv, H, L.xq, L.xd, T, L.qkv, nullptr, EPI_STORE, 0, s)))
        return rc;
    if ((rc = launch_rope_kv(L.qkv, T, Nqkv, 0, nq, Nq, Nq + Nkv, nkv, hd, pos, seq, c.rope_base,
                             k_cache, v_cache, c.cap, s)))
        return rc;
    if ((rc = launch_attention(L.qkv, Nqkv, T, nq, nkv, hd, k_cache, v_cache, c.cap, pos, seq,
                               L.attn, Nq, L.att_ws, L.att_bytes, s)))
        return rc;
    if ((rc = launch_quantize_q8(L.attn, T, Nq, L.xq, L.xd, s))) return rc;
    if ((rc = matmul(w->w_o_q, w->w_o_d, H, Nq, L.xq, L.xd, T, x, x, EPI_STORE, 0, s))) return rc;

    // feed-forward half
    if ((rc = launch_rmsnorm_q8(x, w->gamma_ffn, T, H, c.eps, nullptr, L.xq, L.xd, s))) return rc;
    if ((rc = matmul(w->w_gate_up_q, w->w_gate_up_d, 2 * F, H, L.xq, L.xd, T, L.h, nullptr,
                     EPI_SWIGLU, F, s)))
        return rc;
    if ((rc = launch_quantize_q8(L.h, T, F, L.xq, L.xd, s))) return rc;
    return matmul(w->w_down_q, w->w_down_d, H, F, L.xq, L.xd, T, x, x, EPI_STORE, 0, s);
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
