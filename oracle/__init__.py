"""ctypes view of the CPU oracle (``oracle.cpp``), on numpy arrays.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the GPU library and its
Python binding never do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F32 = ctypes.c_float


def build() -> None:
    """Compile ``oracle.cpp`` (g++ -O2, OpenMP, no fast-math, no contraction)."""
    cmd = ["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", os.path.join(_HERE, "oracle.cpp"), "-o", _SO + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)


class Layer(ctypes.Structure):
    _fields_ = [("w_qkv_q", _P), ("w_qkv_d", _P), ("w_o_q", _P), ("w_o_d", _P),
                ("w_gu_q", _P), ("w_gu_d", _P), ("w_down_q", _P), ("w_down_d", _P),
                ("gamma_attn", _P), ("gamma_ffn", _P)]


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", _I64), ("n_q_heads", _I64), ("n_kv_heads", _I64), ("head_dim", _I64),
                ("ffn", _I64), ("eps", _F32), ("rope_base", _F32), ("cap", _I64)]


_SIGS = {
    "oracle_f32_to_f16": ([_F32], ctypes.c_uint16),
    "oracle_f16_to_f32": ([ctypes.c_uint16], _F32),
    "oracle_f32_to_f16_array": ([_P, _I64, _P], None),
    "oracle_f16_to_f32_array": ([_P, _I64, _P], None),
    "oracle_quantize_q4_0": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "oracle_quantize_q8_0": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "oracle_block_dots_q4_0_q8_0": ([_P, _I64, _I64, _P, _I64, _P], ctypes.c_int),
    "oracle_qmatmul_q4_0_q8_0": ([_P, _P, _I64, _I64, _P, _P, _I64, _P], ctypes.c_int),
    "oracle_rmsnorm": ([_P, _P, _I64, _I64, _F32, _P], ctypes.c_int),
    "oracle_rope": ([_P, _I64, _I64, _I64, _P, _F32], ctypes.c_int),
    "oracle_kv_append": ([_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _I64], ctypes.c_int),
    "oracle_gqa_attention": ([_P, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _P, _P], ctypes.c_int),
    "oracle_swiglu": ([_P, _P, _I64, _P], ctypes.c_int),
    "oracle_embed_lookup": ([_P, _I64, _I64, _P, _I64, _P], ctypes.c_int),
    "oracle_argmax": ([_P, _I64, _I64, _P], ctypes.c_int),
    "oracle_sample": ([_P, _I64, _I64, ctypes.c_int32, ctypes.c_double, ctypes.c_float, _P, _P],
                      ctypes.c_int),
    "oracle_layer_forward": ([ctypes.POINTER(Layer), ctypes.POINTER(LayerCfg), _P, _I64, _P, _P,
                              _P, _P], ctypes.c_int),
    "oracle_moe_route": ([_P, _I64, _I64, _P, _I64, _I32, _P, _P, _P], ctypes.c_int),
    "oracle_moe_expert_ffn": ([_P, _I64, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "oracle_moe_route_and_apply": ([_P, _I64, _I64, _P, _I64, _I32, _P, _P, _P, _P, _I64, _P,
                                    _P, _P], ctypes.c_int),
    "oracle_quantize_rowq": ([_I32, _P, _I64, _I64, _P, _P], ctypes.c_int),
    "oracle_qmatmul_rowq_q8_0": ([_I32, _P, _P, _I64, _I64, _P, _P, _I64, _P], ctypes.c_int),
    "oracle_moe_route_and_apply_rowq": ([_I32, _P, _I64, _I64, _P, _I64, _I32, _P, _P, _P, _P,
                                         _I64, _P, _P, _P], ctypes.c_int),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_SO)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# fp16
# --------------------------------------------------------------------------
def f32_to_f16(x) -> np.ndarray:
    """binary16 bit patterns (uint16) of fp32 values, round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_array(_p(x), x.size, _p(out))
    return out


def f16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_array(_p(h), h.size, _p(out))
    return out


# --------------------------------------------------------------------------
# quantizers and matmul
# --------------------------------------------------------------------------
def quantize_q4_0(w) -> tuple[np.ndarray, np.ndarray]:
    """Q4_0 of an fp32 [n][k] matrix -> (nibbles uint8 [n][k/2], scales uint16 [n][k/32])."""
    w = _c(w, np.float32)
    n, k = w.shape
    wq = np.empty((n, k // 2), np.uint8)
    wd = np.empty((n, k // 32), np.uint16)
    _check(lib().oracle_quantize_q4_0(_p(w), n, k, _p(wq), _p(wd)), "quantize_q4_0")
    return wq, wd


def quantize_q8_0(x) -> tuple[np.ndarray, np.ndarray]:
    """Q8_0 of fp32 [rows][k] -> (int8 [rows][k], fp16 bits [rows][k/32])."""
    x = _c(x, np.float32)
    x2 = x.reshape(-1, x.shape[-1])
    rows, k = x2.shape
    q = np.empty((rows, k), np.int8)
    d = np.empty((rows, k // 32), np.uint16)
    _check(lib().oracle_quantize_q8_0(_p(x2), rows, k, _p(q), _p(d)), "quantize_q8_0")
    return q.reshape(x.shape), d.reshape(x.shape[:-1] + (k // 32,))


def block_dots(wq, k: int, xq) -> np.ndarray:
    """int32 [m][n][k/32] per-block dot products of Q4_0 rows with Q8_0 rows."""
    wq = _c(wq, np.uint8)
    xq = _c(xq, np.int8).reshape(-1, k)
    n, m = wq.shape[0], xq.shape[0]
    out = np.empty((m, n, k // 32), np.int32)
    _check(lib().oracle_block_dots_q4_0_q8_0(_p(wq), n, k, _p(xq), m, _p(out)), "block_dots")
    return out


def qmatmul(wq, wd, xq, xd) -> np.ndarray:
    """y [m][n] = Q4_0 W [n][k] times Q8_0 x [m][k] (fp32 out)."""
    wq = _c(wq, np.uint8)
    wd = _c(wd, np.uint16)
    n, k = wq.shape[0], wq.shape[1] * 2
    xq = _c(xq, np.int8).reshape(-1, k)
    xd = _c(xd, np.uint16).reshape(-1, k // 32)
    m = xq.shape[0]
    y = np.empty((m, n), np.float32)
    _check(lib().oracle_qmatmul_q4_0_q8_0(_p(wq), _p(wd), n, k, _p(xq), _p(xd), m, _p(y)),
           "qmatmul")
    return y


def quantize_rowq(w, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Row-scaled int4 (bits 4) or int2 (bits 2) of an fp32 [n][k] matrix ->
    (codes uint8 [n][k * bits / 8], scales fp32 [n])."""
    w = _c(w, np.float32)
    n, k = w.shape
    wq = np.empty((n, k * bits // 8), np.uint8)
    wr = np.empty(n, np.float32)
    _check(lib().oracle_quantize_rowq(bits, _p(w), n, k, _p(wq), _p(wr)), "quantize_rowq")
    return wq, wr


def qmatmul_rowq(wq, wr, xq, xd, bits: int) -> np.ndarray:
    """y [m][n] = row-scaled int4/int2 W [n][k] times Q8_0 x [m][k] (fp32 out)."""
    wq = _c(wq, np.uint8)
    wr = _c(wr, np.float32)
    n, k = wq.shape[0], wq.shape[1] * 8 // bits
    xq = _c(xq, np.int8).reshape(-1, k)
    xd = _c(xd, np.uint16).reshape(-1, k // 32)
    m = xq.shape[0]
    y = np.empty((m, n), np.float32)
    _check(lib().oracle_qmatmul_rowq_q8_0(bits, _p(wq), _p(wr), n, k, _p(xq), _p(xd), m, _p(y)),
           "qmatmul_rowq")
    return y


# --------------------------------------------------------------------------
# float ops
# --------------------------------------------------------------------------
def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    x = _c(x, np.float32)
    gamma = _c(gamma, np.float32)
    dim = x.shape[-1]
    y = np.empty_like(x)
    _check(lib().oracle_rmsnorm(_p(x), _p(gamma), x.size // dim, dim, eps, _p(y)), "rmsnorm")
    return y


def rope(x, pos, base: float) -> np.ndarray:
    """x [tokens][heads][hd] (copied), rotated in pairs (2i, 2i+1)."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    pos = _c(pos, np.int32)
    t, h, hd = x.shape
    _check(lib().oracle_rope(_p(x), t, h, hd, _p(pos), base), "rope")
    return x


def kv_append(k, v, pos, seq, k_cache, v_cache) -> None:
    """k, v [tokens][n_kv][hd] fp32; caches uint16 [seqs][n_kv][cap][hd], updated in place."""
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    pos = _c(pos, np.int32)
    seq = _c(seq, np.int32)
    t, nkv, hd = k.shape
    cap = k_cache.shape[2]
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    _check(lib().oracle_kv_append(_p(k), _p(v), t, nkv, hd, _p(pos), _p(seq), _p(k_cache),
                                  _p(v_cache), cap), "kv_append")


def gqa_attention(q, k_cache, v_cache, pos, seq) -> np.ndarray:
    """q [tokens][nq][hd]; caches uint16 [seqs][nkv][cap][hd] -> out [tokens][nq][hd]."""
    q = _c(q, np.float32)
    k_cache = _c(k_cache, np.uint16)
    v_cache = _c(v_cache, np.uint16)
    pos = _c(pos, np.int32)
    seq = _c(seq, np.int32)
    t, nq, hd = q.shape
    nkv, cap = k_cache.shape[1], k_cache.shape[2]
    out = np.empty_like(q)
    _check(lib().oracle_gqa_attention(_p(q), t, nq, nkv, hd, _p(k_cache), _p(v_cache), cap,
                                      _p(pos), _p(seq), _p(out)), "gqa_attention")
    return out


def swiglu(gate, up) -> np.ndarray:
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    h = np.empty_like(gate)
    _check(lib().oracle_swiglu(_p(gate), _p(up), gate.size, _p(h)), "swiglu")
    return h


def embed_lookup(table, ids) -> np.ndarray:
    table = _c(table, np.float32)
    ids = _c(ids, np.int32)
    vocab, hidden = table.shape
    x = np.empty((ids.size, hidden), np.float32)
    _check(lib().oracle_embed_lookup(_p(table), vocab, hidden, _p(ids), ids.size, _p(x)), "embed")
    return x


def argmax(logits) -> np.ndarray:
    logits = _c(logits, np.float32)
    vocab = logits.shape[-1]
    rows = logits.size // vocab
    idx = np.empty(rows, np.int32)
    _check(lib().oracle_argmax(_p(logits), rows, vocab, _p(idx)), "argmax")
    return idx


def sample(logits, top_k: int, top_p: float, temperature: float, u, top_p_shift: float = 0.0) -> np.ndarray:
    """Sampler chain (top-k, top-p, temperature, draw with the given uniforms).

    top_p is taken at float32, as the library takes it; top_p_shift moves the
    cut by a small amount past that value (to probe a boundary)."""
    top_p = float(np.float32(top_p)) + top_p_shift
    logits = _c(logits, np.float32)
    vocab = logits.shape[-1]
    rows = logits.size // vocab
    u = _c(np.broadcast_to(np.asarray(u, np.float64), (rows,)), np.float64)
    out = np.empty(rows, np.int32)
    _check(lib().oracle_sample(_p(logits), rows, vocab, top_k, top_p, temperature, _p(u), _p(out)),
           "sample")
    return out


# --------------------------------------------------------------------------
# layer, MoE
# --------------------------------------------------------------------------
def layer_forward(w: dict, cfg: dict, x, pos, seq, k_cache, v_cache) -> np.ndarray:
    """One decoder layer on x [tokens][hidden] (returned as a new array); the
    caches (uint16, [seqs][nkv][cap][hd]) are updated in place.

    ``w`` holds numpy arrays: w_qkv_q, w_qkv_d, w_o_q, w_o_d, w_gu_q, w_gu_d,
    w_down_q, w_down_d, gamma_attn, gamma_ffn.  ``cfg`` holds hidden, n_q_heads,
    n_kv_heads, head_dim, ffn, eps, rope_base, cap."""
    arrs = {k2: np.ascontiguousarray(v2) for k2, v2 in w.items()}
    layer = Layer(**{k2: arrs[k2].ctypes.data for k2 in [f[0] for f in Layer._fields_]})
    c = LayerCfg(cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"],
                 cfg["eps"], cfg["rope_base"], cfg["cap"])
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    pos = _c(pos, np.int32)
    seq = _c(seq, np.int32)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
    _check(lib().oracle_layer_forward(ctypes.byref(layer), ctypes.byref(c), _p(x), x.shape[0],
                                      _p(pos), _p(seq), _p(k_cache), _p(v_cache)), "layer_forward")
    return x


def moe_route(x, w_router, top_k: int, return_logits: bool = False):
    x = _c(x, np.float32)
    w_router = _c(w_router, np.float32)
    t, hidden = x.shape
    e = w_router.shape[1]
    idx = np.empty((t, top_k), np.int32)
    wts = np.empty((t, top_k), np.float32)
    logits = np.empty((t, e), np.float32) if return_logits else None
    _check(lib().oracle_moe_route(_p(x), t, hidden, _p(w_router), e, top_k, _p(idx), _p(wts),
                                  _p(logits)), "moe_route")
    return (idx, wts, logits) if return_logits else (idx, wts)


def moe_expert_ffn(x_row, gu_q, gu_d, dn_q, dn_d) -> np.ndarray:
    x_row = _c(x_row, np.float32)
    hidden = x_row.size
    ffn = gu_q.shape[0] // 2
    y = np.empty(hidden, np.float32)
    _check(lib().oracle_moe_expert_ffn(_p(x_row), hidden, ffn, _p(_c(gu_q, np.uint8)),
                                       _p(_c(gu_d, np.uint16)), _p(_c(dn_q, np.uint8)),
                                       _p(_c(dn_d, np.uint16)), _p(y)), "moe_expert_ffn")
    return y


def moe_route_and_apply(x, w_router, top_k: int, gu_q, gu_d, dn_q, dn_d):
    """Experts stacked: gu_q [E][2F][H/2], gu_d [E][2F][H/32], dn_q [E][H][F/2],
    dn_d [E][H][F/32].  Returns (out [T][H], sel_idx [T][k], sel_w [T][k])."""
    x = _c(x, np.float32)
    w_router = _c(w_router, np.float32)
    t, hidden = x.shape
    e = w_router.shape[1]
    ffn = gu_q.shape[1] // 2
    out = np.empty_like(x)
    idx = np.empty((t, top_k), np.int32)
    wts = np.empty((t, top_k), np.float32)
    _check(lib().oracle_moe_route_and_apply(
        _p(x), t, hidden, _p(w_router), e, top_k, _p(_c(gu_q, np.uint8)), _p(_c(gu_d, np.uint16)),
        _p(_c(dn_q, np.uint8)), _p(_c(dn_d, np.uint16)), ffn, _p(out), _p(idx), _p(wts)),
        "moe_route_and_apply")
    return out, idx, wts


def moe_route_and_apply_rowq(x, w_router, top_k: int, gu_q, gu_r, dn_q, dn_r, bits: int):
    """Row-scaled experts stacked: gu_q [E][2F][H * bits / 8], gu_r [E][2F] fp32,
    dn_q [E][H][F * bits / 8], dn_r [E][H].  Returns (out, sel_idx, sel_w)."""
    x = _c(x, np.float32)
    w_router = _c(w_router, np.float32)
    t, hidden = x.shape
    e = w_router.shape[1]
    ffn = gu_q.shape[1] // 2
    out = np.empty_like(x)
    idx = np.empty((t, top_k), np.int32)
    wts = np.empty((t, top_k), np.float32)
    _check(lib().oracle_moe_route_and_apply_rowq(
        bits, _p(x), t, hidden, _p(w_router), e, top_k, _p(_c(gu_q, np.uint8)), _p(_c(gu_r, np.float32)),
        _p(_c(dn_q, np.uint8)), _p(_c(dn_r, np.float32)), ffn, _p(out), _p(idx), _p(wts)),
        "moe_route_and_apply_rowq")
    return out, idx, wts
