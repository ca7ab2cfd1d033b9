"""Python binding of libqk (``include/qk.h``): the same entry points, on
torch tensors.

This module only marshals arguments: it checks devices, dtypes and
contiguity, hands raw device pointers and the current HIP stream to the C
library, and allocates outputs with torch when the caller gives none.  Every
step of the computation runs in the library's HIP kernels; there is no other
code path, and calls fail loudly when ``libqk.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqk.so")
_lib = None

QK_OK, QK_EINVAL, QK_ESHAPE, QK_EALIGN, QK_EWORKSPACE, QK_EHIP = 0, -1, -2, -3, -4, -5
QK_SCRATCH_BYTES = 8 << 20   # device array behind qk_layer_forward_scratch (include/qk.h)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t


class QKError(RuntimeError):
    def __init__(self, name: str, status: int):
        super().__init__(f"{name} failed: {strerror(status)} (status {status})")
        self.status = status


class Layer(ctypes.Structure):
    _fields_ = [("w_qkv_q", _P), ("w_qkv_d", _P), ("w_o_q", _P), ("w_o_d", _P),
                ("w_gate_up_q", _P), ("w_gate_up_d", _P), ("w_down_q", _P), ("w_down_d", _P),
                ("gamma_attn", _P), ("gamma_ffn", _P)]


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", _I64), ("n_q_heads", _I64), ("n_kv_heads", _I64), ("head_dim", _I64),
                ("ffn", _I64), ("eps", _F32), ("rope_base", _F32), ("cap", _I64)]


class DecoderStruct(ctypes.Structure):
    """qk_decoder of include/qk.h."""
    _fields_ = [("layers", _P), ("n_layers", _I64), ("embed", _P), ("gamma_final", _P),
                ("lm_q", _P), ("lm_d", _P), ("vocab", _I64), ("k_cache", _P), ("v_cache", _P)]


_SIGS = {
    "qk_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "quantize_q8_0": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "qk_quantize_q4_0": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "qk_q4_0_from_blocks": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "qmatmul_q4_0_q8_0": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _P], ctypes.c_int),
    "qk_block_dots_q4_0_q8_0": ([_P, _I64, _I64, _P, _I64, _P, _P], ctypes.c_int),
    "qk_gate_up_swiglu": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _P], ctypes.c_int),
    "rmsnorm": ([_P, _P, _I64, _I64, _F32, _P, _P], ctypes.c_int),
    "rope": ([_P, _I64, _I64, _I64, _P, _F32, _P], ctypes.c_int),
    "swiglu": ([_P, _P, _I64, _P, _P], ctypes.c_int),
    "qk_kv_append": ([_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _P], ctypes.c_int),
    "qk_embed_lookup": ([_P, _I64, _I64, _P, _I64, _P, _P], ctypes.c_int),
    "qk_read_probe": ([_P, _I64, _P, ctypes.c_int32, _P], ctypes.c_int),
    "qk_sample": ([_P, _I64, _I64, ctypes.c_int32, ctypes.c_float, ctypes.c_float, _P, _P, _P],
                  ctypes.c_int),
    "qk_argmax": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "gqa_attention": ([_P, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _SZ, _P],
                      ctypes.c_int),
    "qk_gqa_attention_workspace": ([_I64, _I64, _I64, _I64], _SZ),
    "layer_forward": ([ctypes.POINTER(Layer), ctypes.POINTER(LayerCfg), _P, _I64, _P, _P, _P, _P,
                       _P, _SZ, _P], ctypes.c_int),
    "qk_layer_workspace": ([ctypes.POINTER(LayerCfg), _I64], _SZ),
    "qk_layer_forward_scratch": ([ctypes.POINTER(Layer), ctypes.POINTER(LayerCfg), _P, _I64, _P, _P,
                                  _P, _P, _P], ctypes.c_int),
    "moe_route_and_apply": ([_P, _I64, _I64, _P, _I64, _I32, _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                             _SZ, _P], ctypes.c_int),
    "qk_moe_workspace": ([_I64, _I64, _I64, _I32, _I64], _SZ),
    "qk_quantize_rowq": ([_I32, _P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "qk_qmatmul_rowq_q8_0": ([_I32, _P, _P, _I64, _I64, _P, _P, _I64, _P, _P], ctypes.c_int),
    "qk_moe_route_and_apply_rowq": ([_I32, _P, _I64, _I64, _P, _I64, _I32, _P, _P, _P, _P, _I64, _P,
                                     _P, _P, _P, _SZ, _P], ctypes.c_int),
    "qk_lm_head": ([_P, _P, _F32, _P, _P, _I64, _I64, _I64, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "qk_lm_head_workspace": ([_I64, _I64, _I64], _SZ),
    "qk_ffn_up": ([_P, _P, _F32, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P], ctypes.c_int),
    "qk_ffn_up_workspace": ([_I64, _I64], _SZ),
    "qk_decode_workspace": ([ctypes.POINTER(LayerCfg)], _SZ),
    "qk_decode_greedy": ([ctypes.POINTER(DecoderStruct), ctypes.POINTER(LayerCfg), _P, _P, _I64, _I64,
                          _P, _P, _I64, ctypes.c_uint32, _P, _SZ, _P], ctypes.c_int),
    "qk_decode_error": ([_P, ctypes.POINTER(LayerCfg), _P], ctypes.c_int),
}

EXPORTS = tuple(_SIGS)


def load():
    """Load libqk.so (raises when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return load().qk_strerror(status).decode()


def _check(rc: int, name: str) -> None:
    if rc != QK_OK:
        raise QKError(name, rc)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dev16(t: torch.Tensor, name: str) -> int:
    """fp16 bit patterns: int16 or float16 tensors are both accepted."""
    if t.dtype == torch.float16:
        return _dev(t, torch.float16, name)
    return _dev(t, torch.int16, name)


def _out(out, shape, dtype, like: torch.Tensor):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


# ---------------------------------------------------------------------------
# workspace
# ---------------------------------------------------------------------------
class Workspace:
    """A growable device byte buffer.  Calls that capture a HIP graph should
    size it first (``reserve``) so that no allocation happens during capture."""

    def __init__(self):
        self.buf: torch.Tensor | None = None

    def reserve(self, nbytes: int, device) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws: dict = {}


def _ws(ws, nbytes: int, device):
    if ws is None:
        key = torch.device(device)
        ws = _default_ws.setdefault(key, Workspace())
    if isinstance(ws, Workspace):
        return ws.reserve(nbytes, device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {nbytes} needed")
    return ws


# ---------------------------------------------------------------------------
# quantization and matmul
# ---------------------------------------------------------------------------
def quantize_q8_0(x: torch.Tensor, out_q=None, out_d=None):
    """Q8_0 of fp32 x [..., k] -> (int8 [..., k], fp16 bits as int16 [..., k/32])."""
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    q = _out(out_q, x.shape, torch.int8, x)
    d = _out(out_d, x.shape[:-1] + (k // 32,), torch.int16, x)
    _check(load().quantize_q8_0(_dev(x, torch.float32, "x"), rows, k, _dev(q, torch.int8, "x_q"),
                                _dev16(d, "x_d"), _stream()), "quantize_q8_0")
    return q, d


def qk_quantize_q4_0(w: torch.Tensor, out_q=None, out_d=None):
    """Q4_0 of fp32 w [n][k] -> (uint8 nibbles [n][k/2], fp16 bits as int16 [n][k/32])."""
    n, k = w.shape
    q = _out(out_q, (n, k // 2), torch.uint8, w)
    d = _out(out_d, (n, k // 32), torch.int16, w)
    _check(load().qk_quantize_q4_0(_dev(w, torch.float32, "w"), n, k, _dev(q, torch.uint8, "w_q"),
                                   _dev16(d, "w_d"), _stream()), "qk_quantize_q4_0")
    return q, d


def qmatmul_q4_0_q8_0(w_q, w_d, x_q, x_d, out=None):
    """y [m][n] = Q4_0 W [n][k] times Q8_0 x [m][k]."""
    n, k = w_q.shape[0], w_q.shape[1] * 2
    m = x_q.numel() // k
    y = _out(out, (m, n), torch.float32, x_q)
    _check(load().qmatmul_q4_0_q8_0(_dev(w_q, torch.uint8, "w_q"), _dev16(w_d, "w_d"), n,
                                    k, _dev(x_q, torch.int8, "x_q"), _dev16(x_d, "x_d"), m,
                                    _dev(y, torch.float32, "y"), _stream()), "qmatmul_q4_0_q8_0")
    return y


def qk_quantize_rowq(w: torch.Tensor, bits: int, out_q=None, out_r=None):
    """Row-scaled int4 (bits 4) or int2 (bits 2) of fp32 w [n][k] ->
    (uint8 codes [n][k * bits / 8], fp32 scales [n])."""
    n, k = w.shape
    q = _out(out_q, (n, k * bits // 8), torch.uint8, w)
    r = _out(out_r, (n,), torch.float32, w)
    _check(load().qk_quantize_rowq(bits, _dev(w, torch.float32, "w"), n, k, _dev(q, torch.uint8, "w_q"),
                                   _dev(r, torch.float32, "w_r"), _stream()), "qk_quantize_rowq")
    return q, r


def qk_qmatmul_rowq_q8_0(w_q, w_r, x_q, x_d, bits: int, out=None):
    """y [m][n] = row-scaled int4/int2 W [n][k] times Q8_0 x [m][k]."""
    n, k = w_q.shape[0], w_q.shape[1] * 8 // bits
    m = x_q.numel() // k
    y = _out(out, (m, n), torch.float32, x_q)
    _check(load().qk_qmatmul_rowq_q8_0(bits, _dev(w_q, torch.uint8, "w_q"), _dev(w_r, torch.float32, "w_r"),
                                       n, k, _dev(x_q, torch.int8, "x_q"), _dev16(x_d, "x_d"), m,
                                       _dev(y, torch.float32, "y"), _stream()), "qk_qmatmul_rowq_q8_0")
    return y


def qk_gate_up_swiglu(w_q, w_d, x_q, x_d, out=None):
    """h [m][ffn] = swish(W_gate x) * (W_up x), W = [gate rows; up rows] Q4_0 [2 ffn][k]."""
    ffn, k = w_q.shape[0] // 2, w_q.shape[1] * 2
    m = x_q.numel() // k
    h = _out(out, (m, ffn), torch.float32, x_q)
    _check(load().qk_gate_up_swiglu(_dev(w_q, torch.uint8, "w_q"), _dev16(w_d, "w_d"), ffn, k,
                                    _dev(x_q, torch.int8, "x_q"), _dev16(x_d, "x_d"), m,
                                    _dev(h, torch.float32, "h"), _stream()), "qk_gate_up_swiglu")
    return h


def qk_block_dots_q4_0_q8_0(w_q, x_q, out=None):
    n, k = w_q.shape[0], w_q.shape[1] * 2
    m = x_q.numel() // k
    isum = _out(out, (m, n, k // 32), torch.int32, x_q)
    _check(load().qk_block_dots_q4_0_q8_0(_dev(w_q, torch.uint8, "w_q"), n, k,
                                          _dev(x_q, torch.int8, "x_q"), m,
                                          _dev(isum, torch.int32, "isum"), _stream()),
           "qk_block_dots_q4_0_q8_0")
    return isum


# ---------------------------------------------------------------------------
# element-wise
# ---------------------------------------------------------------------------
def rmsnorm(x, gamma, eps: float, out=None):
    dim = x.shape[-1]
    y = _out(out, x.shape, torch.float32, x)
    _check(load().rmsnorm(_dev(x, torch.float32, "x"), _dev(gamma, torch.float32, "gamma"),
                          x.numel() // dim, dim, eps, _dev(y, torch.float32, "y"), _stream()),
           "rmsnorm")
    return y


def rope(x, pos, base: float):
    """In place on x [tokens][heads][hd]; pos int32 [tokens] on the device."""
    t, h, hd = x.shape
    _check(load().rope(_dev(x, torch.float32, "x"), t, h, hd, _dev(pos, torch.int32, "pos"), base,
                       _stream()), "rope")
    return x


def swiglu(gate, up, out=None):
    h = _out(out, gate.shape, torch.float32, gate)
    _check(load().swiglu(_dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up"),
                         gate.numel(), _dev(h, torch.float32, "h"), _stream()), "swiglu")
    return h


def qk_kv_append(k, v, pos, seq, k_cache, v_cache):
    t, nkv, hd = k.shape
    cap = k_cache.shape[2]
    _check(load().qk_kv_append(_dev(k, torch.float32, "k"), _dev(v, torch.float32, "v"), t, nkv, hd,
                               _dev(pos, torch.int32, "pos"), _dev(seq, torch.int32, "seq"),
                               _dev16(k_cache, "k_cache"),
                               _dev16(v_cache, "v_cache"), cap, _stream()),
           "qk_kv_append")


def qk_embed_lookup(table, ids, out=None):
    vocab, hidden = table.shape
    x = _out(out, (ids.numel(), hidden), torch.float32, table)
    _check(load().qk_embed_lookup(_dev(table, torch.float32, "table"), vocab, hidden,
                                  _dev(ids, torch.int32, "ids"), ids.numel(),
                                  _dev(x, torch.float32, "x"), _stream()), "qk_embed_lookup")
    return x


def qk_sample(logits, top_k: int, top_p: float, temperature: float, u, out=None):
    """Sampler chain over logits [rows][vocab] with uniforms u [rows] (fp64) -> ids."""
    vocab = logits.shape[-1]
    rows = logits.numel() // vocab
    ids = _out(out, (rows,), torch.int32, logits)
    _check(load().qk_sample(_dev(logits, torch.float32, "logits"), rows, vocab, top_k, top_p,
                            temperature, _dev(u, torch.float64, "u"), _dev(ids, torch.int32, "ids"),
                            _stream()), "qk_sample")
    return ids


def qk_read_probe(buf, blocks=2048, out=None):
    """Stream `buf` (a device tensor, a multiple of 16 bytes) through 128-bit
    non-temporal loads; returns the per-workgroup XOR words.  Timing is the
    caller's (a measurement helper, not an operation of the method)."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("qk_read_probe: buf must be a contiguous device tensor")
    words = _out(out, (blocks,), torch.int32, buf)
    _check(load().qk_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                _dev(words, torch.int32, "out"), blocks, _stream()), "qk_read_probe")
    return words


def qk_argmax(logits, out=None):
    vocab = logits.shape[-1]
    rows = logits.numel() // vocab
    idx = _out(out, (rows,), torch.int32, logits)
    _check(load().qk_argmax(_dev(logits, torch.float32, "logits"), rows, vocab,
                            _dev(idx, torch.int32, "idx"), _stream()), "qk_argmax")
    return idx


# ---------------------------------------------------------------------------
# attention, layer, MoE
# ---------------------------------------------------------------------------
def gqa_attention(q, k_cache, v_cache, pos, seq, out=None, ws=None):
    """q [tokens][nq][hd]; caches fp16 bits (int16) [seqs][nkv][cap][hd]."""
    t, nq, hd = q.shape
    nkv, cap = k_cache.shape[1], k_cache.shape[2]
    o = _out(out, q.shape, torch.float32, q)
    need = load().qk_gqa_attention_workspace(t, nq, hd, cap)
    w = _ws(ws, need, q.device)
    _check(load().gqa_attention(_dev(q, torch.float32, "q"), t, nq, nkv, hd,
                                _dev16(k_cache, "k_cache"),
                                _dev16(v_cache, "v_cache"), cap,
                                _dev(pos, torch.int32, "pos"), _dev(seq, torch.int32, "seq"),
                                _dev(o, torch.float32, "out"), w.data_ptr(), need, _stream()),
           "gqa_attention")
    return o


@dataclass
class LayerWeights:
    """Device tensors of one layer in the interface layout (Q4_0 split)."""
    w_qkv_q: torch.Tensor
    w_qkv_d: torch.Tensor
    w_o_q: torch.Tensor
    w_o_d: torch.Tensor
    w_gate_up_q: torch.Tensor
    w_gate_up_d: torch.Tensor
    w_down_q: torch.Tensor
    w_down_d: torch.Tensor
    gamma_attn: torch.Tensor
    gamma_ffn: torch.Tensor

    def struct(self) -> Layer:
        f = lambda t, dt, n: _dev(t, dt, n)  # noqa: E731
        return Layer(f(self.w_qkv_q, torch.uint8, "w_qkv_q"), _dev16(self.w_qkv_d, "w_qkv_d"),
                     f(self.w_o_q, torch.uint8, "w_o_q"), _dev16(self.w_o_d, "w_o_d"),
                     f(self.w_gate_up_q, torch.uint8, "w_gate_up_q"),
                     _dev16(self.w_gate_up_d, "w_gate_up_d"),
                     f(self.w_down_q, torch.uint8, "w_down_q"), _dev16(self.w_down_d, "w_down_d"),
                     f(self.gamma_attn, torch.float32, "gamma_attn"),
                     f(self.gamma_ffn, torch.float32, "gamma_ffn"))


def layer_cfg(hidden, n_q_heads, n_kv_heads, head_dim, ffn, eps, rope_base, cap) -> LayerCfg:
    return LayerCfg(hidden, n_q_heads, n_kv_heads, head_dim, ffn, eps, rope_base, cap)


def qk_layer_workspace(cfg: LayerCfg, tokens: int) -> int:
    return int(load().qk_layer_workspace(ctypes.byref(cfg), tokens))


def layer_forward(w, cfg: LayerCfg, x, pos, seq, k_cache, v_cache, ws=None):
    """x [tokens][hidden] updated in place; w is a LayerWeights or a Layer struct."""
    t = x.shape[0]
    need = qk_layer_workspace(cfg, t)
    wsb = _ws(ws, need, x.device)
    st = w.struct() if isinstance(w, LayerWeights) else w
    _check(load().layer_forward(ctypes.byref(st), ctypes.byref(cfg), _dev(x, torch.float32, "x"), t,
                                _dev(pos, torch.int32, "pos"), _dev(seq, torch.int32, "seq"),
                                _dev16(k_cache, "k_cache"),
                                _dev16(v_cache, "v_cache"), wsb.data_ptr(), need,
                                _stream()), "layer_forward")
    return x


def qk_layer_forward_scratch(w, cfg: LayerCfg, x, pos, seq, k_cache, v_cache):
    """layer_forward without a caller workspace (the library's own device
    array; calls that overlap on one GPU race).  x updated in place."""
    t = x.shape[0]
    st = w.struct() if isinstance(w, LayerWeights) else w
    _check(load().qk_layer_forward_scratch(ctypes.byref(st), ctypes.byref(cfg),
                                           _dev(x, torch.float32, "x"), t,
                                           _dev(pos, torch.int32, "pos"), _dev(seq, torch.int32, "seq"),
                                           _dev16(k_cache, "k_cache"), _dev16(v_cache, "v_cache"),
                                           _stream()), "qk_layer_forward_scratch")
    return x


def qk_ffn_up(x, gamma, eps: float, w_q, w_d, out=None, ws=None):
    """h [T][ffn] = SwiGLU(W_gate . Q8_0(rmsnorm(x)), W_up . Q8_0(rmsnorm(x)))."""
    t, hidden = x.shape
    ffn = w_q.shape[0] // 2
    h = _out(out, (t, ffn), torch.float32, x)
    need = int(load().qk_ffn_up_workspace(hidden, t))
    wsb = _ws(ws, need, x.device)
    _check(load().qk_ffn_up(_dev(x, torch.float32, "x"), _dev(gamma, torch.float32, "gamma"), eps,
                            _dev(w_q, torch.uint8, "w_q"), _dev16(w_d, "w_d"), ffn, hidden, t,
                            _dev(h, torch.float32, "h"), wsb.data_ptr(), need, _stream()),
           "qk_ffn_up")
    return h


def qk_lm_head_workspace(vocab: int, hidden: int, tokens: int) -> int:
    return int(load().qk_lm_head_workspace(vocab, hidden, tokens))


def qk_lm_head(x, gamma, eps: float, w_q, w_d, logits=None, next_ids=None, ws=None):
    """logits [T][V] = W . Q8_0(rmsnorm(x)), next_ids [T] = greedy argmax."""
    t, hidden = x.shape
    vocab = w_q.shape[0]
    lg = _out(logits, (t, vocab), torch.float32, x)
    nx = _out(next_ids, (t,), torch.int32, x)
    need = int(load().qk_lm_head_workspace(vocab, hidden, t))
    wsb = _ws(ws, need, x.device)
    _check(load().qk_lm_head(_dev(x, torch.float32, "x"), _dev(gamma, torch.float32, "gamma"), eps,
                             _dev(w_q, torch.uint8, "w_q"), _dev16(w_d, "w_d"), vocab, hidden, t,
                             _dev(lg, torch.float32, "logits"), _dev(nx, torch.int32, "next"),
                             wsb.data_ptr(), need, _stream()), "qk_lm_head")
    return lg, nx


def qk_moe_workspace(tokens, hidden, n_experts, top_k, ffn) -> int:
    return int(load().qk_moe_workspace(tokens, hidden, n_experts, top_k, ffn))


def moe_route_and_apply(x, w_router, top_k: int, gate_up_q, gate_up_d, down_q, down_d,
                        out=None, sel_idx=None, sel_w=None, ws=None):
    """x [T][H]; w_router [H][E]; experts stacked (see qk.h)."""
    t, hidden = x.shape
    e = w_router.shape[1]
    ffn = gate_up_q.shape[1] // 2
    y = _out(out, (t, hidden), torch.float32, x)
    si = _out(sel_idx, (t, top_k), torch.int32, x)
    sw = _out(sel_w, (t, top_k), torch.float32, x)
    need = qk_moe_workspace(t, hidden, e, top_k, ffn)
    wsb = _ws(ws, need, x.device)
    _check(load().moe_route_and_apply(
        _dev(x, torch.float32, "x"), t, hidden, _dev(w_router, torch.float32, "w_router"), e, top_k,
        _dev(gate_up_q, torch.uint8, "gate_up_q"), _dev16(gate_up_d, "gate_up_d"),
        _dev(down_q, torch.uint8, "down_q"), _dev16(down_d, "down_d"), ffn,
        _dev(y, torch.float32, "y"), _dev(si, torch.int32, "sel_idx"), _dev(sw, torch.float32, "sel_w"),
        wsb.data_ptr(), need, _stream()), "moe_route_and_apply")
    return y, si, sw


def qk_moe_route_and_apply_rowq(x, w_router, top_k: int, gate_up_q, gate_up_r, down_q, down_r,
                                bits: int, out=None, sel_idx=None, sel_w=None, ws=None):
    """x [T][H]; w_router [H][E]; row-scaled experts stacked: gate_up_q
    [E][2F][H * bits / 8], gate_up_r [E][2F], down_q [E][H][F * bits / 8],
    down_r [E][H]."""
    t, hidden = x.shape
    e = w_router.shape[1]
    ffn = gate_up_q.shape[1] // 2
    y = _out(out, (t, hidden), torch.float32, x)
    si = _out(sel_idx, (t, top_k), torch.int32, x)
    sw = _out(sel_w, (t, top_k), torch.float32, x)
    need = qk_moe_workspace(t, hidden, e, top_k, ffn)
    wsb = _ws(ws, need, x.device)
    _check(load().qk_moe_route_and_apply_rowq(
        bits, _dev(x, torch.float32, "x"), t, hidden, _dev(w_router, torch.float32, "w_router"), e,
        top_k, _dev(gate_up_q, torch.uint8, "gate_up_q"), _dev(gate_up_r, torch.float32, "gate_up_r"),
        _dev(down_q, torch.uint8, "down_q"), _dev(down_r, torch.float32, "down_r"), ffn,
        _dev(y, torch.float32, "y"), _dev(si, torch.int32, "sel_idx"), _dev(sw, torch.float32, "sel_w"),
        wsb.data_ptr(), need, _stream()), "qk_moe_route_and_apply_rowq")
    return y, si, sw


# ---------------------------------------------------------------------------
# whole-model greedy decode in one persistent kernel
# ---------------------------------------------------------------------------
def qk_decode_workspace(cfg: LayerCfg) -> int:
    return int(load().qk_decode_workspace(ctypes.byref(cfg)))


def qk_decode_greedy(dec: DecoderStruct, cfg: LayerCfg, n_tokens: int, pos0: int, out_ids,
                     first_id=None, forced=None, logits=None, spin_limit: int = 0, ws=None):
    """n_tokens greedy steps of one sequence from position pos0 (qk_decode_greedy
    of include/qk.h).  out_ids [n_tokens] int32 receives the greedy tokens;
    logits, when given, [rows][vocab] fp32 receives step j in row j % rows."""
    need = qk_decode_workspace(cfg)
    wsb = _ws(ws, need, out_ids.device)
    rows = 0 if logits is None else logits.shape[0]
    _check(load().qk_decode_greedy(ctypes.byref(dec), ctypes.byref(cfg),
                                   None if first_id is None else _dev(first_id, torch.int32, "first_id"),
                                   None if forced is None else _dev(forced, torch.int32, "forced"),
                                   pos0, n_tokens, _dev(out_ids, torch.int32, "out_ids"),
                                   None if logits is None else _dev(logits, torch.float32, "logits"),
                                   rows, spin_limit, wsb.data_ptr(), need, _stream()),
           "qk_decode_greedy")
    return out_ids


def qk_decode_error(cfg: LayerCfg, ws) -> int:
    """The error flag of the last qk_decode_greedy on ws (synchronous)."""
    buf = ws.buf if isinstance(ws, Workspace) else ws
    flag = ctypes.c_int32(0)
    _check(load().qk_decode_error(buf.data_ptr(), ctypes.byref(cfg), ctypes.byref(flag)),
           "qk_decode_error")
    return int(flag.value)
