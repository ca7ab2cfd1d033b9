"""A LLaMA-shaped decoder built from the libqk entry points.

Composition only: embedding lookup, ``layer_forward`` per layer, final
RMSNorm, Q8_0, the LM-head quantized matmul and greedy argmax, all enqueued on
the current stream [kenji.blog TinyLLaMA-in-C++ guide, section 2: embedding,
transformer blocks, RMSNorm, LM head, logits, next token].  Weights arrive as
fp32 host arrays and are quantized to Q4_0 on the device by the library.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (DecoderStruct, Layer, LayerWeights, Workspace, layer_cfg, layer_forward,
               qk_decode_greedy, qk_decode_workspace, qk_embed_lookup, qk_layer_workspace,
               qk_lm_head, qk_lm_head_workspace, qk_quantize_q4_0)


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor (uint16 fp16 bit patterns travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def quantize_on_device(w32: np.ndarray | torch.Tensor, device="cuda"):
    """fp32 [n][k] (host or device) -> Q4_0 (nibbles, scales) on the device."""
    t = w32 if isinstance(w32, torch.Tensor) else to_device(w32, device)
    q, d = qk_quantize_q4_0(t)
    return q, d


def layer_to_device(wf: dict, device="cuda") -> LayerWeights:
    """fp32 layer dict (w_qkv, w_o, w_gate_up, w_down, gamma_attn, gamma_ffn) -> device Q4_0."""
    qkv = quantize_on_device(wf["w_qkv"], device)
    o = quantize_on_device(wf["w_o"], device)
    gu = quantize_on_device(wf["w_gate_up"], device)
    dn = quantize_on_device(wf["w_down"], device)
    return LayerWeights(qkv[0], qkv[1], o[0], o[1], gu[0], gu[1], dn[0], dn[1],
                        to_device(wf["gamma_attn"], device), to_device(wf["gamma_ffn"], device))


@dataclass
class DecoderShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int            # padded to a multiple of 32
    eps: float
    rope_base: float
    layers: int
    vocab: int
    cap: int
    seqs: int = 1


class Decoder:
    """Layers, embedding, final norm and LM head resident on one device, plus
    fp16 KV caches [layer][seqs][n_kv][cap][hd]."""

    def __init__(self, shape: DecoderShape, layers: list[LayerWeights], embed: torch.Tensor,
                 gamma_final: torch.Tensor, lm_q: torch.Tensor, lm_d: torch.Tensor, device="cuda"):
        self.s = shape
        self.layers = layers
        self.structs = [lw.struct() for lw in layers]
        self.embed = embed
        self.gamma_final = gamma_final
        self.lm_q, self.lm_d = lm_q, lm_d
        self.cfg = layer_cfg(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                             shape.ffn, shape.eps, shape.rope_base, shape.cap)
        kv_shape = (shape.layers, shape.seqs, shape.n_kv_heads, shape.cap, shape.head_dim)
        self.k_cache = torch.zeros(kv_shape, dtype=torch.int16, device=device)
        self.v_cache = torch.zeros(kv_shape, dtype=torch.int16, device=device)
        self.ws = Workspace()
        self.head_ws = Workspace()
        self.device = device

    def pack(self, align: int = 4096) -> None:
        """Move every layer's weights and the LM head into one device
        allocation, in the order the step reads them (each slice aligned to
        `align` bytes); the old tensors are released."""
        fields = ["w_qkv_q", "w_qkv_d", "w_o_q", "w_o_d", "w_gate_up_q", "w_gate_up_d",
                  "w_down_q", "w_down_d", "gamma_attn", "gamma_ffn"]
        tensors = [getattr(lw, f) for lw in self.layers for f in fields] + [self.lm_q, self.lm_d]
        sizes = [t.numel() * t.element_size() for t in tensors]
        offs, o = [], 0
        for n in sizes:
            offs.append(o)
            o += (n + align - 1) // align * align
        arena = torch.empty(o, dtype=torch.uint8, device=self.device)
        views = []
        for t, off, n in zip(tensors, offs, sizes):
            v = arena[off:off + n].view(t.dtype).view(t.shape)
            v.copy_(t)
            views.append(v)
        it = iter(views)
        self.layers = [LayerWeights(*[next(it) for _ in fields]) for _ in self.layers]
        self.lm_q, self.lm_d = next(it), next(it)
        self.structs = [lw.struct() for lw in self.layers]
        self.arena = arena
        self._dstruct = None

    def reserve(self, tokens: int) -> None:
        """Size the workspace for calls of up to `tokens` tokens (before graph capture)."""
        self.ws.reserve(qk_layer_workspace(self.cfg, tokens), self.device)
        self.head_ws.reserve(qk_lm_head_workspace(self.s.vocab, self.s.hidden, tokens), self.device)

    def hidden_states(self, ids: torch.Tensor, pos: torch.Tensor, seq: torch.Tensor,
                      x: torch.Tensor | None = None) -> torch.Tensor:
        """Embedding and every layer for the tokens ids [T] at (pos, seq)."""
        x = qk_embed_lookup(self.embed, ids, out=x)
        for li, st in enumerate(self.structs):
            layer_forward(st, self.cfg, x, pos, seq, self.k_cache[li], self.v_cache[li], ws=self.ws)
        return x

    def step(self, ids: torch.Tensor, pos: torch.Tensor, seq: torch.Tensor,
             bufs: dict | None = None) -> tuple[torch.Tensor, torch.Tensor]:
        """One forward over ids [T]: returns (logits [T][V], argmax ids [T])."""
        b = bufs if bufs is not None else {}
        x = self.hidden_states(ids, pos, seq, x=b.get("x"))
        return qk_lm_head(x, self.gamma_final, self.s.eps, self.lm_q, self.lm_d,
                          logits=b.get("logits"), next_ids=b.get("next"), ws=self.head_ws)

    def capture_decode(self, ids: torch.Tensor, positions: list[torch.Tensor], seq: torch.Tensor,
                       logits: torch.Tensor, next_ids: torch.Tensor) -> torch.cuda.CUDAGraph:
        """Capture len(positions) one-token decode steps back to back in one
        HIP graph.  Step j reads its token from ids[j], runs at positions[j],
        writes its logits to logits[j % logits.shape[0]] and its greedy token
        to next_ids[j].  Greedy decoding passes next_ids = ids[1:] (each
        step's argmax is the next step's input); teacher forcing passes ids
        filled beforehand and a separate next_ids."""
        n = len(positions)
        assert ids.numel() >= n and next_ids.numel() >= n
        self.reserve(1)
        x = torch.empty((1, self.s.hidden), dtype=torch.float32, device=self.device)
        rows = logits.shape[0]
        # first launches outside the capture
        self.step(ids[0:1], positions[0], seq, dict(x=x, logits=logits[0:1], next=next_ids[0:1]))
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for j in range(n):
                r = j % rows
                self.step(ids[j:j + 1], positions[j], seq,
                          dict(x=x, logits=logits[r:r + 1], next=next_ids[j:j + 1]))
        return gr

    def decoder_struct(self) -> DecoderStruct:
        """The qk_decoder of this model for qk_decode_greedy (one sequence):
        the layer table is copied to the device once."""
        assert self.s.seqs == 1, "the persistent decode runs one sequence"
        table = (Layer * len(self.structs))(*self.structs)
        raw = bytes(table)
        self.layer_table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)
        self.decode_ws = Workspace()
        self.decode_ws.reserve(qk_decode_workspace(self.cfg), self.device)
        return DecoderStruct(self.layer_table.data_ptr(), len(self.structs), self.embed.data_ptr(),
                             self.gamma_final.data_ptr(), self.lm_q.data_ptr(), self.lm_d.data_ptr(),
                             self.s.vocab, self.k_cache.data_ptr(), self.v_cache.data_ptr())

    def decode_persistent(self, n: int, pos0: int, out_ids: torch.Tensor, first_id=None, forced=None,
                          logits=None, spin_limit: int = 0) -> torch.Tensor:
        """n greedy steps from position pos0 in one persistent kernel launch."""
        if getattr(self, "_dstruct", None) is None:
            self._dstruct = self.decoder_struct()
        return qk_decode_greedy(self._dstruct, self.cfg, n, pos0, out_ids, first_id=first_id,
                                forced=forced, logits=logits, spin_limit=spin_limit,
                                ws=self.decode_ws)

    def step_buffers(self, tokens: int) -> dict:
        """Preallocated buffers so that `step` allocates nothing (graph capture)."""
        dev, H, V = self.device, self.s.hidden, self.s.vocab
        return dict(x=torch.empty((tokens, H), dtype=torch.float32, device=dev),
                    logits=torch.empty((tokens, V), dtype=torch.float32, device=dev),
                    next=torch.empty((tokens,), dtype=torch.int32, device=dev))
