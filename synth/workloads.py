"""The five synthetic workloads: geometry, seeds, and a stream id for every
tensor.  Draws only; no quantization or other arithmetic of the method.

Weights are N(0, 0.02) fp32 draws in [out_rows][in_cols] order (y = W x);
RMSNorm gains are 1 + N(0, 0.02); embeddings and hidden-state inputs are
N(0, 1); token ids are uniform in [0, vocab).  A gate/up/down width that is
not a multiple of 32 is zero-padded to the next multiple: extra gate/up rows
and extra down columns are exactly zero.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import normal, randint

WEIGHT_STD = 0.02
GAMMA_STD = 0.02

# stream ids (per seed)
TID_EMBED = 0
TID_GAMMA_FINAL = 1
TID_LM_HEAD = 2
TID_TOKENS = 3
TID_X = 4
TID_ROUTER = 5
TID_KV = 6           # +layer*2 (+0 K, +1 V) via kv_tensor_id
TID_LAYER0 = 1000    # + 16 * layer + slot
TID_EXPERT0 = 1_000_000  # + 4 * expert + slot
TID_MATMUL0 = 50     # standalone matmul workload

LAYER_SLOTS = {"gamma_attn": 0, "w_q": 1, "w_k": 2, "w_v": 3, "w_o": 4, "gamma_ffn": 5,
               "w_gate": 6, "w_up": 7, "w_down": 8}
EXPERT_SLOTS = {"w_gate": 0, "w_up": 1, "w_down": 2}


def pad32(n: int) -> int:
    return (n + 31) // 32 * 32


@dataclass(frozen=True)
class Geometry:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int                 # as specified
    eps: float = 1e-5
    rope_base: float = 10000.0

    @property
    def ffn_padded(self) -> int:
        return pad32(self.ffn)

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def cfg(self, cap: int) -> dict:
        return dict(hidden=self.hidden, n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, ffn=self.ffn_padded, eps=self.eps,
                    rope_base=self.rope_base, cap=cap)


def layer_tensor_id(layer: int, name: str) -> int:
    return TID_LAYER0 + 16 * layer + LAYER_SLOTS[name]


def expert_tensor_id(expert: int, name: str) -> int:
    return TID_EXPERT0 + 4 * expert + EXPERT_SLOTS[name]


def kv_tensor_id(layer: int, which: int) -> int:
    return TID_KV + 2 * layer + which + 100


def layer_weights_f32(seed: int, layer: int, g: Geometry) -> dict:
    """fp32 weights of one decoder layer, fused as the interface stores them:
    w_qkv [(nq+2nkv)*hd][H] (Q rows, K rows, V rows), w_o [H][nq*hd],
    w_gate_up [2F'][H] (gate rows then up rows), w_down [H][F'], gammas [H];
    F' = F padded to 32 with zero rows/columns."""
    H, hd, F, Fp = g.hidden, g.head_dim, g.ffn, g.ffn_padded
    nq, nkv = g.n_q_heads, g.n_kv_heads
    t = lambda name: layer_tensor_id(layer, name)  # noqa: E731
    w_qkv = np.concatenate([normal(seed, t("w_q"), (nq * hd, H), WEIGHT_STD),
                            normal(seed, t("w_k"), (nkv * hd, H), WEIGHT_STD),
                            normal(seed, t("w_v"), (nkv * hd, H), WEIGHT_STD)], axis=0)
    w_o = normal(seed, t("w_o"), (H, nq * hd), WEIGHT_STD)
    w_gu = np.zeros((2 * Fp, H), np.float32)
    w_gu[:F] = normal(seed, t("w_gate"), (F, H), WEIGHT_STD)
    w_gu[Fp:Fp + F] = normal(seed, t("w_up"), (F, H), WEIGHT_STD)
    w_down = np.zeros((H, Fp), np.float32)
    w_down[:, :F] = normal(seed, t("w_down"), (H, F), WEIGHT_STD)
    return dict(w_qkv=w_qkv, w_o=w_o, w_gate_up=w_gu, w_down=w_down,
                gamma_attn=normal(seed, t("gamma_attn"), H, GAMMA_STD, mean=1.0),
                gamma_ffn=normal(seed, t("gamma_ffn"), H, GAMMA_STD, mean=1.0))


def expert_weights_f32(seed: int, expert: int, hidden: int, ffn: int) -> tuple[np.ndarray, np.ndarray]:
    """(gate_up [2F][H], down [H][F]) fp32 for one MoE expert."""
    gu = np.empty((2 * ffn, hidden), np.float32)
    normal(seed, expert_tensor_id(expert, "w_gate"), (ffn, hidden), WEIGHT_STD, out=gu[:ffn])
    normal(seed, expert_tensor_id(expert, "w_up"), (ffn, hidden), WEIGHT_STD, out=gu[ffn:])
    down = normal(seed, expert_tensor_id(expert, "w_down"), (hidden, ffn), WEIGHT_STD)
    return gu, down


def kv_prefill_f16(seed: int, layer: int, n_kv: int, cap: int, hd: int, filled: int,
                   seqs: int = 1) -> tuple[np.ndarray, np.ndarray]:
    """fp16 caches [seqs][n_kv][cap][hd] whose rows 0..filled-1 hold N(0,1)
    draws (already-rotated keys and values), the rest zero."""
    out = []
    for which in (0, 1):
        c = np.zeros((seqs, n_kv, cap, hd), np.float16)
        vals = normal(seed, kv_tensor_id(layer, which), (seqs, n_kv, filled, hd))
        c[:, :, :filled, :] = vals.astype(np.float16)
        out.append(c)
    return out[0], out[1]


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
# C1: one small decoder layer, 16-token prefill then 16 self-fed decode steps.
LAYER_SMALL = dict(seed=0, geometry=Geometry(256, 8, 2, 32, 688), prompt=16, decode=16, cap=32)
# C2: standalone Q4_0 x Q8_0 matmuls: W[5632x2048] x x[2048]; W[2048x5632] x x[5632]; batch 1 and 8.
MATMUL = dict(seed=1, shapes=[(5632, 2048), (2048, 5632)], batches=[1, 8])
# C3: TinyLLaMA-1.1B-shaped decode: 22 layers, vocab 32000, KV prefilled to 2048, 128 greedy steps.
TINYLLAMA = Geometry(2048, 32, 4, 64, 5632)
DECODE = dict(seed=2, geometry=TINYLLAMA, layers=22, vocab=32000, context=2048, steps=128,
              cap=2176)
# Long context: the same decode with an 8192-row ring cache filled to the
# brim; positions 8192..8319 wrap, so every step attends to 8192 positions.
DECODE_LONG = dict(seed=5, geometry=TINYLLAMA, layers=22, vocab=32000, context=8192, steps=128,
                   cap=8192)
# The same at a 32768-row ring (512 attention chunks per KV head).
DECODE_LONG32K = dict(seed=6, geometry=TINYLLAMA, layers=22, vocab=32000, context=32768, steps=128,
                      cap=32768)
# C4: TinyLLaMA-1.1B-shaped prefill: batch 4 x 512 uniform token ids, causal, full logits.
PREFILL = dict(seed=3, geometry=TINYLLAMA, layers=22, vocab=32000, batch=4, prompt=512, cap=512)
# C5: MoE layer, hidden 6144, 256 experts of width 2048, sigmoid top-8, 64 tokens.
MOE = dict(seed=4, hidden=6144, experts=256, ffn=2048, top_k=8, tokens=64)


def matmul_weight_f32(seed: int, idx: int, n: int, k: int) -> np.ndarray:
    return normal(seed, TID_MATMUL0 + 2 * idx, (n, k), WEIGHT_STD)


def matmul_input_f32(seed: int, idx: int, m: int, k: int) -> np.ndarray:
    return normal(seed, TID_MATMUL0 + 2 * idx + 1, (m, k))
