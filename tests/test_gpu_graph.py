"""Graph capture of the decode step, as the benchmark uses it: several greedy
tokens captured back to back in one HIP graph (each token's argmax writes the
next token's input id in place), replayed several times with eager work and
synchronizations in between; every replay must reproduce the eager run's
logits and tokens bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_q4_q8_amd.model import Decoder, DecoderShape, layer_to_device
from synth import workloads as W
from tests.util import dev, host, say

pytestmark = pytest.mark.gpu


def small_decoder(seed=9, layers=2, vocab=1000, cap=64, pack=False):
    g = W.LAYER_SMALL["geometry"]
    lws = [layer_to_device(W.layer_weights_f32(seed, li, g)) for li in range(layers)]
    embed = synth.normal(seed, W.TID_EMBED, (vocab, g.hidden))
    gamma_f = synth.normal(seed, W.TID_GAMMA_FINAL, g.hidden, W.GAMMA_STD, mean=1.0)
    lm_q, lm_d = oracle.quantize_q4_0(synth.normal(seed, W.TID_LM_HEAD, (vocab, g.hidden), W.WEIGHT_STD))
    shape = DecoderShape(g.hidden, g.n_q_heads, g.n_kv_heads, g.head_dim, g.ffn_padded, g.eps,
                         g.rope_base, layers, vocab, cap, 1)
    dec = Decoder(shape, lws, dev(embed), dev(gamma_f), dev(lm_q), dev(lm_d))
    if pack:
        dec.pack()
    return dec


@pytest.mark.parametrize("pack", [False, True])
def test_decode_graph_replays_match_eager(gpu_lib, pack):
    steps, first = 6, 17
    say(f"decode graph: {steps} tokens in one graph, pack={pack}")
    dec = small_decoder(pack=pack)
    dec.reserve(1)
    bufs = dec.step_buffers(1)
    ids = torch.tensor([first], dtype=torch.int32, device="cuda")
    bufs["next"] = ids                       # argmax writes the next input id in place
    seq = torch.zeros(1, dtype=torch.int32, device="cuda")
    positions = [torch.tensor([j], dtype=torch.int32, device="cuda") for j in range(steps)]

    def reset():
        dec.k_cache.zero_()
        dec.v_cache.zero_()
        ids.fill_(first)

    # eager reference: logits and tokens of every step
    reset()
    want_logits, want_ids = [], []
    for j in range(steps):
        dec.step(ids, positions[j], seq, bufs)
        torch.cuda.synchronize()
        want_logits.append(host(bufs["logits"]).copy())
        want_ids.append(int(host(ids)[0]))
    want_cache = host(dec.k_cache).copy()

    reset()
    dec.step(ids, positions[0], seq, bufs)   # eager warm-up before capture
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for j in range(steps):
            dec.step(ids, positions[j], seq, bufs)
    for rep in range(3):
        reset()                              # eager work between the replays
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert int(host(ids)[0]) == want_ids[-1], f"replay {rep}: final token"
        assert np.array_equal(host(bufs["logits"]), want_logits[-1]), f"replay {rep}: final logits"
        assert np.array_equal(host(dec.k_cache), want_cache), f"replay {rep}: K cache"
