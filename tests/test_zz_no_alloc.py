"""The layer entry point that allocates nothing (qk_layer_forward_scratch,
its workspace a device array inside the library) against layer_forward with
a caller workspace: identical outputs and caches, bit for bit, on two calls
in a row, the second with fewer tokens."""
import numpy as np
import pytest
import torch

import quantized_q4_q8_amd as qk_mod
import synth
from quantized_q4_q8_amd.model import layer_to_device
from synth import workloads as W
from tests.util import dev, host, say

pytestmark = pytest.mark.gpu


def test_scratch_layer_matches_workspace_layer(gpu_lib):
    qk = gpu_lib
    g = W.TINYLLAMA
    cap, ctx = 2176, 2048
    say("qk_layer_forward_scratch: TinyLLaMA-shape layer, 8 then 3 tokens")
    lw = layer_to_device(W.layer_weights_f32(44, 0, g))
    cfg = qk.layer_cfg(**g.cfg(cap))
    kc, vc = W.kv_prefill_f16(44, 0, g.n_kv_heads, cap, g.head_dim, ctx)
    ka, va = dev(kc.view(np.uint16)), dev(vc.view(np.uint16))     # scratch path
    kb, vb = ka.clone(), va.clone()                                 # workspace path
    p0 = ctx
    for tokens in (8, 3):
        x = synth.normal(44, 10 + tokens, (tokens, g.hidden))
        pos = dev(np.arange(p0, p0 + tokens, dtype=np.int32))
        seq = dev(np.zeros(tokens, np.int32))
        xa, xb = dev(x), dev(x)
        qk.qk_layer_forward_scratch(lw, cfg, xa, pos, seq, ka, va)
        qk.layer_forward(lw, cfg, xb, pos, seq, kb, vb)
        torch.cuda.synchronize()
        ga, gb = host(xa), host(xb)
        assert not np.array_equal(ga, x), "the layer ran"
        assert np.array_equal(ga.view(np.uint32), gb.view(np.uint32)), f"{tokens} tokens: outputs differ"
        assert torch.equal(ka, kb) and torch.equal(va, vb), f"{tokens} tokens: caches differ"
        p0 += tokens


def test_scratch_layer_rejects_oversized_calls(gpu_lib):
    """A call whose workspace exceeds the array fails before enqueuing
    anything: the input is left unchanged."""
    qk = gpu_lib
    g = W.TINYLLAMA
    cap = 8192
    need = qk.qk_layer_workspace(qk.layer_cfg(**g.cfg(cap)), 8)
    assert need > qk_mod.QK_SCRATCH_BYTES
    lw = layer_to_device(W.layer_weights_f32(45, 0, W.LAYER_SMALL["geometry"]))
    # the small layer's weights are never read: the size check fails first
    x = dev(synth.normal(45, 1, (8, g.hidden)))
    x0 = x.clone()
    kc = torch.zeros((1, g.n_kv_heads, cap, g.head_dim), dtype=torch.int16, device="cuda")
    pos = dev(np.arange(8, dtype=np.int32))
    seq = dev(np.zeros(8, np.int32))
    with pytest.raises(qk_mod.QKError) as e:
        qk.qk_layer_forward_scratch(lw, qk.layer_cfg(**g.cfg(cap)), x, pos, seq, kc, kc.clone())
    assert e.value.status == qk_mod.QK_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(x, x0)
