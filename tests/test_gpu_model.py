"""Full-size parity: the TinyLLaMA-1.1B-shaped decode and prefill workloads and
the 256-expert MoE layer, against the CPU oracle on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_q4_q8_amd.model import Decoder, DecoderShape, layer_to_device, to_device
from synth import workloads as W
from tests.util import LAYER_TOL, LOGIT_TOL, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def check_tokens(got, logits_o):
    """Greedy tokens agree, except where the oracle's top-2 gap is within the
    logit tolerance (either token is then a correct greedy choice)."""
    want = np.argmax(logits_o, axis=-1)
    for t in range(len(got)):
        if got[t] == want[t]:
            continue
        top2 = np.sort(logits_o[t])[-2:]
        assert top2[1] - top2[0] <= LOGIT_TOL, f"row {t}: token {got[t]} vs {want[t]}"
        assert logits_o[t, got[t]] >= top2[1] - LOGIT_TOL


@pytest.mark.parametrize("vocab,hidden,tokens", [(1000, 256, 1), (32000, 2048, 3), (517, 128, 12)])
def test_lm_head(gpu_lib, vocab, hidden, tokens):
    qk = gpu_lib
    say(f"qk_lm_head vocab={vocab} hidden={hidden} tokens={tokens}")
    x = synth.normal(70, 1, (tokens, hidden))
    g = synth.normal(70, 2, hidden, 0.02, mean=1.0)
    w = synth.normal(70, 3, (vocab, hidden), 0.02)
    wq, wd = oracle.quantize_q4_0(w)
    xq, xd = oracle.quantize_q8_0(oracle.rmsnorm(x, g, 1e-5))
    ref = oracle.qmatmul(wq, wd, xq, xd)
    lg, nx = qk.qk_lm_head(dev(x), dev(g), 1e-5, dev(wq), dev(wd))
    assert np.max(np.abs(host(lg) - ref)) <= LOGIT_TOL
    check_tokens(host(nx), ref)


# ---------------------------------------------------------------------------
# shared TinyLLaMA-shaped model (decode and prefill use different seeds)
# ---------------------------------------------------------------------------
def build(spec, seqs):
    g, seed, L, V, cap = spec["geometry"], spec["seed"], spec["layers"], spec["vocab"], spec["cap"]
    layers, host_layers = [], []
    for li in range(L):
        wf = W.layer_weights_f32(seed, li, g)
        lw = layer_to_device(wf)
        wl = {}
        for name, key in [("w_qkv", "w_qkv"), ("w_o", "w_o"), ("w_gate_up", "w_gu"), ("w_down", "w_down")]:
            wl[key + "_q"], wl[key + "_d"] = oracle.quantize_q4_0(wf[name])
        wl["gamma_attn"], wl["gamma_ffn"] = wf["gamma_attn"], wf["gamma_ffn"]
        if li in (0, L - 1):   # the device quantizer produced the oracle's bytes
            assert np.array_equal(host(lw.w_gate_up_q), wl["w_gu_q"])
            assert np.array_equal(host(lw.w_qkv_d, np.uint16), wl["w_qkv_d"])
        layers.append(lw)
        host_layers.append(wl)
    embed = synth.normal(seed, W.TID_EMBED, (V, g.hidden))
    gamma_f = synth.normal(seed, W.TID_GAMMA_FINAL, g.hidden, W.GAMMA_STD, mean=1.0)
    lm = synth.normal(seed, W.TID_LM_HEAD, (V, g.hidden), W.WEIGHT_STD)
    lm_q, lm_d = oracle.quantize_q4_0(lm)
    shape = DecoderShape(g.hidden, g.n_q_heads, g.n_kv_heads, g.head_dim, g.ffn_padded, g.eps,
                         g.rope_base, L, V, cap, seqs)
    dec = Decoder(shape, layers, dev(embed), dev(gamma_f), dev(lm_q), dev(lm_d))
    hostm = dict(layers=host_layers, embed=embed, gamma_f=gamma_f, lm_q=lm_q, lm_d=lm_d, cfg=g.cfg(cap))
    return dec, hostm


def oracle_forward(hm, ids, pos, seq, kv):
    x = oracle.embed_lookup(hm["embed"], ids)
    for li, wl in enumerate(hm["layers"]):
        x = oracle.layer_forward(wl, hm["cfg"], x, pos, seq, kv[li][0], kv[li][1])
    xq, xd = oracle.quantize_q8_0(oracle.rmsnorm(x, hm["gamma_f"], 1e-5))
    return oracle.qmatmul(hm["lm_q"], hm["lm_d"], xq, xd)


def test_decode_tinyllama_shape_teacher_forced(gpu_lib):
    """22-layer decode from a 2048-row fp16 KV prefill: logits within 1e-2 and
    greedy tokens matching the oracle on every step (teacher-forced).  The
    weights are packed into one arena first, as the benchmark holds them."""
    spec = W.DECODE
    g, L, cap, ctx = spec["geometry"], spec["layers"], spec["cap"], spec["context"]
    say("decode: building the 22-layer model")
    dec, hm = build(spec, 1)
    dec.pack()
    assert all(lw.w_gate_up_q.untyped_storage().data_ptr() == dec.arena.untyped_storage().data_ptr()
               for lw in dec.layers)
    kv = []
    for li in range(L):
        kc, vc = W.kv_prefill_f16(spec["seed"], li, g.n_kv_heads, cap, g.head_dim, ctx)
        dec.k_cache[li].copy_(torch.from_numpy(kc.view(np.int16)))
        dec.v_cache[li].copy_(torch.from_numpy(vc.view(np.int16)))
        kv.append((kc.view(np.uint16).copy(), vc.view(np.uint16).copy()))
    tok = synth.randint(spec["seed"], W.TID_TOKENS, 1, spec["vocab"])
    seq = np.zeros(1, np.int32)
    steps = [0, 1, 2, 3, 127]          # the last decode position of the workload too
    for j in steps:
        say(f"decode step at position {ctx + j}")
        p = np.array([ctx + j], np.int32)
        lo = oracle_forward(hm, tok, p, seq, kv)
        lg, nx = dec.step(dev(tok), dev(p), dev(seq))
        torch.cuda.synchronize()
        assert np.max(np.abs(host(lg) - lo)) <= LOGIT_TOL, f"position {ctx + j}"
        check_tokens(host(nx), lo)
        tok = np.argmax(lo, axis=-1).astype(np.int32)   # teacher forcing: the oracle's token
    # the caches the GPU wrote agree with the oracle's (fp16 rows at the decoded positions)
    for li in (0, L - 1):
        rows = [ctx + j for j in steps]
        got = oracle.f16_to_f32(host(dec.k_cache[li], np.uint16)[0][:, rows])
        want = oracle.f16_to_f32(kv[li][0][0][:, rows])
        assert rel_err(got, want) < LAYER_TOL


def test_decode_long_context_ring_teacher_forced(gpu_lib):
    """22-layer decode past an 8192-row ring cache filled to the brim: every
    step attends to 8192 positions (rows 0..8191 hold positions p - 8191..p),
    logits within 1e-2 and greedy tokens matching the oracle."""
    spec = W.DECODE_LONG
    g, L, cap, ctx = spec["geometry"], spec["layers"], spec["cap"], spec["context"]
    say("long-context decode: building the 22-layer model")
    dec, hm = build(spec, 1)
    kv = []
    for li in range(L):
        kc, vc = W.kv_prefill_f16(spec["seed"], li, g.n_kv_heads, cap, g.head_dim, ctx)
        dec.k_cache[li].copy_(torch.from_numpy(kc.view(np.int16)))
        dec.v_cache[li].copy_(torch.from_numpy(vc.view(np.int16)))
        kv.append((kc.view(np.uint16).copy(), vc.view(np.uint16).copy()))
    tok = synth.randint(spec["seed"], W.TID_TOKENS, 1, spec["vocab"])
    seq = np.zeros(1, np.int32)
    for j in (0, 1, 2):
        say(f"long-context decode step at position {ctx + j}")
        p = np.array([ctx + j], np.int32)
        lo = oracle_forward(hm, tok, p, seq, kv)
        lg, nx = dec.step(dev(tok), dev(p), dev(seq))
        torch.cuda.synchronize()
        assert np.max(np.abs(host(lg) - lo)) <= LOGIT_TOL, f"position {ctx + j}"
        check_tokens(host(nx), lo)
        tok = np.argmax(lo, axis=-1).astype(np.int32)
    # positions 8192..8194 overwrote ring rows 0..2
    for li in (0, L - 1):
        got = oracle.f16_to_f32(host(dec.k_cache[li], np.uint16)[0][:, :3])
        want = oracle.f16_to_f32(kv[li][0][0][:, :3])
        assert rel_err(got, want) < LAYER_TOL


def test_prefill_tinyllama_shape_prefix(gpu_lib):
    """The 4 x 512 causal prefill with full logits; by causality the first 16
    tokens of each sequence must match the oracle's 16-token prefill."""
    spec = W.PREFILL
    B, P, V = spec["batch"], spec["prompt"], spec["vocab"]
    say("prefill: building the 22-layer model")
    dec, hm = build(spec, B)
    ids = synth.randint(spec["seed"], W.TID_TOKENS, (B, P), V)
    pos = np.tile(np.arange(P, dtype=np.int32), B)
    seq = np.repeat(np.arange(B, dtype=np.int32), P)
    say("prefill: 2048 tokens on the GPU")
    lg, nx = dec.step(dev(ids.reshape(-1)), dev(pos), dev(seq))
    torch.cuda.synchronize()
    lg_h = host(lg).reshape(B, P, V)
    assert np.all(np.isfinite(lg_h))
    n = 16
    g = spec["geometry"]
    for b in range(B):
        say(f"prefill: oracle prefix of sequence {b}")
        kv = [(np.zeros((1, g.n_kv_heads, spec["cap"], g.head_dim), np.uint16),
               np.zeros((1, g.n_kv_heads, spec["cap"], g.head_dim), np.uint16)) for _ in range(spec["layers"])]
        lo = oracle_forward(hm, ids[b, :n], np.arange(n, dtype=np.int32), np.zeros(n, np.int32), kv)
        assert np.max(np.abs(lg_h[b, :n] - lo)) <= LOGIT_TOL, f"sequence {b}"
        check_tokens(host(nx).reshape(B, P)[b, :n], lo)


def test_moe_full_size_sampled(gpu_lib):
    """256 experts of three 6144 x 2048 Q4_0 matrices resident on the GPU, 64
    tokens, top-8: routing for every token, outputs for sampled tokens."""
    qk = gpu_lib
    spec = W.MOE
    seed, T, H, E, F, k = spec["seed"], spec["tokens"], spec["hidden"], spec["experts"], spec["ffn"], spec["top_k"]
    say("moe: generating and quantizing 256 experts on the GPU")
    guq = torch.empty((E, 2 * F, H // 2), dtype=torch.uint8, device="cuda")
    gud = torch.empty((E, 2 * F, H // 32), dtype=torch.int16, device="cuda")
    dnq = torch.empty((E, H, F // 2), dtype=torch.uint8, device="cuda")
    dnd = torch.empty((E, H, F // 32), dtype=torch.int16, device="cuda")
    for e in range(E):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        qk.qk_quantize_q4_0(to_device(gu), out_q=guq[e], out_d=gud[e])
        qk.qk_quantize_q4_0(to_device(dn), out_q=dnq[e], out_d=dnd[e])
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), W.WEIGHT_STD)
    say("moe: GPU layer")
    y, sg, wg = qk.moe_route_and_apply(dev(x), dev(wr), k, guq, gud, dnq, dnd)
    torch.cuda.synchronize()
    sel_o, w_o, logits = oracle.moe_route(x, wr, k, return_logits=True)
    sel_g, w_g = host(sg), host(wg)
    from tests.test_gpu_layer import check_routing
    check_routing(sel_g, w_g, sel_o, w_o, logits)
    y_h = host(y)
    checked = 0
    for t in (0, 17, 42, 63):
        if not np.array_equal(sel_g[t], sel_o[t]):
            continue   # a near tie (checked above): either selection is correct
        say(f"moe: oracle token {t}")
        acc = np.zeros(H, np.float64)
        for r in range(k):
            e = int(sel_o[t, r])
            gu, dn = W.expert_weights_f32(seed, e, H, F)
            a, b = oracle.quantize_q4_0(gu)
            c, d = oracle.quantize_q4_0(dn)
            if r == 0:
                assert np.array_equal(host(guq[e]), a) and np.array_equal(host(dnd[e], np.uint16), d)
            acc += np.float64(w_o[t, r]) * oracle.moe_expert_ffn(x[t], a, b, c, d)
        assert rel_err(y_h[t], acc.astype(np.float32)) < LAYER_TOL, f"token {t}"
        checked += 1
    assert checked >= 3


@pytest.mark.parametrize("bits", [4, 2])
def test_moe_rowq_full_size_sampled(gpu_lib, bits):
    """The MoE workload with row-scaled int4 / int2 experts (256 resident,
    64 tokens, top-8): routing for every token, outputs for sampled tokens."""
    qk = gpu_lib
    spec = W.MOE
    seed, T, H, E, F, k = spec["seed"], spec["tokens"], spec["hidden"], spec["experts"], spec["ffn"], spec["top_k"]
    say(f"moe rowq{bits}: generating and quantizing 256 experts on the GPU")
    guq = torch.empty((E, 2 * F, H * bits // 8), dtype=torch.uint8, device="cuda")
    gur = torch.empty((E, 2 * F), dtype=torch.float32, device="cuda")
    dnq = torch.empty((E, H, F * bits // 8), dtype=torch.uint8, device="cuda")
    dnr = torch.empty((E, H), dtype=torch.float32, device="cuda")
    for e in range(E):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        qk.qk_quantize_rowq(to_device(gu), bits, out_q=guq[e], out_r=gur[e])
        qk.qk_quantize_rowq(to_device(dn), bits, out_q=dnq[e], out_r=dnr[e])
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), W.WEIGHT_STD)
    say(f"moe rowq{bits}: GPU layer")
    y, sg, wg = qk.qk_moe_route_and_apply_rowq(dev(x), dev(wr), k, guq, gur, dnq, dnr, bits)
    torch.cuda.synchronize()
    sel_o, w_o, logits = oracle.moe_route(x, wr, k, return_logits=True)
    sel_g, w_g = host(sg), host(wg)
    from tests.test_gpu_layer import check_routing
    check_routing(sel_g, w_g, sel_o, w_o, logits)
    y_h = host(y)
    checked = 0
    for t in (0, 17, 42, 63):
        if not np.array_equal(sel_g[t], sel_o[t]):
            continue   # a near tie (checked above): either selection is correct
        say(f"moe rowq{bits}: oracle token {t}")
        acc = np.zeros(H, np.float64)
        for r in range(k):
            e = int(sel_o[t, r])
            gu, dn = W.expert_weights_f32(seed, e, H, F)
            a, b = oracle.quantize_rowq(gu, bits)
            c, d = oracle.quantize_rowq(dn, bits)
            if r == 0:
                assert np.array_equal(host(guq[e]), a) and np.array_equal(host(dnr[e]), d)
            xq, xd = oracle.quantize_q8_0(x[t:t + 1])
            gup = oracle.qmatmul_rowq(a, b, xq, xd, bits)[0]
            hq, hd = oracle.quantize_q8_0(oracle.swiglu(gup[:F], gup[F:])[None])
            acc += np.float64(w_o[t, r]) * oracle.qmatmul_rowq(c, d, hq, hd, bits)[0]
        assert rel_err(y_h[t], acc.astype(np.float32)) < LAYER_TOL, f"token {t}"
        checked += 1
    assert checked >= 3
