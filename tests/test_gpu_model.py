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


@pytest.mark.parametrize("vocab,hidden,tokens", [(1000, 256, 1), (32000, 2048, 3), (517, 128, 12),
                                                  # K = 6144 in three register chunks, 3 columns
                                                  (4000, 6144, 3)])
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


@pytest.mark.timeout(900)
def test_decode_tinyllama_shape_every_step_graph(gpu_lib):
    """The benchmark's decode path on the full workload: the 128 one-token
    steps (positions 2048..2175) captured back to back in one HIP graph over
    the weights packed into one arena, teacher-forced with the oracle's
    tokens from a device buffer.  Every step's logits are within 1e-2 of the
    oracle's and every greedy token agrees; the K/V rows written at all 128
    positions match the oracle's caches."""
    spec = W.DECODE
    g, L, cap, ctx, n, V = (spec["geometry"], spec["layers"], spec["cap"], spec["context"],
                            spec["steps"], spec["vocab"])
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
    tok = synth.randint(spec["seed"], W.TID_TOKENS, 1, V)
    seq = np.zeros(1, np.int32)
    want = np.empty((n, V), np.float32)
    ids = np.empty(n, np.int32)
    for j in range(n):
        if j % 16 == 0:
            say(f"decode: oracle step {j} (position {ctx + j})")
        ids[j] = tok[0]
        lo = oracle_forward(hm, tok, np.array([ctx + j], np.int32), seq, kv)
        want[j] = lo[0]
        tok = np.argmax(lo, axis=-1).astype(np.int32)   # teacher forcing: the oracle's token
    say("decode: 128 steps in one captured graph on the GPU")
    positions = [dev(np.array([ctx + j], np.int32)) for j in range(n)]
    logits = torch.empty((n, V), dtype=torch.float32, device="cuda")
    nxt = torch.empty(n, dtype=torch.int32, device="cuda")
    gr = dec.capture_decode(dev(ids), positions, dev(seq), logits, nxt)
    gr.replay()
    torch.cuda.synchronize()
    got = host(logits)
    err = np.max(np.abs(got - want), axis=1)
    assert np.all(err <= LOGIT_TOL), f"steps over tolerance: {np.nonzero(err > LOGIT_TOL)[0]}, worst {err.max()}"
    check_tokens(host(nxt), want)
    say(f"decode: worst step logit error {err.max():.2e}")
    # the caches the GPU wrote agree with the oracle's at every decoded position
    rows = list(range(ctx, ctx + n))
    for li in (0, L // 2, L - 1):
        for c in (0, 1):
            gotc = oracle.f16_to_f32(host((dec.k_cache, dec.v_cache)[c][li], np.uint16)[0][:, rows])
            wantc = oracle.f16_to_f32(kv[li][c][0][:, rows])
            assert rel_err(gotc, wantc) < LAYER_TOL, f"layer {li} {'kv'[c]} cache"


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


@pytest.mark.timeout(900)
def test_prefill_tinyllama_shape(gpu_lib):
    """The 4 x 512 causal prefill with full logits.  Every one of the 512
    positions of the last sequence (token tiles 24..31 of the MFMA GEMMs and
    every attention chunk) matches the oracle's 512-token prefill: logits
    within 1e-2, greedy tokens agreeing.  By causality the first 16 tokens
    of the other sequences must match the oracle's 16-token prefills."""
    spec = W.PREFILL
    B, P, V = spec["batch"], spec["prompt"], spec["vocab"]
    g = spec["geometry"]
    say("prefill: building the 22-layer model")
    dec, hm = build(spec, B)
    ids = synth.randint(spec["seed"], W.TID_TOKENS, (B, P), V)
    pos = np.tile(np.arange(P, dtype=np.int32), B)
    seq = np.repeat(np.arange(B, dtype=np.int32), P)
    say("prefill: 2048 tokens on the GPU")
    lg, nx = dec.step(dev(ids.reshape(-1)), dev(pos), dev(seq))
    torch.cuda.synchronize()
    lg_h = host(lg).reshape(B, P, V)
    nx_h = host(nx).reshape(B, P)
    assert np.all(np.isfinite(lg_h))

    def fresh_kv():
        return [(np.zeros((1, g.n_kv_heads, spec["cap"], g.head_dim), np.uint16),
                 np.zeros((1, g.n_kv_heads, spec["cap"], g.head_dim), np.uint16))
                for _ in range(spec["layers"])]

    # the whole last sequence
    b = B - 1
    kv = fresh_kv()
    p_all = np.arange(P, dtype=np.int32)
    x = oracle.embed_lookup(hm["embed"], ids[b])
    for li, wl in enumerate(hm["layers"]):
        if li % 4 == 0:
            say(f"prefill: oracle sequence {b}, layer {li}")
        x = oracle.layer_forward(wl, hm["cfg"], x, p_all, np.zeros(P, np.int32), kv[li][0], kv[li][1])
    xq, xd = oracle.quantize_q8_0(oracle.rmsnorm(x, hm["gamma_f"], 1e-5))
    lo = oracle.qmatmul(hm["lm_q"], hm["lm_d"], xq, xd)
    err = np.max(np.abs(lg_h[b] - lo), axis=1)
    assert np.all(err <= LOGIT_TOL), f"positions over tolerance: {np.nonzero(err > LOGIT_TOL)[0]}"
    check_tokens(nx_h[b], lo)
    say(f"prefill: sequence {b} all {P} positions, worst logit error {err.max():.2e}")
    n = 16
    for b in range(B - 1):
        say(f"prefill: oracle prefix of sequence {b}")
        lo = oracle_forward(hm, ids[b, :n], np.arange(n, dtype=np.int32), np.zeros(n, np.int32), fresh_kv())
        assert np.max(np.abs(lg_h[b, :n] - lo)) <= LOGIT_TOL, f"sequence {b}"
        check_tokens(nx_h[b, :n], lo)


@pytest.mark.timeout(1200)
def test_moe_full_size_every_token(gpu_lib):
    """The MoE workload: 256 resident experts of three 6144 x 2048 matrices,
    64 tokens, top-8, with Q4_0, row-scaled int4 and row-scaled int2
    experts.  Routing of every token, and the output of every token against
    the oracle's expert FFNs (under the GPU's selection where a near tie
    changed it, with that selection's weights)."""
    qk = gpu_lib
    from concurrent.futures import ThreadPoolExecutor

    from tests.test_gpu_layer import check_routing, combine, rowq_expert_ffn, selection_weights
    spec = W.MOE
    seed, T, H, E, F, k = spec["seed"], spec["tokens"], spec["hidden"], spec["experts"], spec["ffn"], spec["top_k"]
    cu = "cuda"
    st = {"q4_0": (torch.empty((E, 2 * F, H // 2), dtype=torch.uint8, device=cu),
                   torch.empty((E, 2 * F, H // 32), dtype=torch.int16, device=cu),
                   torch.empty((E, H, F // 2), dtype=torch.uint8, device=cu),
                   torch.empty((E, H, F // 32), dtype=torch.int16, device=cu))}
    for bits in (4, 2):
        st[bits] = (torch.empty((E, 2 * F, H * bits // 8), dtype=torch.uint8, device=cu),
                    torch.empty((E, 2 * F), dtype=torch.float32, device=cu),
                    torch.empty((E, H, F * bits // 8), dtype=torch.uint8, device=cu),
                    torch.empty((E, H), dtype=torch.float32, device=cu))
    for e in range(E):
        if e % 64 == 0:
            say(f"moe: generating and quantizing experts {e}.. on the GPU (three codecs)")
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        gu_t, dn_t = to_device(gu), to_device(dn)
        a = st["q4_0"]
        qk.qk_quantize_q4_0(gu_t, out_q=a[0][e], out_d=a[1][e])
        qk.qk_quantize_q4_0(dn_t, out_q=a[2][e], out_d=a[3][e])
        for bits in (4, 2):
            a = st[bits]
            qk.qk_quantize_rowq(gu_t, bits, out_q=a[0][e], out_r=a[1][e])
            qk.qk_quantize_rowq(dn_t, bits, out_q=a[2][e], out_r=a[3][e])
        del gu_t, dn_t
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), W.WEIGHT_STD)
    say("moe: GPU layers (Q4_0, int4 per row, int2 per row)")
    res = {"q4_0": qk.moe_route_and_apply(dev(x), dev(wr), k, *st["q4_0"])}
    for bits in (4, 2):
        res[bits] = qk.qk_moe_route_and_apply_rowq(dev(x), dev(wr), k, *st[bits], bits)
    torch.cuda.synchronize()
    sel_o, w_o, logits = oracle.moe_route(x, wr, k, return_logits=True)
    use = {}
    for c, (y, sg, wg) in res.items():
        sel_g, w_g = host(sg), host(wg)
        check_routing(sel_g, w_g, sel_o, w_o, logits)
        wt = np.where((sel_g == sel_o).all(axis=1)[:, None], w_o, selection_weights(logits, sel_g))
        assert np.allclose(w_g, wt, rtol=1e-6, atol=1e-8), f"codec {c}: routing weights"
        use[c] = (sel_g, wt, host(y))
    need = {}
    for c, (sel, _, _) in use.items():
        for t in range(T):
            for e in sel[t]:
                need.setdefault(int(e), set()).add((c, t))
    first = min(need)

    def expert_outputs(e):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        out = {}
        codecs = {c for c, _ in need[e]}
        for c in codecs:
            if c == "q4_0":
                a, b = oracle.quantize_q4_0(gu)
                cq, d = oracle.quantize_q4_0(dn)
                fn = lambda t: oracle.moe_expert_ffn(x[t], a, b, cq, d)
            else:
                a, b = oracle.quantize_rowq(gu, c)
                cq, d = oracle.quantize_rowq(dn, c)
                fn = lambda t, a=a, b=b, cq=cq, d=d, c=c: rowq_expert_ffn(x[t], a, b, cq, d, c)
            if e == first:   # the device quantizer produced the oracle's bytes
                dq = st[c]
                assert np.array_equal(host(dq[0][e]), a) and np.array_equal(host(dq[2][e]), cq)
            for cc, t in need[e]:
                if cc == c:
                    out[(c, t, e)] = fn(t)
        return out

    ys = {}
    with ThreadPoolExecutor(max_workers=4) as ex:
        for i, r in enumerate(ex.map(expert_outputs, sorted(need))):
            if i % 32 == 0:
                say(f"moe: oracle expert FFNs, {i} of {len(need)} experts")
            ys.update(r)
    for c, (sel, wt, y_h) in use.items():
        for t in range(T):
            want = combine([ys[(c, t, int(e))] for e in sel[t]], wt[t])
            assert rel_err(y_h[t], want) < LAYER_TOL, f"codec {c}, token {t}"
    say(f"moe: all {T} tokens match for every codec ({len(need)} distinct experts)")
