"""GPU parity of layer_forward and moe_route_and_apply against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_q4_q8_amd.model import layer_to_device
from synth import workloads as W
from tests.util import LAYER_TOL, assert_same_fp32, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def oracle_layer(wf):
    wl = {}
    for name, key in [("w_qkv", "w_qkv"), ("w_o", "w_o"), ("w_gate_up", "w_gu"), ("w_down", "w_down")]:
        wl[key + "_q"], wl[key + "_d"] = oracle.quantize_q4_0(wf[name])
    wl["gamma_attn"], wl["gamma_ffn"] = wf["gamma_attn"], wf["gamma_ffn"]
    return wl


def check_weights_identical(lw, wl):
    """The device quantizer produced the very bytes the oracle uses."""
    pairs = [(lw.w_qkv_q, wl["w_qkv_q"]), (lw.w_qkv_d, wl["w_qkv_d"]), (lw.w_o_q, wl["w_o_q"]),
             (lw.w_gate_up_q, wl["w_gu_q"]), (lw.w_down_d, wl["w_down_d"])]
    for t, a in pairs:
        assert np.array_equal(host(t, a.dtype), a)


def test_layer_small_prefill_then_self_fed_decode(gpu_lib):
    """The one-layer workload: 16-token prefill (MFMA GEMM path), then 16 decode
    steps (GEMV path) where each side feeds back its own last output."""
    qk = gpu_lib
    spec = W.LAYER_SMALL
    g, seed, cap = spec["geometry"], spec["seed"], spec["cap"]
    say(f"layer_forward small: H={g.hidden} nq={g.n_q_heads} nkv={g.n_kv_heads} F={g.ffn}")
    wf = W.layer_weights_f32(seed, 0, g)
    wl = oracle_layer(wf)
    lw = layer_to_device(wf)
    check_weights_identical(lw, wl)
    cfg = qk.layer_cfg(**g.cfg(cap))
    P = spec["prompt"]
    x = synth.normal(seed, W.TID_X, (P, g.hidden))
    kshape = (1, g.n_kv_heads, cap, g.head_dim)
    kc, vc = np.zeros(kshape, np.uint16), np.zeros(kshape, np.uint16)
    kcg, vcg = dev(kc), dev(vc)
    pos = np.arange(P, dtype=np.int32)
    seq = np.zeros(P, np.int32)
    ref = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
    xg = dev(x)
    qk.layer_forward(lw, cfg, xg, dev(pos), dev(seq), kcg, vcg)
    assert rel_err(host(xg), ref) < LAYER_TOL
    assert_same_fp32(host(xg), ref)
    assert np.mean(host(kcg, np.uint16) == kc) > 0.999
    kf = oracle.f16_to_f32(kc)
    assert rel_err(oracle.f16_to_f32(host(kcg, np.uint16)), kf) < LAYER_TOL
    o_in, g_in = ref[-1:], host(xg)[-1:]
    for step in range(spec["decode"]):
        p = np.array([P + step], np.int32)
        s0 = np.zeros(1, np.int32)
        o_out = oracle.layer_forward(wl, g.cfg(cap), o_in, p, s0, kc, vc)
        xs = dev(g_in)
        qk.layer_forward(lw, cfg, xs, dev(p), dev(s0), kcg, vcg)
        g_out = host(xs)
        assert rel_err(g_out, o_out) < LAYER_TOL, f"decode step {step}"
        assert_same_fp32(g_out, o_out)
        o_in, g_in = o_out, g_out


@pytest.mark.parametrize("tokens", [5, 40])
def test_layer_ragged_sequences(gpu_lib, tokens):
    """Tokens of three sequences at scattered positions, with prefilled caches;
    5 tokens run the GEMV path, 40 the MFMA path."""
    qk = gpu_lib
    g = W.Geometry(512, 16, 4, 32, 352)
    cap = 96
    say(f"layer_forward ragged tokens={tokens}")
    wf = W.layer_weights_f32(40, 1, g)
    wl = oracle_layer(wf)
    lw = layer_to_device(wf)
    kc, vc = W.kv_prefill_f16(40, 1, g.n_kv_heads, cap, g.head_dim, 50, seqs=3)
    kc, vc = kc.view(np.uint16).copy(), vc.view(np.uint16).copy()
    kcg, vcg = dev(kc), dev(vc)
    seq = (np.arange(tokens) % 3).astype(np.int32)
    pos = (50 + np.arange(tokens) // 3).astype(np.int32)
    x = synth.normal(40, 5, (tokens, g.hidden))
    ref = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
    xg = dev(x)
    qk.layer_forward(lw, qk.layer_cfg(**g.cfg(cap)), xg, dev(pos), dev(seq), kcg, vcg)
    assert rel_err(host(xg), ref) < LAYER_TOL
    assert_same_fp32(host(xg), ref)


@pytest.mark.parametrize("tokens", [3, 8])
def test_layer_tinyllama_shape_few_tokens(gpu_lib, tokens):
    """One layer at the TinyLLaMA-1.1B shape (hidden 2048, FFN 5632) with 3
    and 8 tokens of one sequence at positions 100.. over a prefilled cache:
    the fused-prologue GEMVs with several columns per pass, the down
    projection's K = 5632 in three register chunks."""
    qk = gpu_lib
    g = W.Geometry(2048, 32, 4, 64, 5632)
    cap, ctx = 160, 100
    say(f"layer_forward TinyLLaMA shape tokens={tokens}")
    wf = W.layer_weights_f32(43, 0, g)
    wl = oracle_layer(wf)
    lw = layer_to_device(wf)
    kc, vc = W.kv_prefill_f16(43, 0, g.n_kv_heads, cap, g.head_dim, ctx)
    kc, vc = kc.view(np.uint16).copy(), vc.view(np.uint16).copy()
    kcg, vcg = dev(kc), dev(vc)
    pos = (ctx + np.arange(tokens)).astype(np.int32)
    seq = np.zeros(tokens, np.int32)
    x = synth.normal(43, 5, (tokens, g.hidden))
    ref = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
    xg = dev(x)
    qk.layer_forward(lw, qk.layer_cfg(**g.cfg(cap)), xg, dev(pos), dev(seq), kcg, vcg)
    assert rel_err(host(xg), ref) < LAYER_TOL
    assert_same_fp32(host(xg), ref)
    assert np.mean(host(kcg, np.uint16) == kc) > 0.999


@pytest.mark.parametrize("seqs", [1, 3, 12])
def test_layer_decode_through_ring_wrap(gpu_lib, seqs):
    """Decode past the cache capacity (the cache is a ring, position p in row
    p % cap): each sequence is prefilled with 12 tokens into a 20-row cache,
    then all sequences decode 24 steps together, one token each per call, each
    side feeding back its own output.  With 12 sequences the calls take the
    many-token path (MFMA matmuls, tiled attention)."""
    qk = gpu_lib
    g = W.Geometry(256, 8, 2, 32, 160)
    cap, P, steps = 20, 12, 24
    say(f"layer_forward ring wrap seqs={seqs} cap={cap}")
    wf = W.layer_weights_f32(41, 2, g)
    wl = oracle_layer(wf)
    lw = layer_to_device(wf)
    cfg = qk.layer_cfg(**g.cfg(cap))
    kshape = (seqs, g.n_kv_heads, cap, g.head_dim)
    kc, vc = np.zeros(kshape, np.uint16), np.zeros(kshape, np.uint16)
    kcg, vcg = dev(kc), dev(vc)
    o_in, g_in = [], []
    for s in range(seqs):
        x = synth.normal(41, 10 + s, (P, g.hidden))
        pos, seq = np.arange(P, dtype=np.int32), np.full(P, s, np.int32)
        ref = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
        xg = dev(x)
        qk.layer_forward(lw, cfg, xg, dev(pos), dev(seq), kcg, vcg)
        assert_same_fp32(host(xg), ref)
        o_in.append(ref[-1])
        g_in.append(host(xg)[-1])
    o_in, g_in = np.stack(o_in), np.stack(g_in)
    seq = np.arange(seqs, dtype=np.int32)
    for step in range(steps):
        pos = np.full(seqs, P + step, np.int32)
        o_out = oracle.layer_forward(wl, g.cfg(cap), o_in, pos, seq, kc, vc)
        xs = dev(g_in)
        qk.layer_forward(lw, cfg, xs, dev(pos), dev(seq), kcg, vcg)
        g_out = host(xs)
        assert rel_err(g_out, o_out) < LAYER_TOL, f"decode step {step} (position {P + step})"
        assert_same_fp32(g_out, o_out)
        o_in, g_in = o_out, g_out
    assert np.mean(host(kcg, np.uint16) == kc) > 0.999


@pytest.mark.parametrize("cap,tokens,start", [(32768, 2, 32768 + 5),   # one token per sequence, ring wrapped
                                              (16384, 40, 9000)])      # a 40-token run past 8192: tiled path
def test_layer_long_context(gpu_lib, cap, tokens, start):
    """TinyLLaMA attention heads (32 query, 4 KV, head_dim 64) over long fp16
    caches filled with N(0,1) rows: decode of one token per sequence at a
    wrapped position of a 32768-row ring (512 attention chunks per head,
    merged in the merge pass), and a 40-token prefill run at positions
    9000..9039 of a 16384-row cache (the matrix-core attention pass)."""
    qk = gpu_lib
    g = W.Geometry(512, 32, 4, 64, 704)
    one_each = tokens <= 8
    seqs = tokens if one_each else 1
    say(f"layer_forward long context cap={cap} tokens={tokens} start={start}")
    wf = W.layer_weights_f32(43, 1, g)
    wl = oracle_layer(wf)
    lw = layer_to_device(wf)
    kc, vc = W.kv_prefill_f16(43, 1, g.n_kv_heads, cap, g.head_dim, cap, seqs=seqs)
    kc, vc = kc.view(np.uint16).copy(), vc.view(np.uint16).copy()
    kcg, vcg = dev(kc), dev(vc)
    x = synth.normal(43, 7, (tokens, g.hidden))
    if one_each:
        pos = np.full(tokens, start, np.int32) + np.arange(tokens, dtype=np.int32) * 977
        seq = np.arange(tokens, dtype=np.int32)
    else:
        pos = (start + np.arange(tokens)).astype(np.int32)
        seq = np.zeros(tokens, np.int32)
    ref = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
    xg = dev(x)
    qk.layer_forward(lw, qk.layer_cfg(**g.cfg(cap)), xg, dev(pos), dev(seq), kcg, vcg)
    assert rel_err(host(xg), ref) < LAYER_TOL
    assert_same_fp32(host(xg), ref)
    # the rows written at the tokens' positions
    got_k = oracle.f16_to_f32(host(kcg, np.uint16))
    rows = pos % cap
    for t in range(tokens):
        assert rel_err(got_k[seq[t], :, rows[t]], oracle.f16_to_f32(kc[seq[t], :, rows[t]])) < LAYER_TOL


def test_layer_decode_equals_prefill_last_row(gpu_lib):
    qk = gpu_lib
    g = W.LAYER_SMALL["geometry"]
    cap = 32
    say("layer_forward decode == prefill last row (GPU)")
    lw = layer_to_device(W.layer_weights_f32(41, 0, g))
    cfg = qk.layer_cfg(**g.cfg(cap))
    x = synth.normal(41, 1, (12, g.hidden))
    shape = (1, g.n_kv_heads, cap, g.head_dim)
    pos = np.arange(12, dtype=np.int32)
    seq = np.zeros(12, np.int32)
    ka, va = torch.zeros(shape, dtype=torch.int16, device="cuda"), torch.zeros(shape, dtype=torch.int16, device="cuda")
    full = dev(x)
    qk.layer_forward(lw, cfg, full, dev(pos), dev(seq), ka, va)
    kb, vb = torch.zeros_like(ka), torch.zeros_like(va)
    part = dev(x[:11])
    qk.layer_forward(lw, cfg, part, dev(pos[:11]), dev(seq[:11]), kb, vb)
    last = dev(x[11:])
    qk.layer_forward(lw, cfg, last, dev(pos[11:]), dev(seq[11:]), kb, vb)
    assert rel_err(host(last), host(full)[11:]) < LAYER_TOL


# ---------------------------------------------------------------- MoE
def experts_f32(seed, E, H, F):
    gus, dns = [], []
    for e in range(E):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        gus.append(gu)
        dns.append(dn)
    return np.stack(gus), np.stack(dns)


def check_routing(sel_g, w_g, sel_o, w_o, logits):
    """Selections must agree except where the oracle's k-th and (k+1)-th
    logits are within 1e-5 (either choice is correct there)."""
    k = sel_o.shape[1]
    for t in range(sel_o.shape[0]):
        if np.array_equal(sel_g[t], sel_o[t]):
            assert np.allclose(w_g[t], w_o[t], rtol=1e-5, atol=1e-7)
            continue
        srt = np.sort(logits[t])[::-1]
        assert srt[k - 1] - srt[k] < 1e-5, f"token {t}: selection differs without a near tie"


def rowq_expert_ffn(x_row, gu_q, gu_r, dn_q, dn_r, bits):
    """The oracle's expert FFN with row-scaled weights (the expert shape comes
    from the arrays): Q8_0 input, gate/up, SwiGLU, Q8_0, down."""
    F = gu_q.shape[0] // 2
    xq, xd = oracle.quantize_q8_0(np.asarray(x_row, np.float32)[None])
    gup = oracle.qmatmul_rowq(gu_q, gu_r, xq, xd, bits)[0]
    hq, hd = oracle.quantize_q8_0(oracle.swiglu(gup[:F], gup[F:])[None])
    return oracle.qmatmul_rowq(dn_q, dn_r, hq, hd, bits)[0]


def selection_weights(logits, sel):
    """The routing rule's weights for a given selection: s = sigmoid(logit)
    in fp64 for each selected expert, w = s / (sum of s in rank order),
    rounded to fp32."""
    T, k = sel.shape
    w = np.empty((T, k), np.float32)
    for t in range(T):
        s = 1.0 / (1.0 + np.exp(-logits[t, sel[t]].astype(np.float64)))
        tot = 0.0
        for r in range(k):
            tot += s[r]
        w[t] = (s / tot).astype(np.float32)
    return w


def combine(ys, w):
    """sum over ranks, in rank order, of w[r] * ys[r], in fp64, rounded once."""
    acc = np.zeros(len(ys[0]), np.float64)
    for r in range(len(w)):
        acc += np.float64(w[r]) * np.asarray(ys[r], np.float64)
    return acc.astype(np.float32)


def moe_expected(sel_g, w_g, sel_o, out_o, logits, expert_y):
    """Expected output of every token.  Where the GPU chose the oracle's
    experts it is the oracle's output.  Where a near tie gave another
    selection (which check_routing accepted) it is the oracle's expert FFNs
    under the GPU's selection, combined with the routing rule's weights for
    that selection; the GPU's weights must equal those.  expert_y(t, e) is
    the oracle's FFN of expert e on token t."""
    want = np.array(out_o, np.float32, copy=True)
    for t in range(sel_o.shape[0]):
        if np.array_equal(sel_g[t], sel_o[t]):
            continue
        wt = selection_weights(logits[t:t + 1], sel_g[t:t + 1])[0]
        assert np.allclose(w_g[t], wt, rtol=1e-6, atol=1e-8), f"token {t}: weights of the GPU's selection"
        want[t] = combine([expert_y(t, int(e)) for e in sel_g[t]], wt)
    return want


@pytest.mark.parametrize("T,H,E,F,k", [(8, 256, 16, 64, 4), (33, 512, 64, 96, 8), (1, 128, 8, 32, 1),
                                       # 1600 pairs: the grouping's second chunk of 1024,
                                       # about 100 tokens per expert (passes of 8 columns)
                                       (200, 64, 16, 32, 8),
                                       # gate/up rows of 256 blocks: past the expert GEMV's
                                       # 192, so the grouped GEMV's multi-step rows take them;
                                       # the down projection stays on the expert GEMV
                                       (6, 8192, 8, 64, 2)])
def test_moe_matches_oracle(gpu_lib, T, H, E, F, k):
    qk = gpu_lib
    say(f"moe_route_and_apply T={T} H={H} E={E} F={F} k={k}")
    seed = 50 + T
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), 0.02)
    gu, dn = experts_f32(seed, E, H, F)
    guq = np.stack([oracle.quantize_q4_0(a)[0] for a in gu])
    gud = np.stack([oracle.quantize_q4_0(a)[1] for a in gu])
    dnq = np.stack([oracle.quantize_q4_0(a)[0] for a in dn])
    dnd = np.stack([oracle.quantize_q4_0(a)[1] for a in dn])
    out, sel, w = oracle.moe_route_and_apply(x, wr, k, guq, gud, dnq, dnd)
    _, _, logits = oracle.moe_route(x, wr, k, return_logits=True)
    y, sg, wg = qk.moe_route_and_apply(dev(x), dev(wr), k, dev(guq), dev(gud), dev(dnq), dev(dnd))
    sel_g, w_g = host(sg), host(wg)
    check_routing(sel_g, w_g, sel, w, logits)
    want = moe_expected(sel_g, w_g, sel, out, logits,
                        lambda t, e: oracle.moe_expert_ffn(x[t], guq[e], gud[e], dnq[e], dnd[e]))
    assert rel_err(host(y), want) < LAYER_TOL
    if np.array_equal(sel_g, sel):
        assert_same_fp32(host(y), out)
    # every selection is a set of distinct experts and weights sum to 1
    assert all(len(set(r)) == k for r in sel_g)
    assert np.allclose(w_g.sum(1), 1.0, atol=1e-6)


@pytest.mark.parametrize("T,H,E,F,k,skew", [
    (256, 256, 8, 128, 2, False),   # about 64 tokens per expert: every expert on the matrix cores
    (96, 256, 16, 64, 4, True),     # experts 0 and 1 take every token, the rest about 14 each: both paths
    (64, 6144, 16, 512, 8, False),  # the MoE workload's hidden width, 32 tokens per expert
])
def test_moe_mfma_experts(gpu_lib, T, H, E, F, k, skew):
    """Experts with at least 16 tokens run on the grouped int8 MFMA GEMM, the
    others on the grouped GEMV (calls averaging at least 16 tokens per
    expert); every token's output matches the oracle's.
    skew: a router that always ranks experts 0 and 1 first (a large constant
    feature and router weights on it), so that two experts hold every token
    and the others few."""
    qk = gpu_lib
    say(f"moe_route_and_apply (matrix-core experts) T={T} H={H} E={E} F={F} k={k} skew={skew}")
    seed = 70 + T
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), 0.02)
    if skew:
        x[:, 0] = 8.0
        wr[0, :] = 0.0
        wr[0, 0], wr[0, 1] = 1.0, 0.9
    gu, dn = experts_f32(seed, E, H, F)
    guq = np.stack([oracle.quantize_q4_0(a)[0] for a in gu])
    gud = np.stack([oracle.quantize_q4_0(a)[1] for a in gu])
    dnq = np.stack([oracle.quantize_q4_0(a)[0] for a in dn])
    dnd = np.stack([oracle.quantize_q4_0(a)[1] for a in dn])
    del gu, dn
    out, sel, w = oracle.moe_route_and_apply(x, wr, k, guq, gud, dnq, dnd)
    _, _, logits = oracle.moe_route(x, wr, k, return_logits=True)
    counts = np.bincount(sel.ravel(), minlength=E)
    assert counts.max() >= 16, "the case must give some expert the matrix-core path"
    if skew:
        assert counts.min() < 16
    y, sg, wg = qk.moe_route_and_apply(dev(x), dev(wr), k, dev(guq), dev(gud), dev(dnq), dev(dnd))
    sel_g, w_g = host(sg), host(wg)
    check_routing(sel_g, w_g, sel, w, logits)
    want = moe_expected(sel_g, w_g, sel, out, logits,
                        lambda t, e: oracle.moe_expert_ffn(x[t], guq[e], gud[e], dnq[e], dnd[e]))
    assert rel_err(host(y), want) < LAYER_TOL
    if np.array_equal(sel_g, sel):
        assert_same_fp32(host(y), out)


@pytest.mark.parametrize("T,H,E,F,k", [
    (12, 6144, 4, 544, 4),   # every expert holds all 12 tokens: gate/up columns staged 5, 5, 2
    (15, 2048, 8, 96, 3),    # 3 to 8 tokens per expert, 3-block down rows, one row group per workgroup
])
def test_moe_expert_gemv_stages(gpu_lib, T, H, E, F, k):
    """The grouped expert GEMV (fewer than 16 tokens per call on average, so
    no expert goes to the matrix cores) on experts with more columns than it
    stages at once (five at hidden 6144), with an odd number of blocks per
    down row (17 at ffn 544: the scale's half of its 32-bit word changes from
    row to row), and with workgroups that take one or two row groups after
    their pairs; every token matches the oracle."""
    qk = gpu_lib
    say(f"moe_route_and_apply (expert GEMV column stages) T={T} H={H} E={E} F={F} k={k}")
    seed = 90 + T
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), 0.02)
    gu, dn = experts_f32(seed, E, H, F)
    guq = np.stack([oracle.quantize_q4_0(a)[0] for a in gu])
    gud = np.stack([oracle.quantize_q4_0(a)[1] for a in gu])
    dnq = np.stack([oracle.quantize_q4_0(a)[0] for a in dn])
    dnd = np.stack([oracle.quantize_q4_0(a)[1] for a in dn])
    del gu, dn
    out, sel, w = oracle.moe_route_and_apply(x, wr, k, guq, gud, dnq, dnd)
    _, _, logits = oracle.moe_route(x, wr, k, return_logits=True)
    counts = np.bincount(sel.ravel(), minlength=E)
    assert counts.max() > 5 and counts.max() < 16, "some expert needs several column stages"
    y, sg, wg = qk.moe_route_and_apply(dev(x), dev(wr), k, dev(guq), dev(gud), dev(dnq), dev(dnd))
    sel_g, w_g = host(sg), host(wg)
    check_routing(sel_g, w_g, sel, w, logits)
    want = moe_expected(sel_g, w_g, sel, out, logits,
                        lambda t, e: oracle.moe_expert_ffn(x[t], guq[e], gud[e], dnq[e], dnd[e]))
    assert rel_err(host(y), want) < LAYER_TOL
    if np.array_equal(sel_g, sel):
        assert_same_fp32(host(y), out)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("T,H,E,F,k", [(8, 256, 16, 64, 4), (33, 512, 64, 96, 8), (16, 6144, 16, 2048, 8)])
def test_moe_rowq_matches_oracle(gpu_lib, bits, T, H, E, F, k):
    """The MoE layer with row-scaled int4 / int2 experts (the last case has
    the expert shape of the MoE workload, 16 experts)."""
    qk = gpu_lib
    say(f"qk_moe_route_and_apply_rowq bits={bits} T={T} H={H} E={E} F={F} k={k}")
    seed = 60 + T
    x = synth.normal(seed, W.TID_X, (T, H))
    wr = synth.normal(seed, W.TID_ROUTER, (H, E), 0.02)
    gu, dn = experts_f32(seed, E, H, F)
    guq, gur = map(np.stack, zip(*[oracle.quantize_rowq(a, bits) for a in gu]))
    dnq, dnr = map(np.stack, zip(*[oracle.quantize_rowq(a, bits) for a in dn]))
    out, sel, w = oracle.moe_route_and_apply_rowq(x, wr, k, guq, gur, dnq, dnr, bits)
    _, _, logits = oracle.moe_route(x, wr, k, return_logits=True)
    y, sg, wg = qk.qk_moe_route_and_apply_rowq(dev(x), dev(wr), k, dev(guq), dev(gur), dev(dnq),
                                               dev(dnr), bits)
    sel_g, w_g = host(sg), host(wg)
    check_routing(sel_g, w_g, sel, w, logits)
    want = moe_expected(sel_g, w_g, sel, out, logits,
                        lambda t, e: rowq_expert_ffn(x[t], guq[e], gur[e], dnq[e], dnr[e], bits))
    assert rel_err(host(y), want) < LAYER_TOL
    if np.array_equal(sel_g, sel):
        assert_same_fp32(host(y), out)
    assert all(len(set(r)) == k for r in sel_g)


@pytest.mark.parametrize("E,k", [(256, 8), (1001, 32), (37, 5)])
def test_moe_router_exact_ties(gpu_lib, E, k):
    """Router columns repeat seven distinct columns, so every token's logits
    tie exactly in groups; the choice must be the oracle's (largest logit,
    lower expert index among equal logits), for the expert count of the MoE
    workload, the largest supported count with a ragged tail, and a small one."""
    qk = gpu_lib
    T, H, F = 20, 64, 32
    say(f"moe router exact ties E={E} k={k}")
    seed = 70 + E
    x = synth.normal(seed, W.TID_X, (T, H))
    base = synth.normal(seed, W.TID_ROUTER, (H, 7), 0.02)
    wr = np.ascontiguousarray(base[:, np.arange(E) % 7])
    gu, dn = experts_f32(seed, E, H, F)
    guq = np.stack([oracle.quantize_q4_0(a)[0] for a in gu])
    gud = np.stack([oracle.quantize_q4_0(a)[1] for a in gu])
    dnq = np.stack([oracle.quantize_q4_0(a)[0] for a in dn])
    dnd = np.stack([oracle.quantize_q4_0(a)[1] for a in dn])
    out, sel, w = oracle.moe_route_and_apply(x, wr, k, guq, gud, dnq, dnd)
    y, sg, wg = qk.moe_route_and_apply(dev(x), dev(wr), k, dev(guq), dev(gud), dev(dnq), dev(dnd))
    assert np.array_equal(host(sg), sel)
    assert np.allclose(host(wg), w, rtol=1e-6, atol=1e-8)
    assert rel_err(host(y), out) < LAYER_TOL


def test_moe_zero_router_ties(gpu_lib):
    qk = gpu_lib
    T, H, E, F, k = 4, 64, 12, 32, 5
    say("moe zero router")
    x = synth.normal(60, 1, (T, H))
    gu, dn = experts_f32(60, E, H, F)
    guq = np.stack([oracle.quantize_q4_0(a)[0] for a in gu])
    gud = np.stack([oracle.quantize_q4_0(a)[1] for a in gu])
    dnq = np.stack([oracle.quantize_q4_0(a)[0] for a in dn])
    dnd = np.stack([oracle.quantize_q4_0(a)[1] for a in dn])
    wr = np.zeros((H, E), np.float32)
    out, sel, w = oracle.moe_route_and_apply(x, wr, k, guq, gud, dnq, dnd)
    y, sg, wg = qk.moe_route_and_apply(dev(x), dev(wr), k, dev(guq), dev(gud), dev(dnq), dev(dnd))
    assert np.all(host(sg) == np.arange(k)) and np.all(host(wg) == np.float32(1 / k))
    assert rel_err(host(y), out) < LAYER_TOL
