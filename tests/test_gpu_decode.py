"""The whole-model greedy decode in one persistent kernel (qk_decode_greedy)
against the oracle: every step's logits within 1e-2 and every greedy token
agreeing, teacher-forced and free-running, at the TinyLLaMA-1.1B shape and
on small models (ring wrap, several layers); the bounded waits give up when
the host sets a tiny spin limit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quantized_q4_q8_amd.model import Decoder, DecoderShape, layer_to_device
from synth import workloads as W
from tests.test_gpu_model import build, check_tokens, oracle_forward
from tests.util import LAYER_TOL, LOGIT_TOL, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def small_model(seed, g, L, V, cap, ctx):
    """A small decoder with KV caches prefilled with N(0,1) fp16 rows 0..ctx-1."""
    spec = dict(geometry=g, seed=seed, layers=L, vocab=V, cap=cap)
    dec, hm = build(spec, 1)
    kv = []
    for li in range(L):
        kc, vc = W.kv_prefill_f16(seed, li, g.n_kv_heads, cap, g.head_dim, ctx)
        dec.k_cache[li].copy_(torch.from_numpy(kc.view(np.int16)))
        dec.v_cache[li].copy_(torch.from_numpy(vc.view(np.int16)))
        kv.append((kc.view(np.uint16).copy(), vc.view(np.uint16).copy()))
    return dec, hm, kv


def oracle_steps(hm, kv, first, pos0, n, forced=None):
    """n oracle decode steps: logits [n][V]; the input of step j is forced[j]
    when given, else the greedy token of step j - 1."""
    seq = np.zeros(1, np.int32)
    out, tok = [], np.array([first], np.int32)
    for j in range(n):
        if forced is not None:
            tok = np.array([forced[j]], np.int32)
        lo = oracle_forward(hm, tok, np.array([pos0 + j], np.int32), seq, kv)
        out.append(lo[0])
        tok = np.argmax(lo, axis=-1).astype(np.int32)
    return np.stack(out)


def check_steps(got_logits, got_ids, want):
    err = np.max(np.abs(got_logits - want), axis=1)
    assert np.all(err <= LOGIT_TOL), f"steps over tolerance: {np.nonzero(err > LOGIT_TOL)[0]}, worst {err.max()}"
    check_tokens(got_ids, want)
    return float(err.max())


@pytest.mark.parametrize("L,cap,ctx,n", [(2, 64, 20, 12),     # several layers, no wrap
                                         (3, 48, 40, 24)])    # positions 40..63 wrap a 48-row ring
def test_decode_small_teacher_forced(gpu_lib, L, cap, ctx, n):
    g = W.LAYER_SMALL["geometry"]
    V = 1000
    say(f"qk_decode_greedy small: L={L} cap={cap} ctx={ctx} n={n}")
    dec, hm, kv = small_model(80 + L, g, L, V, cap, ctx)
    forced = synth.randint(80 + L, W.TID_TOKENS, n, V).astype(np.int32)
    want = oracle_steps(hm, [(k.copy(), v.copy()) for k, v in kv], 0, ctx, n, forced=forced)
    logits = torch.empty((n, V), dtype=torch.float32, device="cuda")
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    dec.decode_persistent(n, ctx, ids, forced=dev(forced), logits=logits)
    torch.cuda.synchronize()
    assert qk_error(gpu_lib, dec) == 0
    check_steps(host(logits), host(ids), want)
    # the rows written at the decoded positions match the oracle's caches
    ko = [(k.copy(), v.copy()) for k, v in kv]
    oracle_steps(hm, ko, 0, ctx, n, forced=forced)
    for li in range(L):
        rows = [(ctx + j) % cap for j in range(n)]
        got = oracle.f16_to_f32(host(dec.k_cache[li], np.uint16)[0][:, rows])
        want_k = oracle.f16_to_f32(ko[li][0][0][:, rows])
        assert rel_err(got, want_k) < LAYER_TOL


def qk_error(qk, dec):
    return qk.qk_decode_error(dec.cfg, dec.decode_ws)


def test_decode_small_free_running(gpu_lib):
    """Greedy decoding feeding back its own tokens (inside the kernel) gives
    the oracle's greedy sequence, and the same logits."""
    g = W.LAYER_SMALL["geometry"]
    L, V, cap, ctx, n = 2, 517, 64, 10, 16
    say("qk_decode_greedy small free-running")
    dec, hm, kv = small_model(90, g, L, V, cap, ctx)
    first = int(synth.randint(90, W.TID_TOKENS, 1, V)[0])
    want = oracle_steps(hm, [(k.copy(), v.copy()) for k, v in kv], first, ctx, n)
    logits = torch.empty((n, V), dtype=torch.float32, device="cuda")
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    dec.decode_persistent(n, ctx, ids, first_id=dev(np.array([first], np.int32)), logits=logits)
    torch.cuda.synchronize()
    assert qk_error(gpu_lib, dec) == 0
    got_ids = host(ids)
    # a near tie may legitimately change the trajectory: compare up to it
    want_ids = np.argmax(want, axis=-1)
    for j in range(n):
        if got_ids[j] != want_ids[j]:
            top2 = np.sort(want[j])[-2:]
            assert top2[1] - top2[0] <= LOGIT_TOL, f"step {j}"
            n = j + 1
            break
    check_steps(host(logits)[:n], got_ids[:n], want[:n])


def test_decode_repeatable_and_logits_rows(gpu_lib):
    """Two launches on the same workspace give identical tokens (the
    exchange words are cleared per launch), and a one-row logits buffer
    holds the last step's logits."""
    g = W.LAYER_SMALL["geometry"]
    L, V, cap, ctx, n = 2, 1000, 64, 8, 6
    dec, hm, kv = small_model(91, g, L, V, cap, ctx)
    forced = synth.randint(91, W.TID_TOKENS, n, V).astype(np.int32)
    k0, v0 = dec.k_cache.clone(), dec.v_cache.clone()
    outs = []
    for rep in range(2):
        dec.k_cache.copy_(k0)
        dec.v_cache.copy_(v0)
        ids = torch.empty(n, dtype=torch.int32, device="cuda")
        lg = torch.empty((1, V), dtype=torch.float32, device="cuda")
        dec.decode_persistent(n, ctx, ids, forced=dev(forced), logits=lg)
        torch.cuda.synchronize()
        outs.append((host(ids), host(lg)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    want = oracle_steps(hm, [(k.copy(), v.copy()) for k, v in kv], 0, ctx, n, forced=forced)
    assert np.max(np.abs(outs[0][1][0] - want[-1])) <= LOGIT_TOL


def test_decode_bounded_wait_gives_up(gpu_lib):
    """With a spin limit of one poll the kernel's waits give up: the call
    returns, the kernel ends, and the error flag is set.  A later launch with
    the default limit on the same workspace is correct again."""
    g = W.LAYER_SMALL["geometry"]
    L, V, cap, ctx, n = 2, 1000, 64, 8, 4
    dec, hm, kv = small_model(92, g, L, V, cap, ctx)
    forced = synth.randint(92, W.TID_TOKENS, n, V).astype(np.int32)
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    say("qk_decode_greedy with spin_limit 1")
    dec.decode_persistent(n, ctx, ids, forced=dev(forced), spin_limit=1)
    torch.cuda.synchronize()
    assert qk_error(gpu_lib, dec) != 0
    dec.k_cache.zero_()
    dec.v_cache.zero_()
    for li in range(L):
        dec.k_cache[li].copy_(torch.from_numpy(kv[li][0].view(np.int16)))
        dec.v_cache[li].copy_(torch.from_numpy(kv[li][1].view(np.int16)))
    lg = torch.empty((n, V), dtype=torch.float32, device="cuda")
    dec.decode_persistent(n, ctx, ids, forced=dev(forced), logits=lg)
    torch.cuda.synchronize()
    assert qk_error(gpu_lib, dec) == 0
    want = oracle_steps(hm, [(k.copy(), v.copy()) for k, v in kv], 0, ctx, n, forced=forced)
    check_steps(host(lg), host(ids), want)


@pytest.mark.timeout(900)
def test_decode_tinyllama_shape_persistent_every_step(gpu_lib):
    """The decode workload through the persistent kernel as the benchmark
    runs it (TinyLLaMA-1.1B shape, 22 layers, fp16 KV prefilled to 2048,
    positions 2048..2175, weights in one arena), teacher-forced with the
    oracle's tokens: all 128 steps' logits within 1e-2, every greedy token
    agreeing, and the K/V rows of every decoded position."""
    spec = W.DECODE
    g, L, cap, ctx, n, V = (spec["geometry"], spec["layers"], spec["cap"], spec["context"],
                            spec["steps"], spec["vocab"])
    say("persistent decode: building the 22-layer model")
    dec, hm = build(spec, 1)
    dec.pack()
    kv = []
    for li in range(L):
        kc, vc = W.kv_prefill_f16(spec["seed"], li, g.n_kv_heads, cap, g.head_dim, ctx)
        dec.k_cache[li].copy_(torch.from_numpy(kc.view(np.int16)))
        dec.v_cache[li].copy_(torch.from_numpy(vc.view(np.int16)))
        kv.append((kc.view(np.uint16).copy(), vc.view(np.uint16).copy()))
    first = int(synth.randint(spec["seed"], W.TID_TOKENS, 1, V)[0])
    seq = np.zeros(1, np.int32)
    want = np.empty((n, V), np.float32)
    forced = np.empty(n, np.int32)
    tok = np.array([first], np.int32)
    for j in range(n):
        if j % 16 == 0:
            say(f"persistent decode: oracle step {j}")
        forced[j] = tok[0]
        lo = oracle_forward(hm, tok, np.array([ctx + j], np.int32), seq, kv)
        want[j] = lo[0]
        tok = np.argmax(lo, axis=-1).astype(np.int32)
    say("persistent decode: 128 steps in one launch")
    logits = torch.empty((n, V), dtype=torch.float32, device="cuda")
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    dec.decode_persistent(n, ctx, ids, forced=dev(forced), logits=logits)
    torch.cuda.synchronize()
    assert qk_error(gpu_lib, dec) == 0
    worst = check_steps(host(logits), host(ids), want)
    say(f"persistent decode: worst step logit error {worst:.2e}")
    rows = list(range(ctx, ctx + n))
    for li in (0, L // 2, L - 1):
        for c in (0, 1):
            gotc = oracle.f16_to_f32(host((dec.k_cache, dec.v_cache)[c][li], np.uint16)[0][:, rows])
            wantc = oracle.f16_to_f32(kv[li][c][0][:, rows])
            assert rel_err(gotc, wantc) < LAYER_TOL, f"layer {li} {'kv'[c]} cache"
