#!/usr/bin/env python3
"""Throughput benchmark of the Q4_0 x Q8_0 decoder path on one MI355X.

Default workload: TinyLLaMA-1.1B-shaped greedy decode (22 layers, hidden
2048, 32 query / 4 KV heads of 64, SwiGLU 5632, vocab 32000, Q4_0 weights
from N(0, 0.02), fp16 KV cache prefilled with N(0, 1) to context 2048).  One
step is the workload's full 128-token greedy decode (positions 2048..2175):
per token embedding, 22 decoder layers, final RMSNorm, LM head and argmax.
The step's kernels (all 128 tokens, back to back) are captured once in a HIP
graph and replayed; inputs are resident in HBM before timing starts.

Prints one JSON line: throughput (tokens/s), the dominant kernel's HBM
roofline (its average duration from HIP events on its stream), and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def read_ceiling(dev) -> float:
    """Achievable HBM read rate (GB/s): qk_read_probe streaming a 1 GiB
    buffer (four times the memory-side cache) with the GEMV's 128-bit
    non-temporal loads, 10 timed passes after 2 untimed."""
    import torch
    import quantized_q4_q8_amd as qk
    buf = torch.zeros(2**30 // 4, dtype=torch.int32, device=dev)
    words = torch.empty(2048, dtype=torch.int32, device=dev)
    for _ in range(2):
        qk.qk_read_probe(buf, out=words)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        qk.qk_read_probe(buf, out=words)
    b.record()
    torch.cuda.synchronize()
    gbs = 2**30 * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf, words
    log(f"read probe: {gbs:.0f} GB/s achievable (1 GiB, 128-bit non-temporal loads)")
    return gbs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "longctx", "longctx32k", "layer", "matmul", "prefill", "moe",
                             "sample"],
                    help="decode (the headline line); the others measure decode past an "
                         "8192-row or a 32768-row ring cache and the standalone matmul, "
                         "prefill, MoE and sampler workloads")
    ap.add_argument("--codec", default="q4_0", choices=["q4_0", "int4row", "int2row"],
                    help="weight format of the matmul and moe workloads: Q4_0 (fp16 scale per "
                         "32-block) or row-scaled int4 / int2 (fp32 scale per row)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--kernel-rounds", type=int, default=20)
    ap.add_argument("--graph", choices=["token", "step"], default="step",
                    help="decode capture: one HIP graph per token position, or the whole "
                         "step's tokens in one graph")
    ap.add_argument("--no-arena", action="store_true",
                    help="decode: keep each weight in its own allocation instead of one arena "
                         "in step order")
    ap.add_argument("--decode-tokens", type=int, default=128,
                    help="tokens per step; only for short profiling runs (the workload is 128)")
    return ap.parse_args()


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_counters(kernel: str, src_hash: str):
    """Busy fractions from the committed rocprofv3 counter summary, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return {k: rec[k] for k in ("mfma_busy", "valu_busy", "lds_active", "wave_cycles_waiting")}


def stored_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    rec = t.get(kernel)
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# decode workload
# ---------------------------------------------------------------------------
def build_decoder(spec, want_host_q4: bool, seqs: int = 1):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from quantized_q4_q8_amd.model import Decoder, DecoderShape, layer_to_device, to_device
    from synth import normal, randint
    from synth import workloads as W

    g, seed, L, V, cap = spec["geometry"], spec["seed"], spec["layers"], spec["vocab"], spec["cap"]
    ctx = spec.get("context", 0)       # rows of the KV cache prefilled with N(0,1)
    host = {"layers": [], "kv": []} if want_host_q4 else None
    if want_host_q4:
        import oracle
    layers = []
    t0 = time.time()
    for li in range(L):
        wf = W.layer_weights_f32(seed, li, g)
        layers.append(layer_to_device(wf))
        if want_host_q4:
            wl = {}
            for name, key in [("w_qkv", "w_qkv"), ("w_o", "w_o"), ("w_gate_up", "w_gu"),
                              ("w_down", "w_down")]:
                wl[key + "_q"], wl[key + "_d"] = oracle.quantize_q4_0(wf[name])
            wl["gamma_attn"], wl["gamma_ffn"] = wf["gamma_attn"], wf["gamma_ffn"]
            host["layers"].append(wl)
        del wf
    log(f"layers generated and quantized in {time.time() - t0:.1f}s")
    embed = normal(seed, W.TID_EMBED, (V, g.hidden))
    gamma_f = normal(seed, W.TID_GAMMA_FINAL, g.hidden, W.GAMMA_STD, mean=1.0)
    lm = normal(seed, W.TID_LM_HEAD, (V, g.hidden), W.WEIGHT_STD)
    lm_q, lm_d = qk.qk_quantize_q4_0(to_device(lm))
    shape = DecoderShape(g.hidden, g.n_q_heads, g.n_kv_heads, g.head_dim, g.ffn_padded, g.eps,
                         g.rope_base, L, V, cap, seqs)
    dec = Decoder(shape, layers, to_device(embed), to_device(gamma_f), lm_q, lm_d)
    for li in range(L if ctx > 0 else 0):
        kc, vc = W.kv_prefill_f16(seed, li, g.n_kv_heads, cap, g.head_dim, ctx, seqs=seqs)
        dec.k_cache[li].copy_(torch.from_numpy(kc.view(np.int16)))
        dec.v_cache[li].copy_(torch.from_numpy(vc.view(np.int16)))
        if want_host_q4:
            host["kv"].append((kc.view(np.uint16).copy(), vc.view(np.uint16).copy()))
    first = randint(seed, W.TID_TOKENS, 1, V)
    if want_host_q4:
        import oracle
        host["embed"], host["gamma_f"] = embed, gamma_f
        host["lm_q"], host["lm_d"] = oracle.quantize_q4_0(lm)
    del lm
    torch.cuda.synchronize()
    log(f"model resident on the GPU after {time.time() - t0:.1f}s")
    return dec, first, host


def decode_bytes_per_token(spec) -> float:
    """Algorithmic HBM bytes per decode token at the workload's mean context."""
    g, L, V = spec["geometry"], spec["layers"], spec["vocab"]
    H, F = g.hidden, g.ffn_padded
    q4 = 9 / 16  # bytes per Q4_0 weight
    lin = L * (g.n_qkv * H + H * g.n_q_heads * g.head_dim + 2 * F * H + H * F) + V * H
    # cache rows read per layer, averaged over the steps (the ring holds cap)
    mean_ctx = sum(min(spec["context"] + j + 1, spec["cap"]) for j in range(spec["steps"])) / spec["steps"]
    kv = L * 2 * g.n_kv_heads * g.head_dim * 2 * mean_ctx
    norms = (2 * L + 1) * H * 4
    return lin * q4 + kv + norms + H * 4


def run_decode(args, long_context=False):
    """long_context: False (the headline workload), True (8192-row ring) or
    "32k" (32768-row ring)."""
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from synth import normal
    from synth import workloads as W

    spec = (W.DECODE_LONG32K if long_context == "32k" else W.DECODE_LONG) if long_context else W.DECODE
    g, L = spec["geometry"], spec["layers"]
    steps_per_run = max(1, min(args.decode_tokens, spec["steps"]))
    want_cpu = not args.no_cpu_baseline
    dec, first, host = build_decoder(spec, want_cpu)
    dev = dec.device
    if not args.no_arena:   # all weights in one allocation, in the order the step reads them
        dec.pack()
        torch.cuda.synchronize()

    # -- the decode positions (2048 .. 2175) captured in one HIP graph (or
    #    one graph per position with --graph token)
    seq = torch.zeros(1, dtype=torch.int32, device=dev)
    positions = [torch.tensor([spec["context"] + j], dtype=torch.int32, device=dev)
                 for j in range(steps_per_run)]
    t0 = time.time()
    graphs = []
    if args.graph == "step":
        # the step's tokens back to back in one graph: token j reads ids[j],
        # its argmax writes ids[j + 1]
        ids = torch.zeros(steps_per_run + 1, dtype=torch.int32, device=dev)
        ids[0] = int(first[0])
        logits = torch.empty((1, spec["vocab"]), dtype=torch.float32, device=dev)
        graphs.append(dec.capture_decode(ids, positions, seq, logits, ids[1:]))
    else:
        dec.reserve(1)
        bufs = dec.step_buffers(1)
        ids = torch.tensor(first, dtype=torch.int32, device=dev)
        bufs["next"] = ids                     # argmax writes the next input token in place
        dec.step(ids, positions[0], seq, bufs)  # eager warm-up (first launches)
        torch.cuda.synchronize()
        for j in range(steps_per_run):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                dec.step(ids, positions[j], seq, bufs)
            graphs.append(gr)
    torch.cuda.synchronize()
    log(f"captured {len(graphs)} decode graph(s) for {steps_per_run} tokens in {time.time() - t0:.1f}s")

    def one_run():
        for gr in graphs:
            gr.replay()

    if args.graph != "step":
        ids.fill_(int(first[0]))
    for _ in range(args.warmup):
        one_run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        one_run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    tok_s = steps_per_run * args.steps / (ms / 1e3)
    log(f"decode: {ms_per_step:.3f} ms per {steps_per_run}-token step, {tok_s:.1f} tok/s")

    # -- the dominant kernel on its own: the fused RMSNorm + Q8_0 + gate/up +
    #    SwiGLU GEMV (the same kernel instance the decode step runs), once per
    #    layer in turn (the 22 layers' 286 MB exceed the 256 MB MALL),
    #    back-to-back in one captured graph; HIP events on the replay stream
    x = normal(7, 0, (1, g.hidden))
    xg = torch.from_numpy(x).to(dev)
    h = torch.empty((1, g.ffn_padded), dtype=torch.float32, device=dev)
    def ffn_ups():
        for lw in dec.layers:
            qk.qk_ffn_up(xg, lw.gamma_ffn, g.eps, lw.w_gate_up_q, lw.w_gate_up_d, out=h)
    ffn_ups()
    torch.cuda.synchronize()
    kg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(kg):
        ffn_ups()
    kg.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.kernel_rounds):
        kg.replay()
    b.record()
    torch.cuda.synchronize()
    avg_us = a.elapsed_time(b) * 1e3 / (args.kernel_rounds * L)
    H, F = g.hidden, g.ffn_padded
    # weights, Q4_0; x and gamma fp32 read; h fp32 written
    kbytes = 2 * F * H * 9 / 16 + 2 * H * 4 + F * 4
    achieved = kbytes / (avg_us * 1e-6) / 1e9
    kname = "k_gemv<1,4,1,EPI_SWIGLU,PRO_RMSNORM,1,false>"
    src = source_hash([os.path.join(ROOT, "quantized_q4_q8_amd", "csrc", f)
                       for f in ("gemv.hip", "qdot.h", "internal.h", "common.h")])
    traffic = stored_traffic(kname, src)
    log(f"fused gate/up GEMV: {avg_us:.2f} us per launch, {achieved:.0f} GB/s")

    # -- the matmul share of one token: the token's Q4_0 x Q8_0 products
    #    alone (per layer QKV, output projection, gate/up + SwiGLU and down,
    #    then the LM head), each a GEMV on a resident Q8_0 activation row,
    #    back to back in one captured graph
    Nq, Nqkv = g.n_q_heads * g.head_dim, g.n_qkv
    xq, xd = qk.quantize_q8_0(xg)
    hq, hdq = qk.quantize_q8_0(h)
    y_qkv = torch.empty((1, Nqkv), dtype=torch.float32, device=dev)
    y_h = torch.empty((1, H), dtype=torch.float32, device=dev)
    y_lm = torch.empty((1, spec["vocab"]), dtype=torch.float32, device=dev)
    def matmuls():
        for lw in dec.layers:
            qk.qmatmul_q4_0_q8_0(lw.w_qkv_q, lw.w_qkv_d, xq, xd, out=y_qkv)
            qk.qmatmul_q4_0_q8_0(lw.w_o_q, lw.w_o_d, xq, xd, out=y_h)
            qk.qk_gate_up_swiglu(lw.w_gate_up_q, lw.w_gate_up_d, xq, xd, out=h)
            qk.qmatmul_q4_0_q8_0(lw.w_down_q, lw.w_down_d, hq, hdq, out=y_h)
        qk.qmatmul_q4_0_q8_0(dec.lm_q, dec.lm_d, xq, xd, out=y_lm)
    mm_us = graph_time_us(matmuls, 1, args.kernel_rounds)
    mm_bytes = (L * (Nqkv * H + H * Nq + 2 * F * H + H * F) + spec["vocab"] * H) * 9 / 16 \
        + L * (3 * (H + H // 32 * 2) + F + F // 32 * 2) + H + H // 32 * 2
    mm_gbs = mm_bytes / (mm_us * 1e-6) / 1e9
    log(f"matmul step: {mm_us:.1f} us per token, {mm_gbs:.0f} GB/s")

    # -- the attention share of one token: the 22 layers' grouped-query
    #    attention (chunk and merge passes) over the resident caches at the
    #    workload's middle position
    mid = spec["context"] + steps_per_run // 2
    qa = torch.from_numpy(normal(8, 0, (1, g.n_q_heads, g.head_dim))).to(dev)
    pa = torch.tensor([mid], dtype=torch.int32, device=dev)
    oa = torch.empty_like(qa)
    wsa = torch.empty(qk.load().qk_gqa_attention_workspace(1, g.n_q_heads, g.head_dim, spec["cap"]),
                      dtype=torch.uint8, device=dev)
    def attentions():
        for li in range(L):
            qk.gqa_attention(qa, dec.k_cache[li], dec.v_cache[li], pa, seq, out=oa, ws=wsa)
    att_us = graph_time_us(attentions, 1, args.kernel_rounds)
    att_rows = min(mid + 1, spec["cap"])
    att_bytes = L * (2 * g.n_kv_heads * g.head_dim * 2 * att_rows + 2 * Nq * 4)
    att_gbs = att_bytes / (att_us * 1e-6) / 1e9
    log(f"attention step: {att_us:.1f} us per token ({att_us / L:.2f} us per layer), {att_gbs:.0f} GB/s")

    # -- a plain 256 MiB device copy: calibrates the HBM byte counters
    #    (FETCH_SIZE / WRITE_SIZE) of profiling runs against a known size
    cal_src = torch.empty(64 * 2**20, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    read_gbs = read_ceiling(dev)

    step_bytes = decode_bytes_per_token(spec)
    c0, c1 = spec["context"], spec["context"] + steps_per_run - 1
    if long_context:
        metric = f"decode tokens/s at TinyLLaMA-1.1B Q4_0 shape, {spec['cap']}-row ring KV cache"
        workload = (f"tinyllama-1.1b-shape greedy decode, 22 layers, positions {c0}->{c1} "
                    f"through an {spec['cap']}-row ring cache (every step attends {spec['cap']} positions)")
    else:
        metric = "decode tokens/s at TinyLLaMA-1.1B Q4_0 shape"
        workload = f"tinyllama-1.1b-shape greedy decode, 22 layers, context {c0}->{c1}"
    out = {
        "metric": metric,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 x q8_0 (int32 block dots, fp64 accumulate, fp32 activations)",
        "data": "synthetic: seeded N(0,0.02) Q4_0 weights, N(0,1) fp16 KV prefill",
        "config": {"workload": workload, "kv_cap": spec["cap"],
                   "tokens_per_step": steps_per_run, "batch": 1, "layers": L,
                   "hidden": g.hidden, "heads": [g.n_q_heads, g.n_kv_heads, g.head_dim],
                   "ffn": g.ffn, "vocab": spec["vocab"], "kv_cache": "fp16",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": int(kbytes),
                     "avg_us": round(avg_us, 3), "launches_timed": args.kernel_rounds * L,
                     "source_hash": src, "achievable_GBps": round(read_gbs, 1),
                     "frac_of_achievable": round(achieved / read_gbs, 4)},
        "mul_mat_step": {"what": "the token's Q4_0 x Q8_0 GEMVs alone (22 x QKV, output, gate/up, "
                                 "down, and the LM head), one graph",
                         "bytes": int(mm_bytes), "us": round(mm_us, 2), "GBps": round(mm_gbs, 1),
                         "frac": round(mm_gbs / HBM_PEAK_GBS, 4)},
        "attention_step": {"what": f"the token's 22 attention calls (chunk + merge) at position {mid}",
                           "bytes": int(att_bytes), "us": round(att_us, 2),
                           "us_per_layer": round(att_us / L, 3), "GBps": round(att_gbs, 1),
                           "frac": round(att_gbs / HBM_PEAK_GBS, 4)},
        "step_roofline": {"bytes_per_token": int(step_bytes),
                          "achieved_GBps": round(step_bytes * tok_s / 1e9, 1),
                          "frac": round(step_bytes * tok_s / 1e9 / HBM_PEAK_GBS, 4),
                          "roofline_tokens_per_s": round(HBM_PEAK_GBS * 1e9 / step_bytes, 1)},
    }
    if want_cpu:
        out["cpu_baseline"] = cpu_decode_baseline(spec, host, first, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_decode_baseline(spec, host, first, budget_s: float):
    """The oracle decoding tokens of the same workload on the host cores."""
    import numpy as np

    import oracle

    g, L = spec["geometry"], spec["layers"]
    cfg = g.cfg(spec["cap"])
    kv = [(k.copy(), v.copy()) for k, v in host["kv"]]
    tok = int(first[0])
    seq = np.zeros(1, np.int32)
    n, t_total = 0, 0.0
    while n < 64:
        p = np.array([spec["context"] + n], np.int32)
        t0 = time.perf_counter()
        x = oracle.embed_lookup(host["embed"], np.array([tok], np.int32))
        for li in range(L):
            x = oracle.layer_forward(host["layers"][li], cfg, x, p, seq, kv[li][0], kv[li][1])
        xn = oracle.rmsnorm(x, host["gamma_f"], g.eps)
        xq, xd = oracle.quantize_q8_0(xn)
        logits = oracle.qmatmul(host["lm_q"], host["lm_d"], xq, xd)
        tok = int(oracle.argmax(logits)[0])
        t_total += time.perf_counter() - t0
        n += 1
        if t_total >= budget_s:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    log(f"oracle: {n} tokens in {t_total:.1f}s on {threads} threads")
    return {"value": round(n / t_total, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} greedy decode tokens (positions {spec['context']}.."
                      f"{spec['context'] + n - 1}) of the same 22-layer workload, oracle in "
                      f"fp64/exact-int C++ with OpenMP"}


def graph_time_us(fn, launches: int, rounds: int, warm: int = 1) -> float:
    """Average µs per launch of `fn` (which makes `launches` launches),
    captured once in a graph, replayed `warm` times untimed and then `rounds`
    times timed; HIP events on the replay stream."""
    import torch

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(max(1, warm)):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(rounds):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (rounds * launches)


def base_line(args, metric, value, unit, ms_per_step, dtype, config):
    return {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic: seeded N(0,0.02) weights quantized to Q4_0, N(0,1) activations",
            "config": config}


# ---------------------------------------------------------------------------
# small layer: H 256, 8/2 heads of 32, F 688 (704), cap 32; a 16-token
# prefill call, then 16 one-token decode calls (positions 16..31)
# ---------------------------------------------------------------------------
def run_layer(args):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from quantized_q4_q8_amd.model import layer_to_device
    from synth import normal
    from synth import workloads as W

    spec = W.LAYER_SMALL
    g, P, D, cap = spec["geometry"], spec["prompt"], spec["decode"], spec["cap"]
    dev = torch.device("cuda")
    wf = W.layer_weights_f32(spec["seed"], 0, g)
    lw = layer_to_device(wf)
    cfg = qk.layer_cfg(**g.cfg(cap))
    kshape = (1, g.n_kv_heads, cap, g.head_dim)
    kc = torch.zeros(kshape, dtype=torch.int16, device=dev)
    vc = torch.zeros(kshape, dtype=torch.int16, device=dev)
    x0 = normal(spec["seed"], 10, (P, g.hidden))
    xp = torch.from_numpy(x0).to(dev)
    xd = torch.from_numpy(x0[-1:].copy()).to(dev)
    seq_p = torch.zeros(P, dtype=torch.int32, device=dev)
    seq_d = torch.zeros(1, dtype=torch.int32, device=dev)
    pos_p = torch.arange(P, dtype=torch.int32, device=dev)
    pos_d = [torch.tensor([P + j], dtype=torch.int32, device=dev) for j in range(D)]
    ws = torch.empty(qk.qk_layer_workspace(cfg, P), dtype=torch.uint8, device=dev)
    rounds = max(20, args.kernel_rounds)
    pre_us = graph_time_us(lambda: qk.layer_forward(lw, cfg, xp, pos_p, seq_p, kc, vc, ws=ws), 1, rounds)
    dec_us = graph_time_us(lambda: [qk.layer_forward(lw, cfg, xd, p, seq_d, kc, vc, ws=ws) for p in pos_d],
                           D, rounds)
    log(f"layer: prefill call ({P} tokens) {pre_us:.2f} us, decode call {dec_us:.2f} us")
    H, F, Nq = g.hidden, g.ffn_padded, g.n_q_heads * g.head_dim
    wbytes = (g.n_qkv * H + H * Nq + 2 * F * H + H * F) * 9 / 16 + 2 * H * 4
    mid = P + D // 2
    dbytes = wbytes + 2 * g.n_kv_heads * g.head_dim * 2 * (mid + 1) + 2 * H * 4
    gbs = dbytes / (dec_us * 1e-6) / 1e9
    out = base_line(args, "decode layer calls/s, small layer (H 256, 8/2 heads of 32, F 704)",
                    1e6 / dec_us, "calls/s", dec_us / 1e3, "q4_0 x q8_0 (int32 block dots, fp64 accumulate, fp32 activations)",
                    {"workload": f"one pre-norm layer, H {H}, heads 8/2 x 32, F {F}, cap {cap}: a {P}-token "
                                 f"prefill call, then {D} one-token decode calls (positions {P}..{P + D - 1})",
                     "parallelism": "single GPU"})
    out["data"] = "synthetic: seeded N(0,0.02) Q4_0 weights, N(0,1) activations"
    out["prefill_call_us"] = round(pre_us, 2)
    out["roofline"] = {"bound": "hbm", "kernel": "layer_forward, one decode call (six launches)",
                       "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None,
                       "bytes_per_launch": int(dbytes), "avg_us": round(dec_us, 3),
                       "note": "latency-bound: 0.4 MB per call is far below one launch's worth of HBM time"}
    if not args.no_cpu_baseline:
        import oracle
        wl = {}
        for name, key in [("w_qkv", "w_qkv"), ("w_o", "w_o"), ("w_gate_up", "w_gu"), ("w_down", "w_down")]:
            wl[key + "_q"], wl[key + "_d"] = oracle.quantize_q4_0(wf[name])
        wl["gamma_attn"], wl["gamma_ffn"] = wf["gamma_attn"], wf["gamma_ffn"]
        kh = np.zeros(kshape, np.uint16)
        vh = np.zeros(kshape, np.uint16)
        xo = oracle.layer_forward(wl, g.cfg(cap), x0, np.arange(P, dtype=np.int32), np.zeros(P, np.int32), kh, vh)
        t0, n = time.perf_counter(), 0
        xr = xo[-1:]
        while n < D and (time.perf_counter() - t0 < args.cpu_seconds or n == 0):
            xr = oracle.layer_forward(wl, g.cfg(cap), xr, np.array([P + n], np.int32), np.zeros(1, np.int32), kh, vh)
            n += 1
        dt = (time.perf_counter() - t0) / n
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        out["cpu_baseline"] = {"value": round(1.0 / dt, 2), "unit": "calls/s", "cores": threads,
                               "kind": "oracle", "sample": f"{n} oracle decode calls of the same layer "
                                                           f"(positions {P}..{P + n - 1})"}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# standalone matmul workload: W 5632x2048 and 2048x5632, batch 1 and 8
# ---------------------------------------------------------------------------
def run_matmul(args):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from quantized_q4_q8_amd.model import to_device
    from synth import workloads as W

    spec = W.MATMUL
    rows = []
    dev = torch.device("cuda")
    bits = {"q4_0": 0, "int4row": 4, "int2row": 2}[args.codec]
    for idx, (n, k) in enumerate(spec["shapes"]):
        wf = to_device(W.matmul_weight_f32(spec["seed"], idx, n, k))
        if bits:   # row-scaled: codes [n][k bits / 8] and fp32 scales [n]
            wq, wd = qk.qk_quantize_rowq(wf, bits)
            wbytes = n * k * bits // 8 + n * 4
            mm = lambda a, b, xq, xd, out: qk.qk_qmatmul_rowq_q8_0(a, b, xq, xd, bits, out=out)  # noqa: E731
        else:
            wq, wd = qk.qk_quantize_q4_0(wf)
            wbytes = n * k * 9 // 16
            mm = qk.qmatmul_q4_0_q8_0
        del wf
        # distinct copies filling 1 GiB, so that a launch cannot hit the 256 MB
        # memory-side cache left warm by the previous one
        copies = -(-(1 << 30) // wbytes)
        wq_all = wq.unsqueeze(0).repeat(copies, *([1] * wq.dim()))
        wd_all = wd.unsqueeze(0).repeat(copies, *([1] * wd.dim()))
        for m in spec["batches"]:
            xq, xd = qk.quantize_q8_0(to_device(W.matmul_input_f32(spec["seed"], idx, m, k)))
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            nbytes = wbytes + m * k * 34 // 32 + m * n * 4
            cold = graph_time_us(lambda: [mm(wq_all[c], wd_all[c], xq, xd, out=y)
                                          for c in range(copies)], copies, max(2, args.steps))
            hot = graph_time_us(lambda: [mm(wq, wd, xq, xd, out=y)
                                         for _ in range(copies)], copies, max(2, args.steps))
            rec = {"n": n, "k": k, "m": m, "bytes_per_launch": nbytes,
                   "cold_us": round(cold, 3), "cold_GBps": round(nbytes / cold / 1e3, 1),
                   "hot_us": round(hot, 3), "hot_GBps": round(nbytes / hot / 1e3, 1),
                   "int_ops_per_launch": 2 * m * n * k,
                   "cold_TOPs": round(2 * m * n * k / cold / 1e6, 3)}
            log(f"matmul {n}x{k} m={m}: cold {cold:.2f} us {rec['cold_GBps']} GB/s, hot {hot:.2f} us")
            rows.append(rec)
        del wq_all, wd_all
        torch.cuda.empty_cache()
    head = rows[0]
    wname = {"q4_0": "Q4_0", "int4row": "row-scaled int4", "int2row": "row-scaled int2"}[args.codec]
    out = base_line(args, f"{wname} x Q8_0 GEMV GB/s, W 5632x2048 x x[2048], cold memory-side cache",
                    head["cold_GBps"], "GB/s", head["cold_us"] / 1e3,
                    f"{args.codec} x q8_0 (int32 block dots, fp64 accumulate)",
                    {"workload": "standalone matmul: W 5632x2048 and 2048x5632, batch 1 and 8",
                     "codec": args.codec,
                     "copies": "1 GiB of distinct weight copies rotated per launch",
                     "parallelism": "single GPU"})
    if bits:
        out["data"] = f"synthetic: seeded N(0,0.02) weights quantized to row-scaled int{bits}, N(0,1) activations"
    out["roofline"] = {"bound": "hbm", "kernel": "k_gemv_rowq (M=1, store epilogue)" if bits else "k_gemv (M=1, store epilogue)",
                       "achieved": head["cold_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(head["cold_GBps"] / HBM_PEAK_GBS, 4), "traffic": None,
                       "bytes_per_launch": head["bytes_per_launch"], "avg_us": head["cold_us"]}
    read_gbs = read_ceiling(dev)
    out["roofline"]["achievable_GBps"] = round(read_gbs, 1)
    out["roofline"]["frac_of_achievable"] = round(head["cold_GBps"] / read_gbs, 4)
    out["shapes"] = rows
    if not args.no_cpu_baseline:
        import oracle
        w = W.matmul_weight_f32(spec["seed"], 0, 5632, 2048)
        xq, xd = oracle.quantize_q8_0(W.matmul_input_f32(spec["seed"], 0, 1, 2048))
        if bits:
            owq, owr = oracle.quantize_rowq(w, bits)
            omm = lambda: oracle.qmatmul_rowq(owq, owr, xq, xd, bits)  # noqa: E731
        else:
            owq, owd = oracle.quantize_q4_0(w)
            omm = lambda: oracle.qmatmul(owq, owd, xq, xd)  # noqa: E731
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0) or n == 0:
            omm()
            n += 1
        dt = (time.perf_counter() - t0) / n
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        out["cpu_baseline"] = {"value": round(head["bytes_per_launch"] / dt / 1e9, 3), "unit": "GB/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{n} oracle GEMVs of W 5632x2048 x x[2048]"}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# prefill workload: 4 x 512 tokens through the 22-layer model, full logits
# ---------------------------------------------------------------------------
def run_prefill(args):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from synth import randint
    from synth import workloads as W

    spec = W.PREFILL
    g, L, B, P, V = spec["geometry"], spec["layers"], spec["batch"], spec["prompt"], spec["vocab"]
    T = B * P
    want_cpu = not args.no_cpu_baseline
    dec, _, host = build_decoder(spec, want_cpu, seqs=B)
    dev = dec.device
    ids_h = randint(spec["seed"], W.TID_TOKENS, (B, P), V)
    ids = torch.from_numpy(ids_h.reshape(-1).astype(np.int32)).to(dev)
    pos = torch.from_numpy(np.tile(np.arange(P, dtype=np.int32), B)).to(dev)
    seq = torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), P)).to(dev)
    dec.reserve(T)
    bufs = dec.step_buffers(T)
    for _ in range(max(1, args.warmup)):
        dec.step(ids, pos, seq, bufs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dec.step(ids, pos, seq, bufs)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    tok_s = T / (ms / 1e3)
    H, F, Nqkv = g.hidden, g.ffn_padded, g.n_qkv
    lin_macs = L * T * H * (Nqkv + g.n_q_heads * g.head_dim + 2 * F) + L * T * F * H + T * V * H
    log(f"prefill: {ms:.3f} ms per {T}-token step, {tok_s:.0f} tok/s, "
        f"{2 * lin_macs / (ms / 1e3) / 1e12:.1f} TOP/s over the step")

    # the dominant GEMM alone: gate/up + SwiGLU, M = 2048, N = 2 x 5632, K = 2048
    xq, xd = qk.quantize_q8_0(torch.randn((T, H), device=dev))
    h = torch.empty((T, F), dtype=torch.float32, device=dev)
    rounds = max(2, args.kernel_rounds // 4)
    us = graph_time_us(lambda: [qk.qk_gate_up_swiglu(lw.w_gate_up_q, lw.w_gate_up_d, xq, xd, out=h)
                                for lw in dec.layers], L, rounds)
    ops = 2 * T * 2 * F * H
    tops = ops / us / 1e6
    log(f"gate/up GEMM M={T}: {us:.1f} us, {tops:.0f} TOP/s")
    out = base_line(args, "prefill tokens/s at TinyLLaMA-1.1B Q4_0 shape (4 x 512, full logits)",
                    tok_s, "tokens/s", ms, "q4_0 x q8_0 int8 MFMA (int32 block dots, fp64 accumulate)",
                    {"workload": "tinyllama-1.1b-shape causal prefill, batch 4 x 512, 22 layers, full logits",
                     "tokens_per_step": T, "layers": L, "parallelism": "single GPU"})
    out["roofline"] = {"bound": "mfma", "kernel": "k_gemm_mfma<EPI_SWIGLU> (gate/up, M=2048)",
                       "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                       "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": None,
                       "ops_per_launch": ops, "avg_us": round(us, 2)}
    gsrc = source_hash([os.path.join(ROOT, "quantized_q4_q8_amd", "csrc", f) for f in ("gemm.hip", "common.h")])
    out["roofline"]["counters"] = stored_counters("k_gemm_mfma<EPI_SWIGLU>", gsrc)
    out["gemm_counters"] = {"what": "per-SIMD busy fractions from rocprofv3 counters (MFMA busy at 1.0 = "
                                    "the int8 peak), null when the GEMM source changed since",
                            "gate_up": out["roofline"]["counters"],
                            "qkv_o_down_lm": stored_counters("k_gemm_mfma<EPI_STORE>", gsrc)}
    out["step_roofline"] = {"int_ops_per_step": 2 * lin_macs,
                            "achieved_TOPs": round(2 * lin_macs / (ms / 1e3) / 1e12, 1),
                            "frac": round(2 * lin_macs / (ms / 1e3) / 1e12 / INT8_PEAK_TOPS, 4)}
    if want_cpu:
        import oracle
        cfg = g.cfg(spec["cap"])
        n = 8
        kv = [(np.zeros((1, g.n_kv_heads, spec["cap"], g.head_dim), np.uint16),
               np.zeros((1, g.n_kv_heads, spec["cap"], g.head_dim), np.uint16)) for _ in range(L)]
        t0 = time.perf_counter()
        x = oracle.embed_lookup(host["embed"], ids_h[0, :n].astype(np.int32))
        p = np.arange(n, dtype=np.int32)
        s0 = np.zeros(n, np.int32)
        for li in range(L):
            x = oracle.layer_forward(host["layers"][li], cfg, x, p, s0, kv[li][0], kv[li][1])
        xq_o, xd_o = oracle.quantize_q8_0(oracle.rmsnorm(x, host["gamma_f"], g.eps))
        oracle.qmatmul(host["lm_q"], host["lm_d"], xq_o, xd_o)
        dt = time.perf_counter() - t0
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        out["cpu_baseline"] = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"prefill of the first {n} tokens of sequence 0 with full logits"}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# MoE workload: 256 resident experts, 64 tokens, top-8
# ---------------------------------------------------------------------------
def run_moe(args):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from quantized_q4_q8_amd.model import to_device
    from synth import normal
    from synth import workloads as W

    spec = W.MOE
    seed, T, H, E, F, k = spec["seed"], spec["tokens"], spec["hidden"], spec["experts"], spec["ffn"], spec["top_k"]
    dev = torch.device("cuda")
    bits = {"q4_0": 0, "int4row": 4, "int2row": 2}[args.codec]
    t0 = time.time()
    if bits:   # row-scaled experts: codes and one fp32 scale per row
        guq = torch.empty((E, 2 * F, H * bits // 8), dtype=torch.uint8, device=dev)
        gud = torch.empty((E, 2 * F), dtype=torch.float32, device=dev)
        dnq = torch.empty((E, H, F * bits // 8), dtype=torch.uint8, device=dev)
        dnd = torch.empty((E, H), dtype=torch.float32, device=dev)
        quant = lambda w, q, d: qk.qk_quantize_rowq(w, bits, out_q=q, out_r=d)  # noqa: E731
        per_expert = 2 * F * (H * bits // 8 + 4) + H * (F * bits // 8 + 4)
    else:
        guq = torch.empty((E, 2 * F, H // 2), dtype=torch.uint8, device=dev)
        gud = torch.empty((E, 2 * F, H // 32), dtype=torch.int16, device=dev)
        dnq = torch.empty((E, H, F // 2), dtype=torch.uint8, device=dev)
        dnd = torch.empty((E, H, F // 32), dtype=torch.int16, device=dev)
        quant = lambda w, q, d: qk.qk_quantize_q4_0(w, out_q=q, out_d=d)  # noqa: E731
        per_expert = 3 * F * H * 9 // 16
    for e in range(E):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        quant(to_device(gu), guq[e], gud[e])
        quant(to_device(dn), dnq[e], dnd[e])
    torch.cuda.synchronize()
    log(f"{E} experts resident after {time.time() - t0:.1f}s")
    x = to_device(normal(seed, W.TID_X, (T, H)))
    wr = to_device(normal(seed, W.TID_ROUTER, (H, E), W.WEIGHT_STD))
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    sel = torch.empty((T, k), dtype=torch.int32, device=dev)
    sw = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws = torch.empty(qk.qk_moe_workspace(T, H, E, k, F), dtype=torch.uint8, device=dev)
    if bits:
        call = lambda: qk.qk_moe_route_and_apply_rowq(x, wr, k, guq, gud, dnq, dnd, bits, out=y,  # noqa: E731
                                                      sel_idx=sel, sel_w=sw, ws=ws)
    else:
        call = lambda: qk.moe_route_and_apply(x, wr, k, guq, gud, dnq, dnd, out=y, sel_idx=sel,  # noqa: E731
                                              sel_w=sw, ws=ws)
    call()
    torch.cuda.synchronize()
    distinct = int(torch.unique(sel).numel())
    # A layer takes about 1 ms: a few replays would time the clocks settling
    # under the sustained load as much as the layer, so the line times 20 (or
    # --steps) after 10 (or --warmup) untimed ones.
    us = graph_time_us(call, 1, max(20, args.steps), warm=max(10, args.warmup))
    nbytes = distinct * per_expert + H * E * 4 + 2 * T * H * 4
    gbs = nbytes / us / 1e3
    log(f"moe ({args.codec}): {us:.1f} us per layer, {distinct} distinct experts of {per_expert} B, "
        f"{gbs:.0f} GB/s")
    wname = {"q4_0": "Q4_0", "int4row": "row-scaled int4", "int2row": "row-scaled int2"}[args.codec]
    out = base_line(args, f"MoE layer GB/s (256 resident {wname} experts, 64 tokens, top-8)", gbs, "GB/s",
                    us / 1e3, f"{args.codec} x q8_0 (int32 block dots, fp64 accumulate); fp64 router",
                    {"workload": "moe layer: hidden 6144, 256 experts x SwiGLU 2048, 64 tokens, top-8",
                     "codec": args.codec, "bytes_per_expert": per_expert,
                     "distinct_experts": distinct, "parallelism": "single GPU"})
    if bits:
        out["data"] = f"synthetic: seeded N(0,0.02) weights quantized to row-scaled int{bits}, N(0,1) activations"
    out["us_per_layer"] = round(us, 2)
    out["roofline"] = {"bound": "hbm", "kernel": "whole MoE layer (router, top-k, grouping, grouped GEMVs, combine)",
                       "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": nbytes,
                       "avg_us": round(us, 2)}
    read_gbs = read_ceiling(dev)
    out["roofline"]["achievable_GBps"] = round(read_gbs, 1)
    out["roofline"]["frac_of_achievable"] = round(gbs / read_gbs, 4)
    if not args.no_cpu_baseline:
        import oracle
        xs = normal(seed, W.TID_X, (T, H))[:1]
        wrh = normal(seed, W.TID_ROUTER, (H, E), W.WEIGHT_STD)
        experts = []
        sel_o, w_o = oracle.moe_route(xs, wrh, k)
        for r in range(k):
            gu, dn = W.expert_weights_f32(seed, int(sel_o[0, r]), H, F)
            if bits:
                experts.append(oracle.quantize_rowq(gu, bits) + oracle.quantize_rowq(dn, bits))
            else:
                experts.append(oracle.quantize_q4_0(gu) + oracle.quantize_q4_0(dn))

        def expert_ffn(x1, gq, gs, dq, ds):
            if not bits:
                return oracle.moe_expert_ffn(x1, gq, gs, dq, ds)
            xq, xd = oracle.quantize_q8_0(x1[None])
            gu = oracle.qmatmul_rowq(gq, gs, xq, xd, bits)[0]
            hq, hd = oracle.quantize_q8_0(oracle.swiglu(gu[:F], gu[F:])[None])
            return oracle.qmatmul_rowq(dq, ds, hq, hd, bits)[0]

        t1 = time.perf_counter()
        sel_o, w_o = oracle.moe_route(xs, wrh, k)
        acc = np.zeros(H)
        for r in range(k):
            acc += w_o[0, r] * expert_ffn(xs[0], *experts[r])
        dt = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        out["cpu_baseline"] = {"value": round(8 * per_expert / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
                               "kind": "oracle", "sample": "one token through its 8 experts (oracle)"}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# sampler chain over the LM-head logits (vocab 32000): top-k 40, top-p 0.9,
# temperature 0.7, one uniform per row
# ---------------------------------------------------------------------------
def run_sample(args):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from synth import normal, randint

    V, L = 32000, 22
    dev = torch.device("cuda")
    rows_out = []
    for rows in (1, 8):
        lg = [torch.from_numpy(normal(5, 200 + i, (rows, V)) * np.float32(2.5)).to(dev) for i in range(L)]
        u = torch.from_numpy((randint(5, 300, rows, 1 << 30).astype(np.float64) + 0.5) / (1 << 30)).to(dev)
        ids = torch.empty(rows, dtype=torch.int32, device=dev)
        us = graph_time_us(lambda: [qk.qk_sample(x, 40, 0.9, 0.7, u, out=ids) for x in lg], L,
                           max(5, args.steps))
        nbytes = rows * V * 4
        rows_out.append({"rows": rows, "us_per_call": round(us, 3), "GBps": round(nbytes / us / 1e3, 1)})
        log(f"sample rows={rows}: {us:.2f} us per call")
    head = rows_out[0]
    out = base_line(args, "sampler calls/s (32000 logits, top-k 40, top-p 0.9, temperature 0.7)",
                    1e6 / head["us_per_call"], "calls/s", head["us_per_call"] / 1e3,
                    "fp32 logits, fp64 weights and sums",
                    {"workload": "sampler chain over one 32000-logit row (and 8 rows)",
                     "parallelism": "single GPU"})
    out["roofline"] = {"bound": "hbm", "kernel": "k_sample", "achieved": head["GBps"],
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(head["GBps"] / HBM_PEAK_GBS, 5),
                       "traffic": None, "bytes_per_launch": V * 4, "avg_us": head["us_per_call"]}
    out["rows"] = rows_out
    out["data"] = "synthetic: seeded N(0,1) x 2.5 logits, seeded uniforms"
    if not args.no_cpu_baseline:
        import oracle
        x = normal(5, 200, (1, V)) * np.float32(2.5)
        uh = (randint(5, 300, 1, 1 << 30).astype(np.float64) + 0.5) / (1 << 30)
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or n == 0:
            oracle.sample(x, 40, 0.9, 0.7, uh)
            n += 1
        dt = (time.perf_counter() - t0) / n
        out["cpu_baseline"] = {"value": round(1.0 / dt, 2), "unit": "calls/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} oracle sampler calls on one 32000-logit row (single-threaded)"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for {max(args.gpus, world)} GPUs).", flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        sys.exit(1)
    import quantized_q4_q8_amd as qk
    qk.load()
    {"decode": run_decode, "longctx": lambda a: run_decode(a, long_context=True),
     "longctx32k": lambda a: run_decode(a, long_context="32k"), "layer": run_layer, "matmul": run_matmul, "prefill": run_prefill, "moe": run_moe, "sample": run_sample}[args.workload](args)


if __name__ == "__main__":
    main()
