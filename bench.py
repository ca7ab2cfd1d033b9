#!/usr/bin/env python3
"""Throughput benchmark of the Q4_0 x Q8_0 decoder path on one MI355X.

Default workload: TinyLLaMA-1.1B-shaped greedy decode (22 layers, hidden
2048, 32 query / 4 KV heads of 64, SwiGLU 5632, vocab 32000, Q4_0 weights
from N(0, 0.02), fp16 KV cache prefilled with N(0, 1) to context 2048).  One
step is the workload's full 128-token greedy decode (positions 2048..2175):
per token embedding, 22 decoder layers, final RMSNorm, LM head and argmax.
Each token's kernels are captured once in a HIP graph and replayed; inputs
are resident in HBM before timing starts.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="decode", choices=["decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--kernel-rounds", type=int, default=20)
    ap.add_argument("--decode-tokens", type=int, default=128,
                    help="tokens per step; only for short profiling runs (the workload is 128)")
    return ap.parse_args()


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
def build_decoder(spec, want_host_q4: bool):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from quantized_q4_q8_amd.model import Decoder, DecoderShape, layer_to_device, to_device
    from synth import normal, randint
    from synth import workloads as W

    g, seed, L, V, cap = spec["geometry"], spec["seed"], spec["layers"], spec["vocab"], spec["cap"]
    ctx = spec["context"]
    host = {"layers": [], "kv": []} if want_host_q4 else None
    if want_host_q4:
        import oracle
    layers = []
    kshape = (L, 1, g.n_kv_heads, cap, g.head_dim)
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
                         g.rope_base, L, V, cap, 1)
    dec = Decoder(shape, layers, to_device(embed), to_device(gamma_f), lm_q, lm_d)
    for li in range(L):
        kc, vc = W.kv_prefill_f16(seed, li, g.n_kv_heads, cap, g.head_dim, ctx)
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
    mean_ctx = spec["context"] + (spec["steps"] - 1) / 2 + 1       # rows read per layer
    kv = L * 2 * g.n_kv_heads * g.head_dim * 2 * mean_ctx
    norms = (2 * L + 1) * H * 4
    return lin * q4 + kv + norms + H * 4


def run_decode(args):
    import numpy as np
    import torch

    import quantized_q4_q8_amd as qk
    from synth import normal
    from synth import workloads as W

    spec = W.DECODE
    g, L = spec["geometry"], spec["layers"]
    steps_per_run = max(1, min(args.decode_tokens, spec["steps"]))
    want_cpu = not args.no_cpu_baseline
    dec, first, host = build_decoder(spec, want_cpu)
    dev = dec.device

    # -- one HIP graph per decode position (positions 2048 .. 2175)
    dec.reserve(1)
    bufs = dec.step_buffers(1)
    ids = torch.tensor(first, dtype=torch.int32, device=dev)
    bufs["next"] = ids                         # argmax writes the next input token in place
    seq = torch.zeros(1, dtype=torch.int32, device=dev)
    positions = [torch.tensor([spec["context"] + j], dtype=torch.int32, device=dev)
                 for j in range(steps_per_run)]
    dec.step(ids, positions[0], seq, bufs)     # eager warm-up (first launches)
    torch.cuda.synchronize()
    t0 = time.time()
    graphs = []
    for j in range(steps_per_run):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            dec.step(ids, positions[j], seq, bufs)
        graphs.append(gr)
    torch.cuda.synchronize()
    log(f"captured {len(graphs)} decode graphs in {time.time() - t0:.1f}s")

    def one_run():
        for gr in graphs:
            gr.replay()

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
    kname = "k_gemv<1,64,4,1,EPI_SWIGLU,PRO_RMSNORM,1>"
    src = source_hash([os.path.join(ROOT, "quantized_q4_q8_amd", "csrc", f)
                       for f in ("gemv.hip", "internal.h", "common.h")])
    traffic = stored_traffic(kname, src)
    log(f"fused gate/up GEMV: {avg_us:.2f} us per launch, {achieved:.0f} GB/s")

    # -- a plain 256 MiB device copy: calibrates the HBM byte counters
    #    (FETCH_SIZE / WRITE_SIZE) of profiling runs against a known size
    cal_src = torch.empty(64 * 2**20, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    step_bytes = decode_bytes_per_token(spec)
    out = {
        "metric": "decode tokens/s at TinyLLaMA-1.1B Q4_0 shape",
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
        "config": {"workload": "tinyllama-1.1b-shape greedy decode, 22 layers, context 2048->2175",
                   "tokens_per_step": steps_per_run, "batch": 1, "layers": L,
                   "hidden": g.hidden, "heads": [g.n_q_heads, g.n_kv_heads, g.head_dim],
                   "ffn": g.ffn, "vocab": spec["vocab"], "kv_cache": "fp16",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": int(kbytes),
                     "avg_us": round(avg_us, 3), "launches_timed": args.kernel_rounds * L,
                     "source_hash": src},
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
            "sample": f"{n} greedy decode tokens (positions 2048..{2047 + n}) of the same "
                      f"22-layer workload, oracle in fp64/exact-int C++ with OpenMP"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for {max(args.gpus, world)} GPUs).", flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        sys.exit(1)
    import quantized_q4_q8_amd as qk
    qk.load()
    if args.workload == "decode":
        run_decode(args)


if __name__ == "__main__":
    main()
