"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host
code, g++) and driven through every entry point on small edge-case inputs:
ragged multi-sequence prefill, decode past a wrapping ring cache, grouped
and plain multi-head attention, both row-scaled codecs, the sampler's
top-k / top-p / temperature edges and an all-equal logit row.  The driver
runs in a child process with the sanitizer runtimes preloaded; any report
ends it with a non-zero status.

Run as a script (``python test_oracle_sanitized.py <lib>``) it is that driver.
"""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    """Path of a g++ sanitizer runtime, or None."""
    gxx = shutil.which("g++")
    if not gxx:
        return None
    p = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("g++ sanitizer runtimes not available")
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fopenmp", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", so], check=True)
    env = dict(os.environ)
    # the sanitizer runtimes first (ASan requires it), anything preloaded already after them
    env["LD_PRELOAD"] = ":".join([asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, os.path.abspath(__file__), so], env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "all entry points ran" in r.stdout, (r.stdout[-2000:] + r.stderr[-4000:])


# --------------------------------------------------------------------------
# the driver
# --------------------------------------------------------------------------
def _quantized_layer(oracle, wf):
    out = {}
    for name, key in [("w_qkv", "w_qkv"), ("w_o", "w_o"), ("w_gate_up", "w_gu"), ("w_down", "w_down")]:
        out[key + "_q"], out[key + "_d"] = oracle.quantize_q4_0(wf[name])
    out["gamma_attn"] = wf["gamma_attn"]
    out["gamma_ffn"] = wf["gamma_ffn"]
    return out


def _drive(so):
    sys.path.insert(0, ROOT)
    import oracle
    from synth import normal
    from synth import workloads as W

    oracle._SO = so
    oracle.build = lambda: None   # keep the sanitized build
    rng = np.random.default_rng(0)

    # layers: GQA (4 q / 2 kv heads), the small-layer shape, plain multi-head
    for g, cap in [(W.Geometry(128, 4, 2, 32, 96), 40), (W.Geometry(256, 8, 2, 32, 688), 100),
                   (W.Geometry(128, 2, 2, 64, 64), 64)]:
        wl = _quantized_layer(oracle, W.layer_weights_f32(7, 0, g))
        kc = np.zeros((3, g.n_kv_heads, cap, g.head_dim), np.uint16)
        vc = kc.copy()
        x = normal(7, 900, (9, g.hidden))   # three ragged prefills in one call
        pos = np.array([0, 1, 2, 0, 1, 2, 0, 1, 2], np.int32)
        seq = np.array([0, 0, 0, 1, 1, 1, 2, 2, 2], np.int32)
        oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
        for p in [3, cap - 1, cap, cap + 5, 2 * cap + 3]:   # decode, through the ring's wrap
            x1 = normal(7, 901 + p, (3, g.hidden))
            y = oracle.layer_forward(wl, g.cfg(cap), x1, np.array([p, p, p + 1], np.int32),
                                     np.array([0, 1, 2], np.int32), kc, vc)
            assert np.isfinite(y).all()
        q = normal(7, 5, (4, g.n_q_heads, g.head_dim))
        o = oracle.gqa_attention(q, kc, vc, np.array([0, cap - 1, cap + 7, 1], np.int32),
                                 np.array([0, 1, 2, 0], np.int32))
        assert np.isfinite(o).all()

    # matmuls and quantizers, K from one block to the decode down projection
    for n, k in [(1, 32), (7, 64), (33, 5632), (5, 96)]:
        w = normal(1, 2, (n, k))
        xq, xd = oracle.quantize_q8_0(normal(1, 3, (3, k)))
        wq, wd = oracle.quantize_q4_0(w)
        oracle.qmatmul(wq, wd, xq, xd)
        oracle.block_dots(wq, k, xq)
        for bits in (2, 4):
            rq, rr = oracle.quantize_rowq(w, bits)
            oracle.qmatmul_rowq(rq, rr, xq, xd, bits)
    zero = np.zeros((2, 64), np.float32)   # all-zero blocks: zero scales
    oracle.quantize_q8_0(zero)
    oracle.quantize_q4_0(zero)
    oracle.rmsnorm(normal(1, 4, (3, 64)), normal(1, 5, (64,)), 1e-5)
    oracle.rope(normal(1, 6, (3, 2, 32)), np.array([0, 5, 100000], np.int32), 10000.0)
    oracle.swiglu(normal(1, 7, (3, 40)), normal(1, 8, (3, 40)))
    oracle.embed_lookup(normal(1, 9, (50, 64)), np.array([0, 49, 7], np.int32))

    # argmax and the sampler chain, one row of equal logits among them
    lg = normal(1, 10, (4, 517))
    lg[1, :] = 3.0
    oracle.argmax(lg)
    for top_k, top_p, temp in [(1, 0.9, 0.7), (40, 0.9, 0.7), (517, 1.0, 1.0), (13, 0.5, 1.7),
                               (40, 0.9, 0.0), (600, 0.95, 1.3)]:
        oracle.sample(lg, top_k, top_p, temp, rng.random(4))

    # MoE: routing, one expert's FFN, the layer with Q4_0 and row-scaled experts
    H, E, F, T = 256, 16, 64, 9
    xr, wr = normal(2, 1, (T, H)), normal(2, 2, (H, E))
    gus, dns = zip(*[W.expert_weights_f32(2, e, H, F) for e in range(E)])
    gq = [oracle.quantize_q4_0(a) for a in gus]
    dq = [oracle.quantize_q4_0(a) for a in dns]
    oracle.moe_route_and_apply(xr, wr, 4, np.stack([a for a, _ in gq]), np.stack([b for _, b in gq]),
                               np.stack([a for a, _ in dq]), np.stack([b for _, b in dq]))
    oracle.moe_route(xr, wr, E, return_logits=True)   # top-k = every expert
    oracle.moe_expert_ffn(xr[0], gq[0][0], gq[0][1], dq[0][0], dq[0][1])
    for bits in (2, 4):
        gr = [oracle.quantize_rowq(a, bits) for a in gus]
        dr = [oracle.quantize_rowq(a, bits) for a in dns]
        oracle.moe_route_and_apply_rowq(xr, wr, 8, np.stack([a for a, _ in gr]), np.stack([b for _, b in gr]),
                                        np.stack([a for a, _ in dr]), np.stack([b for _, b in dr]), bits)
    print("all entry points ran")


if __name__ == "__main__":
    _drive(sys.argv[1])
