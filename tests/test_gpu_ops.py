"""GPU parity of each libqk entry point against the CPU oracle, through the
C-ABI binding.  Integer and byte outputs are compared bit for bit; fp32
outputs with the relative error of tests/util.py."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
from tests.util import LAYER_TOL, assert_same_fp32, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- quantizers
Q8_SHAPES = [(1, 32), (3, 2048), (5, 5632), (64, 6144), (17, 704), (2, 256)]


@pytest.mark.parametrize("rows,k", Q8_SHAPES)
def test_quantize_q8_0_bit_exact(gpu_lib, rows, k):
    qk = gpu_lib
    say(f"quantize_q8_0 rows={rows} k={k}")
    x = synth.normal(100, rows * 7 + k, (rows, k))
    q, d = qk.quantize_q8_0(dev(x))
    oq, od = oracle.quantize_q8_0(x)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(d, np.uint16), od)


def test_quantize_q8_0_edge_values(gpu_lib):
    qk = gpu_lib
    say("quantize_q8_0 edge values")
    blocks = []
    b = np.zeros(32, np.float32); blocks.append(b)                       # all zero
    b = np.zeros(32, np.float32); b[0] = 127; b[1:9] = [2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -0.0]
    blocks.append(b)                                                      # ties
    blocks.append(np.full(32, 1e-40, np.float32))                         # subnormal inputs
    b = synth.normal(101, 1, 32) * np.float32(1e-6); blocks.append(b)     # fp16-subnormal scale
    b = synth.normal(101, 2, 32) * np.float32(1e-9); blocks.append(b)     # scale underflows fp16
    b = synth.normal(101, 3, 32) * np.float32(1e7); blocks.append(b)      # scale overflows fp16
    b = np.arange(32, dtype=np.float32) - 15.5; blocks.append(b)
    b = np.zeros(32, np.float32); b[31] = -3.0; blocks.append(b)
    # every x/d that lands exactly on a .5 boundary at d = 1
    b = np.concatenate([[127.0], np.arange(31, dtype=np.float32) * 2 + 0.5]).astype(np.float32)
    blocks.append(b)
    x = np.stack(blocks).reshape(1, -1).astype(np.float32)
    q, d = qk.quantize_q8_0(dev(x))
    oq, od = oracle.quantize_q8_0(x)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(d, np.uint16), od)


@pytest.mark.parametrize("n,k", [(7, 64), (384, 256), (2560, 2048), (33, 5632)])
def test_quantize_q4_0_bit_exact(gpu_lib, n, k):
    qk = gpu_lib
    say(f"qk_quantize_q4_0 n={n} k={k}")
    w = synth.normal(102, n + k, (n, k), 0.02)
    w[0, :32] = 0.0
    if n > 1:
        w[1, :32] = np.arange(32, dtype=np.float32) * np.float32(0.5) - 7.0  # ties at delta = 1
    q, d = qk.qk_quantize_q4_0(dev(w))
    oq, od = oracle.quantize_q4_0(w)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(d, np.uint16), od)


@pytest.mark.parametrize("n,k,m", [(5, 32, 1), (64, 2048, 3), (37, 704, 2)])
def test_block_dots_bit_exact_on_any_bytes(gpu_lib, n, k, m):
    qk = gpu_lib
    say(f"qk_block_dots n={n} k={k} m={m}")
    r = np.random.default_rng(n * k + m)
    wq = r.integers(0, 256, (n, k // 2), dtype=np.uint8)     # every nibble, including code -8
    xq = r.integers(-128, 128, (m, k), dtype=np.int8)
    wq[0] = 0x00
    xq[0, :32] = -127
    isum = qk.qk_block_dots_q4_0_q8_0(dev(wq), dev(xq))
    assert np.array_equal(host(isum), oracle.block_dots(wq, k, xq))


# ---------------------------------------------------------------- matmul
MM_CASES = [(5632, 2048, 1), (2048, 5632, 1), (5632, 2048, 8), (2048, 5632, 8),
            (384, 256, 16), (37, 704, 3), (100, 32, 2), (256, 2048, 9), (130, 2048, 33),
            (300, 6144, 130), (64, 256, 1), (4096, 6144, 2),
            # the MFMA path with K stages not filled (3 and 65 blocks), ragged rows and tokens
            (70, 96, 33), (129, 2080, 65), (200, 32, 100),
            # rows longer than one load step (K > 6144: 2 and 3 steps, the
            # last one ragged)
            (300, 8192, 4), (129, 12320, 1), (64, 8192, 8)]


@pytest.mark.parametrize("n,k,m", MM_CASES)
def test_qmatmul_matches_oracle(gpu_lib, n, k, m):
    qk = gpu_lib
    say(f"qmatmul n={n} k={k} m={m}")
    w = synth.normal(103, n + 3 * k, (n, k), 0.02)
    x = synth.normal(104, n + 5 * k + m, (m, k))
    wq, wd = oracle.quantize_q4_0(w)
    xq, xd = oracle.quantize_q8_0(x)
    y = qk.qmatmul_q4_0_q8_0(dev(wq), dev(wd), dev(xq), dev(xd))
    ref = oracle.qmatmul(wq, wd, xq, xd)
    assert rel_err(host(y), ref) < 1e-5
    assert_same_fp32(host(y), ref)


# ------------------------------------------------- row-scaled int4 / int2
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("n,k", [(7, 64), (384, 256), (2048, 6144), (33, 2048)])
def test_quantize_rowq_bit_exact(gpu_lib, bits, n, k):
    qk = gpu_lib
    say(f"qk_quantize_rowq bits={bits} n={n} k={k}")
    w = synth.normal(140, bits * 100 + n, (n, k), 0.02)
    w[min(3, n - 1)] = 0.0                                   # a zero row
    q, r = qk.qk_quantize_rowq(dev(w), bits)
    oq, orr = oracle.quantize_rowq(w, bits)
    assert np.array_equal(host(q, np.uint8), oq)
    assert np.array_equal(host(r), orr)


ROWQ_MM = [(5, 32, 1), (64, 2048, 3), (37, 704, 2), (2048, 6144, 1), (300, 8192, 4), (96, 256, 13),
           (64, 8192, 13),
           (4096, 2048, 8)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("n,k,m", ROWQ_MM)
def test_qmatmul_rowq_matches_oracle(gpu_lib, bits, n, k, m):
    """Row-scaled weights through the GEMV: single and several columns,
    ragged rows, rows past one load step (k 8192), and more than 8 columns
    (two passes)."""
    qk = gpu_lib
    say(f"qk_qmatmul_rowq_q8_0 bits={bits} n={n} k={k} m={m}")
    w = synth.normal(141, bits * 100 + n + 3 * k, (n, k), 0.02)
    x = synth.normal(142, n + 5 * k + m, (m, k))
    wq, wr = oracle.quantize_rowq(w, bits)
    xq, xd = oracle.quantize_q8_0(x)
    y = qk.qk_qmatmul_rowq_q8_0(dev(wq), dev(wr), dev(xq), dev(xd), bits)
    ref = oracle.qmatmul_rowq(wq, wr, xq, xd, bits)
    assert rel_err(host(y), ref) < 1e-5
    assert_same_fp32(host(y), ref)


def test_rowq_rejects_bad_bits(gpu_lib):
    qk = gpu_lib
    L = qk.load()
    w = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    q = torch.zeros((2, 32), dtype=torch.uint8, device="cuda")
    r = torch.zeros(2, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for bits in (0, 3, 8):
        assert L.qk_quantize_rowq(bits, w.data_ptr(), 2, 64, q.data_ptr(), r.data_ptr(), s) == qk.QK_EINVAL
    assert L.qk_quantize_rowq(4, w.data_ptr(), 2, 48, q.data_ptr(), r.data_ptr(), s) == qk.QK_ESHAPE


def test_qmatmul_workload_seeded(gpu_lib):
    """The standalone matmul workload as generated (seed 1): W 5632x2048 and
    the transposed-shape 2048x5632, at batch 1 and 8, quantized on the GPU."""
    qk = gpu_lib
    spec = W.MATMUL
    for idx, (n, k) in enumerate(spec["shapes"]):
        w = W.matmul_weight_f32(spec["seed"], idx, n, k)
        wq, wd = oracle.quantize_q4_0(w)
        wqg, wdg = qk.qk_quantize_q4_0(dev(w))
        assert np.array_equal(host(wqg), wq) and np.array_equal(host(wdg, np.uint16), wd)
        for m in spec["batches"]:
            say(f"matmul workload n={n} k={k} m={m}")
            x = W.matmul_input_f32(spec["seed"], idx, m, k)
            xq, xd = oracle.quantize_q8_0(x)
            xqg, xdg = qk.quantize_q8_0(dev(x))
            assert np.array_equal(host(xqg), xq) and np.array_equal(host(xdg, np.uint16), xd)
            y = qk.qmatmul_q4_0_q8_0(wqg, wdg, xqg, xdg)
            ref = oracle.qmatmul(wq, wd, xq, xd)
            assert rel_err(host(y), ref) < LAYER_TOL
            assert_same_fp32(host(y), ref)


@pytest.mark.parametrize("ffn,k,m", [(5632, 2048, 1), (704, 256, 16), (96, 64, 5), (2048, 6144, 3),
                                     (100, 96, 70)])
def test_gate_up_swiglu(gpu_lib, ffn, k, m):
    qk = gpu_lib
    say(f"qk_gate_up_swiglu ffn={ffn} k={k} m={m}")
    w = synth.normal(112, ffn + k, (2 * ffn, k), 0.02)
    x = synth.normal(113, ffn + k + m, (m, k))
    wq, wd = oracle.quantize_q4_0(w)
    xq, xd = oracle.quantize_q8_0(x)
    h = qk.qk_gate_up_swiglu(dev(wq), dev(wd), dev(xq), dev(xd))
    gu = oracle.qmatmul(wq, wd, xq, xd)
    ref = oracle.swiglu(gu[:, :ffn], gu[:, ffn:])
    assert rel_err(host(h), ref) < 1e-5
    assert_same_fp32(host(h), ref)


@pytest.mark.parametrize("ffn,hidden,tokens", [(5632, 2048, 1), (704, 256, 3), (96, 128, 20)])
def test_ffn_up(gpu_lib, ffn, hidden, tokens):
    qk = gpu_lib
    say(f"qk_ffn_up ffn={ffn} hidden={hidden} tokens={tokens}")
    x = synth.normal(114, 1, (tokens, hidden))
    g = synth.normal(114, 2, hidden, 0.02, mean=1.0)
    wq, wd = oracle.quantize_q4_0(synth.normal(114, 3, (2 * ffn, hidden), 0.02))
    xq, xd = oracle.quantize_q8_0(oracle.rmsnorm(x, g, 1e-5))
    gu = oracle.qmatmul(wq, wd, xq, xd)
    ref = oracle.swiglu(gu[:, :ffn], gu[:, ffn:])
    h = qk.qk_ffn_up(dev(x), dev(g), 1e-5, dev(wq), dev(wd))
    assert rel_err(host(h), ref) < 1e-5
    assert_same_fp32(host(h), ref)


def test_qmatmul_zero_and_empty(gpu_lib):
    qk = gpu_lib
    say("qmatmul zero weights, m = 0")
    wq = np.full((40, 64), 0x88, np.uint8)
    wd = np.zeros((40, 4), np.uint16)
    x = synth.normal(105, 0, (3, 128))
    xq, xd = oracle.quantize_q8_0(x)
    y = qk.qmatmul_q4_0_q8_0(dev(wq), dev(wd), dev(xq), dev(xd))
    assert np.all(host(y) == 0)
    empty = torch.empty((0, 128), dtype=torch.int8, device="cuda")
    emptyd = torch.empty((0, 4), dtype=torch.int16, device="cuda")
    assert qk.qmatmul_q4_0_q8_0(dev(wq), dev(wd), empty, emptyd).shape == (0, 40)


# ---------------------------------------------------------------- element-wise
@pytest.mark.parametrize("rows,dim", [(16, 256), (3, 2048), (1, 6144), (5, 8)])
def test_rmsnorm(gpu_lib, rows, dim):
    qk = gpu_lib
    say(f"rmsnorm rows={rows} dim={dim}")
    x = synth.normal(106, dim, (rows, dim))
    g = synth.normal(106, 1, dim, 0.02, mean=1.0)
    y = qk.rmsnorm(dev(x), dev(g), 1e-5)
    assert rel_err(host(y), oracle.rmsnorm(x, g, 1e-5)) < 2e-6
    assert_same_fp32(host(y), oracle.rmsnorm(x, g, 1e-5))


@pytest.mark.parametrize("tokens,heads,hd", [(16, 12, 32), (3, 36, 64), (1, 1, 2)])
def test_rope(gpu_lib, tokens, heads, hd):
    qk = gpu_lib
    say(f"rope tokens={tokens} heads={heads} hd={hd}")
    x = synth.normal(107, heads, (tokens, heads, hd))
    pos = np.concatenate([[0], synth.randint(107, 2, tokens - 1, 2176)]).astype(np.int32)
    xg = dev(x)
    qk.rope(xg, dev(pos), 10000.0)
    ref = oracle.rope(x, pos, 10000.0)
    got = host(xg)
    assert np.array_equal(got[0], x[0])       # position 0 is the identity
    assert rel_err(got, ref) < 2e-6
    assert_same_fp32(got, ref)


def test_swiglu(gpu_lib):
    qk = gpu_lib
    say("swiglu")
    g = synth.normal(108, 0, 5000) * np.float32(6)
    u = synth.normal(108, 1, 5000)
    h = qk.swiglu(dev(g), dev(u))
    assert rel_err(host(h), oracle.swiglu(g, u)) < 2e-6
    assert_same_fp32(host(h), oracle.swiglu(g, u))


def test_kv_append_bit_exact(gpu_lib):
    qk = gpu_lib
    say("qk_kv_append")
    nkv, cap, hd = 4, 40, 64
    k = synth.normal(109, 0, (6, nkv, hd))
    v = synth.normal(109, 1, (6, nkv, hd))
    pos = np.array([0, 39, 5, 5, 17, 2], np.int32)
    seq = np.array([0, 0, 1, 2, 2, 1], np.int32)
    kc = np.zeros((3, nkv, cap, hd), np.uint16)
    vc = np.zeros_like(kc)
    kcg, vcg = dev(kc), dev(vc)
    qk.qk_kv_append(dev(k), dev(v), dev(pos), dev(seq), kcg, vcg)
    oracle.kv_append(k, v, pos, seq, kc, vc)
    assert np.array_equal(host(kcg, np.uint16), kc)
    assert np.array_equal(host(vcg, np.uint16), vc)
    # past cap, one token per sequence: ring rows pos % cap
    pos = np.array([40, 1000, 79], np.int32)
    seq = np.array([0, 1, 2], np.int32)
    qk.qk_kv_append(dev(k[:3]), dev(v[:3]), dev(pos), dev(seq), kcg, vcg)
    oracle.kv_append(k[:3], v[:3], pos, seq, kc, vc)
    assert np.array_equal(host(kcg, np.uint16), kc)
    assert np.array_equal(host(vcg, np.uint16), vc)


@pytest.mark.parametrize("tokens,cap", [(6, 300), (13, 300), (6, 8192)])
def test_negative_positions_read_and_write_nothing(gpu_lib, tokens, cap):
    """Negative positions (padding tokens) as the header states them: the KV
    store skips their rows and attention gives them zero rows, on the
    few-token chunk/merge pass (6 tokens: the one-wave merge at 300 rows, the
    two-wave merge at 8192) and on the tiled pass (13).  The other tokens
    equal the oracle over them alone (the oracle takes non-negative
    positions only; a token's result depends on its own position, sequence
    and query and on the cache)."""
    qk = gpu_lib
    say(f"negative positions, {tokens} tokens, cap {cap}")
    nq, nkv, hd, seqs = 8, 2, 64, 2
    neg = np.arange(tokens) % 3 == 1
    pos = synth.randint(112, 4, tokens, cap).astype(np.int32)
    pos[neg] = -1 - 37 * np.arange(int(neg.sum()), dtype=np.int32)   # -1, -38, ...
    seq = (np.arange(tokens) % seqs).astype(np.int32)
    # KV store: one token per (sequence, position) so that the result does
    # not depend on the order of the stores
    k = synth.normal(112, 5, (tokens, nkv, hd))
    v = synth.normal(112, 6, (tokens, nkv, hd))
    kpos = np.where(neg, pos, np.arange(tokens, dtype=np.int32) * 7)
    kc, vc = _cache(112, seqs, nkv, cap, hd, cap // 2)
    kcg, vcg = dev(kc), dev(vc)
    qk.qk_kv_append(dev(k), dev(v), dev(kpos), dev(seq), kcg, vcg)
    oracle.kv_append(k[~neg], v[~neg], kpos[~neg], seq[~neg], kc, vc)
    assert np.array_equal(host(kcg, np.uint16), kc)
    assert np.array_equal(host(vcg, np.uint16), vc)
    # attention over the updated caches
    q = synth.normal(112, 3, (tokens, nq, hd))
    out = host(qk.gqa_attention(dev(q), kcg, vcg, dev(pos), dev(seq)))
    assert np.all(out[neg] == 0.0)
    ref = oracle.gqa_attention(q[~neg], kc, vc, pos[~neg], seq[~neg])
    assert rel_err(out[~neg], ref) < 1e-5
    assert_same_fp32(out[~neg], ref)


def test_embed_and_argmax(gpu_lib):
    qk = gpu_lib
    say("qk_embed_lookup, qk_argmax")
    table = synth.normal(110, 0, (1000, 64))
    ids = synth.randint(110, 1, 9, 1000)
    x = qk.qk_embed_lookup(dev(table), dev(ids))
    assert np.array_equal(host(x), oracle.embed_lookup(table, ids))
    logits = synth.normal(110, 2, (5, 32000))
    logits[1, 77] = logits[1, 9000] = 50.0          # tie -> lowest index
    logits[2, :] = -3.0                              # all equal -> 0
    logits[3, 31999] = 60.0                          # last element
    idx = qk.qk_argmax(dev(logits))
    assert host(idx).tolist() == oracle.argmax(logits).tolist()
    assert host(idx)[1] == 77 and host(idx)[2] == 0 and host(idx)[3] == 31999


# ---------------------------------------------------------------- attention
def _cache(seed, seqs, nkv, cap, hd, filled):
    kc = np.zeros((seqs, nkv, cap, hd), np.uint16)
    vc = np.zeros_like(kc)
    kc[:, :, :filled] = synth.normal(seed, 1, (seqs, nkv, filled, hd)).astype(np.float16).view(np.uint16)
    vc[:, :, :filled] = synth.normal(seed, 2, (seqs, nkv, filled, hd)).astype(np.float16).view(np.uint16)
    return kc, vc


ATT_CASES = [
    # (tokens, nq, nkv, hd, cap, seqs, pos recipe)
    (16, 8, 2, 32, 32, 1, "prefill"),
    (1, 32, 4, 64, 2176, 1, "decode2048"),
    (6, 32, 4, 64, 2176, 3, "ragged"),
    (3, 8, 8, 64, 130, 1, "mha"),
    (2, 16, 1, 32, 70, 2, "mqa"),
    (6, 16, 2, 32, 4096, 3, "ragged"),    # head_dim 32, 64 chunks: the one-wave merge's limit
    (1, 32, 4, 64, 2176, 1, "first"),
    # many tokens: the tiled pass (runs of one sequence inside 8-token tiles)
    (64, 8, 2, 64, 200, 1, "prefill"),
    (40, 32, 4, 64, 300, 3, "runs"),
    (37, 16, 1, 32, 130, 2, "random"),
    (12, 32, 4, 64, 2176, 1, "long"),
    # past cap the cache is a ring: one token per sequence, any position
    (3, 32, 4, 64, 4096, 3, "ring"),
    (2, 32, 4, 64, 8192, 2, "ring"),
    (3, 8, 2, 64, 100, 3, "ring"),
    (12, 16, 2, 64, 100, 12, "ring"),     # many tokens: the tiled pass
    # long contexts: up to 512 chunks per head in the merge pass
    (2, 32, 4, 64, 32768, 2, "ring"),
    (2, 16, 2, 32, 32768, 2, "ring"),
    # merge forms by records per head: 65..128 in one wave, two records a
    # lane (8192 rows); 129..255 on the four-wave merge (12000 rows)
    (3, 16, 2, 32, 8192, 3, "ring"),
    (3, 32, 4, 64, 12000, 3, "ring"),
    (2, 16, 2, 32, 12000, 2, "ring"),
    (3, 16, 2, 32, 16384, 3, "spread"),   # the long pass's 64 records, head_dim 32
    (40, 32, 4, 64, 16384, 1, "long9k"),  # many tokens past 8192: the tiled pass
    # caches of 256 chunks and more: four chunks per chunk-pass workgroup and
    # record; positions at chunk and four-chunk boundaries give records of
    # one to four chunks and workgroups with nothing to read
    (8, 32, 4, 64, 32768, 8, "spread"),
    (3, 32, 4, 64, 16384, 3, "spread"),
    (8, 16, 2, 32, 32768, 8, "spread"),
    # head groups that do not divide the 64 query rows of a tiled-pass workgroup
    (24, 12, 4, 64, 100, 2, "random"),    # G = 3: 21 tokens x 3 heads per workgroup
    (25, 24, 4, 32, 90, 1, "prefill"),    # G = 6, head_dim 32
]


@pytest.mark.parametrize("tokens,nq,nkv,hd,cap,seqs,recipe", ATT_CASES)
def test_gqa_attention(gpu_lib, tokens, nq, nkv, hd, cap, seqs, recipe):
    qk = gpu_lib
    say(f"gqa_attention {recipe} tokens={tokens} nq={nq} nkv={nkv} hd={hd} cap={cap}")
    kc, vc = _cache(111, seqs, nkv, cap, hd, cap)
    q = synth.normal(111, 3, (tokens, nq, hd))
    if recipe == "prefill":
        pos = np.arange(tokens, dtype=np.int32)
    elif recipe == "decode2048":
        pos = np.array([2048], np.int32)
    elif recipe == "first":
        pos = np.array([0], np.int32)
    elif recipe == "ragged":
        pos = np.array([2175, 0, 63, 64, 1000, 129], np.int32)
    elif recipe == "runs":   # sequences in runs of 14 tokens at consecutive positions
        seq = (np.arange(tokens) // 14 % seqs).astype(np.int32)
        pos = np.array([90 * (t // 14) + t % 14 + 3 for t in range(tokens)], np.int32)
    elif recipe == "long":
        pos = (2100 + np.arange(tokens)).astype(np.int32)
    elif recipe == "long9k":
        pos = (9000 + np.arange(tokens)).astype(np.int32)
    elif recipe == "spread":
        pos = np.array([cap // 2 - 1, 255, cap - 700, 0, 63, 64, 256, 5000], np.int32)[:tokens]
    elif recipe == "ring":
        pos = np.array([cap - 1, cap, 2 * cap + 37, 5 * cap + 3] * 3, np.int32)[:tokens] + \
            (synth.randint(111, 5, tokens, 7)).astype(np.int32)
    else:
        pos = (synth.randint(111, 4, tokens, cap)).astype(np.int32)
    if recipe != "runs":
        seq = (np.arange(tokens) % seqs).astype(np.int32)
    out = qk.gqa_attention(dev(q), dev(kc), dev(vc), dev(pos), dev(seq))
    ref = oracle.gqa_attention(q, kc, vc, pos, seq)
    assert rel_err(host(out), ref) < 1e-5
    assert_same_fp32(host(out), ref)


# ---------------------------------------------------------------- errors
def test_error_codes_and_nothing_enqueued(gpu_lib):
    qk = gpu_lib
    say("error paths")
    L = qk.load()
    x = torch.full((2, 40), 7.0, dtype=torch.float32, device="cuda")
    q = torch.full((2, 40), 5, dtype=torch.int8, device="cuda")
    d = torch.full((2, 2), 3, dtype=torch.int16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.quantize_q8_0(x.data_ptr(), 2, 40, q.data_ptr(), d.data_ptr(), s) == qk.QK_ESHAPE
    assert L.quantize_q8_0(x.data_ptr() + 4, 1, 32, q.data_ptr(), d.data_ptr(), s) == qk.QK_EALIGN
    assert L.quantize_q8_0(None, 1, 32, q.data_ptr(), d.data_ptr(), s) == qk.QK_EINVAL
    qa = torch.zeros((4, 2, 32), dtype=torch.float32, device="cuda")
    kc = torch.zeros((1, 1, 8, 32), dtype=torch.int16, device="cuda")
    pos = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.full((4, 2, 32), 9.0, dtype=torch.float32, device="cuda")
    rc = L.gqa_attention(qa.data_ptr(), 4, 2, 1, 32, kc.data_ptr(), kc.data_ptr(), 8,
                         pos.data_ptr(), pos.data_ptr(), out.data_ptr(), ws.data_ptr(), 16, s)
    assert rc == qk.QK_EWORKSPACE
    rc = L.gqa_attention(qa.data_ptr(), 4, 3, 2, 32, kc.data_ptr(), kc.data_ptr(), 8,
                         pos.data_ptr(), pos.data_ptr(), out.data_ptr(), ws.data_ptr(), 16, s)
    assert rc == qk.QK_ESHAPE
    torch.cuda.synchronize()
    # nothing was enqueued: outputs untouched
    assert torch.all(q == 5) and torch.all(d == 3) and torch.all(out == 9.0)


# ---------------------------------------------------------------- sampler chain
def _sample_agrees(qk_ids, logits, top_k, top_p, temp, u):
    """GPU ids equal the oracle's, except where u lies within 1e-9 of a
    cumulative boundary or the top-p cut within 1e-12 of a running
    probability: there the fp64 exp and the order of the fp64 sums of either
    side may decide."""
    want = oracle.sample(logits, top_k, top_p, temp, u)
    for r in np.nonzero(qk_ids != want)[0]:
        alt = {int(oracle.sample(logits[r], top_k, top_p, temp, [min(u[r] + d, 1 - 1e-16)])[0])
               for d in (-1e-9, 1e-9)}
        alt |= {int(oracle.sample(logits[r], top_k, top_p, temp, [u[r]], top_p_shift=d)[0]) for d in (-1e-12, 1e-12)}
        assert int(qk_ids[r]) in alt, f"row {r}: {qk_ids[r]} vs {want[r]}"
    return float(np.mean(qk_ids == want))


@pytest.mark.parametrize("rows,vocab,top_k,top_p,temp", [
    (8, 32000, 40, 0.9, 0.7),      # the chain of the llama.cpp guide
    (5, 32000, 256, 1.0, 1.0),
    (7, 1000, 1, 0.9, 0.7),        # greedy by top-k
    (6, 517, 13, 0.5, 1.7),
    (4, 32000, 40, 0.9, 0.0),      # greedy by temperature
    (3, 5001, 40, 0.9, 0.7),       # rows not a multiple of 4 logits: 4-byte loads
    (3, 3000, 256, 0.95, 1.3),     # between 1024 and 4096 logits
    (2, 32768, 40, 0.9, 0.7),      # the largest row
])
def test_sampler_chain(gpu_lib, rows, vocab, top_k, top_p, temp):
    qk = gpu_lib
    say(f"qk_sample rows={rows} vocab={vocab} k={top_k} p={top_p} T={temp}")
    logits = synth.normal(130, rows + vocab, (rows, vocab)) * np.float32(2.5)
    logits[0, 5] = logits[0, 900 % vocab] = np.float32(40.0)   # a tie at the top
    u = (synth.randint(130, 1, rows, 1 << 30).astype(np.float64) + 0.5) / (1 << 30)
    ids = host(qk.qk_sample(dev(logits), top_k, top_p, temp, dev(u)))
    assert _sample_agrees(ids, logits, top_k, top_p, temp, u) >= 0.99


def test_sampler_ties_and_grid(gpu_lib):
    """All-equal logits keep the lowest ids; a grid of u reproduces the
    oracle's draws token for token."""
    qk = gpu_lib
    say("qk_sample ties and u grid")
    flat = np.zeros((3, 300), np.float32)
    u = np.array([0.1, 0.5, 0.9])
    assert host(qk.qk_sample(dev(flat), 4, 1.0, 1.0, dev(u))).tolist() == [0, 2, 3]
    logits = np.tile(synth.normal(131, 1, 64) * np.float32(1.5), (400, 1)).astype(np.float32)
    ug = (np.arange(400) + 0.5) / 400
    ids = host(qk.qk_sample(dev(logits), 64, 0.95, 0.8, dev(ug)))
    assert _sample_agrees(ids, logits, 64, 0.95, 0.8, ug) >= 0.99


@pytest.mark.parametrize("levels,top_k", [(4, 256), (4, 40), (50, 256), (50, 7)])
def test_sampler_heavy_ties(gpu_lib, levels, top_k):
    """Integer-valued logits over 32000 ids: thousands of ids share the top
    value (levels 4), or a few hundred do (levels 50).  The kept set is the
    lowest ids among equal logits in both regimes."""
    qk = gpu_lib
    say(f"qk_sample heavy ties levels={levels} k={top_k}")
    rows, vocab = 4, 32000
    logits = synth.randint(132, levels, (rows, vocab), levels).astype(np.float32)
    u = (synth.randint(133, 1, rows, 1 << 30).astype(np.float64) + 0.5) / (1 << 30)
    for temp in (0.0, 0.7):
        ids = host(qk.qk_sample(dev(logits), top_k, 0.9, temp, dev(u)))
        assert _sample_agrees(ids, logits, top_k, 0.9, temp, u) >= 0.99


def test_sampler_rejects_bad_top_k(gpu_lib):
    qk = gpu_lib
    L = qk.load()
    x = torch.zeros((1, 10), dtype=torch.float32, device="cuda")
    u = torch.zeros(1, dtype=torch.float64, device="cuda")
    o = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.qk_sample(x.data_ptr(), 1, 10, 0, 0.9, 0.7, u.data_ptr(), o.data_ptr(), s) == qk.QK_EINVAL
    assert L.qk_sample(x.data_ptr(), 1, 10, 257, 0.9, 0.7, u.data_ptr(), o.data_ptr(), s) == qk.QK_EINVAL


@pytest.mark.parametrize("nbytes,blocks", [(2**20 + 48, 7), (16 * 1000, 2048), (16, 3)])
def test_read_probe_reads_every_word_once(gpu_lib, nbytes, blocks):
    """The bandwidth probe covers the buffer exactly once: the XOR of its
    per-workgroup words equals the XOR of every 32-bit word of the buffer."""
    qk = gpu_lib
    say(f"qk_read_probe bytes={nbytes} blocks={blocks}")
    rng = np.random.default_rng(nbytes + blocks)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).to("cuda")
    out = qk.qk_read_probe(buf, blocks=blocks)
    got = np.bitwise_xor.reduce(host(out).view(np.uint32))
    want = np.bitwise_xor.reduce(words)
    assert int(got) == int(want)
    L = qk.load()
    s = torch.cuda.current_stream().cuda_stream
    assert L.qk_read_probe(buf.data_ptr(), 24, out.data_ptr(), blocks, s) == qk.QK_ESHAPE
    assert L.qk_read_probe(buf.data_ptr(), 16, out.data_ptr(), 0, s) == qk.QK_EINVAL
