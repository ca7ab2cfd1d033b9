"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, invariants, numpy's IEEE binary16 conversion, or fp64 brute force on
tiny inputs.  No GPU is used.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# IEEE binary16
# ---------------------------------------------------------------------------
def test_half_to_float_all_65536_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy_rne():
    r = rng(1)
    parts = [
        r.standard_normal(200_000).astype(np.float32) * np.float32(10.0) ** r.integers(-9, 6, 200_000),
        np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e9, -1e9, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11),
                  np.inf, -np.inf, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 5.960464477539063e-08,
                  2.9802322387695312e-08], dtype=np.float32),
    ]
    # every half-way point between adjacent binary16 values (ties to even)
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    x = np.concatenate(parts).astype(np.float32)
    ours = oracle.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Q8_0 activations
# ---------------------------------------------------------------------------
def test_q8_0_golden_blocks():
    """Hand-worked blocks (tests/golden/q8_0_blocks.json)."""
    with open(os.path.join(GOLDEN, "q8_0_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = np.array(case["x"], np.float32)[None, :]
        q, d = oracle.quantize_q8_0(x)
        assert q[0].tolist() == case["q"], case["name"]
        assert int(d[0, 0]) == int(case["d_f16_bits"], 16), case["name"]


def test_q8_0_half_away_from_zero_with_unit_scale():
    # max|x| = 127 gives d = 1 exactly, so the codes are the rounded inputs.
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:9] = [2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -3.49]
    q, d = oracle.quantize_q8_0(x[None])
    assert q[0, :9].tolist() == [127, 3, -3, 1, -1, 2, -2, 127, -3]
    assert oracle.f16_to_f32(d)[0, 0] == 1.0


@pytest.mark.parametrize("c", [1e-3, 0.75, -3.0, 200.0])
def test_q8_0_single_nonzero(c):
    for j in (0, 7, 31):
        x = np.zeros(64, np.float32)
        x[32 + j] = c
        q, d = oracle.quantize_q8_0(x[None])
        assert np.all(q[0, :32] == 0) and d[0, 0] == 0
        expect = np.zeros(32, np.int8)
        expect[j] = 127 if c > 0 else -127
        assert np.array_equal(q[0, 32:], expect)
        assert d[0, 1] == np.float16(np.float32(abs(c)) / np.float32(127)).view(np.uint16)


def test_q8_0_error_bound_random():
    x = synth.normal(11, 0, (64, 512))
    x[3] *= 1e-3
    x[5] *= 1e3
    q, d = oracle.quantize_q8_0(x)
    dd = oracle.f16_to_f32(d).astype(np.float64)
    xb = x.reshape(64, 16, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    recon = dd[..., None] * q.reshape(64, 16, 32)
    bound = d32 / 2 + 127 * np.abs(dd - d32)
    assert np.all(np.abs(xb - recon) <= bound[..., None] * (1 + 1e-6) + 1e-30)
    assert np.abs(q).max() == 127 and q.min() >= -127


# ---------------------------------------------------------------------------
# Q4_0 weights
# ---------------------------------------------------------------------------
def unpack_q4(wq):
    """nibbles -> int codes in [0, 15], element order (numpy bit ops)."""
    n, kh = wq.shape
    b = wq.reshape(n, kh // 16, 16)
    lo = b & 0x0F
    hi = b >> 4
    return np.concatenate([lo, hi], axis=-1).reshape(n, kh * 2).astype(np.int32)


def test_q4_0_unit_scale_codes_and_layout():
    # max|w| = 7 gives delta = 1: codes are the rounded weights, +8.
    w = np.zeros((1, 32), np.float32)
    w[0, :10] = [7.0, 2.5, -2.5, 0.5, -0.5, 1.49, -6.5, 3.0, -7.0, 0.0]
    w[0, 16] = 4.0
    w[0, 31] = -1.0
    wq, wd = oracle.quantize_q4_0(w)
    assert oracle.f16_to_f32(wd)[0, 0] == 1.0
    codes = [15, 11, 5, 9, 7, 9, 1, 11, 1, 8]
    assert unpack_q4(wq)[0, :10].tolist() == codes
    # byte j: low nibble element j, high nibble element j + 16
    assert wq[0, 0] == (15 | (12 << 4))
    assert wq[0, 15] == (8 | (7 << 4))


def test_q4_0_zero_block_and_never_code_minus_8():
    w = synth.normal(5, 1, (64, 256), 0.02)
    w[7, 32:64] = 0.0
    wq, wd = oracle.quantize_q4_0(w)
    codes = unpack_q4(wq)
    assert np.all(codes[7, 32:64] == 8) and wd[7, 1] == 0
    assert codes.min() >= 1  # delta = max|w|/7 never reaches the code -8
    assert codes.max() == 15


def test_q4_0_error_bound_random():
    w = synth.normal(6, 2, (128, 256), 0.02)
    wq, wd = oracle.quantize_q4_0(w)
    dl = oracle.f16_to_f32(wd).astype(np.float64)
    wb = w.reshape(128, 8, 32).astype(np.float64)
    d32 = (np.abs(w.reshape(128, 8, 32)).max(-1) / np.float32(7)).astype(np.float64)
    recon = dl[..., None] * (unpack_q4(wq).reshape(128, 8, 32) - 8)
    bound = d32 / 2 + 7 * np.abs(dl - d32)
    assert np.all(np.abs(wb - recon) <= bound[..., None] * (1 + 1e-6))


# ---------------------------------------------------------------------------
# row-scaled int4 / int2 (COLIBRI: int4 container with per-row scales,
# int4/int2 packing)
# ---------------------------------------------------------------------------
def unpack_rowq(wq, bits):
    """Signed codes in element order from the documented packing (numpy)."""
    n, nbytes = wq.shape
    if bits == 4:
        return unpack_q4(wq) - 8
    g = wq.reshape(n, nbytes // 8, 8).astype(np.int32)
    parts = [(g >> (2 * s)) & 3 for s in range(4)]        # elements j + 8 s
    return np.concatenate(parts, axis=-1).reshape(n, nbytes * 4) - 2


def test_rowq_unit_scale_codes_and_layout():
    """max|w| = 7 (int4) or 1 (int2) gives delta 1 exactly, so the codes are
    the weights rounded half away from zero; the bytes follow the documented
    order (worked by hand)."""
    w4 = np.array([[-7, -2.5, 2.5, 0.5, -0.5, 7, 1.49, 3.51] * 4], np.float32)
    q4, r4 = oracle.quantize_rowq(w4, 4)
    assert r4.tolist() == [1.0]
    assert q4[0, :8].tolist() == [0x11, 0x55, 0xBB, 0x99, 0x77, 0xFF, 0x99, 0xCC]
    # nibble of element i = i % 16  ->  byte j = j | j << 4
    w4b = np.array([[(i % 16) - 8 for i in range(32)]], np.float32)
    w4b[0, 0] = w4b[0, 16] = -7.0                            # keep max|w| = 7 (code -8 never made)
    q4b, _ = oracle.quantize_rowq(w4b, 4)
    assert q4b[0].tolist() == [0x11] + [j | (j << 4) for j in range(1, 16)]
    w2 = np.array([[-1, 0, 1, 0.5, -0.5, 0.49, -0.49, 0.2] * 4], np.float32)
    q2, r2 = oracle.quantize_rowq(w2, 2)
    assert r2.tolist() == [1.0]
    assert q2[0].tolist() == [0x55, 0xAA, 0xFF, 0xFF, 0x55, 0xAA, 0xAA, 0xAA]
    # stored code of element i = 1 + (i // 8) % 3  ->  byte j = 1 | 2 << 2 | 3 << 4 | 1 << 6
    w2b = np.array([[((i // 8) % 3) - 1 for i in range(32)]], np.float32)
    q2b, _ = oracle.quantize_rowq(w2b, 2)
    assert q2b[0].tolist() == [0x79] * 8


@pytest.mark.parametrize("bits", [4, 2])
def test_rowq_zero_row_extremes_and_error_bound(bits):
    hi = 7 if bits == 4 else 1
    w = synth.normal(35, bits, (64, 256), 0.02)
    w[3] = 0.0
    wq, wr = oracle.quantize_rowq(w, bits)
    q = unpack_rowq(wq, bits)
    assert wr[3] == 0 and np.all(q[3] == 0)
    assert q.min() >= -hi and q.max() <= hi                 # -8 / -2 never made
    amax = np.abs(w).max(1)
    delta = (amax / np.float32(hi)).astype(np.float32)
    assert np.array_equal(wr, delta)
    arg = np.abs(w).argmax(1)
    assert np.all(np.abs(q[np.arange(64), arg])[amax > 0] == hi)
    recon = wr.astype(np.float64)[:, None] * q
    assert np.all(np.abs(w - recon) <= wr.astype(np.float64)[:, None] / 2 * (1 + 1e-6))


@pytest.mark.parametrize("bits", [4, 2])
def test_qmatmul_rowq_equals_fp64_dequantized_bruteforce(bits):
    """y = delta_r * sum_b dx_b * isum_b equals the fp64 product of the
    dequantized matrices (to fp64 rounding), with exactly representable
    weights (w = 2^-6 q) and random ones."""
    hi = 7 if bits == 4 else 1
    n, k, m = 9, 96, 3
    codes = synth.randint(36, bits, (n, k), 2 * hi + 1).astype(np.int32) - hi
    codes[:, 5] = hi                                         # max|w| = hi * delta
    w_exact = (codes * 2.0 ** -6).astype(np.float32)
    x = synth.normal(36, 10 + bits, (m, k))
    xq, xd = oracle.quantize_q8_0(x)
    xdeq = oracle.f16_to_f32(xd).astype(np.float64).repeat(32, 1) * xq
    for w in (w_exact, synth.normal(36, 20 + bits, (n, k), 0.02)):
        wq, wr = oracle.quantize_rowq(w, bits)
        y = oracle.qmatmul_rowq(wq, wr, xq, xd, bits)
        wdeq = wr.astype(np.float64)[:, None] * unpack_rowq(wq, bits)
        assert np.allclose(y, xdeq @ wdeq.T, rtol=1e-6, atol=1e-9)
    assert np.array_equal(unpack_rowq(oracle.quantize_rowq(w_exact, bits)[0], bits), codes)
    # zero weights give zero exactly
    assert np.all(oracle.qmatmul_rowq(*oracle.quantize_rowq(np.zeros((4, k), np.float32), bits),
                                      xq, xd, bits) == 0)


# ---------------------------------------------------------------------------
# block dots and the quantized matmul
# ---------------------------------------------------------------------------
def test_block_dot_extremes_and_one_hot():
    k = 64
    xq = np.full((1, k), -127, np.int8)
    wq = np.zeros((2, k // 2), np.uint8)          # nibble 0 -> weight code -8
    wq[1] = 0xFF                                    # nibble 15 -> +7
    s = oracle.block_dots(wq, k, xq)
    assert s[0, 0].tolist() == [32512, 32512]       # 32 * 8 * 127
    assert s[0, 1].tolist() == [-28448, -28448]     # 32 * 7 * -127
    # one-hot: weight +1 (nibble 9) at element i, activation one-hot at j
    for i in (0, 5, 15, 16, 21, 31):
        w = np.full(32, 8, np.int64)
        w[i] = 9
        packed = (w[:16] | (w[16:] << 4)).astype(np.uint8)[None]
        for j in (0, 5, 16, 31):
            x = np.zeros((1, 32), np.int8)
            x[0, j] = 77
            assert oracle.block_dots(packed, 32, x)[0, 0, 0] == (77 if i == j else 0)


def test_qmatmul_equals_fp64_dequantized_bruteforce():
    r = rng(3)
    for (n, k, m) in [(8, 64, 1), (5, 96, 3), (16, 256, 4)]:
        w = synth.normal(7, n + k, (n, k), 0.02)
        x = synth.normal(8, n + k + m, (m, k))
        wq, wd = oracle.quantize_q4_0(w)
        xq, xd = oracle.quantize_q8_0(x)
        y = oracle.qmatmul(wq, wd, xq, xd)
        Wd = (oracle.f16_to_f32(wd).astype(np.float64).repeat(32, 1)) * (unpack_q4(wq) - 8)
        Xd = (oracle.f16_to_f32(xd).astype(np.float64).repeat(32, 1)) * xq.astype(np.float64)
        ref = Xd @ Wd.T
        assert np.allclose(y, ref.astype(np.float32), rtol=0, atol=0) or \
            np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)) < 2 ** -23
        # and it approximates the unquantized product within the triangle bound
        exact = x.astype(np.float64) @ w.astype(np.float64).T
        bound = np.abs(Xd) @ np.abs(Wd - w).T + np.abs(Xd - x) @ np.abs(w.astype(np.float64)).T
        assert np.all(np.abs(ref - exact) <= bound * (1 + 1e-9) + 1e-12)
    del r


def test_qmatmul_zero_weights_give_zero():
    wq = np.full((4, 64), 0x88, np.uint8)
    wd = np.zeros((4, 4), np.uint16)
    x = synth.normal(9, 0, (2, 128))
    xq, xd = oracle.quantize_q8_0(x)
    assert np.all(oracle.qmatmul(wq, wd, xq, xd) == 0.0)


# ---------------------------------------------------------------------------
# RMSNorm, RoPE, SwiGLU
# ---------------------------------------------------------------------------
def test_rmsnorm_constant_vector_closed_form():
    for c in (0.5, -3.0, 1e-3):
        x = np.full((1, 64), c, np.float32)
        g = synth.normal(2, 9, 64, 0.02, mean=1.0)
        y = oracle.rmsnorm(x, g, 1e-5)
        cc = float(np.float32(c))
        ref = cc / np.sqrt(cc * cc + float(np.float32(1e-5))) * g.astype(np.float64)
        assert np.allclose(y, ref, rtol=1e-6, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = synth.normal(3, 3, (8, 2048))
    g = np.ones(2048, np.float32)
    y = oracle.rmsnorm(x, g, 1e-5)
    rms = np.sqrt((y.astype(np.float64) ** 2).mean(-1))
    assert np.allclose(rms, 1.0, atol=1e-5)
    # scaling x by a leaves the output unchanged except through eps:
    # y(a x) = y(x) * sqrt(ms + eps) / sqrt(ms + eps / a^2)
    a = 64.0
    y2 = oracle.rmsnorm(x * np.float32(a), g, 1e-5)
    ms = (x.astype(np.float64) ** 2).mean(-1, keepdims=True)
    e = float(np.float32(1e-5))
    assert np.allclose(y2, y * np.sqrt(ms + e) / np.sqrt(ms + e / a ** 2), rtol=1e-6, atol=1e-7)
    assert not np.allclose(y2, y, rtol=1e-6, atol=0)   # the eps term is really there


def test_rope_position_zero_is_identity_and_norm_preserving():
    x = synth.normal(4, 4, (3, 5, 64))
    y0 = oracle.rope(x, np.zeros(3, np.int32), 10000.0)
    assert np.array_equal(y0, x)
    pos = np.array([1, 77, 2047], np.int32)
    y = oracle.rope(x, pos, 10000.0)
    n0 = np.hypot(x[..., 0::2].astype(np.float64), x[..., 1::2])
    n1 = np.hypot(y[..., 0::2].astype(np.float64), y[..., 1::2])
    assert np.allclose(n0, n1, rtol=1e-6)


def test_rope_angles_and_relative_position():
    hd = 64
    # unit vector on every pair: pair i at position m turns by m * base^(-2i/hd)
    e = np.zeros((1, 1, hd), np.float32)
    e[..., 0::2] = 1.0
    for m in (1, 3, 100):
        y = oracle.rope(e, np.array([m], np.int32), 10000.0)[0, 0]
        ang = np.arctan2(y[1::2], y[0::2])
        i = np.arange(hd // 2)
        ref = np.angle(np.exp(1j * m * 10000.0 ** (-2.0 * i / hd)))
        assert np.allclose(ang, ref, atol=2e-6)
    assert np.isclose(np.arctan2(*oracle.rope(e, np.array([1], np.int32), 1e4)[0, 0, [1, 0]]), 1.0)
    # <R_m q, R_n k> depends on m - n only
    q = synth.normal(5, 5, (1, 1, hd))
    k = synth.normal(5, 6, (1, 1, hd))
    dots = []
    for (m, n) in [(10, 3), (17, 10), (1007, 1000)]:
        a = oracle.rope(q, np.array([m], np.int32), 1e4).astype(np.float64)
        b = oracle.rope(k, np.array([n], np.int32), 1e4).astype(np.float64)
        dots.append(float((a * b).sum()))
    assert np.allclose(dots, dots[0], rtol=1e-5)


def test_swiglu_limits_and_library_sigmoid():
    from scipy.special import expit
    g = np.array([0.0, 50.0, -50.0, 1.0, -2.0, 3.5], np.float32)
    u = np.ones_like(g)
    h = oracle.swiglu(g, u)
    assert h[0] == 0.0 and np.isclose(h[1], 50.0) and abs(h[2]) < 1e-18
    gg = synth.normal(6, 7, 1000) * np.float32(4)
    uu = synth.normal(6, 8, 1000)
    ref = gg.astype(np.float64) * expit(gg.astype(np.float64)) * uu
    assert np.allclose(oracle.swiglu(gg, uu), ref, rtol=1e-6, atol=1e-30)


# ---------------------------------------------------------------------------
# KV append and attention
# ---------------------------------------------------------------------------
def test_kv_append_rows_and_fp16_rounding():
    nkv, cap, hd = 2, 8, 32
    kc = np.zeros((2, nkv, cap, hd), np.uint16)
    vc = np.zeros_like(kc)
    k = synth.normal(7, 1, (3, nkv, hd))
    v = synth.normal(7, 2, (3, nkv, hd))
    pos = np.array([0, 5, 5], np.int32)
    seq = np.array([0, 0, 1], np.int32)
    oracle.kv_append(k, v, pos, seq, kc, vc)
    for t in range(3):
        assert np.array_equal(kc[seq[t], :, pos[t]], k[t].astype(np.float16).view(np.uint16))
        assert np.array_equal(vc[seq[t], :, pos[t]], v[t].astype(np.float16).view(np.uint16))
    touched = np.zeros((2, cap), bool)
    touched[seq, pos] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~touched] == 0)


def _caches(seed, seqs, nkv, cap, hd):
    kc = synth.normal(seed, 1, (seqs, nkv, cap, hd)).astype(np.float16).view(np.uint16)
    vc = synth.normal(seed, 2, (seqs, nkv, cap, hd)).astype(np.float16).view(np.uint16)
    return kc, vc


def test_attention_invariants():
    nq, nkv, hd, cap = 4, 2, 32, 16
    q = synth.normal(8, 3, (3, nq, hd))
    kc, vc = _caches(8, 1, nkv, cap, hd)
    seq = np.zeros(3, np.int32)
    # single row -> o = v0
    o = oracle.gqa_attention(q, kc, vc, np.zeros(3, np.int32), seq)
    v0 = oracle.f16_to_f32(vc[0, :, 0])           # [nkv][hd]
    assert np.allclose(o, np.repeat(v0[None], 2, axis=1).reshape(1, nq, hd).repeat(3, 0), atol=0)
    # all-ones V -> weights sum to 1
    ones = np.full_like(vc, np.float16(1.0).view(np.uint16))
    o1 = oracle.gqa_attention(q, kc, ones, np.array([3, 9, 15], np.int32), seq)
    assert np.allclose(o1, 1.0, atol=1e-7)
    # identical keys -> mean of values
    kc_same = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    om = oracle.gqa_attention(q, kc_same, vc, np.array([7, 7, 7], np.int32), seq)
    vm = oracle.f16_to_f32(vc[0, :, :8]).astype(np.float64).mean(1)
    assert np.allclose(om, np.repeat(vm, 2, axis=0)[None].repeat(3, 0), atol=1e-6)
    # causality: rows after pos do not matter
    p = np.array([4, 4, 4], np.int32)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, 5:] ^= 0x1234
    vc2[:, :, 5:] ^= 0x0BAD
    assert np.array_equal(oracle.gqa_attention(q, kc, vc, p, seq), oracle.gqa_attention(q, kc2, vc2, p, seq))


def test_gqa_single_kv_head_equals_broadcast_mha():
    nq, hd, cap = 4, 32, 12
    q = synth.normal(9, 3, (2, nq, hd))
    kc, vc = _caches(9, 1, 1, cap, hd)
    pos = np.array([6, 11], np.int32)
    seq = np.zeros(2, np.int32)
    gqa = oracle.gqa_attention(q, kc, vc, pos, seq)
    mha = oracle.gqa_attention(q, np.repeat(kc, nq, 1), np.repeat(vc, nq, 1), pos, seq)
    assert np.array_equal(gqa, mha)


def test_attention_fp64_bruteforce():
    from scipy.special import softmax
    nq, nkv, hd, cap = 6, 3, 32, 10
    q = synth.normal(10, 3, (2, nq, hd))
    kc, vc = _caches(10, 2, nkv, cap, hd)
    pos = np.array([9, 4], np.int32)
    seq = np.array([1, 0], np.int32)
    o = oracle.gqa_attention(q, kc, vc, pos, seq)
    K = oracle.f16_to_f32(kc).astype(np.float64)
    V = oracle.f16_to_f32(vc).astype(np.float64)
    for t in range(2):
        for h in range(nq):
            g = h // (nq // nkv)
            Kt, Vt = K[seq[t], g, :pos[t] + 1], V[seq[t], g, :pos[t] + 1]
            p = softmax(Kt @ q[t, h].astype(np.float64) / np.sqrt(hd))
            assert np.allclose(o[t, h], p @ Vt, rtol=1e-6, atol=1e-7)


def test_ring_cache_decode_is_sliding_window_bruteforce():
    """ENGINE 8 (the KV arena holds the longest context and is used as a ring
    buffer): decoding past cap one token at a time, position p sits in row
    p % cap, and attention at p equals softmax attention over the positions
    p - cap + 1 .. p of the whole history, brute force in fp64."""
    from scipy.special import softmax
    nq, nkv, hd, cap, steps = 4, 2, 32, 8, 21
    ks = synth.normal(30, 1, (steps, nkv, hd))
    vs = synth.normal(30, 2, (steps, nkv, hd))
    qs = synth.normal(30, 3, (steps, nq, hd))
    kc = np.zeros((1, nkv, cap, hd), np.uint16)
    vc = np.zeros_like(kc)
    seq = np.zeros(1, np.int32)
    Kh = ks.astype(np.float16).astype(np.float64)   # the history as the cache stores it
    Vh = vs.astype(np.float16).astype(np.float64)
    for p in range(steps):
        pos = np.array([p], np.int32)
        oracle.kv_append(ks[p:p + 1], vs[p:p + 1], pos, seq, kc, vc)
        assert np.array_equal(kc[0, :, p % cap], ks[p].astype(np.float16).view(np.uint16))
        o = oracle.gqa_attention(qs[p:p + 1], kc, vc, pos, seq)
        lo = max(0, p - cap + 1)
        for h in range(nq):
            g = h // (nq // nkv)
            w = softmax(Kh[lo:p + 1, g] @ qs[p, h].astype(np.float64) / np.sqrt(hd))
            assert np.allclose(o[0, h], w @ Vh[lo:p + 1, g], rtol=1e-6, atol=1e-7), (p, h)


def test_ring_cache_rejects_multi_token_wrap():
    """Past the wrap, a call holding several tokens of one sequence would
    overwrite rows its own earlier tokens attend to: such calls are
    rejected; one token per sequence is accepted at any position."""
    nkv, hd, cap = 1, 32, 8
    kc = np.zeros((2, nkv, cap, hd), np.uint16)
    vc = np.zeros_like(kc)
    k = synth.normal(31, 1, (2, nkv, hd))
    q = synth.normal(31, 2, (2, 2, hd))
    oracle.kv_append(k, k, np.array([6, 7], np.int32), np.array([0, 0], np.int32), kc, vc)
    oracle.kv_append(k, k, np.array([100, 9], np.int32), np.array([0, 1], np.int32), kc, vc)
    assert np.array_equal(kc[0, 0, 100 % cap], k[0, 0].astype(np.float16).view(np.uint16))
    with pytest.raises(ValueError):
        oracle.kv_append(k, k, np.array([7, 8], np.int32), np.array([0, 0], np.int32), kc, vc)
    with pytest.raises(ValueError):
        oracle.gqa_attention(q, kc, vc, np.array([8, 9], np.int32), np.array([1, 1], np.int32))
    with pytest.raises(ValueError):
        oracle.kv_append(k, k, np.array([-1, 0], np.int32), np.array([0, 1], np.int32), kc, vc)


# ---------------------------------------------------------------------------
# embedding, argmax
# ---------------------------------------------------------------------------
def test_embed_and_argmax():
    table = synth.normal(12, 0, (50, 32))
    ids = np.array([3, 0, 49, 3], np.int32)
    assert np.array_equal(oracle.embed_lookup(table, ids), table[ids])
    logits = np.array([[1.0, 3.0, 3.0, -1.0], [-5, -5, -5, -5], [0, 0, 0, 1]], np.float32)
    assert oracle.argmax(logits).tolist() == [1, 0, 3]
    big = synth.normal(12, 1, (7, 32000))
    assert np.array_equal(oracle.argmax(big), np.argmax(big, axis=1))


# ---------------------------------------------------------------------------
# the decoder layer
# ---------------------------------------------------------------------------
def quantize_layer(wf):
    out = {}
    for name, key in [("w_qkv", "w_qkv"), ("w_o", "w_o"), ("w_gate_up", "w_gu"), ("w_down", "w_down")]:
        q, d = oracle.quantize_q4_0(wf[name])
        out[key + "_q"], out[key + "_d"] = q, d
    out["gamma_attn"] = wf["gamma_attn"]
    out["gamma_ffn"] = wf["gamma_ffn"]
    return out


SMALL = W.Geometry(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=96)


def _np_q8(x):
    """Q8_0 in numpy (float32 division, half away from zero), for the composition check."""
    xb = x.reshape(x.shape[0], -1, 32).astype(np.float32)
    d = np.abs(xb).max(-1) / np.float32(127)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(d[..., None] > 0, xb / d[..., None], 0).astype(np.float32)
    q = np.clip(np.sign(v) * np.floor(np.abs(v) + np.float32(0.5)), -127, 127)
    dh = d.astype(np.float16).astype(np.float64)
    return (q * dh[..., None]).reshape(x.shape)


def _np_layer(wf, g: W.Geometry, x, pos, kcache, vcache):
    """Layer composition in numpy fp64 on dequantized weights (brute force)."""
    def deq(name):
        q, d = oracle.quantize_q4_0(wf[name])
        return (unpack_q4(q) - 8) * oracle.f16_to_f32(d).astype(np.float64).repeat(32, 1)

    def rms(v, gam):
        return v / np.sqrt((v * v).mean(-1, keepdims=True) + np.float32(g.eps)) * gam

    H, nq, nkv, hd, F = g.hidden, g.n_q_heads, g.n_kv_heads, g.head_dim, g.ffn_padded
    T = x.shape[0]
    x = x.astype(np.float64)
    qkv = _np_q8(rms(x, wf["gamma_attn"]).astype(np.float32)) @ deq("w_qkv").T
    q = qkv[:, :nq * hd].reshape(T, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(T, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(T, nkv, hd)
    i = np.arange(hd // 2)
    ang = pos[:, None].astype(np.float64) * g.rope_base ** (-2.0 * i / hd)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]

    def rot(a):
        out = a.copy()
        out[..., 0::2] = a[..., 0::2] * c - a[..., 1::2] * s
        out[..., 1::2] = a[..., 0::2] * s + a[..., 1::2] * c
        return out
    q, k = rot(q), rot(k)
    K = oracle.f16_to_f32(kcache[0]).astype(np.float64)
    V = oracle.f16_to_f32(vcache[0]).astype(np.float64)
    K[:, pos] = k.astype(np.float32).astype(np.float16).astype(np.float64).transpose(1, 0, 2)
    V[:, pos] = v.astype(np.float32).astype(np.float16).astype(np.float64).transpose(1, 0, 2)
    o = np.zeros((T, nq, hd))
    for t in range(T):
        for h in range(nq):
            gi = h // (nq // nkv)
            sc = K[gi, :pos[t] + 1] @ q[t, h] / np.sqrt(hd)
            p = np.exp(sc - sc.max())
            o[t, h] = (p / p.sum()) @ V[gi, :pos[t] + 1]
    x1 = x + _np_q8(o.reshape(T, -1).astype(np.float32)) @ deq("w_o").T
    gu = _np_q8(rms(x1, wf["gamma_ffn"]).astype(np.float32)) @ deq("w_gate_up").T
    gg, uu = gu[:, :F], gu[:, F:]
    hh = gg / (1 + np.exp(-gg)) * uu
    return x1 + _np_q8(hh.astype(np.float32)) @ deq("w_down").T


def test_layer_matches_fp64_composition():
    g = SMALL
    wf = W.layer_weights_f32(21, 0, g)
    wl = quantize_layer(wf)
    cap = 16
    x = synth.normal(21, W.TID_X, (6, g.hidden))
    pos = np.arange(6, dtype=np.int32) + 3
    seq = np.zeros(6, np.int32)
    kc, vc = W.kv_prefill_f16(21, 0, g.n_kv_heads, cap, g.head_dim, 3)
    kc, vc = kc.view(np.uint16), vc.view(np.uint16)
    ref = _np_layer(wf, g, x, pos, kc.copy(), vc.copy())
    out = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
    err = np.abs(out - ref) / np.maximum(np.abs(ref), np.sqrt((ref ** 2).mean()))
    assert err.max() < 1e-4


def test_layer_with_zero_output_weights_is_identity():
    g = SMALL
    wl = quantize_layer(W.layer_weights_f32(22, 0, g))
    wl["w_o_q"][:] = 0x88
    wl["w_down_q"][:] = 0x88
    cap = 8
    x = synth.normal(22, 1, (4, g.hidden))
    kc = np.zeros((1, g.n_kv_heads, cap, g.head_dim), np.uint16)
    vc = kc.copy()
    out = oracle.layer_forward(wl, g.cfg(cap), x, np.arange(4, dtype=np.int32), np.zeros(4, np.int32), kc, vc)
    assert np.array_equal(out, x)


def test_layer_ffn_padding_is_exact():
    """Padding F with zero gate/up rows and zero down columns leaves the layer unchanged."""
    g = SMALL                                   # F = 96 (already a multiple of 32)
    wf = W.layer_weights_f32(23, 0, g)
    F = g.ffn_padded
    wpad = dict(wf)
    gu = np.zeros((2 * (F + 32), g.hidden), np.float32)
    gu[:F] = wf["w_gate_up"][:F]
    gu[F + 32:F + 32 + F] = wf["w_gate_up"][F:]
    wpad["w_gate_up"] = gu
    wpad["w_down"] = np.concatenate([wf["w_down"], np.zeros((g.hidden, 32), np.float32)], 1)
    cap = 8
    x = synth.normal(23, 1, (3, g.hidden))
    pos = np.arange(3, dtype=np.int32)
    seq = np.zeros(3, np.int32)
    outs = []
    for wset, ffn in [(wf, F), (wpad, F + 32)]:
        kc = np.zeros((1, g.n_kv_heads, cap, g.head_dim), np.uint16)
        vc = kc.copy()
        cfg = g.cfg(cap)
        cfg["ffn"] = ffn
        outs.append(oracle.layer_forward(quantize_layer(wset), cfg, x, pos, seq, kc, vc))
    assert np.array_equal(outs[0], outs[1])


def test_layer_decode_equals_last_row_of_prefill():
    g = SMALL
    wl = quantize_layer(W.layer_weights_f32(24, 0, g))
    cap = 16
    x = synth.normal(24, 1, (7, g.hidden))
    pos = np.arange(7, dtype=np.int32)
    seq = np.zeros(7, np.int32)
    shape = (1, g.n_kv_heads, cap, g.head_dim)
    kc, vc = np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)
    full = oracle.layer_forward(wl, g.cfg(cap), x, pos, seq, kc, vc)
    kc2, vc2 = np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)
    oracle.layer_forward(wl, g.cfg(cap), x[:6], pos[:6], seq[:6], kc2, vc2)
    last = oracle.layer_forward(wl, g.cfg(cap), x[6:], pos[6:], seq[6:], kc2, vc2)
    assert np.array_equal(full[6], last[0])
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------
def _experts(seed, E, H, F):
    gq, gd, dq, dd = [], [], [], []
    for e in range(E):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        a, b = oracle.quantize_q4_0(gu)
        c, d = oracle.quantize_q4_0(dn)
        gq.append(a), gd.append(b), dq.append(c), dd.append(d)
    return np.stack(gq), np.stack(gd), np.stack(dq), np.stack(dd)


def test_moe_zero_router_picks_first_k_uniformly():
    T, H, E, F, k = 3, 64, 16, 32, 4
    x = synth.normal(30, 1, (T, H))
    idx, w = oracle.moe_route(x, np.zeros((H, E), np.float32), k)
    assert np.all(idx == np.arange(k)) and np.all(w == np.float32(1 / k))


def test_moe_router_ranking_fp64():
    T, H, E, k = 16, 256, 64, 8
    x = synth.normal(31, 1, (T, H))
    wr = synth.normal(31, 2, (H, E), 0.02)
    idx, w, logits = oracle.moe_route(x, wr, k, return_logits=True)
    r = x.astype(np.float64) @ wr.astype(np.float64)
    assert np.allclose(logits, r, rtol=1e-6, atol=1e-6)
    ref_idx = np.argsort(-r, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref_idx)
    s = 1 / (1 + np.exp(-np.take_along_axis(r, ref_idx, 1)))
    assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=1e-6)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def test_moe_sparse_equals_dense_bruteforce():
    T, H, E, F, k = 4, 64, 8, 32, 3
    x = synth.normal(32, 1, (T, H))
    wr = synth.normal(32, 2, (H, E), 0.3)
    gq, gd, dq, dd = _experts(32, E, H, F)
    out, idx, w = oracle.moe_route_and_apply(x, wr, k, gq, gd, dq, dd)
    # dense: every expert on every token, then select and combine
    dense = np.stack([[oracle.moe_expert_ffn(x[t], gq[e], gd[e], dq[e], dd[e]) for e in range(E)]
                      for t in range(T)])                     # [T][E][H]
    r = x.astype(np.float64) @ wr.astype(np.float64)
    sel = np.argsort(-r, axis=1, kind="stable")[:, :k]
    s = 1 / (1 + np.exp(-np.take_along_axis(r, sel, 1)))
    ww = s / s.sum(1, keepdims=True)
    ref = np.einsum("tk,tkh->th", ww, np.take_along_axis(dense, sel[:, :, None], 1).astype(np.float64))
    assert np.array_equal(idx, sel)
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-7)


def test_moe_identical_experts_give_single_expert_output():
    T, H, E, F, k = 3, 64, 6, 32, 4
    x = synth.normal(33, 1, (T, H))
    wr = synth.normal(33, 2, (H, E), 0.1)
    gq, gd, dq, dd = _experts(33, 1, H, F)
    rep = lambda a: np.repeat(a, E, 0)  # noqa: E731
    out, _, _ = oracle.moe_route_and_apply(x, wr, k, rep(gq), rep(gd), rep(dq), rep(dd))
    for t in range(T):
        single = oracle.moe_expert_ffn(x[t], gq[0], gd[0], dq[0], dd[0])
        assert np.allclose(out[t], single, rtol=1e-6, atol=1e-8)


def _experts_rowq(seed, E, H, F, bits):
    gq, gr, dq, dr = [], [], [], []
    for e in range(E):
        gu, dn = W.expert_weights_f32(seed, e, H, F)
        a, b = oracle.quantize_rowq(gu, bits)
        c, d = oracle.quantize_rowq(dn, bits)
        gq.append(a), gr.append(b), dq.append(c), dr.append(d)
    return np.stack(gq), np.stack(gr), np.stack(dq), np.stack(dr)


@pytest.mark.parametrize("bits", [4, 2])
def test_moe_rowq_sparse_equals_dense_bruteforce(bits):
    """Row-scaled experts: the routed layer equals evaluating every expert on
    every token (Q8_0, row-scaled matmul, SwiGLU, Q8_0, row-scaled matmul),
    then selecting and combining in fp64."""
    T, H, E, F, k = 4, 64, 8, 32, 3
    x = synth.normal(37, 1, (T, H))
    wrt = synth.normal(37, 2, (H, E), 0.3)
    gq, gr, dq, dr = _experts_rowq(37, E, H, F, bits)
    out, idx, w = oracle.moe_route_and_apply_rowq(x, wrt, k, gq, gr, dq, dr, bits)

    def expert(t, e):
        xq, xd = oracle.quantize_q8_0(x[t:t + 1])
        gu = oracle.qmatmul_rowq(gq[e], gr[e], xq, xd, bits)[0]
        h = oracle.swiglu(gu[:F], gu[F:])
        hq, hd = oracle.quantize_q8_0(h[None])
        return oracle.qmatmul_rowq(dq[e], dr[e], hq, hd, bits)[0]

    dense = np.stack([[expert(t, e) for e in range(E)] for t in range(T)])
    r = x.astype(np.float64) @ wrt.astype(np.float64)
    sel = np.argsort(-r, axis=1, kind="stable")[:, :k]
    s = 1 / (1 + np.exp(-np.take_along_axis(r, sel, 1)))
    ww = s / s.sum(1, keepdims=True)
    ref = np.einsum("tk,tkh->th", ww, np.take_along_axis(dense, sel[:, :, None], 1).astype(np.float64))
    assert np.array_equal(idx, sel)
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-7)


def test_expert_ffn_fp64_bruteforce():
    H, F = 64, 64
    x = synth.normal(34, 1, H)
    gu, dn = W.expert_weights_f32(34, 0, H, F)
    a, b = oracle.quantize_q4_0(gu)
    c, d = oracle.quantize_q4_0(dn)
    y = oracle.moe_expert_ffn(x, a, b, c, d)
    deq = lambda q, s: (unpack_q4(q) - 8) * oracle.f16_to_f32(s).astype(np.float64).repeat(32, 1)  # noqa
    g = deq(a, b) @ _np_q8(x[None])[0]
    h = g[:F] / (1 + np.exp(-g[:F])) * g[F:]
    ref = deq(c, d) @ _np_q8(h[None].astype(np.float32))[0]
    assert np.allclose(y, ref, rtol=1e-4, atol=1e-6)


# ---------------------------------------------------------------- sampler chain
def test_sampler_golden_worked_example():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sampler_chain.json")))
    for c in g["cases"]:
        got = oracle.sample(np.array(c["logits"], np.float32), c["top_k"], c["top_p"], c["temperature"], [c["u"]])
        assert int(got[0]) == c["token"], c


def test_sampler_greedy_limits_equal_argmax():
    """top_k = 1, or temperature 0, or top_p tiny: the argmax for every u."""
    logits = synth.normal(120, 1, (6, 300)) * np.float32(3.0)
    logits[2, 10] = logits[2, 200] = 50.0               # tie: the lower id
    want = oracle.argmax(logits)
    for u in (0.0, 0.37, 0.999999):
        assert np.array_equal(oracle.sample(logits, 1, 0.9, 0.7, u), want)
        assert np.array_equal(oracle.sample(logits, 40, 0.9, 0.0, u), want)
        assert np.array_equal(oracle.sample(logits, 40, 1e-9, 1.5, u), want)


def _grid_counts(logits, top_k, top_p, temp, n=20000):
    u = (np.arange(n) + 0.5) / n
    toks = oracle.sample(np.tile(logits, (n, 1)), top_k, top_p, temp, u)
    return np.bincount(toks, minlength=logits.size) / n


def test_sampler_draw_is_softmax_at_temperature():
    """With every id kept, the inverse-CDF draw over a uniform grid of u
    reproduces softmax(l / T) (scipy) to within the grid spacing per id."""
    from scipy.special import softmax
    logits = (synth.normal(121, 1, 37) * np.float32(1.3)).astype(np.float32)
    for temp in (1.0, 2.0, 0.7):
        freq = _grid_counts(logits, 37, 1.0, temp)
        ref = softmax(logits.astype(np.float64) / temp)
        assert np.max(np.abs(freq - ref)) <= 1.0 / 20000 + 1e-12


def test_sampler_top_p_and_top_k_truncation():
    """Probabilities 0.5, 0.3, 0.15, 0.05: top_p = 0.75 keeps the first two,
    which are then drawn with weights 0.625 / 0.375; top_k = 3 with top_p = 1
    renormalizes the first three."""
    p = np.array([0.05, 0.5, 0.15, 0.3])                 # ids 1, 3, 2, 0 by rank
    logits = np.log(p).astype(np.float32)
    freq = _grid_counts(logits, 4, 0.75, 1.0)
    assert abs(freq[1] - 0.625) <= 1e-4 and abs(freq[3] - 0.375) <= 1e-4 and freq[0] == freq[2] == 0
    freq = _grid_counts(logits, 3, 1.0, 1.0)
    assert freq[0] == 0 and abs(freq[1] - 0.5 / 0.95) <= 1e-4 and abs(freq[2] - 0.15 / 0.95) <= 1e-4


def test_sampler_ties_keep_lowest_ids():
    logits = np.zeros(100, np.float32)
    freq = _grid_counts(logits, 2, 1.0, 1.0, n=1000)
    assert abs(freq[0] - 0.5) <= 1e-3 and abs(freq[1] - 0.5) <= 1e-3 and freq[2:].sum() == 0
