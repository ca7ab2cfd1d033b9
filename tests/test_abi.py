"""The C-ABI library without a GPU: it loads, exports every entry point that
include/qk.h declares, and its host-only helpers behave as documented.
Nothing here enqueues device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import quantized_q4_q8_amd as qk
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qk.h")


def declared_functions():
    """Names of the functions the header declares (a return type at the start
    of a line, then the name and an opening parenthesis)."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    pat = re.compile(r"^(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*|void)\s*\*?\s*(\w+)\s*\(", re.M)
    return sorted(set(pat.findall(text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qk.LIB_PATH):
        from quantized_q4_q8_amd import build as b
        b.build()
    return qk.load()


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("quantize_q8_0", "qmatmul_q4_0_q8_0", "rmsnorm", "rope", "gqa_attention",
              "swiglu", "moe_route_and_apply", "layer_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(qk.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_binding_covers_the_header(lib):
    assert set(qk.EXPORTS) == set(declared_functions())


def test_strerror_host_only(lib):
    for code in (0, -1, -2, -3, -4, -5):
        s = qk.strerror(code)
        assert isinstance(s, str) and s
    assert qk.strerror(-99)          # unknown codes still give text


def test_q4_0_from_blocks_host(lib):
    """Interleaved 18-byte blocks (fp16 scale, 16 nibble bytes) to the split
    layout, on host memory: the inverse of packing the oracle's split output."""
    n, k = 7, 96
    w = synth.normal(5, 1, (n, k), 0.02)
    wq, wd = oracle.quantize_q4_0(w)
    nb = k // 32
    aos = np.zeros((n, nb, 18), np.uint8)
    aos[:, :, 0:2] = wd.reshape(n, nb, 1).view(np.uint8).reshape(n, nb, 2)
    aos[:, :, 2:] = wq.reshape(n, nb, 16)
    out_q = np.zeros_like(wq)
    out_d = np.zeros_like(wd)
    f = lib.qk_q4_0_from_blocks
    st = f(aos.ctypes.data_as(ctypes.c_void_p), n, k, out_q.ctypes.data_as(ctypes.c_void_p),
           out_d.ctypes.data_as(ctypes.c_void_p))
    assert st == 0
    assert np.array_equal(out_q, wq) and np.array_equal(out_d, wd)
    assert f(aos.ctypes.data_as(ctypes.c_void_p), n, 33, out_q.ctypes.data_as(ctypes.c_void_p),
             out_d.ctypes.data_as(ctypes.c_void_p)) == -2


def test_workspace_queries_host_only(lib):
    """Size queries are pure host arithmetic: positive for valid shapes and
    non-decreasing in the token count."""
    cfg = qk.layer_cfg(hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=64, ffn=5632,
                       eps=1e-5, rope_base=1e4, cap=2176)
    a = lib.qk_layer_workspace(ctypes.byref(cfg), 1)
    b = lib.qk_layer_workspace(ctypes.byref(cfg), 512)
    assert 0 < a <= b
    assert lib.qk_ffn_up_workspace(2048, 1) > 0
    assert lib.qk_lm_head_workspace(32000, 2048, 1) > 0
    assert lib.qk_gqa_attention_workspace(4, 32, 64, 2176) > 0
    assert lib.qk_moe_workspace(64, 6144, 256, 8, 2048) > 0


def test_scratch_size_constant_matches_header():
    """The binding's QK_SCRATCH_BYTES is the header's."""
    m = re.search(r"#define QK_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == qk.QK_SCRATCH_BYTES


def test_decode_greedy_validation_host_only(lib):
    """qk_decode_greedy checks its arguments on the host before it touches the
    device: missing pointers, too many layers, a logits buffer without rows
    and misaligned tables give their codes, and zero tokens return at once."""
    cfg = qk.layer_cfg(hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=64, ffn=5632,
                       eps=1e-5, rope_base=1e4, cap=2176)
    fake = 4096   # never dereferenced: every call below returns before any device work

    def dec(**kw):
        f = dict(layers=fake, n_layers=22, embed=fake, gamma_final=fake, lm_q=fake, lm_d=fake,
                 vocab=32000, k_cache=fake, v_cache=fake)
        f.update(kw)
        return qk.DecoderStruct(**f)

    def call(m, n_tokens=4, first=fake, forced=None, out=fake, logits=None, rows=0):
        return lib.qk_decode_greedy(ctypes.byref(m) if m is not None else None, ctypes.byref(cfg),
                                    first, forced, 2048, n_tokens, out, logits, rows, 0, None, 0, None)

    assert call(None) == qk.QK_EINVAL
    assert call(dec(n_layers=0)) == qk.QK_EINVAL
    assert call(dec(n_layers=65)) == qk.QK_ESHAPE           # more layers than the kernel's table holds
    assert call(dec(), n_tokens=0) == qk.QK_OK               # nothing to do, nothing enqueued
    assert call(dec(), n_tokens=-1) == qk.QK_EINVAL
    assert call(dec(embed=None)) == qk.QK_EINVAL
    assert call(dec(), out=None) == qk.QK_EINVAL
    assert call(dec(), first=None, forced=None) == qk.QK_EINVAL   # no first id and no forced ids
    assert call(dec(), logits=fake, rows=0) == qk.QK_EINVAL
    assert call(dec(embed=fake + 4)) == qk.QK_EALIGN
    assert lib.qk_decode_workspace(None) == 0
    flag = ctypes.c_int32(7)
    assert lib.qk_decode_error(None, ctypes.byref(cfg), ctypes.byref(flag)) == qk.QK_EINVAL
    assert flag.value == 7


C_PROGRAM = r"""
#include <stdio.h>
#include "qk.h"

int main(void) {
    qk_layer_cfg cfg = {2048, 32, 4, 64, 5632, 1e-5f, 10000.0f, 2176};
    size_t one = qk_layer_workspace(&cfg, 1), many = qk_layer_workspace(&cfg, 512);
    size_t att = qk_gqa_attention_workspace(4, 32, 64, 2176);
    printf("%s|%s|%d|%d\n", qk_strerror(QK_OK), qk_strerror(QK_ESHAPE),
           one > 0 && one <= many, att > 0);
    return 0;
}
"""


def test_header_is_c_and_links_from_c(lib, tmp_path):
    """The header is plain C: a C11 program (pedantic, warnings as errors)
    includes it, links libqk.so and calls its host-only entry points."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    src, exe = tmp_path / "abi.c", tmp_path / "abi"
    src.write_text(C_PROGRAM)
    libdir = os.path.dirname(qk.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-lqk", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=60).stdout
    ok, eshape, ws_ok, att_ok = out.strip().split("|")
    assert ok == lib.qk_strerror(qk.QK_OK).decode() and eshape == lib.qk_strerror(qk.QK_ESHAPE).decode()
    assert ws_ok == "1" and att_ok == "1"
