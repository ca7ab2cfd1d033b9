"""The C ABI from a plain C11 caller, with no Python or torch in the
process: gcc builds a program against include/qk.h and the HIP runtime API
that allocates device memory, runs quantize_q8_0 and qmatmul_q4_0_q8_0 on
the GPU (default stream) and writes the results; they equal the oracle's
(Q8_0 bit-exact, the matmul to the last fp32 bit).  A call with k % 32 != 0
returns QK_ESHAPE."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth
from tests.util import assert_same_fp32, rel_err, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

C_SOURCE = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "qk.h"

static void* load(const char* dir, const char* name, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    void* b = malloc(n ? n : 1);
    size_t got = f && b ? fread(b, 1, n, f) : 0;
    if (f) fclose(f);
    return got == n ? b : NULL;
}

static int save(const char* dir, const char* name, const void* b, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    size_t put = f ? fwrite(b, 1, n, f) : 0;
    if (f) fclose(f);
    return put == n;
}

#define HIP_OK(call) do { if ((call) != hipSuccess) { printf("hip error at %d\n", __LINE__); return 3; } } while (0)

int main(int argc, char** argv) {
    if (argc != 5) return 2;
    const char* dir = argv[1];
    const int64_t n = atol(argv[2]), k = atol(argv[3]), m = atol(argv[4]);
    const size_t wq_b = (size_t)(n * k / 2), wd_b = (size_t)(n * (k / 32)) * 2;
    const size_t x_b = (size_t)(m * k) * 4, xq_b = (size_t)(m * k), xd_b = (size_t)(m * (k / 32)) * 2;
    const size_t y_b = (size_t)(m * n) * 4;
    void* wq = load(dir, "wq.bin", wq_b);
    void* wd = load(dir, "wd.bin", wd_b);
    void* x = load(dir, "x.bin", x_b);
    void *xq = malloc(xq_b), *xd = malloc(xd_b), *y = malloc(y_b);
    if (!wq || !wd || !x || !xq || !xd || !y) return 2;
    void *d_wq, *d_wd, *d_x, *d_xq, *d_xd, *d_y;
    HIP_OK(hipMalloc(&d_wq, wq_b));
    HIP_OK(hipMalloc(&d_wd, wd_b));
    HIP_OK(hipMalloc(&d_x, x_b));
    HIP_OK(hipMalloc(&d_xq, xq_b));
    HIP_OK(hipMalloc(&d_xd, xd_b));
    HIP_OK(hipMalloc(&d_y, y_b));
    HIP_OK(hipMemcpy(d_wq, wq, wq_b, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_wd, wd, wd_b, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, x_b, hipMemcpyHostToDevice));
    int rc = quantize_q8_0((const float*)d_x, m, k, (int8_t*)d_xq, (uint16_t*)d_xd, NULL);
    if (rc != QK_OK) { printf("quantize_q8_0: %s\n", qk_strerror(rc)); return 1; }
    rc = qmatmul_q4_0_q8_0((const uint8_t*)d_wq, (const uint16_t*)d_wd, n, k, (const int8_t*)d_xq,
                           (const uint16_t*)d_xd, m, (float*)d_y, NULL);
    if (rc != QK_OK) { printf("qmatmul_q4_0_q8_0: %s\n", qk_strerror(rc)); return 1; }
    const int bad = qmatmul_q4_0_q8_0((const uint8_t*)d_wq, (const uint16_t*)d_wd, n, 40,
                                      (const int8_t*)d_xq, (const uint16_t*)d_xd, m, (float*)d_y, NULL);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(xq, d_xq, xq_b, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(xd, d_xd, xd_b, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, d_y, y_b, hipMemcpyDeviceToHost));
    if (!save(dir, "xq.out", xq, xq_b) || !save(dir, "xd.out", xd, xd_b) || !save(dir, "y.out", y, y_b))
        return 2;
    printf("ok %d\n", bad);
    hipFree(d_wq); hipFree(d_wd); hipFree(d_x); hipFree(d_xq); hipFree(d_xd); hipFree(d_y);
    free(wq); free(wd); free(x); free(xq); free(xd); free(y);
    return 0;
}
"""


@pytest.fixture(scope="module")
def c_caller(gpu_lib, tmp_path_factory):
    """The C program, built with gcc (C11, warnings as errors)."""
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("c_caller")
    src, exe = d / "caller.c", d / "caller"
    src.write_text(C_SOURCE)
    libdir = os.path.dirname(gpu_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), "-L", libdir, "-lqk", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], check=True)
    return str(exe)


@pytest.mark.gpu
@pytest.mark.parametrize("n,k,m", [(300, 2048, 1), (64, 5632, 5), (96, 256, 20)])
def test_c_caller_quantize_and_matmul(c_caller, tmp_path, n, k, m):
    say(f"C caller: quantize_q8_0 + qmatmul_q4_0_q8_0 n={n} k={k} m={m}")
    w = synth.normal(113, n + k, (n, k), 0.02)
    x = synth.normal(114, n + k + m, (m, k))
    wq, wd = oracle.quantize_q4_0(w)
    (tmp_path / "wq.bin").write_bytes(np.ascontiguousarray(wq, np.uint8).tobytes())
    (tmp_path / "wd.bin").write_bytes(np.ascontiguousarray(wd, np.uint16).tobytes())
    (tmp_path / "x.bin").write_bytes(np.ascontiguousarray(x, np.float32).tobytes())
    r = subprocess.run([c_caller, str(tmp_path), str(n), str(k), str(m)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split() == ["ok", "-2"], r.stdout   # QK_ESHAPE for k = 40
    xq = np.fromfile(tmp_path / "xq.out", np.int8).reshape(m, k)
    xd = np.fromfile(tmp_path / "xd.out", np.uint16).reshape(m, k // 32)
    y = np.fromfile(tmp_path / "y.out", np.float32).reshape(m, n)
    oq, od = oracle.quantize_q8_0(x)
    assert np.array_equal(xq, oq) and np.array_equal(xd, od)
    ref = oracle.qmatmul(wq, wd, oq, od)
    assert rel_err(y, ref) < 1e-5
    assert_same_fp32(y, ref)
