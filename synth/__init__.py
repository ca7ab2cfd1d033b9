"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.

This package draws numbers and lays out the workloads' tensors; it holds none
of the method's arithmetic.  The draws themselves (splitmix64, uniform,
Box-Muller) live in ``synth.c``; ``workloads`` names every tensor of every
workload and gives it a stream id.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> None:
    """Compile ``synth.c`` into ``libsynth.so`` (gcc, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_SO)
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_void_p]
        lib.synth_normal_f32.restype = None
        lib.synth_uniform_i32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_uniform_i32.restype = None
        lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_u64.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def normal(seed: int, tensor_id: int, shape, std: float = 1.0, mean: float = 0.0,
           offset: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """fp32 draws of N(mean, std^2): elements [offset, offset + prod(shape)) of
    the stream (seed, tensor_id), in row-major order."""
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    n = int(np.prod(shape)) if shape else 1
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_f32(seed, tensor_id, offset, n, float(mean), float(std),
                             out.ctypes.data)
    return out


def randint(seed: int, tensor_id: int, shape, bound: int, offset: int = 0) -> np.ndarray:
    """int32 draws uniform in [0, bound) from the stream (seed, tensor_id)."""
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(shape, dtype=np.int32)
    _load().synth_uniform_i32(seed, tensor_id, offset, n, bound, out.ctypes.data)
    return out


def u64(seed: int, tensor_id: int, n: int) -> int:
    """The raw n-th splitmix64 output of the stream (seed, tensor_id)."""
    return int(_load().synth_u64(seed, tensor_id, n))
