"""CPU oracle for the multi-scale deformable attention core.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``scale_deformable_attention_03_amd``) never imports it, and the two
share no source.

The arithmetic lives in ``msda_oracle.c`` (plain scalar C, float64
accumulation, built with ``-O2 -ffp-contract=off``).  This module only builds
that file with gcc, loads it with ctypes and marshals numpy arrays.

Every float input is widened exactly to float32 by the caller (fp16/bf16 ->
fp32 is exact); outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msda_oracle.c")
_LIB = os.path.join(_HERE, "libmsda_oracle.so")

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def build() -> str:
    """Compile the oracle with gcc (OpenMP, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_forward.argtypes = [_i64] * 7 + [_ptr] * 6 + [ctypes.c_int]
        lib.oracle_forward.restype = None
        lib.oracle_backward.argtypes = [_i64] * 7 + [_ptr] * 9 + [ctypes.c_int]
        lib.oracle_backward.restype = None
        lib.oracle_forward_one.argtypes = [_i64] * 6 + [_ptr] * 5 + [_i64] * 3 + [_ptr]
        lib.oracle_forward_one.restype = None
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle takes float32 inputs (exactly widened), got {a.dtype}")
    return a


def _dims(spatial_shapes, level_start_index, value, loc):
    shapes = np.ascontiguousarray(np.asarray(spatial_shapes, dtype=np.int64).reshape(-1, 2))
    starts = np.ascontiguousarray(np.asarray(level_start_index, dtype=np.int64).reshape(-1))
    bs, K, M, D = value.shape
    bs2, Q, M2, L, P, two = loc.shape
    if bs2 != bs or M2 != M or two != 2 or shapes.shape[0] != L or starts.shape[0] != L:
        raise ValueError("inconsistent shapes")
    return shapes, starts, (bs, K, M, D, L, P, Q)


def threads(nthreads: int = 0) -> int:
    """Threads an oracle call with this ``nthreads`` uses (0 = OpenMP default)."""
    return int(_load().oracle_threads(int(nthreads)))


def forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
            nthreads: int = 0) -> np.ndarray:
    """Oracle forward; returns float64 ``[bs, Q, M*D]``."""
    lib = _load()
    value, loc, w = _f32(value), _f32(sampling_locations), _f32(attention_weights)
    shapes, starts, (bs, K, M, D, L, P, Q) = _dims(spatial_shapes, level_start_index, value, loc)
    if w.shape != (bs, Q, M, L, P):
        raise ValueError("attention_weights shape")
    out = np.empty((bs, Q, M * D), dtype=np.float64)
    lib.oracle_forward(bs, K, M, D, L, P, Q, shapes.ctypes.data, starts.ctypes.data,
                       value.ctypes.data, loc.ctypes.data, w.ctypes.data, out.ctypes.data,
                       int(nthreads))
    return out


def forward_one(value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights, b: int, q: int, m: int) -> np.ndarray:
    """Oracle forward at one (b, q, m); returns float64 ``[D]``."""
    lib = _load()
    value, loc, w = _f32(value), _f32(sampling_locations), _f32(attention_weights)
    shapes, starts, (bs, K, M, D, L, P, Q) = _dims(spatial_shapes, level_start_index, value, loc)
    if not (0 <= b < bs and 0 <= q < Q and 0 <= m < M):
        raise IndexError("(b, q, m) out of range")
    out = np.empty((D,), dtype=np.float64)
    lib.oracle_forward_one(K, M, D, L, P, Q, shapes.ctypes.data, starts.ctypes.data,
                           value.ctypes.data, loc.ctypes.data, w.ctypes.data, b, q, m,
                           out.ctypes.data)
    return out


def backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
             grad_output, nthreads: int = 0):
    """Oracle backward; returns float64 ``(grad_value, grad_loc, grad_w)``."""
    lib = _load()
    value, loc, w = _f32(value), _f32(sampling_locations), _f32(attention_weights)
    g = _f32(grad_output)
    shapes, starts, (bs, K, M, D, L, P, Q) = _dims(spatial_shapes, level_start_index, value, loc)
    if w.shape != (bs, Q, M, L, P) or g.shape != (bs, Q, M * D):
        raise ValueError("attention_weights / grad_output shape")
    gv = np.empty((bs, K, M, D), dtype=np.float64)
    gl = np.empty((bs, Q, M, L, P, 2), dtype=np.float64)
    gw = np.empty((bs, Q, M, L, P), dtype=np.float64)
    lib.oracle_backward(bs, K, M, D, L, P, Q, shapes.ctypes.data, starts.ctypes.data,
                        value.ctypes.data, loc.ctypes.data, w.ctypes.data, g.ctypes.data,
                        gv.ctypes.data, gl.ctypes.data, gw.ctypes.data, int(nthreads))
    return gv, gl, gw
