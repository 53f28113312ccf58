"""ctypes binding of libmsda_micro.so (include/msda_micro.h): the gather and
atomic-scatter measurement kernels, plus the host-side corner table they
read.  Used by bench.py to measure the ceilings of the core's two access
patterns; no part of the MSDeformAttn computation runs here.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsda_micro.so")
EXPORTS = ("msda_micro_gather", "msda_micro_scatter")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m scale_deformable_attention_03_amd.build`")
    import torch  # noqa: F401  (PyTorch's HIP runtime first, as for libmsda.so)
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.msda_micro_gather.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.msda_micro_gather.restype = ctypes.c_int
    lib.msda_micro_scatter.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.msda_micro_scatter.restype = ctypes.c_int
    return lib


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def corner_table(sampling_locations: np.ndarray, spatial_shapes, level_start_index, num_keys: int,
                 lanes: int) -> np.ndarray:
    """uint32 [batch * heads * queries, levels * points * 4]: for every
    (plane, query) group in the core's plane-major order and every sample,
    the first 16-byte vector of its four corner rows (top-left, top-right,
    bottom-left, bottom-right) in a value tensor [batch, keys, heads, D] with
    `lanes` vectors per row.  Pixel coordinates as the core forms them
    (x = loc_x * W - 0.5 and y likewise, float32); corners off the map are
    clamped onto it, so every index is in bounds (the core skips those rows
    instead)."""
    loc = np.asarray(sampling_locations, dtype=np.float32)
    bs, Q, M, L, P, _ = loc.shape
    shapes = np.asarray(spatial_shapes, dtype=np.int64).reshape(L, 2)
    starts = np.asarray(level_start_index, dtype=np.int64).reshape(L)
    H = shapes[:, 0].astype(np.float32)[None, None, None, :, None]
    W = shapes[:, 1].astype(np.float32)[None, None, None, :, None]
    lx = np.nan_to_num(loc[..., 0], nan=-2.0, posinf=2.0, neginf=-2.0)
    ly = np.nan_to_num(loc[..., 1], nan=-2.0, posinf=2.0, neginf=-2.0)
    x = (lx * W).astype(np.float32) - np.float32(0.5)
    y = (ly * H).astype(np.float32) - np.float32(0.5)
    x0 = np.clip(np.floor(x), -2, W + 1).astype(np.int64)
    y0 = np.clip(np.floor(y), -2, H + 1).astype(np.int64)
    Wi = shapes[:, 1][None, None, None, :, None]
    Hi = shapes[:, 0][None, None, None, :, None]
    st = starts[None, None, None, :, None]
    b = np.arange(bs, dtype=np.int64)[:, None, None, None, None]
    m = np.arange(M, dtype=np.int64)[None, None, :, None, None]
    out = np.empty((bs, Q, M, L, P, 4), dtype=np.int64)
    for c, (dy, dx) in enumerate(((0, 0), (0, 1), (1, 0), (1, 1))):
        xc = np.clip(x0 + dx, 0, Wi - 1)
        yc = np.clip(y0 + dy, 0, Hi - 1)
        row = (b * num_keys + st + yc * Wi + xc) * M + m
        out[..., c] = row * lanes
    # plane-major group order: (b, m, q)
    out = out.transpose(0, 2, 1, 3, 4, 5).reshape(bs * M * Q, L * P * 4)
    nvec = bs * num_keys * M * lanes
    if out.min() < 0 or out.max() + lanes > nvec:
        raise ValueError("corner table out of bounds")
    return out.astype(np.uint32)


def gather(rows_ptr: int, table_ptr: int, out_ptr: int, ngroups: int, samples: int, lanes: int, with_fma: bool,
           stream: int) -> None:
    st = lib().msda_micro_gather(rows_ptr, table_ptr, out_ptr, ngroups, samples, lanes, int(with_fma), stream)
    if st != 0:
        raise RuntimeError(f"msda_micro_gather: status {st}")


def scatter(dst_ptr: int, table_ptr: int, ngroups: int, samples: int, lanes: int, lane_contiguous: bool,
            stream: int) -> None:
    st = lib().msda_micro_scatter(dst_ptr, table_ptr, ngroups, samples, lanes, int(lane_contiguous), stream)
    if st != 0:
        raise RuntimeError(f"msda_micro_scatter: status {st}")
