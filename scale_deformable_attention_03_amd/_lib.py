"""ctypes binding of libmsda.so (the C ABI declared in include/msda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind these calls.  There is no fallback: if the library is missing
the import of this module fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsda.so")

MSDA_F32, MSDA_F16, MSDA_BF16 = 0, 1, 2
# mixed precision: fp16 / bf16 value side, float32 per-sample tensors
MSDA_F16_F32, MSDA_BF16_F32 = 3, 4
STATUS = {0: "MSDA_SUCCESS", 1: "MSDA_ERROR_INVALID_VALUE", 2: "MSDA_ERROR_NOT_SUPPORTED",
          3: "MSDA_ERROR_MISALIGNED", 4: "MSDA_ERROR_HIP"}
EXPORTS = ("msda_validate", "msda_forward", "msda_backward_workspace_bytes", "msda_backward",
           "msda_backward_accumulate", "msda_backward_profile", "msda_forward_fused",
           "msda_backward_fused", "msda_status_string", "msda_abi_version",
           "msda_backward_noalloc", "msda_backward_noalloc_max_workspace", "msda_forward_train",
           "msda_backward_counted", "msda_backward_counted_profile")
BACKWARD_STAGES = ("zero_fill", "count", "scan", "gradient", "accumulate", "narrow")


class MsdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Problem(ctypes.Structure):
    """msda_problem_t."""
    _fields_ = [("batch", ctypes.c_int32), ("num_keys", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("embed_dims", ctypes.c_int32),
                ("num_levels", ctypes.c_int32), ("num_points", ctypes.c_int32),
                ("num_queries", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("spatial_shapes", ctypes.POINTER(ctypes.c_int64)),
                ("level_start_index", ctypes.POINTER(ctypes.c_int64))]


def make_problem(batch, num_keys, num_heads, embed_dims, num_levels, num_points, num_queries,
                 dtype: int, spatial_shapes, level_start_index):
    """Build a Problem; returns (problem, keepalive) -- keep the second alive
    for as long as the first is used (it owns the host shape arrays)."""
    shapes = np.ascontiguousarray(np.asarray(spatial_shapes, dtype=np.int64).reshape(-1))
    starts = np.ascontiguousarray(np.asarray(level_start_index, dtype=np.int64).reshape(-1))
    p = Problem(int(batch), int(num_keys), int(num_heads), int(embed_dims), int(num_levels),
                int(num_points), int(num_queries), int(dtype),
                shapes.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return p, (shapes, starts)


def _hip_runtimes() -> set:
    """Paths of every HIP runtime (libamdhip64) mapped into this process."""
    with open("/proc/self/maps") as f:
        return {line.split()[-1] for line in f if "libamdhip64" in line}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m scale_deformable_attention_03_amd.build`")
    # PyTorch ships its own HIP runtime.  Load it first, so that libmsda.so's
    # dependency on libamdhip64.so.7 resolves to that same, already loaded
    # runtime (matched by soname).  Loaded the other way round, the process
    # would hold two HIP runtimes, and handles of one (streams, allocations)
    # would be passed to the other.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("more than one HIP runtime is loaded in this process "
                          f"({sorted(runtimes)}); import torch before anything that loads "
                          "/opt/rocm's libamdhip64")
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    lib.msda_validate.argtypes = [P]
    lib.msda_validate.restype = ctypes.c_int
    lib.msda_forward.argtypes = [P, vp, vp, vp, vp, vp]
    lib.msda_forward.restype = ctypes.c_int
    lib.msda_backward_workspace_bytes.argtypes = [P]
    lib.msda_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.msda_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msda_backward.restype = ctypes.c_int
    lib.msda_backward_accumulate.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msda_backward_accumulate.restype = ctypes.c_int
    lib.msda_backward_profile.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.msda_backward_profile.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.msda_forward_fused.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.msda_forward_fused.restype = ctypes.c_int
    lib.msda_backward_fused.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msda_backward_fused.restype = ctypes.c_int
    lib.msda_backward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.msda_backward_noalloc.restype = ctypes.c_int
    lib.msda_backward_noalloc_max_workspace.argtypes = []
    lib.msda_backward_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.msda_forward_train.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msda_forward_train.restype = ctypes.c_int
    lib.msda_backward_counted.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msda_backward_counted.restype = ctypes.c_int
    lib.msda_backward_counted_profile.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.msda_backward_counted_profile.restype = ctypes.c_int
    lib.msda_status_string.argtypes = [ctypes.c_int]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_abi_version.argtypes = []
    lib.msda_abi_version.restype = ctypes.c_int32
    return lib


lib = _load()


def validate(problem: Problem) -> int:
    return lib.msda_validate(ctypes.byref(problem))


def workspace_bytes(problem: Problem) -> int:
    return int(lib.msda_backward_workspace_bytes(ctypes.byref(problem)))


def forward(problem: Problem, value: int, loc: int, w: int, out: int, stream: int) -> None:
    st = lib.msda_forward(ctypes.byref(problem), value, loc, w, out, stream)
    if st != 0:
        raise MsdaError(st, "msda_forward")


def backward(problem: Problem, value: int, loc: int, w: int, gout: int, gvalue: int, gloc: int,
             gw: int, workspace: int, workspace_bytes_: int, stream: int) -> None:
    st = lib.msda_backward(ctypes.byref(problem), value, loc, w, gout, gvalue, gloc, gw,
                           workspace, workspace_bytes_, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward")


def forward_train(problem: Problem, value: int, loc: int, w: int, out: int, workspace: int,
                  workspace_bytes_: int, stream: int) -> None:
    """msda_forward that also counts the backward's records into the
    workspace, for a following backward_counted on the same workspace."""
    st = lib.msda_forward_train(ctypes.byref(problem), value, loc, w, out, workspace, workspace_bytes_, stream)
    if st != 0:
        raise MsdaError(st, "msda_forward_train")


def backward_counted(problem: Problem, value: int, loc: int, w: int, gout: int, gvalue: int, gloc: int,
                     gw: int, workspace: int, workspace_bytes_: int, stream: int) -> None:
    """msda_backward after forward_train on the same locations and workspace."""
    st = lib.msda_backward_counted(ctypes.byref(problem), value, loc, w, gout, gvalue, gloc, gw,
                                   workspace, workspace_bytes_, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward_counted")


def backward_accumulate(problem: Problem, value: int, loc: int, w: int, gout: int, gacc: int,
                        gloc: int, gw: int, workspace: int, workspace_bytes_: int, stream: int) -> None:
    st = lib.msda_backward_accumulate(ctypes.byref(problem), value, loc, w, gout, gacc, gloc, gw,
                                      workspace, workspace_bytes_, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward_accumulate")


def backward_noalloc(problem: Problem, value: int, loc: int, w: int, gout: int, gvalue: int, gloc: int,
                     gw: int, stream: int) -> None:
    """msda_backward with the library's own scratch memory as its workspace
    (no allocation; at most noalloc_max_workspace() bytes of workspace)."""
    st = lib.msda_backward_noalloc(ctypes.byref(problem), value, loc, w, gout, gvalue, gloc, gw, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward_noalloc")


def noalloc_max_workspace() -> int:
    return int(lib.msda_backward_noalloc_max_workspace())


def backward_profile(problem: Problem, value: int, loc: int, w: int, gout: int, gvalue: int, gloc: int,
                     gw: int, workspace: int, workspace_bytes_: int, events, stream: int) -> None:
    """msda_backward with HIP events recorded between its stages (events: a
    ctypes array of len(BACKWARD_STAGES) + 1 hipEvent_t handles)."""
    st = lib.msda_backward_profile(ctypes.byref(problem), value, loc, w, gout, gvalue, gloc, gw,
                                   workspace, workspace_bytes_, events, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward_profile")


def backward_counted_profile(problem: Problem, value: int, loc: int, w: int, gout: int, gvalue: int, gloc: int,
                             gw: int, workspace: int, workspace_bytes_: int, events, stream: int) -> None:
    """backward_counted with the stage events of backward_profile."""
    st = lib.msda_backward_counted_profile(ctypes.byref(problem), value, loc, w, gout, gvalue, gloc, gw,
                                           workspace, workspace_bytes_, events, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward_counted_profile")


def forward_fused(problem: Problem, ref_dims: int, value: int, mask: int, ref: int, off: int, logits: int,
                  out: int, stream: int) -> None:
    """mask: device address of the uint8 key padding mask, or 0 for none."""
    st = lib.msda_forward_fused(ctypes.byref(problem), ref_dims, value, mask, ref, off, logits, out, stream)
    if st != 0:
        raise MsdaError(st, "msda_forward_fused")


def backward_fused(problem: Problem, ref_dims: int, value: int, mask: int, ref: int, off: int, logits: int,
                   gout: int, gvalue: int, goff: int, glogits: int, workspace: int, workspace_bytes_: int,
                   stream: int) -> None:
    st = lib.msda_backward_fused(ctypes.byref(problem), ref_dims, value, mask, ref, off, logits, gout, gvalue,
                                 goff, glogits, workspace, workspace_bytes_, stream)
    if st != 0:
        raise MsdaError(st, "msda_backward_fused")
