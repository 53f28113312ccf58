"""Host-only checks of the C ABI (no GPU needed, no kernel launched).

  * libmsda.so loads and exports every function include/msda.h declares;
  * msda_validate enforces the envelope of the Ascend DrivingSDK API page
    (constraints: num_levels*num_points <= 64, num_heads <= 8,
    embed_dims <= 256; parameter list: embed_dims a multiple of 8) and the
    consistency MSDeformAttn.forward asserts in the Deformable DETR
    walkthrough (section 2.2.4: sum of H*W equals the flattened length);
  * pointer checks (NULL, misalignment) and the workspace size check return
    before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from scale_deformable_attention_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")

OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3

DETR = [(100, 134), (50, 67), (25, 34), (13, 17)]


def starts(shapes):
    hw = [h * w for h, w in shapes]
    return [int(sum(hw[:i])) for i in range(len(hw))]


def prob(bs=2, shapes=DETR, M=8, D=32, P=4, Q=300, dtype=0, K=None, st=None):
    K = sum(h * w for h, w in shapes) if K is None else K
    st = starts(shapes) if st is None else st
    return _lib.make_problem(bs, K, M, D, len(shapes), P, Q, dtype, shapes, st)


def test_every_declared_symbol_is_exported():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\S.*?\b(msda_[a-z_]+)\s*\(", text, flags=re.M))
    assert declared == set(_lib.EXPORTS), declared
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert _lib.lib.msda_abi_version() == 1


def test_status_strings():
    for code, name in _lib.STATUS.items():
        assert _lib.lib.msda_status_string(code).decode() == name
    assert _lib.lib.msda_status_string(99).decode() == "MSDA_UNKNOWN_STATUS"


@pytest.mark.parametrize("kw", [dict(), dict(dtype=1), dict(dtype=2), dict(dtype=3), dict(dtype=4), dict(D=8),
                                dict(D=256),
                                dict(M=1), dict(M=8), dict(P=16), dict(shapes=[(1, 1)], P=64),
                                dict(bs=0), dict(Q=0), dict(shapes=[(3, 1)] * 64, P=1)])
def test_valid_descriptors(kw):
    p, keep = prob(**kw)
    assert _lib.validate(p) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(D=12), UNSUPPORTED),            # not a multiple of 8
    (dict(D=264), UNSUPPORTED),           # > 256
    (dict(M=9), UNSUPPORTED),             # > 8 heads
    (dict(P=17), UNSUPPORTED),            # L*P = 68 > 64
    (dict(D=0), INVALID),
    (dict(M=0), INVALID),
    (dict(P=0), INVALID),
    (dict(bs=-1), INVALID),
    (dict(Q=-3), INVALID),
    (dict(dtype=7), INVALID),
    (dict(dtype=5), INVALID),
    (dict(K=17820), INVALID),             # sum of H*W differs from num_keys
    (dict(st=[0, 13400, 16750, 17601]), INVALID),   # not the exclusive prefix sum
    (dict(st=[1, 13401, 16751, 17601]), INVALID),
    (dict(shapes=[(0, 5)], K=0), INVALID),
    (dict(shapes=[(4, -2)], K=-8), INVALID),
])
def test_invalid_descriptors(kw, code):
    p, keep = prob(**kw)
    assert _lib.validate(p) == code


def test_index_range_limit():
    # per batch, value and output bytes stay below 2^31 (32-bit byte offsets)
    p, keep = prob(shapes=[(4096, 2048)], M=8, D=256, P=1, Q=1)
    assert _lib.validate(p) == UNSUPPORTED
    p, keep = prob(shapes=[(4096, 2048)], M=1, D=64, P=1, Q=1)              # 2^31 bytes exactly
    assert _lib.validate(p) == UNSUPPORTED
    p, keep = prob(shapes=[(4096, 2048)], M=1, D=64, P=1, Q=1, dtype=1)     # fp16: 2^30 bytes
    assert _lib.validate(p) == OK
    p, keep = prob(shapes=[(64, 64)], K=None, M=8, D=256, P=1, Q=1 << 18)   # output 2^31 bytes
    assert _lib.validate(p) == UNSUPPORTED


def test_null_descriptor_and_null_shape_arrays():
    lib = _lib.lib
    assert lib.msda_validate(None) == INVALID
    p, keep = prob()
    p.spatial_shapes = ctypes.POINTER(ctypes.c_int64)()
    assert _lib.validate(p) == INVALID


def test_workspace_bytes():
    # fp32: the binned transpose only (up to 4 records of 12 bytes per sample,
    # plus counts, cursors and the unit list); fp16/bf16 add a float32
    # grad_value accumulator.
    p, keep = prob(dtype=0)
    f32 = _lib.workspace_bytes(p)
    samples = 2 * 300 * 8 * 4 * 4
    assert 48 * samples <= f32 < 48 * samples + (8 << 20)
    for dt in (1, 2, 3, 4):          # fp16, bf16 and the mixed codes (16-bit values)
        p, keep = prob(dtype=dt)
        assert _lib.workspace_bytes(p) == f32 + 2 * 17821 * 8 * 32 * 4
    p, keep = prob(dtype=1, D=12)
    assert _lib.workspace_bytes(p) == 0   # invalid descriptor
    p, keep = prob(bs=0)
    assert _lib.workspace_bytes(p) == 0   # empty problem


def _fwd(p, v, loc, w, out):
    return _lib.lib.msda_forward(ctypes.byref(p), v, loc, w, out, None)


def test_forward_pointer_checks_return_before_launch():
    p, keep = prob()
    good = 0x10000
    assert _fwd(p, None, good, good, good) == INVALID
    assert _fwd(p, good, good, good, None) == INVALID
    assert _fwd(p, good + 4, good, good, good) == MISALIGNED
    assert _fwd(p, good, good, good + 8, good) == MISALIGNED
    bad, keep2 = prob(D=12)
    assert _fwd(bad, good, good, good, good) == UNSUPPORTED


def test_backward_pointer_and_workspace_checks_return_before_launch():
    lib = _lib.lib
    good = 0x10000
    p, keep = prob(dtype=2)
    need = _lib.workspace_bytes(p)
    assert need > 0
    args = [good] * 7
    assert lib.msda_backward(ctypes.byref(p), *args, None, need, None) == INVALID      # no workspace
    assert lib.msda_backward(ctypes.byref(p), *args, good, need - 16, None) == INVALID  # too small
    assert lib.msda_backward(ctypes.byref(p), *args, good + 2, need, None) == MISALIGNED
    for i in range(7):
        a = list(args)
        a[i] = None
        assert lib.msda_backward(ctypes.byref(p), *a, good, need, None) == INVALID, i
        a[i] = good + 4
        assert lib.msda_backward(ctypes.byref(p), *a, good, need, None) == MISALIGNED, i


def test_empty_tensors_may_be_null():
    # Q = 0: locations / weights / output have no elements and may be NULL;
    # nothing is enqueued by the forward.
    p, keep = prob(Q=0)
    assert _fwd(p, 0x10000, None, None, None) == OK


def test_single_hip_runtime_in_process():
    """libmsda.so must share PyTorch's HIP runtime (one libamdhip64 mapped)."""
    assert len(_lib._hip_runtimes()) == 1, _lib._hip_runtimes()


def test_noalloc_rejects_problems_beyond_its_scratch():
    """msda_backward_noalloc refuses, before anything is enqueued, a problem
    whose workspace exceeds its scratch array (the encoder's is over 200 MB)."""
    lib = _lib.lib
    assert _lib.noalloc_max_workspace() == 64 << 20
    p, keep = prob(Q=17821)
    assert _lib.workspace_bytes(p) > _lib.noalloc_max_workspace()
    good = 0x10000
    assert lib.msda_backward_noalloc(ctypes.byref(p), *([good] * 7), None) == UNSUPPORTED
    bad, keep2 = prob(D=12)
    assert lib.msda_backward_noalloc(ctypes.byref(bad), *([good] * 7), None) == UNSUPPORTED
    assert lib.msda_backward_noalloc(ctypes.byref(p), None, *([good] * 6), None) == INVALID


def test_training_pair_checks_return_before_launch():
    """msda_forward_train checks its workspace like the backward (missing,
    short, misaligned) and msda_backward_counted has msda_backward's checks,
    all before anything is enqueued."""
    lib = _lib.lib
    good = 0x10000
    p, keep = prob(dtype=0)
    need = _lib.workspace_bytes(p)
    assert need > 0
    ft = lib.msda_forward_train
    assert ft(ctypes.byref(p), good, good, good, good, None, need, None) == INVALID        # no workspace
    assert ft(ctypes.byref(p), good, good, good, good, good, need - 16, None) == INVALID   # too small
    assert ft(ctypes.byref(p), good, good, good, good, good + 2, need, None) == MISALIGNED
    assert ft(ctypes.byref(p), None, good, good, good, good, need, None) == INVALID
    assert ft(ctypes.byref(p), good, good, good + 4, good, good, need, None) == MISALIGNED
    bad, keep2 = prob(D=12)
    assert ft(ctypes.byref(bad), good, good, good, good, good, need, None) == UNSUPPORTED
    args = [good] * 7
    bc = lib.msda_backward_counted
    assert bc(ctypes.byref(p), *args, None, need, None) == INVALID
    assert bc(ctypes.byref(p), *args, good, need - 16, None) == INVALID
    for i in range(7):
        a = list(args)
        a[i] = None
        assert bc(ctypes.byref(p), *a, good, need, None) == INVALID, i
    assert lib.msda_backward_counted_profile(ctypes.byref(p), *args, good, need, None, None) == INVALID  # no events
