"""PyTorch-facing entry points of the MSDeformAttn core.

Signature and layouts follow the Ascend DrivingSDK API page for
multi_scale_deformable_attn (prototype and parameter list):

    ms_deform_attn(value, spatial_shapes, level_start_index,
                   sampling_locations, attention_weights) -> output

    value               [bs, num_keys, num_heads, embed_dims]
    spatial_shapes      [num_levels, 2] (H, W), int32/int64, any device
    level_start_index   [num_levels],  int32/int64, any device
    sampling_locations  [bs, num_queries, num_heads, num_levels, num_points, 2]
    attention_weights   [bs, num_queries, num_heads, num_levels, num_points]
    output              [bs, num_queries, num_heads * embed_dims]

The autograd backward returns gradients for value, sampling_locations and
attention_weights and None for the two integer tensors, as
MSDeformAttnFunction.backward does on the "DQ-DETR ops directory" CSDN page
(section 2(3)).

The fused form takes what MSDeformAttn.forward has before it forms the
locations and weights ("Deformable DETR walkthrough", section 2.2.4):

    ms_deform_attn_fused(value, spatial_shapes, level_start_index,
                         reference_points, sampling_offsets, attention_logits,
                         key_padding_mask=None)

    reference_points    [bs, num_queries, num_levels, 2 or 4]
    sampling_offsets    like sampling_locations
    attention_logits    like attention_weights (softmax over levels * points)
    key_padding_mask    None or bool/uint8 [bs, num_keys], True = padded key
                        (its value row reads as zero)

and differentiates with respect to value, sampling_offsets and
attention_logits (reference points and the mask get no gradient).

Float types: every float tensor in one of float32, float16, bfloat16; or
mixed precision, with value, output and their gradients in float16 or
bfloat16 and the per-sample tensors (locations or offsets, weights or
logits, reference points and their gradients) in float32.

This module only marshals arguments: PyTorch supplies device memory and the
current stream, the HIP library computes.  The shape tensors are read on the
host (a device copy is fetched once per call, which synchronises).
"""
from __future__ import annotations

import weakref

import numpy as np
import torch

from . import _lib

DTYPE_CODE = {torch.float32: _lib.MSDA_F32, torch.float16: _lib.MSDA_F16,
              torch.bfloat16: _lib.MSDA_BF16}


MIXED_CODE = {torch.float16: _lib.MSDA_F16_F32, torch.bfloat16: _lib.MSDA_BF16_F32}


def dtype_code(value_dtype, sample_dtype) -> int:
    """The library's dtype code for value-side and per-sample float types."""
    if value_dtype == sample_dtype and value_dtype in DTYPE_CODE:
        return DTYPE_CODE[value_dtype]
    if sample_dtype == torch.float32 and value_dtype in MIXED_CODE:
        return MIXED_CODE[value_dtype]
    raise TypeError(f"unsupported float types: value {value_dtype}, per-sample tensors {sample_dtype} "
                    "(one type for all, or float16/bfloat16 values with float32 per-sample tensors)")


# Host copies of device shape tensors (spatial_shapes, level_start_index):
# copying one to the host synchronises the device, so each tensor is copied
# once and the copy kept, keyed by the tensor object (a weak reference, so a
# new tensor at a reused address never hits) and its version counter (an
# in-place change invalidates the copy).
_HOST_COPIES: dict = {}
_HOST_COPIES_MAX = 64


def _host_int64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            ent = _HOST_COPIES.get(id(x))
            if ent is not None and ent[0]() is x and ent[1] == x._version:
                return ent[2]
        host = np.ascontiguousarray(x.detach().to("cpu").numpy().astype(np.int64, copy=False))
        if x.device.type != "cpu":
            host.setflags(write=False)
            if len(_HOST_COPIES) >= _HOST_COPIES_MAX:
                _HOST_COPIES.clear()
            _HOST_COPIES[id(x)] = (weakref.ref(x), x._version, host)
        return host
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _check(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype} (one dtype for all float tensors)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def problem_for(value: torch.Tensor, spatial_shapes, level_start_index,
                sampling_locations: torch.Tensor):
    """(Problem, keepalive) for tensors laid out as in the module docstring."""
    if value.dim() != 4 or sampling_locations.dim() != 6 or sampling_locations.shape[-1] != 2:
        raise ValueError("value must be [bs, K, M, D] and sampling_locations [bs, Q, M, L, P, 2]")
    code = dtype_code(value.dtype, sampling_locations.dtype)
    bs, K, M, D = value.shape
    bs2, Q, M2, L, P, _ = sampling_locations.shape
    if bs2 != bs or M2 != M:
        raise ValueError("batch / heads of value and sampling_locations differ")
    shapes = _host_int64(spatial_shapes).reshape(-1, 2)
    starts = _host_int64(level_start_index).reshape(-1)
    if shapes.shape[0] != L or starts.shape[0] != L:
        raise ValueError("spatial_shapes / level_start_index do not match num_levels")
    return _lib.make_problem(bs, K, M, D, L, P, Q, code, shapes, starts)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """One msda_forward call on the current stream; returns output."""
    prob, keep = problem_for(value, spatial_shapes, level_start_index, sampling_locations)
    dev, dt, st = value.device, value.dtype, sampling_locations.dtype
    bs, K, M, D = value.shape
    _, Q, _, L, P, _ = sampling_locations.shape
    _check(value, "value", dt, dev)
    _check(sampling_locations, "sampling_locations", st, dev)
    _check(attention_weights, "attention_weights", st, dev, (bs, Q, M, L, P))
    if out is None:
        out = torch.empty((bs, Q, M * D), dtype=dt, device=dev)
    _check(out, "output", dt, dev, (bs, Q, M * D))
    _lib.forward(prob, value.data_ptr(), sampling_locations.data_ptr(),
                 attention_weights.data_ptr(), out.data_ptr(), _stream(dev))
    return out


def forward_train(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """One msda_forward_train call on the current stream: the forward, which
    also leaves the backward's record counts in the workspace.  Returns
    (output, workspace); pass that workspace to backward(..., counted=True)
    with the same locations."""
    prob, keep = problem_for(value, spatial_shapes, level_start_index, sampling_locations)
    dev, dt, st = value.device, value.dtype, sampling_locations.dtype
    bs, K, M, D = value.shape
    _, Q, _, L, P, _ = sampling_locations.shape
    _check(value, "value", dt, dev)
    _check(sampling_locations, "sampling_locations", st, dev)
    _check(attention_weights, "attention_weights", st, dev, (bs, Q, M, L, P))
    if out is None:
        out = torch.empty((bs, Q, M * D), dtype=dt, device=dev)
    _check(out, "output", dt, dev, (bs, Q, M * D))
    need = _lib.workspace_bytes(prob)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _lib.forward_train(prob, value.data_ptr(), sampling_locations.data_ptr(), attention_weights.data_ptr(),
                       out.data_ptr(), workspace.data_ptr() if need > 0 else 0, need, _stream(dev))
    return out, workspace


def backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
             grad_output, grads=None, workspace: torch.Tensor | None = None, counted: bool = False):
    """One msda_backward call on the current stream; returns
    (grad_value, grad_sampling_locations, grad_attention_weights).  With
    counted=True it is msda_backward_counted on the workspace that
    forward_train returned for the same locations."""
    prob, keep = problem_for(value, spatial_shapes, level_start_index, sampling_locations)
    dev, dt, st = value.device, value.dtype, sampling_locations.dtype
    bs, K, M, D = value.shape
    _, Q, _, L, P, _ = sampling_locations.shape
    _check(value, "value", dt, dev)
    _check(sampling_locations, "sampling_locations", st, dev)
    _check(attention_weights, "attention_weights", st, dev, (bs, Q, M, L, P))
    _check(grad_output, "grad_output", dt, dev, (bs, Q, M * D))
    if grads is None:
        grads = (torch.empty_like(value), torch.empty_like(sampling_locations),
                 torch.empty_like(attention_weights))
    gv, gl, gw = grads
    _check(gv, "grad_value", dt, dev, value.shape)
    _check(gl, "grad_sampling_locations", st, dev, sampling_locations.shape)
    _check(gw, "grad_attention_weights", st, dev, attention_weights.shape)
    need = _lib.workspace_bytes(prob)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        if counted:
            raise ValueError("backward(counted=True) needs the workspace forward_train returned")
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if (need > 0) else 0
    call = _lib.backward_counted if counted else _lib.backward
    call(prob, value.data_ptr(), sampling_locations.data_ptr(), attention_weights.data_ptr(),
         grad_output.data_ptr(), gv.data_ptr(), gl.data_ptr(), gw.data_ptr(), ws_ptr, need, _stream(dev))
    return gv, gl, gw


class MSDeformAttnFunction(torch.autograd.Function):
    """Autograd wrapper.  When a gradient is wanted, forward =
    msda_forward_train and backward = msda_backward_counted on the workspace
    the forward filled (held from the forward to the backward; the saved
    locations cannot change in between: autograd checks their version);
    otherwise forward = msda_forward."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_locations, attention_weights):
        shapes = _host_int64(spatial_shapes)
        starts = _host_int64(level_start_index)
        ctx.workspace = None
        if any(ctx.needs_input_grad):
            out, ctx.workspace = forward_train(value, shapes, starts, sampling_locations, attention_weights)
        else:
            out = forward(value, shapes, starts, sampling_locations, attention_weights)
        ctx.save_for_backward(value, sampling_locations, attention_weights)
        ctx.host_shapes = (shapes, starts)
        return out

    @staticmethod
    def backward(ctx, grad_output):
        value, loc, w = ctx.saved_tensors
        shapes, starts = ctx.host_shapes
        counted = ctx.workspace is not None
        gv, gl, gw = backward(value, shapes, starts, loc, w, grad_output.contiguous(), workspace=ctx.workspace,
                              counted=counted)
        return gv, None, None, gl, gw


def ms_deform_attn(value, spatial_shapes, level_start_index, sampling_locations, attention_weights):
    """Differentiable MSDeformAttn core (see the module docstring)."""
    return MSDeformAttnFunction.apply(value, spatial_shapes, level_start_index,
                                      sampling_locations, attention_weights)


def _mask_ptr(value, key_padding_mask) -> int:
    if key_padding_mask is None:
        return 0
    bs, K = value.shape[:2]
    if key_padding_mask.dtype not in (torch.bool, torch.uint8):
        raise TypeError("key_padding_mask must be bool or uint8")
    _check(key_padding_mask, "key_padding_mask", key_padding_mask.dtype, value.device, (bs, K))
    return key_padding_mask.data_ptr()      # bool is stored as one byte, 0 or 1


def _check_fused(value, reference_points, sampling_offsets, attention_logits):
    dev, dt, st = value.device, value.dtype, sampling_offsets.dtype
    bs, K, M, D = value.shape
    _, Q, _, L, P, _ = sampling_offsets.shape
    _check(value, "value", dt, dev)
    _check(sampling_offsets, "sampling_offsets", st, dev)
    _check(attention_logits, "attention_logits", st, dev, (bs, Q, M, L, P))
    if reference_points.dim() != 4 or reference_points.shape[-1] not in (2, 4):
        raise ValueError("reference_points must be [bs, num_queries, num_levels, 2 or 4]")
    _check(reference_points, "reference_points", st, dev, (bs, Q, L, reference_points.shape[-1]))
    return int(reference_points.shape[-1])


def forward_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                  attention_logits, key_padding_mask=None, out: torch.Tensor | None = None) -> torch.Tensor:
    """One msda_forward_fused call on the current stream; returns output."""
    prob, keep = problem_for(value, spatial_shapes, level_start_index, sampling_offsets)
    ref_dims = _check_fused(value, reference_points, sampling_offsets, attention_logits)
    mask = _mask_ptr(value, key_padding_mask)
    bs, K, M, D = value.shape
    Q = sampling_offsets.shape[1]
    if out is None:
        out = torch.empty((bs, Q, M * D), dtype=value.dtype, device=value.device)
    _check(out, "output", value.dtype, value.device, (bs, Q, M * D))
    _lib.forward_fused(prob, ref_dims, value.data_ptr(), mask, reference_points.data_ptr(),
                       sampling_offsets.data_ptr(), attention_logits.data_ptr(), out.data_ptr(),
                       _stream(value.device))
    return out


def backward_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                   attention_logits, grad_output, key_padding_mask=None, grads=None,
                   workspace: torch.Tensor | None = None):
    """One msda_backward_fused call on the current stream; returns
    (grad_value, grad_sampling_offsets, grad_attention_logits)."""
    prob, keep = problem_for(value, spatial_shapes, level_start_index, sampling_offsets)
    ref_dims = _check_fused(value, reference_points, sampling_offsets, attention_logits)
    mask = _mask_ptr(value, key_padding_mask)
    dev, dt = value.device, value.dtype
    bs, K, M, D = value.shape
    Q = sampling_offsets.shape[1]
    _check(grad_output, "grad_output", dt, dev, (bs, Q, M * D))
    if grads is None:
        grads = (torch.empty_like(value), torch.empty_like(sampling_offsets),
                 torch.empty_like(attention_logits))
    gv, go, gl = grads
    _check(gv, "grad_value", dt, dev, value.shape)
    _check(go, "grad_sampling_offsets", sampling_offsets.dtype, dev, sampling_offsets.shape)
    _check(gl, "grad_attention_logits", sampling_offsets.dtype, dev, attention_logits.shape)
    need = _lib.workspace_bytes(prob)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if (need > 0) else 0
    _lib.backward_fused(prob, ref_dims, value.data_ptr(), mask, reference_points.data_ptr(),
                        sampling_offsets.data_ptr(), attention_logits.data_ptr(), grad_output.data_ptr(),
                        gv.data_ptr(), go.data_ptr(), gl.data_ptr(), ws_ptr, need, _stream(dev))
    return gv, go, gl


class MSDeformAttnFusedFunction(torch.autograd.Function):
    """Autograd wrapper: forward = msda_forward_fused, backward = msda_backward_fused."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                attention_logits, key_padding_mask=None):
        shapes = _host_int64(spatial_shapes)
        starts = _host_int64(level_start_index)
        out = forward_fused(value, shapes, starts, reference_points, sampling_offsets, attention_logits,
                            key_padding_mask)
        ctx.save_for_backward(value, reference_points, sampling_offsets, attention_logits, key_padding_mask)
        ctx.host_shapes = (shapes, starts)
        return out

    @staticmethod
    def backward(ctx, grad_output):
        value, ref, off, logits, mask = ctx.saved_tensors
        shapes, starts = ctx.host_shapes
        gv, go, gl = backward_fused(value, shapes, starts, ref, off, logits, grad_output.contiguous(), mask)
        return gv, None, None, None, go, gl, None


def ms_deform_attn_fused(value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
                         attention_logits, key_padding_mask=None):
    """Differentiable MSDeformAttn core with the fused prologue (see the module docstring)."""
    return MSDeformAttnFusedFunction.apply(value, spatial_shapes, level_start_index, reference_points,
                                           sampling_offsets, attention_logits, key_padding_mask)
