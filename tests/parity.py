"""Shared helpers of the parity tests: run a workload through the HIP library
(via the C ABI) and through the CPU oracle, and compare element by element.

Tolerances (the bar an element must meet: |gpu - ref| <= rtol*|ref| + atol):
  fp32 forward            rtol 1e-5, atol 1e-6
  fp32 backward           rtol 1e-4, atol 1e-4 * RMS(ref tensor)
                          (float32 atomics reorder the grad_value sums)
  fp16 / bf16, all        rtol 1e-2, atol 1e-2 * RMS(ref tensor)
                          (against the float64 oracle fed the same 16-bit inputs)
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {
    ("f32", "fwd"): (1e-5, None, 1e-6),
    ("f32", "bwd"): (1e-4, 1e-4, None),
    ("f16", "fwd"): (1e-2, 1e-2, None),
    ("f16", "bwd"): (1e-2, 1e-2, None),
    ("bf16", "fwd"): (1e-2, 1e-2, None),
    ("bf16", "bwd"): (1e-2, 1e-2, None),
}


def assert_close(name, gpu, ref, rtol, atol_rms=None, atol=None):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    if atol is None:
        atol = atol_rms * float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(gpu - ref)
    bound = rtol * np.abs(ref) + atol
    bad = ~(err <= bound)            # NaN in gpu counts as bad
    norm = float(np.linalg.norm((gpu - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))
    # the normwise relative error, reported beside the elementwise bar (shown with pytest -s)
    print(f"[parity] {name}: normwise rel err {norm:.3g}, max abs err {float(np.nanmax(err)):.3g}", flush=True)
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err - bound, -np.inf))), ref.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{ref.size} elements out of tolerance "
            f"(rtol {rtol:g}, atol {atol:.3g}); worst at {i}: gpu {gpu[i]!r} ref {ref[i]!r}; "
            f"normwise rel err {norm:.3g}")


def to_device(wl, device="cuda"):
    return dict(value=wl.value.to(device), loc=wl.sampling_locations.to(device),
                w=wl.attention_weights.to(device), g=wl.grad_output.to(device))


def gpu_forward(wl, t=None):
    from scale_deformable_attention_03_amd import ops
    t = t or to_device(wl)
    out = ops.forward(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"], t["w"])
    torch.cuda.synchronize()
    return out


def gpu_backward(wl, t=None):
    from scale_deformable_attention_03_amd import ops
    t = t or to_device(wl)
    gv, gl, gw = ops.backward(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"], t["w"], t["g"])
    torch.cuda.synchronize()
    return gv, gl, gw


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_forward(wl, nthreads=0):
    return oracle.forward(wl.f32("value"), wl.spatial_shapes, wl.level_start_index,
                          wl.f32("sampling_locations"), wl.f32("attention_weights"), nthreads)


def oracle_backward(wl, nthreads=0):
    return oracle.backward(wl.f32("value"), wl.spatial_shapes, wl.level_start_index,
                           wl.f32("sampling_locations"), wl.f32("attention_weights"),
                           wl.f32("grad_output"), nthreads)


def sample_tol(wl, kind):
    """Tolerance of the per-sample gradients: their own type's (float32 in
    mixed precision: computed in float32 from the same widened 16-bit rows
    as the oracle's, and stored as float32)."""
    return TOL[(wl.sample_dtype or wl.dtype, kind)]


def tag(wl):
    return f"{wl.name}/{wl.dtype}" + (f"+{wl.sample_dtype}" if wl.sample_dtype else "")


def check_forward(wl, out=None):
    out = gpu_forward(wl) if out is None else out
    rtol, arms, atol = TOL[(wl.dtype, "fwd")]
    assert_close(f"{tag(wl)}/output", f64(out), oracle_forward(wl), rtol, arms, atol)
    return out


def check_backward(wl, grads=None):
    gv, gl, gw = gpu_backward(wl) if grads is None else grads
    rgv, rgl, rgw = oracle_backward(wl)
    rtol, arms, atol = sample_tol(wl, "bwd")
    assert_close(f"{tag(wl)}/grad_attention_weights", f64(gw), rgw, rtol, arms, atol)
    assert_close(f"{tag(wl)}/grad_sampling_locations", f64(gl), rgl, rtol, arms, atol)
    rtol, arms, atol = TOL[(wl.dtype, "bwd")]
    assert_close(f"{tag(wl)}/grad_value", f64(gv), rgv, rtol, arms, atol)
    return gv, gl, gw


# ---- fused prologue ---------------------------------------------------------------

def fused_to_device(wl, device="cuda"):
    return dict(value=wl.value.to(device), ref=wl.reference_points.to(device),
                off=wl.sampling_offsets.to(device), logits=wl.attention_logits.to(device),
                g=wl.grad_output.to(device),
                mask=None if wl.key_padding_mask is None else wl.key_padding_mask.to(device))


def gpu_forward_fused(wl, t=None):
    from scale_deformable_attention_03_amd import ops
    t = t or fused_to_device(wl)
    out = ops.forward_fused(t["value"], wl.spatial_shapes, wl.level_start_index, t["ref"], t["off"], t["logits"],
                            t["mask"])
    torch.cuda.synchronize()
    return out


def gpu_backward_fused(wl, t=None):
    from scale_deformable_attention_03_amd import ops
    t = t or fused_to_device(wl)
    grads = ops.backward_fused(t["value"], wl.spatial_shapes, wl.level_start_index, t["ref"], t["off"],
                               t["logits"], t["g"], t["mask"])
    torch.cuda.synchronize()
    return grads


def oracle_fused_args(wl):
    return (wl.f32("value"), wl.spatial_shapes, wl.level_start_index, wl.f32("reference_points"),
            wl.f32("sampling_offsets"), wl.f32("attention_logits"))


def oracle_mask(wl):
    return None if wl.key_padding_mask is None else wl.key_padding_mask.numpy()


def check_forward_fused(wl, out=None):
    out = gpu_forward_fused(wl) if out is None else out
    rtol, arms, atol = TOL[(wl.dtype, "fwd")]
    assert_close(f"{tag(wl)}/ref{wl.ref_dims}/output", f64(out),
                 oracle.forward_fused(*oracle_fused_args(wl), oracle_mask(wl)), rtol, arms, atol)
    return out


def check_backward_fused(wl, grads=None):
    gv, goff, glog = gpu_backward_fused(wl) if grads is None else grads
    rgv, rgoff, rglog = oracle.backward_fused(*oracle_fused_args(wl), wl.f32("grad_output"), oracle_mask(wl))
    t = f"{tag(wl)}/ref{wl.ref_dims}"
    rtol, arms, atol = sample_tol(wl, "bwd")
    assert_close(f"{t}/grad_attention_logits", f64(glog), rglog, rtol, arms, atol)
    assert_close(f"{t}/grad_sampling_offsets", f64(goff), rgoff, rtol, arms, atol)
    rtol, arms, atol = TOL[(wl.dtype, "bwd")]
    assert_close(f"{t}/grad_value", f64(gv), rgv, rtol, arms, atol)
    return gv, goff, glog
