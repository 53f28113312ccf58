"""The whole MSDeformAttn module step around the fused core.

"Deformable DETR walkthrough" (zhangshiyu.com/post/59697), section 2.2.4,
MSDeformAttn: four Linears around the core --

    value   = value_proj(input_flatten), padded keys zero-filled, viewed [N, K, M, D]
    offsets = sampling_offsets(query)     viewed [N, Q, M, L, P, 2]
    logits  = attention_weights(query)    viewed [N, Q, M, L, P]
    out     = core(value, locations(reference_points, offsets), softmax(logits))
    output  = output_proj(out)

Every view is a zero-copy reinterpretation of the Linear's output (the
feature dimension is ordered head, level, point, coordinate), so the fused
core (``ms_deform_attn_fused``: locations, softmax, key padding and the
sampling in the HIP kernels) reads the GEMM outputs in place.  The four
Linears are plain dense GEMMs and run through PyTorch's ROCm BLAS (hipBLASLt)
with autograd; the core's backward is the C ABI's.

Parameters are initialised as the walkthrough's _reset_parameters describes
for sampling_offsets (zero weight; bias = head direction scaled so the larger
component is 1, times point index + 1) -- plus, because a step with random
weights is what is measured here, seeded uniform weights for all four Linears
(``init_weight_scale``), so that every query samples its own pattern.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

from . import ops
from .workloads import offset_directions


def module_parameters(d_model: int, n_levels: int, n_heads: int, n_points: int, seed: int,
                      init_weight_scale: float = 0.02) -> dict:
    """Seeded parameters as float64 numpy arrays (name -> array), shapes as
    nn.Linear's: weight [out, in], bias [out].

    value_proj / output_proj: Xavier-uniform weights, zero bias (the
    walkthrough's _reset_parameters); sampling_offsets: bias = the initial
    sampling pattern, weight U(-s, s); attention_weights: zero bias, weight
    U(-s, s), s = init_weight_scale."""
    rng = np.random.default_rng(seed)
    M, L, P, C = n_heads, n_levels, n_points, d_model

    def xavier(out_f, in_f):
        a = math.sqrt(6.0 / (in_f + out_f))
        return rng.uniform(-a, a, size=(out_f, in_f))

    return {
        "value_proj.weight": xavier(C, C), "value_proj.bias": np.zeros(C),
        "sampling_offsets.weight": rng.uniform(-init_weight_scale, init_weight_scale, size=(M * L * P * 2, C)),
        "sampling_offsets.bias": offset_directions(M, L, P).reshape(-1),
        "attention_weights.weight": rng.uniform(-init_weight_scale, init_weight_scale, size=(M * L * P, C)),
        "attention_weights.bias": np.zeros(M * L * P),
        "output_proj.weight": xavier(C, C), "output_proj.bias": np.zeros(C),
    }


class MSDeformAttnModule:
    """The module with its parameters as tensors (requires_grad) on a device.

    forward(query [N, Q, C], reference_points [N, Q, L, 2 or 4],
            input_flatten [N, K, C], spatial_shapes, level_start_index,
            input_padding_mask [N, K] bool or None) -> [N, Q, C]
    """

    def __init__(self, d_model: int = 256, n_levels: int = 4, n_heads: int = 8, n_points: int = 4,
                 device="cuda", dtype=torch.float32, seed: int = 7, params: dict | None = None):
        if d_model % n_heads != 0:
            raise ValueError("d_model must be a multiple of n_heads")
        self.d_model, self.n_levels, self.n_heads, self.n_points = d_model, n_levels, n_heads, n_points
        params = params if params is not None else module_parameters(d_model, n_levels, n_heads, n_points, seed)
        self.params = {k: torch.tensor(v, dtype=dtype, device=device).requires_grad_() for k, v in params.items()}

    def parameters(self):
        return list(self.params.values())

    def _linear(self, x, name):
        return F.linear(x, self.params[name + ".weight"], self.params[name + ".bias"])

    def forward(self, query, reference_points, input_flatten, spatial_shapes, level_start_index,
                input_padding_mask=None):
        N, Q, _ = query.shape
        _, K, _ = input_flatten.shape
        M, L, P = self.n_heads, self.n_levels, self.n_points
        value = self._linear(input_flatten, "value_proj").view(N, K, M, self.d_model // M)
        offsets = self._linear(query, "sampling_offsets").view(N, Q, M, L, P, 2)
        logits = self._linear(query, "attention_weights").view(N, Q, M, L, P)
        out = ops.ms_deform_attn_fused(value, spatial_shapes, level_start_index, reference_points.contiguous(),
                                       offsets, logits, input_padding_mask)
        return self._linear(out, "output_proj")

    __call__ = forward
