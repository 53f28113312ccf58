"""Pins of the oracle's module step (oracle.module_forward / module_backward).

The module is MSDeformAttn of the Deformable DETR walkthrough
(zhangshiyu.com/post/59697, section 2.2.4): value_proj, sampling_offsets and
attention_weights Linears, the core, output_proj.  The oracle writes the
Linears' backward out by hand (dx = dy W, dW = dy^T x, db = column sums);
here torch's float64 autograd derives it instead, through nn.Linear's
functional form, masked_fill, the location formula, torch.softmax and
grid_sample.  Dyadic inputs (multiples of 1/8 and 1/64) keep every Linear
output exact in float32, so the oracle's float32 intermediates equal torch's
float64 ones and the comparison is tight.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from scale_deformable_attention_03_amd import workloads as W
from tests.test_oracle_pins import grid_sample_core


def torch_module(wl, params, query, inp, mask):
    """float64 module with torch ops only (no oracle code)."""
    N, Q, C = query.shape
    K = inp.shape[1]
    M, L, P = wl.n_heads, wl.n_levels, wl.n_points
    shapes = wl.spatial_shapes
    value = F.linear(inp, params["value_proj.weight"], params["value_proj.bias"])
    if mask is not None:
        value = value.masked_fill(torch.tensor(mask)[..., None], 0.0)
    value = value.view(N, K, M, C // M)
    off = F.linear(query, params["sampling_offsets.weight"], params["sampling_offsets.bias"]).view(N, Q, M, L, P, 2)
    lg = F.linear(query, params["attention_weights.weight"], params["attention_weights.bias"])
    w = torch.softmax(lg.view(N, Q, M, L * P), -1).view(N, Q, M, L, P)
    ref = torch.tensor(wl.reference_points.numpy(), dtype=torch.float64)[:, :, None, :, None, :]
    if ref.shape[-1] == 2:
        norm = torch.tensor(np.stack([shapes[:, 1], shapes[:, 0]], -1), dtype=torch.float64)
        loc = ref + off / norm[None, None, None, :, None, :]
    else:
        loc = ref[..., :2] + off / P * ref[..., 2:] * 0.5
    Wd = torch.tensor(shapes[:, 1], dtype=torch.float64)[None, None, None, :, None]
    Hd = torch.tensor(shapes[:, 0], dtype=torch.float64)[None, None, None, :, None]
    core = grid_sample_core(value, shapes, loc[..., 0] * Wd - 0.5, loc[..., 1] * Hd - 0.5, w)
    return F.linear(core, params["output_proj.weight"], params["output_proj.bias"])


@pytest.mark.parametrize("ref_dims,masked", [(2, False), (4, False), (2, True)])
def test_module_autograd_cross_check(ref_dims, masked):
    wl = W.make_module("pin", 2, [(8, 16), (4, 8), (2, 4)], 32, 4, 2, 13, seed=5, ref_dims=ref_dims,
                       dyadic=True, valid=[(1.0, 1.0), (0.75, 0.5)] if masked else None)
    # dyadic reference points (and powers-of-two maps): every float32
    # location operation of the oracle is exact too
    wl.reference_points = torch.round(wl.reference_points * 64) / 64
    mask = None if wl.key_padding_mask is None else wl.key_padding_mask.numpy()
    if masked:
        assert mask.any() and not mask.all()
    args = (wl.params, wl.query.numpy(), wl.reference_points.numpy(), wl.input_flatten.numpy(), wl.spatial_shapes,
            wl.level_start_index)
    out, _ = oracle.module_forward(*args, wl.n_heads, wl.n_levels, wl.n_points, mask)
    grads = oracle.module_backward(*args, wl.grad_output.numpy(), wl.n_heads, wl.n_levels, wl.n_points, mask)

    params = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in wl.params.items()}
    q = torch.tensor(wl.query.numpy(), dtype=torch.float64, requires_grad=True)
    x = torch.tensor(wl.input_flatten.numpy(), dtype=torch.float64, requires_grad=True)
    ref_out = torch_module(wl, params, q, x, mask)
    ref_out.backward(torch.tensor(wl.grad_output.numpy(), dtype=torch.float64))

    np.testing.assert_allclose(out, ref_out.detach().numpy(), rtol=1e-9, atol=1e-9)
    # the oracle rounds the core's input gradient (a float32 tensor in the
    # module) to float32: 6e-8 relative
    for name, t in list(params.items()) + [("query", q), ("input_flatten", x)]:
        ref = t.grad.numpy()
        scale = float(np.abs(ref).max())
        np.testing.assert_allclose(grads[name], ref, rtol=1e-6, atol=1e-6 * scale, err_msg=name)
    if masked:
        # padded rows reach no gradient of value_proj's input
        np.testing.assert_array_equal(grads["input_flatten"][mask], 0.0)


def test_dyadic_intermediates_are_exact():
    """The dyadic recipe's claim: value, offsets and logits computed in
    float64 are already float32 numbers."""
    wl = W.make_module("exact", 2, [(8, 16), (4, 8)], 64, 4, 2, 30, seed=6, dyadic=True)
    q, x = wl.query.numpy().astype(np.float64), wl.input_flatten.numpy().astype(np.float64)
    for name, src in (("value_proj", x), ("sampling_offsets", q), ("attention_weights", q)):
        y = src @ wl.params[name + ".weight"].astype(np.float64).T + wl.params[name + ".bias"]
        np.testing.assert_array_equal(y.astype(np.float32).astype(np.float64), y)
