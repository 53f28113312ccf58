"""GPU parity of the whole MSDeformAttn module step (module.MSDeformAttnModule:
PyTorch hipBLASLt Linears around the fused core through the C ABI) against
the oracle's module step, forward output and the gradients of every
parameter, the query and input_flatten.

Inputs are dyadic (workloads.make_module(dyadic=True)): the Linear outputs
that set the sampling locations are then exact in float32 on both sides, so
the two sides sample at identical locations and the float32 bars apply
element by element (a location differing in its last bit could move a sample
across a bilinear cell edge, where the location gradient jumps)."""
import numpy as np
import pytest
import torch

import oracle
from scale_deformable_attention_03_amd import workloads as W
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def run_module(wl):
    from scale_deformable_attention_03_amd.module import MSDeformAttnModule
    print(f"[gpu] module {wl.name} {tuple(wl.query.shape)} {tuple(wl.input_flatten.shape)} "
          f"ref{wl.reference_points.shape[-1]} masked {wl.key_padding_mask is not None}", flush=True)
    m = MSDeformAttnModule(wl.d_model, wl.n_levels, wl.n_heads, wl.n_points, device="cuda", params=wl.params)
    q = wl.query.cuda().requires_grad_()
    x = wl.input_flatten.cuda().requires_grad_()
    mask = None if wl.key_padding_mask is None else wl.key_padding_mask.cuda()
    out = m(q, wl.reference_points.cuda(), x, wl.spatial_shapes, wl.level_start_index, mask)
    out.backward(wl.grad_output.cuda())
    torch.cuda.synchronize()

    omask = None if wl.key_padding_mask is None else wl.key_padding_mask.numpy()
    args = (wl.params, wl.query.numpy(), wl.reference_points.numpy(), wl.input_flatten.numpy(), wl.spatial_shapes,
            wl.level_start_index)
    ref, _ = oracle.module_forward(*args, wl.n_heads, wl.n_levels, wl.n_points, omask)
    grads = oracle.module_backward(*args, wl.grad_output.numpy(), wl.n_heads, wl.n_levels, wl.n_points, omask)
    f64 = lambda t: t.detach().double().cpu().numpy()
    rtol, _, atol = TOL[("f32", "fwd")]
    assert_close(f"{wl.name}/output", f64(out), ref, rtol, atol=atol * max(1.0, float(np.abs(ref).max())))
    rtol, arms, _ = TOL[("f32", "bwd")]
    for name, t in list(m.params.items()) + [("query", q), ("input_flatten", x)]:
        assert_close(f"{wl.name}/grad {name}", f64(t.grad), grads[name], rtol, arms)


@pytest.mark.parametrize("ref_dims", [2, 4])
def test_module_decoder_like(ref_dims):
    """d_model 256 (8 heads x 32), 4 levels, 4 points, 300 queries per image
    on a small pyramid."""
    run_module(W.make_module("module_dec", 2, [(24, 32), (12, 16), (6, 8), (3, 4)], 256, 8, 4, 300, seed=61,
                             ref_dims=ref_dims, dyadic=True))


def test_module_encoder_like_padded():
    """Encoder-style: queries are the keys (pixel-centre reference points over
    the valid extent), two images padded to one size, key padding mask."""
    shapes = [(16, 20), (8, 10), (4, 5), (2, 3)]
    K = sum(h * w for h, w in shapes)
    run_module(W.make_module("module_enc", 2, shapes, 256, 8, 4, K, seed=62, ref_dist="encoder", dyadic=True,
                             valid=[(1.0, 1.0), (0.7, 0.55)]))


def test_module_generic_heads_levels():
    """Other module widths: d_model 64 (4 heads x 16), 3 levels, 3 points."""
    run_module(W.make_module("module_small", 2, [(11, 13), (6, 7), (3, 4)], 64, 4, 3, 90, seed=63, dyadic=True))
