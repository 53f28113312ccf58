"""GPU parity of the fused prologue (msda_forward_fused / msda_backward_fused)
against the oracle's fused functions, element by element, on seeded inputs:
reference points (2-d and 4-d), raw offsets and logits in every dtype, on
problems of several workgroups with a ragged tail, the L = P = 4 kernels and
the generic ones, samples pushed off the map, the float-atomic fallback, an
empty problem, key padding masks (padded images with valid-ratio-scaled
reference points, random masks, masks on segments split over several
accumulation units), the DETR encoder and decoder shapes at full size and the
autograd wrapper."""
import numpy as np
import pytest
import torch

from scale_deformable_attention_03_amd import workloads as W
from tests.parity import (check_backward_fused, check_forward_fused, fused_to_device, gpu_backward_fused,
                          gpu_forward_fused)

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def run(wl):
    masked = "" if wl.key_padding_mask is None else f" masked {int(wl.key_padding_mask.sum())}"
    print(f"[gpu] fused {wl.name} {wl.dtype} ref{wl.ref_dims} {tuple(wl.sampling_offsets.shape)}{masked}",
          flush=True)
    t = fused_to_device(wl)
    check_forward_fused(wl, gpu_forward_fused(wl, t))
    check_backward_fused(wl, gpu_backward_fused(wl, t))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ref_dims", [2, 4])
def test_generic_levels_points(dtype, ref_dims):
    """L = 3, P = 3 (the generic kernels), 150 queries: several workgroups per
    (batch, head) plane and a ragged last one."""
    run(W.make_fused("generic", 2, [(11, 13), (6, 7), (3, 4)], 4, 32, 3, 150, dtype, seed=31,
                     ref_dims=ref_dims))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ref_dims", [2, 4])
def test_four_levels_four_points(dtype, ref_dims):
    """L = P = 4 (the unrolled kernels), 8 heads x 32 dims, 203 queries."""
    run(W.make_fused("l4p4", 2, [(20, 27), (10, 14), (5, 7), (3, 4)], 8, 32, 4, 203, dtype, seed=32,
                     ref_dims=ref_dims))


@pytest.mark.parametrize("ref_dims", [2, 4])
def test_off_map_samples(ref_dims):
    """Offsets of ~20 pixels on small maps: many samples fall off the map
    (zero output and offset gradients) yet their weights still enter every
    logit gradient of the head."""
    run(W.make_fused("offmap", 2, [(6, 8), (3, 4)], 4, 16, 4, 70, "f32", seed=33, ref_dims=ref_dims,
                     offset_sigma=20.0))


@pytest.mark.parametrize("D", [8, 64, 256])
def test_row_widths(D):
    """Other lane splits of the kernels (embed_dims 8, 64, 256), 2-d refs."""
    run(W.make_fused(f"width{D}", 1, [(9, 10), (5, 5)], 2, D, 2, 77, "f32", seed=34 + D))


def test_fallback_path():
    """A 1 x 600000 level exceeds the binned backward's segment count: the
    float-atomic path with the fused prologue."""
    run(W.make_fused("fallback", 1, [(1, 600000)], 1, 8, 1, 64, "f32", seed=35))


@pytest.mark.parametrize("ref_dims", [2, 4])
def test_empty_queries(ref_dims):
    from scale_deformable_attention_03_amd import ops
    wl = W.make_fused("empty", 2, [(5, 6)], 2, 16, 2, 0, "f32", seed=36, ref_dims=ref_dims)
    t = fused_to_device(wl)
    out = ops.forward_fused(t["value"], wl.spatial_shapes, wl.level_start_index, t["ref"], t["off"], t["logits"])
    assert out.shape == (2, 0, 32)
    gv = torch.full_like(t["value"], 7.0)
    ops.backward_fused(t["value"], wl.spatial_shapes, wl.level_start_index, t["ref"], t["off"], t["logits"],
                       t["g"], grads=(gv, torch.empty_like(t["off"]), torch.empty_like(t["logits"])))
    torch.cuda.synchronize()
    assert torch.all(gv == 0)


@pytest.mark.parametrize("make", [lambda: W.detr_encoder_fused(), lambda: W.detr_decoder_fused("f32", 4),
                                  lambda: W.detr_decoder_fused("f32", 2), lambda: W.detr_decoder_fused("bf16", 4)],
                         ids=["encoder_f32_ref2", "decoder_f32_ref4", "decoder_f32_ref2", "decoder_bf16_ref4"])
def test_detr_shapes_full_size(make):
    run(make())


PADDED = [(1.0, 1.0), (0.7, 0.55)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ref_dims", [2, 4])
def test_padded_images_encoder(dtype, ref_dims):
    """Two images padded to one size (the second to 70% x 55%): per-level
    masks by nearest downsampling, encoder reference points over the valid
    extent scaled by each level's valid ratio; L = P = 4."""
    shapes = [(16, 20), (8, 10), (4, 5), (2, 3)]
    K = sum(h * w for h, w in shapes)
    run(W.make_fused("padded_enc", 2, shapes, 8, 32, 4, K, dtype, seed=41, ref_dims=ref_dims,
                     ref_dist="encoder", valid=PADDED))


@pytest.mark.parametrize("ref_dims", [2, 4])
def test_padded_images_decoder(ref_dims):
    run(W.make_fused("padded_dec", 2, [(15, 21), (8, 11), (4, 6)], 4, 32, 3, 130, "f32", seed=42,
                     ref_dims=ref_dims, valid=PADDED))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_random_mask(dtype):
    """A mask with no structure (30% of keys), generic kernels."""
    wl = W.make_fused("random_mask", 2, [(11, 13), (6, 7), (3, 4)], 4, 32, 3, 150, dtype, seed=43)
    wl.key_padding_mask = torch.from_numpy(np.random.default_rng(44).random(wl.value.shape[:2]) < 0.3)
    run(wl)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mask_on_split_segments(dtype):
    """2000 queries on a 4x4 level: its segments are split over several
    accumulation units (rows added with atomics), with a random mask."""
    wl = W.make_fused("split_mask", 2, [(4, 4), (30, 40)], 2, 16, 4, 2000, dtype, seed=45)
    wl.key_padding_mask = torch.from_numpy(np.random.default_rng(46).random(wl.value.shape[:2]) < 0.3)
    run(wl)


def test_mask_on_fallback_path():
    wl = W.make_fused("fallback_mask", 1, [(1, 600000)], 1, 8, 1, 64, "f32", seed=47)
    m = np.zeros(wl.value.shape[:2], dtype=bool)
    m[:, ::3] = True
    wl.key_padding_mask = torch.from_numpy(m)
    run(wl)


def test_autograd_function():
    from scale_deformable_attention_03_amd import ms_deform_attn_fused
    wl = W.make_fused("autograd", 2, [(11, 13), (6, 7)], 4, 32, 3, 40, "f32", seed=37, ref_dims=4)
    t = fused_to_device(wl)
    v = t["value"].clone().requires_grad_()
    off = t["off"].clone().requires_grad_()
    lg = t["logits"].clone().requires_grad_()
    mask = torch.from_numpy(np.random.default_rng(38).random(wl.value.shape[:2]) < 0.2).cuda()
    wl.key_padding_mask = mask.cpu()
    out = ms_deform_attn_fused(v, wl.spatial_shapes, wl.level_start_index, t["ref"], off, lg, mask)
    out.backward(t["g"])
    torch.cuda.synchronize()
    check_forward_fused(wl, out.detach())
    check_backward_fused(wl, (v.grad, off.grad, lg.grad))


@pytest.mark.parametrize("ref_dims", [2, 4])
def test_max_envelope_fused(ref_dims):
    """The envelope's corner: L * P = 64 (4 levels x 16 points), 8 heads x 64
    dims, fp16, large offsets (many samples off the map)."""
    run(W.make_fused("max_fused", 1, [(40, 40), (20, 20), (10, 10), (5, 5)], 8, 64, 16, 120, "f16", seed=71,
                     ref_dims=ref_dims, offset_sigma=6.0))


def test_fallback_path_box_refs_mixed():
    """The float-atomic fallback with 4-d reference points, bf16 values and
    float32 per-sample tensors, and a padding mask."""
    wl = W.make_fused("fallback_mixed", 1, [(1, 600000)], 1, 8, 2, 64, "bf16", seed=72, ref_dims=4,
                      sample_dtype="f32")
    m = np.zeros(wl.value.shape[:2], dtype=bool)
    m[:, 1::4] = True
    wl.key_padding_mask = torch.from_numpy(m)
    run(wl)
