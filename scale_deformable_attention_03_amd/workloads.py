"""Seeded synthetic inputs shaped like the Deformable DETR workloads.

This module draws inputs only; it holds none of the core's arithmetic (no
bilinear sampling, no weighted sum).  The same bytes feed the HIP library and
the CPU oracle.

Shapes come from the pages:
  * Ascend DrivingSDK API page for multi_scale_deformable_attn, usage example:
    bs 1, one 100x100 level, 4 heads, 8 points, 16 queries, 32 dims,
    value = U[0,1)*0.01, locations = 0.005, weights = U[0,1) + 1e-5, and a
    backward with an all-ones output gradient;
  * Deformable DETR walkthrough (zhangshiyu.com/post/59697), section 2.2.4:
    d_model 256 = 8 heads x 32 dims, 4 levels, 4 points; encoder queries are
    the flattened pixels themselves with pixel-centre reference points
    ((j + 0.5)/W, (i + 0.5)/H) (get_reference_points, valid ratios 1);
    attention weights are a softmax over the L*P logits of one head;
    section 2.3: 300 decoder queries; section 2.1.1: backbone strides
    8/16/32/64.

Recipe (identical for every consumer):
  * numpy ``default_rng(seed)`` (PCG64); draws happen in the fixed order
    value, reference points, offsets / locations, logits / weights,
    grad_output;
  * every float is drawn in float64 and cast once to the workload dtype
    (through torch's round-to-nearest-even conversion);
  * the softmax of the weight logits is part of input preparation (the core
    takes weights as given and never normalises them).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    """One problem instance on the host (torch CPU tensors, workload dtype)."""

    name: str
    dtype: str                       # "f32" | "f16" | "bf16"
    spatial_shapes: np.ndarray       # int64 [L, 2] = (H, W)
    level_start_index: np.ndarray    # int64 [L]
    value: torch.Tensor              # [bs, K, M, D]
    sampling_locations: torch.Tensor  # [bs, Q, M, L, P, 2]
    attention_weights: torch.Tensor  # [bs, Q, M, L, P]
    grad_output: torch.Tensor        # [bs, Q, M*D]
    meta: dict = field(default_factory=dict)
    sample_dtype: str | None = None  # per-sample tensors' type when it differs (mixed precision)

    @property
    def dims(self):
        bs, K, M, D = self.value.shape
        _, Q, _, L, P, _ = self.sampling_locations.shape
        return dict(bs=bs, num_keys=K, num_heads=M, embed_dims=D, num_levels=L,
                    num_points=P, num_queries=Q)

    def f32(self, name: str) -> np.ndarray:
        """The named float tensor widened exactly to float32 (oracle input)."""
        return getattr(self, name).to(torch.float32).numpy()


def level_starts(shapes) -> np.ndarray:
    """Exclusive prefix sum of H*W over levels (flattened level offsets)."""
    shapes = np.asarray(shapes, dtype=np.int64).reshape(-1, 2)
    hw = shapes[:, 0] * shapes[:, 1]
    return np.concatenate([[0], np.cumsum(hw)[:-1]]).astype(np.int64)


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(DTYPES[dtype]).contiguous()


def _softmax_last(x: np.ndarray) -> np.ndarray:
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def pixel_centre_refs(shapes) -> np.ndarray:
    """[K, 2] normalised (x, y) pixel centres of every flattened key, level by
    level, row-major within a level (valid ratios 1)."""
    refs = []
    for H, W in np.asarray(shapes, dtype=np.int64).reshape(-1, 2):
        ys, xs = np.meshgrid((np.arange(H) + 0.5) / H, (np.arange(W) + 0.5) / W, indexing="ij")
        refs.append(np.stack([xs.reshape(-1), ys.reshape(-1)], axis=-1))
    return np.concatenate(refs, axis=0)


def make(name: str, bs: int, shapes, heads: int, dims: int, points: int, queries: int,
         dtype: str, seed: int, value_dist: str = "normal", loc_dist: str = "uniform",
         loc_args: tuple = (0.0, 1.0), weight_dist: str = "softmax", grad_dist: str = "normal",
         meta: dict | None = None, sample_dtype: str | None = None) -> Workload:
    """General seeded generator.

    dtype is the value-side type (value, grad_output); sample_dtype, when
    given, the per-sample tensors' type (mixed precision: "f32"), else dtype.
    The draws are the same either way.

    value_dist:  "normal" N(0,1) | "u001" U[0,1)*0.01
    loc_dist:    "uniform" U[lo,hi]^2 i.i.d. per sample (loc_args = (lo, hi))
                 "encoder" pixel-centre ref of query q (queries = keys) +
                           N(0, sigma) offsets, clamped (loc_args = (sigma, lo, hi))
                 "decoder" per-query ref U[0,1]^2 shared over heads/levels/points
                           + N(0, sigma) offsets (loc_args = (sigma,))
                 "const"   every coordinate equals loc_args[0]
    weight_dist: "softmax" softmax over L*P of N(0,1) logits | "u+1e-5" U[0,1)+1e-5
    grad_dist:   "normal" N(0,1) | "ones"
    """
    shapes = np.asarray(shapes, dtype=np.int64).reshape(-1, 2)
    L = shapes.shape[0]
    K = int((shapes[:, 0] * shapes[:, 1]).sum())
    M, D, P, Q = heads, dims, points, queries
    rng = np.random.default_rng(seed)

    if value_dist == "normal":
        value = rng.standard_normal((bs, K, M, D))
    elif value_dist == "u001":
        value = rng.random((bs, K, M, D)) * 0.01
    else:
        raise ValueError(value_dist)

    lshape = (bs, Q, M, L, P, 2)
    if loc_dist == "uniform":
        lo, hi = loc_args
        loc = rng.uniform(lo, hi, size=lshape)
    elif loc_dist == "encoder":
        sigma, lo, hi = loc_args
        if Q != K:
            raise ValueError("encoder locations need queries == keys")
        ref = pixel_centre_refs(shapes)                      # [K, 2]
        loc = ref[None, :, None, None, None, :] + rng.normal(0.0, sigma, size=lshape)
        loc = np.clip(loc, lo, hi)
    elif loc_dist == "decoder":
        (sigma,) = loc_args
        ref = rng.random((bs, Q, 2))
        loc = ref[:, :, None, None, None, :] + rng.normal(0.0, sigma, size=lshape)
    elif loc_dist == "const":
        loc = np.full(lshape, float(loc_args[0]))
    else:
        raise ValueError(loc_dist)

    if weight_dist == "softmax":
        logits = rng.standard_normal((bs, Q, M, L * P))
        w = _softmax_last(logits).reshape(bs, Q, M, L, P)
    elif weight_dist == "u+1e-5":
        w = rng.random((bs, Q, M, L, P)) + 1e-5
    else:
        raise ValueError(weight_dist)

    if grad_dist == "normal":
        g = rng.standard_normal((bs, Q, M * D))
    elif grad_dist == "ones":
        g = np.ones((bs, Q, M * D))
    else:
        raise ValueError(grad_dist)

    sdt = sample_dtype or dtype
    return Workload(name=name, dtype=dtype, spatial_shapes=shapes,
                    level_start_index=level_starts(shapes),
                    value=_cast(value, dtype), sampling_locations=_cast(loc, sdt),
                    attention_weights=_cast(w, sdt), grad_output=_cast(g, dtype),
                    meta=dict(meta or {}, seed=seed),
                    sample_dtype=None if sdt == dtype else sdt)


# --- the five named workloads -------------------------------------------------

DETR_LEVELS = [(100, 134), (50, 67), (25, 34), (13, 17)]
LARGE_LEVELS = [(128, 128), (64, 64), (32, 32), (16, 16)]
STRESS_LEVELS = [(200, 200), (100, 100), (50, 50), (25, 25)]


def tiny_single_level(kink: bool = False) -> Workload:
    """bs 1, one 100x100 level, 4 heads x 32 dims, 8 points, 16 queries, fp32;
    value U[0,0.01), locations U[0,1]^2 (or the constant 0.005 of the usage
    example when ``kink``), weights U[0,1)+1e-5, grad_output ones."""
    return make("tiny_single_level" + ("_kink" if kink else ""), 1, [(100, 100)], 4, 32, 8, 16,
                "f32", 1001, value_dist="u001",
                loc_dist="const" if kink else "uniform",
                loc_args=(0.005,) if kink else (0.0, 1.0),
                weight_dist="u+1e-5", grad_dist="ones")


def detr_encoder(bs: int = 2, dtype: str = "f32", sigma: float = 0.02, seed: int = 1002,
                 sample_dtype: str | None = None) -> Workload:
    """Deformable-DETR encoder self-attention: 4 levels (100,134) (50,67)
    (25,34) (13,17), K = Q = 17821, 8 heads x 32 dims, 4 points."""
    K = sum(h * w for h, w in DETR_LEVELS)
    return make("detr_encoder", bs, DETR_LEVELS, 8, 32, 4, K, dtype, seed,
                loc_dist="encoder", loc_args=(sigma, -0.05, 1.05), sample_dtype=sample_dtype)


def detr_decoder(dtype: str = "f32", sample_dtype: str | None = None) -> Workload:
    """Deformable-DETR decoder cross-attention: the encoder's 4-level value,
    bs 2, 300 queries, 4 points; refs U[0,1]^2 + N(0, 0.05) offsets."""
    return make("detr_decoder", 2, DETR_LEVELS, 8, 32, 4, 300, dtype, 1003,
                loc_dist="decoder", loc_args=(0.05,), sample_dtype=sample_dtype)


def large_batch_encoder(bs: int = 8, dtype: str = "bf16") -> Workload:
    """bs 8 encoder on the 1024x1024 pyramid (128,128) (64,64) (32,32) (16,16),
    K = Q = 21760, 8 heads x 32 dims, 4 points, bf16."""
    K = sum(h * w for h, w in LARGE_LEVELS)
    return make("large_batch_encoder", bs, LARGE_LEVELS, 8, 32, 4, K, dtype, 1004,
                loc_dist="encoder", loc_args=(0.02, -0.05, 1.05))


def max_constraint(dtype: str = "f16") -> Workload:
    """bs 4, 8 heads x 64 dims, 4 levels x 16 points (L*P = 64), levels
    (200,200) (100,100) (50,50) (25,25), K = 53125, 900 queries, fp16;
    locations U[-0.1, 1.1]^2."""
    return make("max_constraint", 4, STRESS_LEVELS, 8, 64, 16, 900, dtype, 1005,
                loc_dist="uniform", loc_args=(-0.1, 1.1))


# Levels whose value bytes per batch (8 heads x 32 dims: 1 KiB per key in
# float32, 512 B in fp16 / bf16) fall within 4 MiB below 2^31, the envelope's
# per-batch byte limit.
OFFSET_LIMIT_LEVELS = {4: [(1448, 1446), (4, 5)], 2: [(2048, 2046), (4, 5)]}


def offset_limit(dtype: str = "f32", seed: int = 1031, queries: int = 48) -> Workload:
    """bs 2 at the per-batch byte limit of the envelope: two levels (the
    large one sized for the dtype, then (4, 5)), 8 heads x 32 dims
    (2,144,079,872 value bytes per batch in float32, 2,145,396,736 in 16-bit;
    batch 1 starts 2 GiB into the tensor), 4 points, `queries` queries.
    Level-0 locations U[0.97, 1.02]^2 (the map's last rows and columns, some
    corners off the map), level-1 locations U[-0.1, 1.1]^2 (the last keys of
    the batch).  value is U[-1, 1), drawn directly in float32 to keep the
    draw cheap, then rounded to the dtype; weights and grad_output as in
    make()."""
    shapes = np.asarray(OFFSET_LIMIT_LEVELS[4 if dtype == "f32" else 2], dtype=np.int64)
    K = int((shapes[:, 0] * shapes[:, 1]).sum())
    bs, M, D, L, P, Q = 2, 8, 32, 2, 4, queries
    rng = np.random.default_rng(seed)
    v = rng.random((bs, K, M, D), dtype=np.float32)
    v *= 2.0
    v -= 1.0
    value = torch.from_numpy(v).to(DTYPES[dtype])
    del v
    loc = np.empty((bs, Q, M, L, P, 2))
    loc[:, :, :, 0] = rng.uniform(0.97, 1.02, size=(bs, Q, M, P, 2))
    loc[:, :, :, 1] = rng.uniform(-0.1, 1.1, size=(bs, Q, M, P, 2))
    w = _softmax_last(rng.standard_normal((bs, Q, M, L * P))).reshape(bs, Q, M, L, P)
    g = rng.standard_normal((bs, Q, M * D))
    return Workload(f"offset_limit_{dtype}", dtype, shapes, level_starts(shapes), value, _cast(loc, dtype),
                    _cast(w, dtype), _cast(g, dtype))


NAMED = {
    "tiny_single_level": tiny_single_level,
    "detr_encoder": detr_encoder,
    "detr_decoder": detr_decoder,
    "detr_decoder_f16": lambda: detr_decoder("f16"),
    "large_batch_encoder": large_batch_encoder,
    "max_constraint": max_constraint,
    # mixed precision: bf16 value side, float32 locations and weights
    "detr_encoder_bf16_f32": lambda: detr_encoder(dtype="bf16", sample_dtype="f32"),
}


# --- inputs of the fused prologue ----------------------------------------------

@dataclass
class FusedWorkload:
    """Inputs of the fused form: reference points, raw sampling offsets and
    attention logits instead of locations and weights (host tensors)."""

    name: str
    dtype: str
    spatial_shapes: np.ndarray       # int64 [L, 2] = (H, W)
    level_start_index: np.ndarray    # int64 [L]
    value: torch.Tensor              # [bs, K, M, D]
    reference_points: torch.Tensor   # [bs, Q, L, 2 or 4]
    sampling_offsets: torch.Tensor   # [bs, Q, M, L, P, 2]
    attention_logits: torch.Tensor   # [bs, Q, M, L, P]
    grad_output: torch.Tensor        # [bs, Q, M*D]
    key_padding_mask: torch.Tensor | None = None   # bool [bs, K] or None
    meta: dict = field(default_factory=dict)
    sample_dtype: str | None = None  # per-sample tensors' type when it differs (mixed precision)

    @property
    def ref_dims(self) -> int:
        return int(self.reference_points.shape[-1])

    def f32(self, name: str) -> np.ndarray:
        return getattr(self, name).to(torch.float32).numpy()


def offset_directions(heads: int, levels: int, points: int) -> np.ndarray:
    """[M, L, P, 2] pixel offsets of the module's initial sampling pattern
    (walkthrough section 2.2.4, _reset_parameters): head m looks along the
    angle 2 pi m / M, its direction scaled so that the larger component is
    1, and point p goes p + 1 steps along it, on every level."""
    th = np.arange(heads) * (2.0 * np.pi / heads)
    d = np.stack([np.cos(th), np.sin(th)], -1)
    d = d / np.abs(d).max(-1, keepdims=True)
    steps = np.arange(1, points + 1, dtype=np.float64)
    return np.broadcast_to(d[:, None, None, :] * steps[None, None, :, None], (heads, levels, points, 2)).copy()


def padding_masks(shapes, valid) -> tuple[np.ndarray, np.ndarray]:
    """Key padding of a batch of images padded to one size (walkthrough
    section 2.1: the backbone downsamples the image mask to every level with
    F.interpolate, nearest; section 2.2.4: the valid ratios are the unpadded
    fraction of each level's width and height).

    valid: per batch element, the unpadded fraction (h, w) of the padded
    image, whose size is 8x the first level's.  Returns the mask
    [bs, K] (True = padded key) and the valid ratios [bs, L, 2] as (x, y)."""
    import torch.nn.functional as F
    shapes = np.asarray(shapes, dtype=np.int64).reshape(-1, 2)
    Hi, Wi = int(shapes[0, 0]) * 8, int(shapes[0, 1]) * 8
    img = torch.zeros(len(valid), Hi, Wi, dtype=torch.bool)
    for b, (fh, fw) in enumerate(valid):
        img[b, int(round(fh * Hi)):, :] = True
        img[b, :, int(round(fw * Wi)):] = True
    masks, ratios = [], []
    for H, W in shapes:
        m = F.interpolate(img[None].float(), size=(int(H), int(W))).to(torch.bool)[0]     # [bs, H, W]
        vh = (~m[:, :, 0]).sum(1).double() / float(H)
        vw = (~m[:, 0, :]).sum(1).double() / float(W)
        masks.append(m.reshape(len(valid), -1))
        ratios.append(torch.stack([vw, vh], -1))
    return torch.cat(masks, 1).numpy(), torch.stack(ratios, 1).numpy()


def make_fused(name: str, bs: int, shapes, heads: int, dims: int, points: int, queries: int,
               dtype: str, seed: int, ref_dims: int = 2, ref_dist: str = "uniform",
               offset_sigma: float = 1.0, valid=None, meta: dict | None = None,
               sample_dtype: str | None = None) -> FusedWorkload:
    """Seeded inputs of the fused form.

    ref_dist:  "encoder" the pixel centre of query q (queries = keys), the
                         same on every level (valid ratios 1), as the encoder's
                         get_reference_points gives;
               "uniform" U[0,1]^2 per query, the same on every level (the
                         decoder's reference points).
    ref_dims 4 appends a box size U[0.05, 0.5]^2 per query.
    valid (per batch element (h, w) fractions, see padding_masks) adds a key
    padding mask and scales the reference points by the valid ratios the way
    the encoder (get_reference_points: pixel centres over the valid extent,
    times each level's ratio) and the decoder (reference times the ratios;
    the box by the ratios too) do; None means no padding.
    Offsets: the initial sampling pattern (offset_directions) plus
    N(0, offset_sigma) pixels per sample -- the 4-d form reads the same
    numbers in units of P half box sizes.  Logits: N(0, 1).
    Draw order: value, reference points, box sizes, offsets, logits,
    grad_output.  sample_dtype as for make.
    """
    shapes = np.asarray(shapes, dtype=np.int64).reshape(-1, 2)
    L = shapes.shape[0]
    K = int((shapes[:, 0] * shapes[:, 1]).sum())
    M, D, P, Q = heads, dims, points, queries
    rng = np.random.default_rng(seed)
    value = rng.standard_normal((bs, K, M, D))
    if valid is not None:
        if len(valid) != bs:
            raise ValueError("valid needs one (h, w) pair per batch element")
        mask, ratios = padding_masks(shapes, valid)
    else:
        mask, ratios = None, np.ones((bs, L, 2))
    if ref_dist == "encoder":
        if Q != K:
            raise ValueError("encoder reference points need queries == keys")
        # pixel centres of each query's own level over that level's valid extent
        lvl_of_key = np.repeat(np.arange(L), shapes[:, 0] * shapes[:, 1])
        xy = pixel_centre_refs(shapes)[None] / ratios[:, lvl_of_key, :]          # [bs, K, 2]
    elif ref_dist == "uniform":
        xy = rng.random((bs, Q, 2))
    else:
        raise ValueError(ref_dist)
    ref = xy[:, :, None, :] * ratios[:, None, :, :]
    if ref_dims == 4:
        wh = rng.uniform(0.05, 0.5, size=(bs, Q, 2))
        ref = np.concatenate([ref, wh[:, :, None, :] * ratios[:, None, :, :]], -1)
    elif ref_dims != 2:
        raise ValueError(ref_dims)
    off = offset_directions(M, L, P)[None, None] + rng.normal(0.0, offset_sigma, size=(bs, Q, M, L, P, 2))
    logits = rng.standard_normal((bs, Q, M, L, P))
    g = rng.standard_normal((bs, Q, M * D))
    sdt = sample_dtype or dtype
    return FusedWorkload(name=name, dtype=dtype, spatial_shapes=shapes, level_start_index=level_starts(shapes),
                         value=_cast(value, dtype), reference_points=_cast(ref, sdt),
                         sampling_offsets=_cast(off, sdt), attention_logits=_cast(logits, sdt),
                         grad_output=_cast(g, dtype),
                         key_padding_mask=None if mask is None else torch.from_numpy(mask),
                         meta=dict(meta or {}, seed=seed), sample_dtype=None if sdt == dtype else sdt)


def detr_encoder_fused(bs: int = 2, dtype: str = "f32", seed: int = 1012) -> FusedWorkload:
    """The DETR encoder shapes in the fused form: pixel-centre reference
    points (2-d), offsets around the initial pattern, logits."""
    K = sum(h * w for h, w in DETR_LEVELS)
    return make_fused("detr_encoder_fused", bs, DETR_LEVELS, 8, 32, 4, K, dtype, seed, 2, "encoder")


def detr_decoder_fused(dtype: str = "f32", ref_dims: int = 4, seed: int = 1013) -> FusedWorkload:
    """The DETR decoder shapes in the fused form (bs 2, 300 queries), with
    4-d box reference points (two-stage / box refinement) by default."""
    return make_fused("detr_decoder_fused", 2, DETR_LEVELS, 8, 32, 4, 300, dtype, seed, ref_dims, "uniform")


# --- inputs of the whole module step ------------------------------------------

@dataclass
class ModuleWorkload:
    """Inputs and parameters of one MSDeformAttn module step (host, float32)."""

    name: str
    spatial_shapes: np.ndarray
    level_start_index: np.ndarray
    d_model: int
    n_heads: int
    n_levels: int
    n_points: int
    params: dict                     # name -> float32 array, nn.Linear layouts
    query: torch.Tensor              # [bs, Q, C]
    input_flatten: torch.Tensor      # [bs, K, C]
    reference_points: torch.Tensor   # [bs, Q, L, 2 or 4]
    grad_output: torch.Tensor        # [bs, Q, C]
    key_padding_mask: torch.Tensor | None = None
    meta: dict = field(default_factory=dict)


def make_module(name: str, bs: int, shapes, d_model: int, n_heads: int, n_points: int, queries: int,
                seed: int, ref_dims: int = 2, ref_dist: str = "uniform", valid=None,
                dyadic: bool = False) -> ModuleWorkload:
    """Seeded module inputs.  Parameters: ``module.module_parameters``, or with
    ``dyadic`` every weight a multiple of 1/64 in [-1/4, 1/4] and the offset
    bias rounded to 1/64, with query and input_flatten multiples of 1/8 in
    [-2, 2]: then value, offsets and logits (sums of 256 products) are exact
    in float32 whatever the summation order, so every consumer forms the same
    sampling locations.  Otherwise query and input_flatten are N(0, 1).
    Reference points and padding as in make_fused (queries = keys for
    ref_dist "encoder").  grad_output N(0, 1).
    Draw order: parameters (own seed), query, input_flatten, reference points,
    box sizes, grad_output."""
    from .module import module_parameters
    shapes = np.asarray(shapes, dtype=np.int64).reshape(-1, 2)
    L = shapes.shape[0]
    K = int((shapes[:, 0] * shapes[:, 1]).sum())
    C, Q = d_model, queries
    rng = np.random.default_rng(seed)
    if dyadic:
        M, P = n_heads, n_points
        params = {
            "value_proj.weight": rng.integers(-16, 17, size=(C, C)) / 64, "value_proj.bias": np.zeros(C),
            "sampling_offsets.weight": rng.integers(-16, 17, size=(M * L * P * 2, C)) / 64,
            "sampling_offsets.bias": np.round(offset_directions(M, L, P).reshape(-1) * 64) / 64,
            "attention_weights.weight": rng.integers(-16, 17, size=(M * L * P, C)) / 64,
            "attention_weights.bias": np.zeros(M * L * P),
            "output_proj.weight": rng.integers(-16, 17, size=(C, C)) / 64, "output_proj.bias": np.zeros(C),
        }
        query = rng.integers(-16, 17, size=(bs, Q, C)) / 8
        inp = rng.integers(-16, 17, size=(bs, K, C)) / 8
    else:
        params = module_parameters(C, L, n_heads, n_points, seed + 1)
        query = rng.standard_normal((bs, Q, C))
        inp = rng.standard_normal((bs, K, C))
    params = {k: np.asarray(v, dtype=np.float32) for k, v in params.items()}
    if valid is not None:
        mask, ratios = padding_masks(shapes, valid)
    else:
        mask, ratios = None, np.ones((bs, L, 2))
    if ref_dist == "encoder":
        if Q != K:
            raise ValueError("encoder reference points need queries == keys")
        lvl_of_key = np.repeat(np.arange(L), shapes[:, 0] * shapes[:, 1])
        xy = pixel_centre_refs(shapes)[None] / ratios[:, lvl_of_key, :]
    else:
        xy = rng.random((bs, Q, 2))
    ref = xy[:, :, None, :] * ratios[:, None, :, :]
    if ref_dims == 4:
        wh = rng.uniform(0.05, 0.5, size=(bs, Q, 2))
        ref = np.concatenate([ref, wh[:, :, None, :] * ratios[:, None, :, :]], -1)
    g = rng.standard_normal((bs, Q, C))
    return ModuleWorkload(name=name, spatial_shapes=shapes, level_start_index=level_starts(shapes), d_model=C,
                          n_heads=n_heads, n_levels=L, n_points=n_points, params=params,
                          query=_cast(query, "f32"), input_flatten=_cast(inp, "f32"),
                          reference_points=_cast(ref, "f32"), grad_output=_cast(g, "f32"),
                          key_padding_mask=None if mask is None else torch.from_numpy(mask),
                          meta=dict(seed=seed, dyadic=dyadic))


def detr_encoder_module(bs: int = 2, seed: int = 1022) -> ModuleWorkload:
    """One encoder layer's MSDeformAttn step at the DETR encoder shapes:
    d_model 256 (8 heads x 32), 4 levels, 4 points, K = Q = 17821,
    pixel-centre reference points."""
    K = sum(h * w for h, w in DETR_LEVELS)
    return make_module("detr_encoder_module", bs, DETR_LEVELS, 256, 8, 4, K, seed, 2, "encoder")
