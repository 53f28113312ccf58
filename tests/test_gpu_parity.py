"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
identical seeded inputs, element by element (tolerances in tests/parity.py).

Covers the five named workloads at full size, fwd and bwd, in their dtypes,
plus edge cases: tiny and degenerate maps (1x1, 1xW, Hx1), one level / one
point, fully and partly off-map samples, exact pixel centres and kinks,
NaN/Inf locations, every lane split of the kernels (embed_dims 8..256 in each
dtype), ragged tails, empty problems, the maximum envelope, non-default
streams and the autograd wrapper.
"""
import json
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from scale_deformable_attention_03_amd import workloads as W
from tests.parity import (TOL, assert_close, check_backward, check_forward, f64, gpu_backward,
                          gpu_forward, oracle_backward, oracle_forward, to_device)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import scale_deformable_attention_03_amd._lib as lib
    assert os.path.exists(lib.LIB_PATH)
    print(f"[gpu] device {torch.cuda.get_device_name(0)}", flush=True)


# ---------------------------------------------------------------------------
# the five named workloads, full size
# ---------------------------------------------------------------------------

NAMED = [
    ("tiny_single_level", lambda: W.tiny_single_level()),
    ("tiny_single_level_kink", lambda: W.tiny_single_level(kink=True)),
    ("detr_encoder_f32", lambda: W.detr_encoder()),
    ("detr_decoder_f32", lambda: W.detr_decoder("f32")),
    ("detr_decoder_f16", lambda: W.detr_decoder("f16")),
    ("large_batch_encoder_bf16", lambda: W.large_batch_encoder()),
    ("max_constraint_f16", lambda: W.max_constraint()),
]


@pytest.mark.parametrize("name,make", NAMED, ids=[n for n, _ in NAMED])
def test_named_workload(name, make):
    print(f"[gpu] workload {name}", flush=True)
    wl = make()
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


# ---------------------------------------------------------------------------
# closed forms through the GPU
# ---------------------------------------------------------------------------

def test_golden_2x2_on_gpu():
    gold = json.load(open(os.path.join(GOLDEN, "bilinear_2x2.json")))
    cases = gold["cases"]
    n = len(cases)
    D = 8                                  # the map, replicated over 8 channels
    vmap = torch.tensor(gold["map"], dtype=torch.float32).reshape(1, 4, 1, 1).expand(1, 4, 1, D)
    loc = torch.tensor([c["loc"] for c in cases], dtype=torch.float32).reshape(1, n, 1, 1, 1, 2)
    w = torch.ones(1, n, 1, 1, 1)
    g = torch.zeros(1, n, D)
    g[..., 0] = 1.0                         # grad_output selects channel 0
    wl = W.Workload("golden2x2", "f32", np.array([[2, 2]]), np.array([0]), vmap.contiguous(), loc, w, g)
    out = f64(gpu_forward(wl))
    gv, gl, gw = gpu_backward(wl)
    for i, c in enumerate(cases):
        assert out[0, i, 0] == pytest.approx(c["sample"], abs=1e-6), c
        assert f64(gl)[0, i, 0, 0, 0] == pytest.approx(c["grad_loc"], abs=1e-5), c
        assert f64(gw)[0, i, 0, 0, 0] == pytest.approx(c["sample"], abs=1e-6), c


def test_ascend_example_closed_form_on_gpu():
    """Locations 0.005 on a 100x100 map land exactly on pixel (0, 0): the
    output is value row 0 times the weight sum (exact floor decision)."""
    wl = W.tiny_single_level(kink=True)
    out = f64(gpu_forward(wl))
    V = wl.f32("value").astype(np.float64)
    w = wl.f32("attention_weights").astype(np.float64)
    expect = (w.sum(axis=(3, 4))[..., None] * V[0, 0][None, None]).reshape(1, 16, 128)
    assert_close("ascend_example", out, expect, 1e-5, atol=1e-7)
    gv, gl, gw = gpu_backward(wl)
    gvn = f64(gv)
    assert np.all(gvn[0, 1:] == 0.0), "only row 0 receives gradient"
    G = wl.f32("grad_output").astype(np.float64).reshape(1, 16, 4, 32)
    dx = np.einsum("bqmd,md->bqm", G, V[0, 1] - V[0, 0])[..., None, None]
    assert_close("ascend_example/grad_loc_x", f64(gl)[..., 0], 100 * w * dx, 1e-4, atol=1e-6)


# ---------------------------------------------------------------------------
# edge cases and every kernel instantiation
# ---------------------------------------------------------------------------

EDGE = [
    # (id, bs, shapes, M, D, P, Q, dtype, loc_dist, loc_args)
    ("map1x1", 2, [(1, 1)], 3, 8, 3, 37, "f32", "uniform", (-0.5, 1.5)),
    ("row1xW_colHx1", 1, [(1, 9), (7, 1)], 2, 16, 2, 50, "f32", "uniform", (-0.3, 1.3)),
    ("one_level_one_point", 3, [(13, 17)], 1, 32, 1, 101, "f32", "uniform", (-0.1, 1.1)),
    ("far_off_map", 1, [(10, 10), (5, 5)], 4, 32, 4, 30, "f32", "uniform", (-3.0, 4.0)),
    ("D8_f16", 2, [(12, 9), (6, 5)], 8, 8, 4, 77, "f16", "uniform", (-0.1, 1.1)),
    ("D16_bf16", 2, [(12, 9), (6, 5)], 5, 16, 3, 65, "bf16", "uniform", (-0.1, 1.1)),
    ("D24_f32_masked_lanes", 1, [(9, 14), (4, 7)], 3, 24, 2, 70, "f32", "uniform", (-0.1, 1.1)),
    ("D24_f16", 1, [(9, 14), (4, 7)], 3, 24, 2, 70, "f16", "uniform", (-0.1, 1.1)),
    ("D40_f32", 2, [(8, 8)], 2, 40, 5, 33, "f32", "uniform", (-0.1, 1.1)),
    ("D64_f32", 2, [(20, 30), (10, 15)], 8, 64, 4, 129, "f32", "uniform", (-0.1, 1.1)),
    ("D128_bf16", 1, [(20, 30), (10, 15), (5, 8)], 4, 128, 2, 45, "bf16", "uniform", (-0.1, 1.1)),
    ("D256_f32_max_dims", 1, [(16, 16), (8, 8)], 8, 256, 32, 9, "f32", "uniform", (-0.1, 1.1)),
    ("D256_f16", 1, [(16, 16)], 2, 256, 3, 21, "f16", "uniform", (-0.1, 1.1)),
    ("LP64_max_envelope", 2, [(30, 40), (15, 20), (8, 10), (4, 5)], 8, 32, 16, 61, "f32", "uniform", (-0.1, 1.1)),
    ("L64_P1", 1, [(2 + i % 3, 3 + i % 4) for i in range(64)], 2, 8, 1, 19, "f32", "uniform", (-0.1, 1.1)),
    ("ragged_tail_L4P4", 1, [(17, 23), (9, 12), (5, 6), (3, 3)], 8, 32, 4, 33, "f32", "uniform", (-0.1, 1.1)),
    ("ragged_tail_bf16", 3, [(17, 23), (9, 12), (5, 6), (3, 3)], 7, 32, 4, 13, "bf16", "uniform", (-0.1, 1.1)),
    # more than 64 (batch, head) planes: the accumulation's plane lookup reads
    # a second chunk of unit prefixes; sparse (few records per key) and dense
    ("planes72_sparse", 9, [(20, 27), (10, 14)], 8, 16, 2, 40, "f32", "uniform", (-0.1, 1.1)),
    ("planes130_dense", 26, [(6, 7), (3, 4)], 5, 8, 4, 300, "f32", "uniform", (-0.1, 1.1)),
    ("planes72_dense_bf16", 9, [(8, 9), (4, 5)], 8, 16, 4, 150, "bf16", "uniform", (-0.1, 1.1)),
    # the fixed L4P4 / L4P16 kernels at other lane splits: samples per lane in
    # the prologues (2 for float32, 4 for 16-bit), samples kept per lane for
    # the grad_loc / grad_w stores (16- and 32-byte grad_loc), and none
    ("L4P4_f32_D16", 2, [(12, 14), (6, 7), (3, 4), (2, 2)], 4, 16, 4, 70, "f32", "uniform", (-0.1, 1.1)),
    ("L4P4_bf16_D16", 2, [(12, 14), (6, 7), (3, 4), (2, 2)], 4, 16, 4, 70, "bf16", "uniform", (-0.1, 1.1)),
    ("L4P4_f16_D64", 2, [(12, 14), (6, 7), (3, 4), (2, 2)], 4, 64, 4, 70, "f16", "uniform", (-0.1, 1.1)),
    ("L4P4_f32_D64", 1, [(12, 14), (6, 7), (3, 4), (2, 2)], 4, 64, 4, 70, "f32", "uniform", (-0.1, 1.1)),
    ("L4P16_f32_D16", 2, [(12, 14), (6, 7), (3, 4), (2, 2)], 4, 16, 16, 45, "f32", "uniform", (-0.1, 1.1)),
    ("L4P16_bf16_D32", 2, [(12, 14), (6, 7), (3, 4), (2, 2)], 4, 32, 16, 45, "bf16", "uniform", (-0.1, 1.1)),
    ("L4P16_f16_D64", 1, [(12, 14), (6, 7), (3, 4), (2, 2)], 8, 64, 16, 45, "f16", "uniform", (-0.1, 1.1)),
    # level extents at the binned path's limit (16-bit cell fields: x0 + 1 and
    # y0 + 1 up to 65534)
    ("width65534_binned", 1, [(2, 65534)], 1, 8, 2, 3000, "f32", "uniform", (-0.05, 1.05)),
    ("height65534_binned", 1, [(65534, 2)], 1, 8, 2, 3000, "f32", "uniform", (-0.05, 1.05)),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_case(case):
    name, bs, shapes, M, D, P, Q, dtype, dist, args = case
    print(f"[gpu] edge {name}", flush=True)
    wl = W.make(name, bs, shapes, M, D, P, Q, dtype, seed=zlib.crc32(name.encode()) % 10000, loc_dist=dist, loc_args=args)
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


@pytest.mark.parametrize("levels,dtype,binned", [
    ([(512, 1024)], "f32", True),                # 2048 segments of 256 keys: the LDS histogram's size
    ([(512, 1024)], "bf16", True),
    ([(512, 1024), (2, 64)], "f32", False),      # 2052 segments: float atomics instead
    ([(512, 1024), (1, 1)], "f32", False),       # 2049 segments, and one hot row per head
], ids=["2048_f32", "2048_bf16", "2052_f32", "2049_hot_row_f32"])
def test_segment_limit(levels, dtype, binned):
    """The binned backward at its segment limit: embed_dims 8 and few records
    per key give segments of 256 keys, so a level of 512 x 1024 keys fills
    exactly the 2048 histogram slots per plane; a second level of 2 x 64 keys
    (four more segments) takes the float-atomic backward.  The path taken
    shows in the workspace size (float32 problems need none without
    records).  A 1 x 1 second level makes its single row per head the sum of
    all 8,000 of that head's samples on the level (largely cancelling, as
    grad_output is N(0, 1)): added one corner at a time in arbitrary order,
    its float32 rounding missed the elementwise bar (relative error 1.6e-4 on
    one element); the gradient workgroup's pre-reduction makes it about 32
    adds of merged partial sums per element."""
    from scale_deformable_attention_03_amd import _lib, ops
    wl = W.make(f"segments_{dtype}", 1, levels, 2, 8, 4, 2000, dtype, seed=1041, loc_args=(-0.05, 1.05))
    print(f"[gpu] segment limit {levels} {dtype}", flush=True)
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_locations)
    ws = _lib.workspace_bytes(prob)
    if dtype == "f32":
        assert (ws > 0) == binned
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


def test_query_field_limit():
    """2^24 - 1 queries in one plane, the most the binned records' 24-bit
    query field holds (one head, one level of 64 x 64 keys, one point,
    embed_dims 8): every query index up to the field's maximum is packed
    into a record and read back as a grad_output row."""
    from scale_deformable_attention_03_amd import _lib, ops
    Q = (1 << 24) - 1
    wl = W.make("query_limit", 1, [(64, 64)], 1, 8, 1, Q, "f32", seed=1042, loc_args=(-0.05, 1.05),
                weight_dist="u+1e-5")
    print(f"[gpu] query field limit: Q {Q}", flush=True)
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_locations)
    assert _lib.workspace_bytes(prob) > 0, "binned backward"
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_byte_offset_limit(dtype):
    """Per batch, value bytes within 4 MiB below 2^31 (the envelope's limit on
    32-bit byte offsets; one past the last byte is the off-map sentinel), bs
    2 so that batch 1's rows lie beyond 2^31 bytes from the tensor start;
    samples on the map's last rows and columns and in the last level.  At
    this size the backward scatters with float atomics (more keys than the
    binned records address), for fp16 into a float32 workspace of more than
    2^31 elements that is then rounded.  Forward, grad_loc and grad_w in full
    against the oracle; grad_value on every row either side touched, the
    tolerance's RMS taken over the whole tensor, and every other row exactly
    zero."""
    from scale_deformable_attention_03_amd import _lib, ops
    wl = W.offset_limit(dtype)
    bs, K, M, D = wl.value.shape
    per_batch = K * M * D * wl.value.element_size()
    assert 2 ** 31 - (4 << 20) < per_batch < 2 ** 31
    print(f"[gpu] offset limit {dtype}: bs {bs} K {K} bytes per batch {per_batch}", flush=True)
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_locations)
    assert _lib.validate(prob) == 0
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    gv, gl, gw = gpu_backward(wl, t)
    del t
    rgv, rgl, rgw = oracle_backward(wl)
    rtol, arms, atol = TOL[(dtype, "bwd")]
    assert_close(f"{wl.name}/grad_attention_weights", f64(gw), rgw, rtol, arms)
    assert_close(f"{wl.name}/grad_sampling_locations", f64(gl), rgl, rtol, arms)
    ref_rows = rgv.reshape(bs * K, M * D)
    ref_touched = np.flatnonzero(np.any(ref_rows != 0.0, axis=1))
    gpu_rows = gv.view(bs * K, M * D)
    gpu_touched = torch.nonzero(gpu_rows.abs().amax(dim=1) != 0).flatten().cpu().numpy()
    rows = np.union1d(ref_touched, gpu_touched)
    assert rows.size > 0 and rows.max() >= K, "batch 1 holds touched rows"
    rms = float(np.sqrt(np.sum(ref_rows[ref_touched] ** 2) / ref_rows.size))
    got = gpu_rows[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    assert_close(f"{wl.name}/grad_value (touched rows)", got, ref_rows[rows], rtol, atol=arms * rms)
    assert np.setdiff1d(gpu_touched, ref_touched).size == 0


def test_pixel_centres_and_kinks():
    """Locations on exact pixel centres (integer pixel coordinates: every
    sample is a kink) on non-power-of-two maps: same floor decisions as the
    oracle, so the gradients agree too."""
    rng = np.random.default_rng(7)
    shapes = np.array([(100, 134), (13, 17)])
    wl = W.make("centres", 1, shapes, 4, 32, 4, 64, "f32", seed=7)
    loc = np.empty((1, 64, 4, 2, 4, 2))
    for lvl, (H, Wd) in enumerate(shapes):
        loc[..., lvl, :, 0] = (rng.integers(0, Wd, (1, 64, 4, 4)) + 0.5) / Wd
        loc[..., lvl, :, 1] = (rng.integers(0, H, (1, 64, 4, 4)) + 0.5) / H
    wl.sampling_locations = torch.tensor(loc, dtype=torch.float32)
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


def test_nan_inf_locations_contribute_nothing():
    wl = W.make("naninf", 1, [(6, 8)], 2, 16, 3, 10, "f32", seed=3)
    loc = wl.sampling_locations.clone()
    loc[0, 0, 0, 0, 0, 0] = float("nan")
    loc[0, 1, 1, 0, 1, 1] = float("inf")
    loc[0, 2, 0, 0, 2, 0] = float("-inf")
    loc[0, 3, 1, 0, 0, :] = 1e30
    wl.sampling_locations = loc
    t = to_device(wl)
    out = check_forward(wl, gpu_forward(wl, t))
    assert torch.isfinite(out).all()
    gv, gl, gw = check_backward(wl, gpu_backward(wl, t))
    assert torch.isfinite(gv).all() and torch.isfinite(gl).all() and torch.isfinite(gw).all()


# ---------------------------------------------------------------------------
# empty problems, determinism, streams, autograd
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bs,Q", [(0, 5), (2, 0)])
def test_empty_problem(bs, Q, dtype):
    from scale_deformable_attention_03_amd import ops
    dt = W.DTYPES[dtype]
    shapes = np.array([(4, 5)])
    v = torch.randn(bs, 20, 2, 8, device="cuda").to(dt)
    loc = torch.rand(bs, Q, 2, 1, 2, 2, device="cuda").to(dt)
    w = torch.rand(bs, Q, 2, 1, 2, device="cuda").to(dt)
    out = ops.forward(v, shapes, [0], loc, w)
    assert out.shape == (bs, Q, 16)
    gv = torch.full_like(v, 7.0)
    g = torch.randn(bs, Q, 16, device="cuda").to(dt)
    gv, gl, gw = ops.backward(v, shapes, [0], loc, w, g, grads=(gv, torch.empty_like(loc), torch.empty_like(w)))
    torch.cuda.synchronize()
    assert (gv == 0).all(), "grad_value is zeroed even when no query samples it"


def test_backward_accumulate_without_queries_leaves_buffer():
    """Q = 0 through msda_backward_accumulate adds nothing."""
    from scale_deformable_attention_03_amd import _lib, ops
    shapes = np.array([(4, 5)])
    v = torch.randn(2, 20, 2, 8, device="cuda")
    loc = torch.rand(2, 0, 2, 1, 2, 2, device="cuda")
    w = torch.rand(2, 0, 2, 1, 2, device="cuda")
    g = torch.randn(2, 0, 16, device="cuda")
    prob, keep = ops.problem_for(v, shapes, [0], loc)
    need = max(_lib.workspace_bytes(prob), 16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    acc = torch.full(v.shape, 0.5, dtype=torch.float32, device="cuda")
    _lib.backward_accumulate(prob, v.data_ptr(), loc.data_ptr(), w.data_ptr(), g.data_ptr(), acc.data_ptr(),
                             loc.data_ptr(), w.data_ptr(), ws.data_ptr(), need,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (acc == 0.5).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_segments_split_over_units(dtype):
    """A 4x4 level sampled 16,000 times per head: each segment holds far more
    records than one accumulation unit, so its rows are zeroed, added with
    float atomics and (16-bit) rounded from the float32 workspace, while a
    sparse 30x40 level beside it is written straight from the tile."""
    wl = W.make("split_units", 2, [(4, 4), (30, 40)], 2, 16, 4, 2000, dtype, seed=21,
                loc_dist="uniform", loc_args=(-0.05, 1.05))
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


def test_forward_bitwise_repeatable_and_backward_stable():
    wl = W.detr_decoder("f32")
    t = to_device(wl)
    a = gpu_forward(wl, t).clone()
    b = gpu_forward(wl, t)
    assert torch.equal(a, b)
    gv1, gl1, gw1 = [x.clone() for x in gpu_backward(wl, t)]
    gv2, gl2, gw2 = gpu_backward(wl, t)
    assert torch.equal(gl1, gl2) and torch.equal(gw1, gw2)
    assert_close("grad_value run-to-run", f64(gv2), f64(gv1), 1e-5, atol=1e-6)


def test_non_default_stream():
    from scale_deformable_attention_03_amd import ops
    wl = W.detr_decoder("f32")
    t = to_device(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = ops.forward(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"], t["w"])
    s.synchronize()
    check_forward(wl, out)


def test_autograd_function():
    from scale_deformable_attention_03_amd import ms_deform_attn
    wl = W.make("autograd", 2, [(11, 13), (6, 7)], 4, 32, 3, 40, "f32", seed=5)
    t = to_device(wl)
    v = t["value"].clone().requires_grad_()
    loc = t["loc"].clone().requires_grad_()
    w = t["w"].clone().requires_grad_()
    shapes_dev = torch.tensor(wl.spatial_shapes, device="cuda")       # device shape tensors work too
    starts_dev = torch.tensor(wl.level_start_index, device="cuda")
    out = ms_deform_attn(v, shapes_dev, starts_dev, loc, w)
    out.backward(t["g"])
    check_forward(wl, out.detach())
    check_backward(wl, (v.grad, loc.grad, w.grad))


def test_sampled_outputs_one_by_one_at_full_size():
    """The benchmark's workload (DETR encoder, fp32, bs 2) checked on outputs
    the oracle computes one (b, q, m) at a time, spread over every level's
    queries and both batches."""
    wl = W.detr_encoder()
    out = f64(gpu_forward(wl))
    rng = np.random.default_rng(0)
    value, loc, w = wl.f32("value"), wl.f32("sampling_locations"), wl.f32("attention_weights")
    D = 32
    for _ in range(200):
        b, q, m = int(rng.integers(2)), int(rng.integers(17821)), int(rng.integers(8))
        ref = oracle.forward_one(value, wl.spatial_shapes, wl.level_start_index, loc, w, b, q, m)
        assert_close(f"out[{b},{q},{m}]", out[b, q, m * D:(m + 1) * D], ref, 1e-5, atol=1e-6)


def test_atomic_fallback_path():
    """A level with more key segments than the binned backward supports
    (one 1 x 600000 map) takes the float-atomic path; it must agree too."""
    wl = W.make("fallback", 1, [(1, 600000)], 1, 8, 1, 64, "f32", seed=21)
    t = to_device(wl)
    check_forward(wl, gpu_forward(wl, t))
    check_backward(wl, gpu_backward(wl, t))


@pytest.mark.parametrize("dtype,levels,P,Q", [
    ("f32", [(20, 30), (10, 15)], 4, 90),
    ("bf16", [(20, 30), (10, 15)], 4, 90),
    ("f32", [(30, 40), (3, 4)], 8, 3000),      # 4,000 records per key of the 3 x 4 level:
    ("bf16", [(30, 40), (3, 4)], 8, 3000),     # its segment spans many units
], ids=["f32", "bf16", "hot_level_f32", "hot_level_bf16"])
def test_backward_accumulate_adds(dtype, levels, P, Q):
    """msda_backward_accumulate adds grad_value into a float32 buffer: two
    calls on a pre-filled buffer give prefill + 2 * grad_value (also for a
    level whose segment is split over many accumulation units)."""
    from scale_deformable_attention_03_amd import _lib, ops
    wl = W.make("accumulate", 2, levels, 4, 32, P, Q, dtype, seed=8)
    t = to_device(wl)
    prob, keep = ops.problem_for(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"])
    need = _lib.workspace_bytes(prob)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    acc = torch.full(t["value"].shape, 0.25, dtype=torch.float32, device="cuda")
    gl = torch.empty_like(t["loc"])
    gw = torch.empty_like(t["w"])
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        _lib.backward_accumulate(prob, t["value"].data_ptr(), t["loc"].data_ptr(), t["w"].data_ptr(),
                                 t["g"].data_ptr(), acc.data_ptr(), gl.data_ptr(), gw.data_ptr(),
                                 ws.data_ptr(), need, stream)
    torch.cuda.synchronize()
    rgv, rgl, rgw = oracle_backward(wl)
    rtol, arms, atol = TOL[("f32", "bwd")] if dtype == "f32" else TOL[(dtype, "bwd")]
    assert_close("accumulate/grad_value", f64(acc), 0.25 + 2 * rgv, rtol, arms, atol)
    assert_close("accumulate/grad_w", f64(gw), rgw, *TOL[(dtype, "bwd")])


def test_device_shape_tensors_copied_to_host_once():
    """Device spatial_shapes / level_start_index are copied to the host once
    per tensor (the copy synchronises the device) and reused; an in-place
    change of the tensor, or a new tensor, is copied afresh."""
    from scale_deformable_attention_03_amd import ops
    t = torch.tensor([[100, 134], [50, 67]], dtype=torch.int64, device="cuda")
    a = ops._host_int64(t)
    assert ops._host_int64(t) is a
    t.mul_(1)                                        # bumps the version counter
    b = ops._host_int64(t)
    assert b is not a and np.array_equal(a, b)
    u = torch.tensor([[7, 9], [3, 4]], dtype=torch.int64, device="cuda")
    assert np.array_equal(ops._host_int64(u), [[7, 9], [3, 4]])
