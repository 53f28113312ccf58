"""GPU parity of the backward's record merging.

The records of a query's samples on one level that share an image row and an
x-pair become one record with summed weights, at four points per level on
planes counted apart from the scan.  These tests use problems where most
records merge and check the plain backward and the training pair against the
CPU oracle:
- tiny levels, where a query's four points often fall in one cell or in
  vertically adjacent cells;
- all four points of a level at one location (every row merges);
- points one, two and three pixels below the first (rows shared between
  neighbouring cells);
and the accumulating and no-alloc entry points on merged records.
"""
import pytest
import torch

from scale_deformable_attention_03_amd import workloads as W
from tests.parity import check_backward, check_forward, to_device

pytestmark = pytest.mark.gpu

LEVELS = [(8, 10), (4, 5), (2, 3), (1, 2)]


def clustered(mode, dtype, sample_dtype, seed):
    """700 queries (11,200 samples per plane: counted apart from the scan,
    so the records merge), 2 heads of 32 channels, L4P4."""
    wl = W.make(f"merge_{mode}", 1, LEVELS, 2, 32, 4, 700, dtype, seed=seed, loc_args=(-0.1, 1.1),
                sample_dtype=sample_dtype)
    loc = wl.sampling_locations.to(torch.float32)      # [bs, Q, M, L, P, 2]
    if mode == "same":
        loc = loc[..., :1, :].expand_as(loc).clone()
    elif mode == "column":
        H = torch.tensor([float(h) for h, _ in LEVELS]).view(1, 1, 1, len(LEVELS))
        for p in range(1, 4):
            loc[..., p, 0] = loc[..., 0, 0]
            loc[..., p, 1] = loc[..., 0, 1] + p / H
    wl.sampling_locations = loc.to(wl.sampling_locations.dtype)
    return wl


CASES = [(mode, dt, sdt) for mode in ("uniform", "same", "column")
         for dt, sdt in (("f32", None), ("bf16", None), ("f16", "f32"))]


@pytest.mark.parametrize("mode,dt,sdt", CASES, ids=[f"{m}_{d}{'_' + s if s else ''}" for m, d, s in CASES])
def test_merged_records_match_oracle(mode, dt, sdt):
    from scale_deformable_attention_03_amd import ops
    print(f"[gpu] merged records {mode} {dt} {sdt}", flush=True)
    wl = clustered(mode, dt, sdt, seed=1301)
    # plain backward: the count kernel and the gradient kernel merge
    check_backward(wl)
    # training pair: the counting forward merges
    t = to_device(wl)
    out, ws = ops.forward_train(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"], t["w"])
    grads = ops.backward(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"], t["w"], t["g"],
                         workspace=ws, counted=True)
    torch.cuda.synchronize()
    check_forward(wl, out)
    check_backward(wl, grads)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_merged_records_accumulate_and_noalloc(dt):
    """Merged records through msda_backward_accumulate (every unit adds its
    rows with float atomics: two calls on a pre-filled buffer give prefill
    + 2 * grad_value) and through msda_backward_noalloc (the library's own
    workspace; outputs pre-filled with NaN, so every element must be
    written)."""
    from scale_deformable_attention_03_amd import _lib, ops
    from tests.parity import TOL, assert_close, f64, oracle_backward
    print(f"[gpu] merged records, accumulating and no-alloc entry points, {dt}", flush=True)
    wl = clustered("same", dt, None, seed=1302)
    t = to_device(wl)
    prob, keep = ops.problem_for(t["value"], wl.spatial_shapes, wl.level_start_index, t["loc"])
    need = _lib.workspace_bytes(prob)
    assert 0 < need <= _lib.noalloc_max_workspace()
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    acc = torch.full(t["value"].shape, 0.25, dtype=torch.float32, device="cuda")
    gl, gw = torch.empty_like(t["loc"]), torch.empty_like(t["w"])
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        _lib.backward_accumulate(prob, t["value"].data_ptr(), t["loc"].data_ptr(), t["w"].data_ptr(),
                                 t["g"].data_ptr(), acc.data_ptr(), gl.data_ptr(), gw.data_ptr(),
                                 ws.data_ptr(), need, stream)
    got = [torch.full_like(x, float("nan")) for x in (t["value"], t["loc"], t["w"])]
    _lib.backward_noalloc(prob, t["value"].data_ptr(), t["loc"].data_ptr(), t["w"].data_ptr(), t["g"].data_ptr(),
                          got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), stream)
    torch.cuda.synchronize()
    rgv, rgl, rgw = oracle_backward(wl)
    rtol, arms, atol = TOL[("f32", "bwd")] if dt == "f32" else TOL[(dt, "bwd")]
    assert_close("merge/accumulate/grad_value", f64(acc), 0.25 + 2 * rgv, rtol, arms, atol)
    rtol, arms, atol = TOL[(dt, "bwd")]
    for name, g, r in zip(("grad_value", "grad_sampling_locations", "grad_attention_weights"), got, (rgv, rgl, rgw)):
        assert_close(f"merge/noalloc/{name}", f64(g), r, rtol, arms, atol)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_one_query_last_tile(dt):
    """2049 queries: the gradient kernel's last query tile (32 queries per
    workgroup at float32, 64 at bf16) holds a single query, for which the
    record epilogue's multiply-high division by the tile's query count is
    replaced by the index itself."""
    print(f"[gpu] one-query last tile, {dt}", flush=True)
    wl = W.make("one_query_tile", 1, LEVELS, 2, 32, 4, 2049, dt, seed=1303, loc_args=(-0.1, 1.1))
    check_backward(wl)
