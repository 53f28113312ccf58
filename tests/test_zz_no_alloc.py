"""msda_backward_noalloc (the backward whose workspace is the library's own
scratch array) against msda_backward with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller problem, in float32 and
bf16; results to the parity bars (the order of grad_value's float sums may
differ between the two entry points)."""
import numpy as np
import pytest
import torch

from scale_deformable_attention_03_amd import _lib, ops
from scale_deformable_attention_03_amd import workloads as W
from tests.parity import TOL, assert_close, f64, to_device

pytestmark = pytest.mark.gpu


def _both(wl):
    t = to_device(wl)
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_locations)
    need = _lib.workspace_bytes(prob)
    assert 0 < need <= _lib.noalloc_max_workspace(), need
    stream = torch.cuda.current_stream().cuda_stream
    ref = [torch.empty_like(t["value"]), torch.empty_like(t["loc"]), torch.empty_like(t["w"])]
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _lib.backward(prob, t["value"].data_ptr(), t["loc"].data_ptr(), t["w"].data_ptr(), t["g"].data_ptr(),
                  ref[0].data_ptr(), ref[1].data_ptr(), ref[2].data_ptr(), ws.data_ptr(), need, stream)
    # outputs pre-filled with NaN: every element must be written
    got = [torch.full_like(r, float("nan")) for r in ref]
    _lib.backward_noalloc(prob, t["value"].data_ptr(), t["loc"].data_ptr(), t["w"].data_ptr(), t["g"].data_ptr(),
                          got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), stream)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_backward_twice(dtype):
    first = W.make(f"noalloc_big_{dtype}", 2, W.DETR_LEVELS, 8, 32, 4, 300, dtype, seed=1051)
    second = W.make(f"noalloc_small_{dtype}", 1, [(20, 30), (10, 15)], 4, 32, 4, 90, dtype, seed=1052)
    for wl in (first, second):
        print(f"[gpu] no-alloc backward {wl.name}", flush=True)
        ref, got = _both(wl)
        rtol, arms, atol = TOL[(dtype, "bwd")]
        for name, r, g in zip(("grad_value", "grad_sampling_locations", "grad_attention_weights"), ref, got):
            assert_close(f"noalloc/{wl.name}/{name}", f64(g), f64(r), rtol, arms, atol)
        # the per-sample gradients do not depend on summation order
        assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])
