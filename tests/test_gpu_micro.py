"""The measurement kernels of libmsda_micro.so compute what they claim, so
that the ceilings bench.py reports are the costs of the stated access
patterns: the gather with FMAs sums 0.25 * (every corner row of a group),
the scatter adds 0.25 to every element of every corner row (each corner
once per appearance), on a small table built from real sampling locations.
Checked against numpy on the host."""
import numpy as np
import pytest
import torch

from scale_deformable_attention_03_amd import _micro
from scale_deformable_attention_03_amd import workloads as W

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


@pytest.mark.parametrize("D,samples_pts", [(32, 4), (16, 3), (64, 2)])
def test_gather_and_scatter(D, samples_pts):
    wl = W.make("micro", 2, [(9, 11), (5, 6)], 3, D, samples_pts, 37, "f32", seed=71, loc_args=(-0.1, 1.1))
    bs, K, M, _ = wl.value.shape
    loc = wl.sampling_locations.numpy()
    Q, L, P = loc.shape[1], loc.shape[3], loc.shape[4]
    lanes = D // 4
    print(f"[gpu] micro D {D} L {L} P {P}", flush=True)
    tab = _micro.corner_table(loc, wl.spatial_shapes, wl.level_start_index, K, lanes)
    ngroups, samples = bs * M * Q, L * P
    rows = wl.value.numpy().reshape(-1, 4)                       # 16-byte vectors
    stream = torch.cuda.current_stream().cuda_stream

    dev_rows = torch.from_numpy(rows.copy()).cuda()
    dev_tab = torch.from_numpy(tab.view(np.int32)).cuda()
    out = torch.zeros(ngroups * lanes * 4, dtype=torch.float32, device="cuda")
    _micro.gather(dev_rows.data_ptr(), dev_tab.data_ptr(), out.data_ptr(), ngroups, samples, lanes, True, stream)
    torch.cuda.synchronize()
    # group g, lane li: sum over its corners of 0.25 * rows[corner + li]
    idx = tab.astype(np.int64)[:, :, None] + np.arange(lanes)[None, None, :]      # [groups, 4*samples, lanes]
    ref = 0.25 * rows[idx].astype(np.float64).sum(axis=1)                        # [groups, lanes, 4]
    np.testing.assert_allclose(out.cpu().numpy().reshape(ngroups, lanes, 4), ref, rtol=1e-5, atol=1e-5)

    for contiguous in (True, False):
        dst = torch.zeros(rows.shape[0] * 4, dtype=torch.float32, device="cuda")
        _micro.scatter(dst.data_ptr(), dev_tab.data_ptr(), ngroups, samples, lanes, contiguous, stream)
        torch.cuda.synchronize()
        expect = np.zeros(rows.shape[0] * 4)
        elems = (tab.astype(np.int64).reshape(-1)[:, None] * 4 + np.arange(4 * lanes)[None, :]).reshape(-1)
        np.add.at(expect, elems, 0.25)
        np.testing.assert_array_equal(dst.cpu().numpy(), expect)
