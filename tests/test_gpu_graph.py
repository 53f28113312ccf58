"""The C ABI under HIP graph capture: a forward + backward captured once on a
stream (torch.cuda.graph) and replayed.  The library allocates nothing,
synchronises nothing and clears its counters with kernels (no memset nodes),
so its launches record into a graph.  Every replay is checked against the
eager result, with eager work and synchronisations between replays: outputs
are overwritten with NaN before each replay, so a replay that skipped a write
would show."""
import numpy as np
import pytest
import torch

from scale_deformable_attention_03_amd import _lib, ops
from scale_deformable_attention_03_amd import workloads as W
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


CASES = [
    ("decoder_f32", lambda: W.detr_decoder("f32")),
    ("decoder_bf16_f32", lambda: W.detr_decoder("bf16", sample_dtype="f32")),
    ("small_dense_f16", lambda: W.make("graph_dense", 2, [(6, 7), (3, 4)], 4, 32, 4, 400, "f16", seed=81)),
    ("fallback_f32", lambda: W.make("graph_fallback", 1, [(1, 600000)], 1, 8, 1, 64, "f32", seed=82)),
    # more than 8192 samples per (batch, head): counted apart from the scan
    ("counted_planes_f32", lambda: W.make("graph_counted", 1, [(40, 56), (20, 28), (10, 14), (5, 7)], 2, 32, 4, 700,
                                          "f32", seed=83)),
]


@pytest.mark.parametrize("counted", [False, True], ids=["plain", "training_pair"])
@pytest.mark.parametrize("make", [c[1] for c in CASES], ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(make, counted):
    wl = make()
    print(f"[gpu] graph {wl.name}", flush=True)
    dev = torch.device("cuda")
    v, loc, w, g = (t.to(dev) for t in (wl.value, wl.sampling_locations, wl.attention_weights, wl.grad_output))
    prob, keep = ops.problem_for(v, wl.spatial_shapes, wl.level_start_index, loc)
    ws = torch.empty(max(_lib.workspace_bytes(prob), 16), dtype=torch.uint8, device=dev)
    bs, K, M, D = v.shape
    Q = loc.shape[1]
    out = torch.empty(bs, Q, M * D, dtype=v.dtype, device=dev)
    grads = (torch.empty_like(v), torch.empty_like(loc), torch.empty_like(w))

    def step():
        if counted:      # msda_forward_train + msda_backward_counted (zero kernel, no memset node)
            ops.forward_train(v, wl.spatial_shapes, wl.level_start_index, loc, w, out=out, workspace=ws)
        else:
            ops.forward(v, wl.spatial_shapes, wl.level_start_index, loc, w, out=out)
        ops.backward(v, wl.spatial_shapes, wl.level_start_index, loc, w, g, grads=grads, workspace=ws,
                     counted=counted)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, *grads)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                     # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    names = ("output", "grad_value", "grad_sampling_locations", "grad_attention_weights")
    for rep in range(3):
        for t in (out, *grads):
            t.fill_(float("nan"))                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, (out, *grads), ref):
            a64, b64 = a.double().cpu().numpy(), b.double().cpu().numpy()
            assert not np.isnan(a64).any(), f"replay {rep}: {name} not written"
            if name == "grad_value":
                # float32 atomics on segments split over several units may
                # reorder additions: compare at the backward bar
                kind = (wl.dtype, "bwd")
                assert_close(f"replay {rep} {name}", a64, b64, *TOL[kind])
            else:
                np.testing.assert_array_equal(a64, b64, err_msg=f"replay {rep}: {name}")
