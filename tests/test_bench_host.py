"""Host logic of bench.py, on the CPU (no GPU, no HIP call): the one-GPU
rule, the minimal-byte model behind the bench line's effective GB/s and
roofline, the comment-blind digest that keys the committed counter runs, and
the lookup of those runs."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from scale_deformable_attention_03_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 exits with status 2 and says why, before any GPU work
    and without a JSON line."""
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True,
                           text=True, timeout=300, env={**os.environ, **env})
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def brute_force_rows(wl) -> int:
    """Distinct (batch, key, head) rows that an in-map bilinear corner
    reaches, one sample at a time (pixel coordinates x = loc_x * W - 0.5 in
    float32, as the pages map them)."""
    loc = wl.sampling_locations.float().numpy()
    bs, Q, M, L, P, _ = loc.shape
    rows = set()
    for b in range(bs):
        for q in range(Q):
            for m in range(M):
                for lvl, (H, Wd) in enumerate(wl.spatial_shapes):
                    s0 = int(wl.level_start_index[lvl])
                    for p in range(P):
                        x = np.float32(np.float32(loc[b, q, m, lvl, p, 0]) * np.float32(Wd)) - np.float32(0.5)
                        y = np.float32(np.float32(loc[b, q, m, lvl, p, 1]) * np.float32(H)) - np.float32(0.5)
                        x0, y0 = int(np.floor(x)), int(np.floor(y))
                        for yc in (y0, y0 + 1):
                            for xc in (x0, x0 + 1):
                                if 0 <= xc < Wd and 0 <= yc < H:
                                    rows.add((b, s0 + yc * Wd + xc, m))
    return len(rows)


def test_touched_rows_against_brute_force():
    """The compulsory value rows of a sparse problem (16 queries on a 100x100
    map: most rows untouched) and of a two-level one with off-map samples."""
    tiny = W.tiny_single_level()
    assert bench.touched_rows(tiny) == brute_force_rows(tiny) < tiny.value.shape[0] * 10000 * tiny.value.shape[2]
    two = W.make("rows_two_levels", 2, [(9, 13), (4, 7)], 3, 8, 3, 40, "f32", seed=5, loc_args=(-0.2, 1.2))
    assert bench.touched_rows(two) == brute_force_rows(two)


def test_encoder_minimal_bytes():
    """The encoder's minimal bytes: reference points at every pixel centre of
    every level reach every value row, so the value side is read whole; the
    forward reads value, locations and weights and writes the output, the
    backward also reads grad_output and writes the three gradients."""
    wl = W.detr_encoder()
    bs, K, M, D = 2, 17821, 8, 32
    rows = bench.touched_rows(wl)
    assert rows == bs * K * M
    samples = bs * K * M * 4 * 4                  # num_queries = num_keys, 4 levels x 4 points
    loc, w, tensor = samples * 2 * 4, samples * 4, bs * K * M * D * 4
    ab = bench.algorithmic_bytes(wl, rows)
    assert ab["fwd"] == tensor + loc + w + tensor
    assert ab["bwd"] == (tensor + loc + w + tensor) + (tensor + loc + w)
    assert ab["grad"] == tensor + loc + w + tensor + loc + w
    assert ab["accum"] == loc + w + tensor + tensor
    assert ab["total"] == 346_725_376


def test_digest_ignores_comments_and_layout():
    a = "int f(int x) { return x + 1; }  // adds one\n/* block\n comment */ int g;"
    b = "int f(int x) {\n    return x + 1;     // another remark\n}\nint g;"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("x + 1", "x + 2"))
    d = bench.kernel_digest()
    assert len(d) == 16 and int(d, 16) >= 0


def test_traffic_lookup_is_keyed_by_digest_and_workload(tmp_path, monkeypatch):
    rec = {"kernel_digest": "00ff", "workloads": {"wl": {"kern": {"hbm_bytes_per_launch": 1234}}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic("00ff", "kern", "wl") == 1234
    assert bench.load_traffic("00fe", "kern", "wl") is None      # other kernel sources
    assert bench.load_traffic("00ff", "kern", "other") is None   # not profiled for this workload
    assert bench.load_traffic("00ff", "other", "wl") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic("00ff", "kern", "wl") is None


def test_percentiles():
    p = bench.percentiles(np.arange(101, dtype=float))
    assert p == {"p10": 10.0, "p50": 50.0, "p90": 90.0}


def test_profile_commands_run_committed_files_only():
    """Every profiling command runs bench.py from the repository root (REPO)
    under rocprofv3, with the program itself after `--`."""
    for name in bench.PROFILE_COMMANDS:
        cmd = bench.profile_command(name, "detr_encoder")
        assert cmd.startswith("rocprofv3 ")
        assert " -- python3 REPO/bench.py" in cmd
        assert "WL" not in cmd
