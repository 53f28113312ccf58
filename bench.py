#!/usr/bin/env python3
"""Throughput of the MSDeformAttn core, forward + backward, on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input,
as a training step runs it: msda_forward_train (the forward, which also
counts the backward's records per key segment) followed by
msda_backward_counted (scan, gradient kernel, accumulation and, for 16-bit
dtypes, the float32 -> dtype conversion of split segments), both through the
C ABI on torch's current stream.  Inputs are resident in HBM before timing
starts, and the timed steps are enqueued with nothing between them (the
forward / backward split comes from a second, evented pass).
To keep the 256 MB Infinity Cache from serving a whole step's working set,
steps rotate over several identical copies of every buffer.

Default workload: Deformable-DETR encoder self-attention, fp32, bs 2, levels
(100,134) (50,67) (25,34) (13,17), 17821 queries = keys, 8 heads x 32 dims,
4 points, seeded synthetic inputs (scale_deformable_attention_03_amd.workloads).

Prints one JSON line: queries/s (bs * num_queries per step / seconds per
step), plus the roofline of the dominant kernel (algorithmic bytes per launch
over its HIP-event-timed average duration against 8 TB/s) and the CPU oracle
timed on the host cores as a reported baseline.  A second object,
"fused_prologue", times the fused form on the same shapes (reference points,
offsets and logits in; msda_forward_fused + msda_backward_fused) beside the
module path it replaces (PyTorch ops for the locations and the softmax and
their backward around the core).  "graph_replay_ms_per_step" is the same step
captured as HIP graphs and replayed (no host launch cost).  A third, "mixed_precision", times the
encoder step with bf16 value-side tensors and float32 per-sample tensors; a
fourth, "module_step", the whole MSDeformAttn module (Linears through
PyTorch's hipBLASLt GEMMs around the fused core) forward and backward.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E peak
MALL_BYTES = 256 << 20       # Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "scale_deformable_attention_03_amd", "csrc", f)
                  for f in ("msda_api.hip", "msda_types.hpp", "msda_plan.hpp", "msda_forward.hpp",
                            "msda_backward.hpp", "msda_device.hpp",
                            "msda_launch.hpp", "msda_launch_impl.hpp", "msda_kernels_f32.hip",
                            "msda_kernels_f16.hip", "msda_kernels_bf16.hip", "msda_kernels_f16_f32.hip",
                            "msda_kernels_bf16_f32.hip")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace collapsed, so that
    edits to comments leave the digest (and the counter runs keyed by it)
    valid.  String literals in these sources hold no comment markers."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def percentiles(us) -> dict:
    """p10 / p50 / p90 of per-step event times (microseconds)."""
    return {f"p{p}": round(float(np.percentile(us, p)), 2) for p in (10, 50, 90)}


def kernel_digest() -> str:
    """Digest of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(_code_only(open(f).read()).encode())
    return h.hexdigest()[:16]


def touched_rows(wl) -> int:
    """Number of (batch, key, head) value rows that at least one in-map
    bilinear corner reads (the compulsory part of the value traffic)."""
    import torch
    loc = wl.sampling_locations.to(torch.float32).numpy()
    bs, Q, M, L, P, _ = loc.shape
    K = wl.value.shape[1]
    seen = np.zeros((bs, K, M), dtype=bool)
    bi = np.broadcast_to(np.arange(bs)[:, None, None, None], (bs, Q, M, P))
    mi = np.broadcast_to(np.arange(M)[None, None, :, None], (bs, Q, M, P))
    for lvl, (H, W) in enumerate(wl.spatial_shapes):
        s0 = int(wl.level_start_index[lvl])
        x = (loc[:, :, :, lvl, :, 0] * np.float32(W)).astype(np.float32) - np.float32(0.5)
        y = (loc[:, :, :, lvl, :, 1] * np.float32(H)).astype(np.float32) - np.float32(0.5)
        ok = (x > -1) & (x < W) & (y > -1) & (y < H)
        x0 = np.floor(np.where(ok, x, 0)).astype(np.int64)
        y0 = np.floor(np.where(ok, y, 0)).astype(np.int64)
        for dy in (0, 1):
            for dx in (0, 1):
                xc, yc = x0 + dx, y0 + dy
                v = ok & (xc >= 0) & (xc < W) & (yc >= 0) & (yc < H)
                seen[bi[v], (s0 + yc * W + xc)[v], mi[v]] = True
    return int(seen.sum())


def algorithmic_bytes(wl, rows: int) -> dict:
    e = wl.value.element_size()                      # value side
    es = wl.sampling_locations.element_size()        # per-sample tensors (float32 in mixed precision)
    bs, K, M, D = wl.value.shape
    Q = wl.sampling_locations.shape[1]
    L, P = wl.sampling_locations.shape[3:5]
    value_rows = rows * D * e
    loc = bs * Q * M * L * P * 2 * es
    w = bs * Q * M * L * P * es
    out = bs * Q * M * D * e
    full_value = bs * K * M * D * e
    fwd = value_rows + loc + w + out
    bwd = value_rows + loc + w + out + full_value + loc + w   # + grad_out; writes gv, gloc, gw
    # the backward's two big kernels: the gather (value rows, loc, w,
    # grad_out in; grad_loc, grad_w out) and the accumulation (loc, w,
    # grad_out in; grad_value out)
    grad = value_rows + loc + w + out + loc + w
    accum = loc + w + out + full_value
    return dict(fwd=fwd, bwd=bwd, total=fwd + bwd, grad=grad, accum=accum)


def load_traffic(digest: str, kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they were taken on other kernel sources or not for this workload."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_digest") != digest:
        return None
    ent = rec.get("workloads", {}).get(workload, {}).get(kernel)
    return ent.get("hbm_bytes_per_launch") if isinstance(ent, dict) else None


# The profiling commands whose output --ingest-profiles reads (REPO is the
# repository root, DIR the directory later handed to --ingest-profiles; run
# from /tmp with TMPDIR=/tmp).
_BENCH_ARGS = "--workload WL --no-cpu-baseline --no-fused --no-mixed --no-module --no-ceilings --no-other-workloads"
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o run -- "
             f"python3 REPO/bench.py --steps 30 --warmup 5 {_BENCH_ARGS}",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o run -- "
             f"python3 REPO/bench.py --steps 4 --warmup 1 {_BENCH_ARGS}",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o run -- "
             f"python3 REPO/bench.py --steps 4 --warmup 1 {_BENCH_ARGS}",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copy_fetch -o run -- "
                  "python3 REPO/bench.py --calibrate-copy",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/copy_write -o run -- "
                  "python3 REPO/bench.py --calibrate-copy",
    "cache": "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum TA_TA_BUSY_sum TD_TD_BUSY_sum TCP_TOTAL_CACHE_ACCESSES_sum "
             "TCP_TCC_READ_REQ_sum GRBM_GUI_ACTIVE --output-format csv -d DIR/cache -o run -- "
             f"python3 REPO/bench.py --steps 4 --warmup 1 {_BENCH_ARGS}",
    "micro_trace": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/micro_trace -o run -- "
                   "python3 REPO/bench.py --workload WL --steps 4 --warmup 1 --no-cpu-baseline --no-fused --no-mixed "
                   "--no-module --no-other-workloads",
    "sq": "rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE "
          "SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d DIR/sq -o run -- "
          f"python3 REPO/bench.py --steps 4 --warmup 1 {_BENCH_ARGS}",
}


def profile_command(name: str, workload: str) -> str:
    """The rocprofv3 command PROFILE_COMMANDS[name] for one workload (REPO,
    DIR left as placeholders)."""
    return PROFILE_COMMANDS[name].replace("WL", workload)


# MI355X: 256 compute units in 8 XCDs, 4 SIMDs per CU (GRBM_GUI_ACTIVE is
# summed over the XCDs; TA/TD/TCP counters over the CUs).
N_XCD, N_CU, N_SIMD = 8, 256, 1024
COPY_BYTES = 512 << 20           # one --calibrate-copy dispatch reads and writes this much


def _short(name: str) -> str:
    """Kernel name without template arguments and parameters."""
    base = name.split("(")[0].replace("void ", "").strip()
    return base.split("<")[0].split("::")[-1]


def _counter_csv(d: str, counter: str) -> dict:
    """{kernel: [values per dispatch]} of one rocprofv3 --pmc CSV run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    out = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _counters_by_kernel(d: str) -> dict:
    """{short kernel name: {counter: mean per dispatch}} of one --pmc run
    (msda kernels only)."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if "msda" not in r["Kernel_Name"]:
                continue
            acc.setdefault(_short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return {k: {c: float(np.mean(v)) for c, v in cs.items()} for k, cs in acc.items()}


def counters_summary(d: str, workload: str, digest: str) -> list:
    """Markdown lines: cache hit rates, texture-path, VALU and LDS activity
    per msda kernel, from the "cache" and "sq" --pmc runs under d.  Busy
    shares are relative to the kernel's own GPU cycles per XCD
    (GRBM_GUI_ACTIVE / 8, taken in the same run)."""
    cache = _counters_by_kernel(os.path.join(d, "cache"))
    sq = _counters_by_kernel(os.path.join(d, "sq"))
    if not cache or not sq:
        return []

    def pct(num, den):
        """Share num / den as a percentage; a dash when a counter is missing."""
        if num is None or den is None or den <= 0:
            return "—"
        return f"{100.0 * num / den:.0f}%"

    md = [f"# Cache, texture-path, VALU and LDS counters per launch, msda kernels, workload {workload}", "",
          f"Kernel sources digest {digest}. Means over the dispatches of two rocprofv3 --pmc runs;",
          f"cycles = GRBM_GUI_ACTIVE / {N_XCD} (GPU cycles of the launch per XCD, same run).",
          "- L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS); L1 hit = 1 - TCP_TCC_READ_REQ / TCP_TOTAL_CACHE_ACCESSES;",
          f"- TA busy, TD busy = TA_TA_BUSY_sum, TD_TD_BUSY_sum / {N_CU} / cycles;",
          f"- VALU issue = SQ_INSTS_VALU * 4 / {N_SIMD} / cycles (a wave64 VALU instruction holds its",
          "  16-lane SIMD for 4 cycles);",
          f"- LDS active = SQ_LDS_IDX_ACTIVE / {N_CU} / cycles; bank and address conflicts as shares of",
          "  the LDS-active cycles (SQ_LDS_BANK_CONFLICT, SQ_LDS_ADDR_CONFLICT: same-address atomics);",
          "- waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of wave lifetime spent waiting).", "",
          "Commands (REPO = repository root, DIR = output directory; run from /tmp, TMPDIR=/tmp):", "",
          f"    {profile_command('cache', workload)}", f"    {profile_command('sq', workload)}", "",
          "| kernel | waves | cycles | L2 hit | L1 hit | TA busy | TD busy | VALU issue | LDS active | "
          "LDS bank conflict | LDS address conflict | waiting |",
          "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(set(cache) & set(sq)):
        c, q = cache[k], sq[k]
        cyc_c = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        cyc_q = q.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        if cyc_c <= 0 or cyc_q <= 0:
            continue
        hit, miss = c.get("TCC_HIT_sum"), c.get("TCC_MISS_sum")
        l1_acc, l1_miss = c.get("TCP_TOTAL_CACHE_ACCESSES_sum"), c.get("TCP_TCC_READ_REQ_sum")
        l1_hits = None if l1_acc is None or l1_miss is None else l1_acc - l1_miss
        valu = q.get("SQ_INSTS_VALU")
        lds = q.get("SQ_LDS_IDX_ACTIVE")
        waves = q.get("SQ_WAVES")
        md.append(
            f"| {k} | {'—' if waves is None else f'{waves:.0f}'} | {cyc_q:.0f} | "
            f"{pct(hit, None if hit is None or miss is None else hit + miss)} | {pct(l1_hits, l1_acc)} | "
            f"{pct(c.get('TA_TA_BUSY_sum'), N_CU * cyc_c)} | {pct(c.get('TD_TD_BUSY_sum'), N_CU * cyc_c)} | "
            f"{pct(None if valu is None else valu * 4, N_SIMD * cyc_q)} | {pct(lds, N_CU * cyc_q)} | "
            f"{pct(q.get('SQ_LDS_BANK_CONFLICT'), lds)} | {pct(q.get('SQ_LDS_ADDR_CONFLICT'), lds)} | "
            f"{pct(q.get('SQ_WAIT_ANY'), q.get('SQ_WAVE_CYCLES'))} |")
    return md


def ingest_profiles(d: str, workload: str) -> None:
    """Turn the raw rocprofv3 output of PROFILE_COMMANDS (under d) into the
    short text summaries and profiles/traffic.json (HBM bytes per launch of
    each msda kernel, for the roofline's traffic field).

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for a plain copy of COPY_BYTES (the runtime's copy kernel):
    scale = COPY_BYTES / (counter KiB * 1024)."""
    import csv
    import glob
    digest = kernel_digest()
    cf = _counter_csv(os.path.join(d, "copy_fetch"), "FETCH_SIZE")
    cw = _counter_csv(os.path.join(d, "copy_write"), "WRITE_SIZE")
    copy_k = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()]
    if not copy_k:
        raise RuntimeError("no copy kernel in the calibration runs")
    kc = max(copy_k, key=lambda k: np.mean(cf[k]))
    fetch_scale = COPY_BYTES / (np.mean(cf[kc]) * 1024.0)
    write_scale = COPY_BYTES / (np.mean(cw[kc]) * 1024.0)
    fetch = _counter_csv(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _counter_csv(os.path.join(d, "write"), "WRITE_SIZE")
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {}
    if rec.get("kernel_digest") != digest or "workloads" not in rec:
        rec = {"kernel_digest": digest, "workloads": {}}
    rec["calibration"] = {"copy_kernel": _short(kc), "copy_bytes": COPY_BYTES,
                          "fetch_kib": round(float(np.mean(cf[kc])), 1), "fetch_scale": round(fetch_scale, 4),
                          "write_kib": round(float(np.mean(cw[kc])), 1), "write_scale": round(write_scale, 4)}
    rec["commands"] = {k: PROFILE_COMMANDS[k] for k in ("fetch", "write", "copy_fetch", "copy_write")}
    rec["commands"]["note"] = "WL: the workload's name (--workload)"
    rows = []
    ents = {}
    for k in sorted(set(fetch) | set(write)):
        if "msda" not in k:
            continue
        f_kib = float(np.mean(fetch.get(k, [0.0])))
        w_kib = float(np.mean(write.get(k, [0.0])))
        hbm = f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale
        ent = {"dispatches": len(fetch.get(k, [])), "fetch_kib": round(f_kib, 1),
               "write_kib": round(w_kib, 1), "hbm_bytes_per_launch": int(round(hbm))}
        ents.setdefault(_short(k), ent)
        rows.append((_short(k), k, ent))
    rec["workloads"][workload] = ents
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    md = [f"# HBM traffic per launch, msda kernels, workload {workload}", "",
          f"Kernel sources digest {digest}. FETCH_SIZE / WRITE_SIZE are rocprofv3 per-dispatch",
          "values in KiB, averaged over the dispatches of the run; bytes = KiB * 1024 * scale, with the",
          f"scale taken from a plain {COPY_BYTES >> 20} MiB device copy ({_short(kc)}):",
          f"FETCH_SIZE read {rec['calibration']['fetch_kib']} KiB -> scale {fetch_scale:.4f};",
          f"WRITE_SIZE read {rec['calibration']['write_kib']} KiB -> scale {write_scale:.4f}.",
          "The counters see traffic between L2 and the memory side (Infinity Cache included).", "",
          "Commands (REPO = repository root, DIR = output directory; run from /tmp, TMPDIR=/tmp):", ""]
    md += [f"    {profile_command(k, workload)}" for k in ("fetch", "write", "copy_fetch", "copy_write")]
    md += ["", "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes per launch (scaled) |",
           "|---|---|---|---|---|"]
    for short, _, e in rows:
        md.append(f"| {short} | {e['dispatches']} | {e['fetch_kib']} | {e['write_kib']} | "
                  f"{e['hbm_bytes_per_launch'] / 1e6:.1f} MB |")
    with open(os.path.join(ROOT, "profiles", f"msda_kernels_{workload}_hbm_traffic.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    stats = glob.glob(os.path.join(d, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        md = [f"# Kernel trace statistics, workload {workload}", "",
              f"Kernel sources digest {digest}. rocprofv3 --stats over a short bench run",
              "(30 timed + 5 warm-up steps, plus the per-stage profiling pass).", "",
              "Command (REPO = repository root, DIR = output directory; run from /tmp, TMPDIR=/tmp):", "",
              f"    {profile_command('trace', workload)}", "",
              "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
        for r in csv.DictReader(open(stats[0])):
            ns = {k: float(r.get(k) or "nan") for k in ("AverageNs", "MinNs", "MaxNs", "Percentage")}
            md.append(f"| {r.get('Name', '?')[:110]} | {r.get('Calls', '?')} | {ns['AverageNs'] / 1e3:.2f} | "
                      f"{ns['MinNs'] / 1e3:.2f} | {ns['MaxNs'] / 1e3:.2f} | {ns['Percentage']:.1f}% |")
        with open(os.path.join(ROOT, "profiles", f"msda_kernels_{workload}_kernel_trace.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
    stats = glob.glob(os.path.join(d, "micro_trace", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        md = [f"# Measurement kernels (gather only, atomic scatter), workload {workload}", "",
              "rocprofv3 --stats of a short bench run with its ceilings leg: the gather and scatter kernels of",
              "libmsda_micro.so on the workload's own corner rows (gather: loads only, then with FMAs;",
              "scatter: lanes on adjacent addresses, then 16 bytes apart), beside the core's kernels.", "",
              "Command (REPO = repository root, DIR = output directory; run from /tmp, TMPDIR=/tmp):", "",
              f"    {profile_command('micro_trace', workload)}", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        for r in csv.DictReader(open(stats[0])):
            name = r.get("Name", "?")
            if not any(t in name for t in ("gather_kernel", "scatter_kernel", "msda_forward_kernel",
                                           "msda_backward_kernel", "msda_accumulate_kernel")):
                continue
            ns = {k: float(r.get(k) or "nan") for k in ("AverageNs", "MinNs", "MaxNs")}
            md.append(f"| {name[:110]} | {r.get('Calls', '?')} | {ns['AverageNs'] / 1e3:.2f} | "
                      f"{ns['MinNs'] / 1e3:.2f} | {ns['MaxNs'] / 1e3:.2f} |")
        with open(os.path.join(ROOT, "profiles", f"micro_gather_scatter_{workload}_kernel_trace.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
    if os.path.isdir(os.path.join(d, "cache")) and os.path.isdir(os.path.join(d, "sq")):
        md = counters_summary(d, workload, digest)
        if md:
            with open(os.path.join(ROOT, "profiles", f"msda_kernels_{workload}_counters.md"), "w") as fh:
                fh.write("\n".join(md) + "\n")
    print(json.dumps(rec, indent=1))


def ceilings_leg(wl, dev, fwd_us: float, step_gbps: float) -> dict:
    """The secondary ceilings of the core's access patterns, measured on the
    same workload with the kernels of libmsda_micro.so (include/msda_micro.h):

    - gather only: the forward's corner-row loads (same groups, same rows,
      16-byte lane loads, four samples in flight), loads only and with the
      fp32 FMAs;
    - atomic scatter: one float32 atomic add per element of every corner
      row, lanes on adjacent addresses and lanes 16 bytes apart (a
      per-sample backward scattering grad_value directly);
    - a streaming device copy of 512 MiB (read + write bytes / time)."""
    import torch
    from scale_deformable_attention_03_amd import _micro

    bs, K, M, D = wl.value.shape
    Q, L, P = wl.sampling_locations.shape[1], wl.sampling_locations.shape[3], wl.sampling_locations.shape[4]
    e = wl.value.element_size()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ngroups, samples = bs * M * Q, L * P

    def timed(fn, reps, warm=1):
        for _ in range(warm):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    res = {}
    loc = wl.sampling_locations.float().numpy()
    lanes = D * e // 16
    if lanes in (2, 4, 8, 16):
        tab = torch.from_numpy(_micro.corner_table(loc, wl.spatial_shapes, wl.level_start_index, K,
                                                   lanes).view(np.int32)).to(dev)
        rows = wl.value.to(dev)
        out = torch.empty(ngroups * lanes * 4, dtype=torch.float32, device=dev)
        row_bytes = ngroups * samples * 4 * lanes * 16
        g_only = timed(lambda: _micro.gather(rows.data_ptr(), tab.data_ptr(), out.data_ptr(), ngroups, samples,
                                             lanes, False, sp), 5, 2)
        res.update({"corner_row_bytes": row_bytes, "gather_only_us": round(g_only, 2),
                    "gather_request_tbps": round(row_bytes / (g_only * 1e-6) / 1e12, 2),
                    "fwd_over_gather_only": round(fwd_us / g_only, 3)})
        if e == 4:
            g_fma = timed(lambda: _micro.gather(rows.data_ptr(), tab.data_ptr(), out.data_ptr(), ngroups, samples,
                                                lanes, True, sp), 5, 2)
            res["gather_fma_us"] = round(g_fma, 2)
        del rows, out, tab
    lanes32 = D // 4                             # float32 rows (grad_value or its workspace)
    if lanes32 in (2, 4, 8, 16):
        tab = torch.from_numpy(_micro.corner_table(loc, wl.spatial_shapes, wl.level_start_index, K,
                                                   lanes32).view(np.int32)).to(dev)
        dst = torch.zeros(bs * K * M * D, dtype=torch.float32, device=dev)
        n_atomic = ngroups * samples * 4 * D
        sc = {}
        for name, contig in (("lane_contiguous", True), ("lane_stride_16B", False)):
            sc[name] = timed(lambda: _micro.scatter(dst.data_ptr(), tab.data_ptr(), ngroups, samples, lanes32,
                                                    contig, sp), 3, 1)
        res["scatter_atomic_us"] = {k: round(v, 1) for k, v in sc.items()}
        res["scatter_atomics"] = n_atomic
        res["atomic_g_per_s"] = {k: round(n_atomic / (v * 1e-6) / 1e9, 1) for k, v in sc.items()}
        del dst, tab
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    c_us = timed(lambda: dst.copy_(src), 5, 2)
    res["copy_gbps"] = round(2 * src.numel() * 4 / (c_us * 1e-6) / 1e9, 1)
    res["step_pct_of_copy_ceiling"] = round(100 * step_gbps / res["copy_gbps"], 2)
    return res


def device_info(props) -> dict:
    """What the run's device reports: name, architecture, compute units, L2
    and memory sizes, peak engine and memory clocks (kHz, from the HIP
    runtime torch loaded), HIP version."""
    import torch
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
            "l2_bytes": getattr(props, "L2_cache_size", None), "memory_bytes": props.total_memory,
            "hip": torch.version.hip}
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        dev = torch.cuda.current_device()
        for key, attr in (("clock_khz", 5), ("memory_clock_khz", 60)):    # hipDeviceAttribute values
            v = ctypes.c_int()
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) == 0:
                info[key] = v.value
    except OSError:
        pass
    return info


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _query_slice(wl, nq: int):
    """The first nq queries of every batch of the workload (same value map)."""
    class Slice:
        pass
    sl = Slice()
    sl.value = wl.value
    sl.spatial_shapes, sl.level_start_index = wl.spatial_shapes, wl.level_start_index
    sl.sampling_locations = wl.sampling_locations[:, :nq].contiguous()
    sl.attention_weights = wl.attention_weights[:, :nq].contiguous()
    sl.grad_output = wl.grad_output[:, :nq].contiguous()
    sl.f32 = lambda name: wl.__class__.f32(sl, name)
    return sl


def cpu_baseline(wl, seconds: float) -> dict:
    """The oracle (float64 scalar C) as it stands, on the host cores: forward
    and backward timed separately, with all threads on the whole workload and
    with one thread on a slice of its queries.  About `seconds` of CPU time."""
    import oracle
    cores = oracle.threads(0)
    bs, Q = wl.sampling_locations.shape[:2]

    def rate(w, fn, nthreads, budget):
        args = (w.f32("value"), w.spatial_shapes, w.level_start_index,
                w.f32("sampling_locations"), w.f32("attention_weights"))
        g = w.f32("grad_output")
        call = (lambda: oracle.forward(*args, nthreads)) if fn == "fwd" else \
               (lambda: oracle.backward(*args, g, nthreads))
        reps, t0 = 0, time.perf_counter()
        while True:
            call()
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
        nq = w.sampling_locations.shape[0] * w.sampling_locations.shape[1]
        return reps * nq / dt, reps, dt

    q = seconds / 4
    fa, fr, _ = rate(wl, "fwd", 0, q)
    ba, br, _ = rate(wl, "bwd", 0, q)
    nq1 = max(1, min(Q, 1024))
    sl = _query_slice(wl, nq1)
    f1, _, _ = rate(sl, "fwd", 1, q)
    b1, _, _ = rate(sl, "bwd", 1, q)
    step_all = 1.0 / (1.0 / fa + 1.0 / ba)
    step_one = 1.0 / (1.0 / f1 + 1.0 / b1)
    return {"value": round(step_all, 1), "unit": "queries/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "fwd_queries_per_s": {"all_threads": round(fa, 1), "one_thread": round(f1, 1)},
            "bwd_queries_per_s": {"all_threads": round(ba, 1), "one_thread": round(b1, 1)},
            "one_thread_step_queries_per_s": round(step_one, 1),
            "sample": f"all {cores} threads: {fr} forward and {br} backward passes over the whole workload "
                      f"({bs}x{Q} queries); one thread: the first {nq1} queries of each batch, same value map; "
                      f"~{q:.0f} s each, float64 scalar C (OpenMP); value = fwd+bwd step rate with all threads"}


def fused_prologue_leg(wl_core, dev, steps: int, warmup: int, nsets: int) -> dict:
    """The fused form on the same shapes (msda_forward_fused +
    msda_backward_fused: reference points, offsets and logits in, offset and
    logit gradients out) against the module path it replaces: PyTorch forms
    the locations and the softmax, the core runs through the C ABI, and
    autograd carries the gradients back through PyTorch's ops."""
    import torch
    from scale_deformable_attention_03_amd import _lib, ops
    from scale_deformable_attention_03_amd import workloads as W

    bs, K, M, D = wl_core.value.shape
    Q, L, P = wl_core.sampling_locations.shape[1], wl_core.sampling_locations.shape[3], \
        wl_core.sampling_locations.shape[4]
    ref_dist = "encoder" if Q == K else "uniform"
    wl = W.make_fused(wl_core.name + "_fused", bs, wl_core.spatial_shapes, M, D, P, Q, wl_core.dtype,
                      seed=1012, ref_dims=2, ref_dist=ref_dist)
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_offsets)
    need_ws = _lib.workspace_bytes(prob)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    sets = []
    for _ in range(nsets):
        s = dict(value=wl.value.to(dev), ref=wl.reference_points.to(dev), off=wl.sampling_offsets.to(dev),
                 lg=wl.attention_logits.to(dev), g=wl.grad_output.to(dev))
        s["out"] = torch.empty(bs, Q, M * D, dtype=wl.value.dtype, device=dev)
        s["gv"] = torch.empty_like(s["value"])
        s["goff"] = torch.empty_like(s["off"])
        s["glg"] = torch.empty_like(s["lg"])
        s["ws"] = torch.empty(max(need_ws, 16), dtype=torch.uint8, device=dev)
        s["ptr"] = {k: v.data_ptr() for k, v in s.items() if isinstance(v, torch.Tensor)}
        sets.append(s)

    def fused(s):
        p = s["ptr"]
        _lib.forward_fused(prob, 2, p["value"], 0, p["ref"], p["off"], p["lg"], p["out"], sp)
        _lib.backward_fused(prob, 2, p["value"], 0, p["ref"], p["off"], p["lg"], p["g"], p["gv"], p["goff"],
                            p["glg"], p["ws"] if need_ws else 0, need_ws, sp)

    shapes = torch.as_tensor(wl.spatial_shapes, device=dev)
    norm = torch.stack([shapes[:, 1], shapes[:, 0]], -1).to(wl.value.dtype)

    def module_path(s):
        off = s["off"].detach().requires_grad_()
        lg = s["lg"].detach().requires_grad_()
        loc = s["ref"][:, :, None, :, None, :] + off / norm[None, None, None, :, None, :]
        w = torch.softmax(lg.view(bs, Q, M, L * P), -1).view(bs, Q, M, L, P)
        out = ops.MSDeformAttnFunction.apply(s["value"], wl.spatial_shapes, wl.level_start_index,
                                             loc.contiguous(), w.contiguous())
        out.backward(s["g"])

    def timed(fn):
        for i in range(warmup):
            fn(sets[i % nsets])
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            fn(sets[i % nsets])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    fused_ms = timed(fused)
    module_ms = timed(module_path)
    log(f"[bench] fused prologue: {fused_ms * 1e3:.1f} us/step; module path {module_ms * 1e3:.1f} us/step")
    return {"workload": wl.name, "reference_points": "2-d", "fused_ms_per_step": round(fused_ms, 5),
            "fused_queries_per_s": round(bs * Q / (fused_ms * 1e-3), 1),
            "module_path_ms_per_step": round(module_ms, 5),
            "speedup_vs_module_path": round(module_ms / fused_ms, 3)}


def mixed_precision_leg(dev, steps: int, warmup: int, nsets: int) -> dict:
    """The encoder step with bf16 value, output and value gradient and
    float32 locations, weights and their gradients (MSDA_BF16_F32), same
    shapes and draws as the float32 headline workload."""
    import torch
    from scale_deformable_attention_03_amd import _lib, ops
    from scale_deformable_attention_03_amd import workloads as W

    wl = W.detr_encoder(dtype="bf16", sample_dtype="f32")
    bs, K, M, D = wl.value.shape
    Q = wl.sampling_locations.shape[1]
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_locations)
    need_ws = _lib.workspace_bytes(prob)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    sets = []
    for _ in range(nsets):
        s = dict(value=wl.value.to(dev), loc=wl.sampling_locations.to(dev), w=wl.attention_weights.to(dev),
                 g=wl.grad_output.to(dev))
        s["out"] = torch.empty(bs, Q, M * D, dtype=wl.value.dtype, device=dev)
        s["gv"] = torch.empty_like(s["value"])
        s["gl"] = torch.empty_like(s["loc"])
        s["gw"] = torch.empty_like(s["w"])
        s["ws"] = torch.empty(max(need_ws, 16), dtype=torch.uint8, device=dev)
        s["ptr"] = {k: v.data_ptr() for k, v in s.items() if isinstance(v, torch.Tensor)}
        sets.append(s)

    def step(s):
        p = s["ptr"]
        _lib.forward_train(prob, p["value"], p["loc"], p["w"], p["out"], p["ws"] if need_ws else 0, need_ws, sp)
        _lib.backward_counted(prob, p["value"], p["loc"], p["w"], p["g"], p["gv"], p["gl"], p["gw"],
                              p["ws"] if need_ws else 0, need_ws, sp)

    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        step(sets[i % nsets])
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    log(f"[bench] mixed precision (bf16 value, f32 samples): {ms * 1e3:.1f} us/step")
    return {"workload": "detr_encoder", "dtype": "bf16 value/output/grad_value, f32 locations/weights/grads",
            "ms_per_step": round(ms, 5), "queries_per_s": round(bs * Q / (ms * 1e-3), 1)}


def module_step_leg(dev, steps: int, warmup: int) -> dict:
    """One MSDeformAttn module step (value_proj, sampling_offsets,
    attention_weights Linears through PyTorch's hipBLASLt GEMMs, the fused
    core through the C ABI, output_proj; forward and backward with autograd)
    at the DETR encoder shapes, float32, random weights."""
    import torch
    from scale_deformable_attention_03_amd import workloads as W
    from scale_deformable_attention_03_amd.module import MSDeformAttnModule

    wl = W.detr_encoder_module()
    m = MSDeformAttnModule(wl.d_model, wl.n_levels, wl.n_heads, wl.n_points, device=dev, params=wl.params)
    q = wl.query.to(dev).requires_grad_()
    x = wl.input_flatten.to(dev).requires_grad_()
    ref = wl.reference_points.to(dev)
    g = wl.grad_output.to(dev)
    shapes, starts = wl.spatial_shapes, wl.level_start_index
    stream = torch.cuda.current_stream(dev)

    def step():
        for p in m.parameters():
            p.grad = None
        q.grad = x.grad = None
        m(q, ref, x, shapes, starts).backward(g)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    bs, Q = wl.query.shape[:2]
    K = wl.input_flatten.shape[1]
    C, M, L, P = wl.d_model, wl.n_heads, wl.n_levels, wl.n_points
    rows_q, rows_k = bs * Q, bs * K
    # fwd: 4 GEMMs; bwd: 2 per Linear (input and weight gradients), 2 * rows * in * out flops each
    linear_flops = 2 * (rows_k * C * C + rows_q * C * (M * L * P * 2) + rows_q * C * (M * L * P) + rows_q * C * C)
    log(f"[bench] module step (Linears + fused core, fwd+bwd): {ms * 1e3:.1f} us/step")
    return {"workload": wl.name, "dtype": "f32", "ms_per_step": round(ms, 5),
            "queries_per_s": round(rows_q / (ms * 1e-3), 1), "linear_gflop_per_step": round(3 * linear_flops / 1e9, 2)}


def measure_workload(wl, name: str, dev, steps: int, warmup: int, extras: bool) -> dict:
    """Time `steps` forward + backward steps of one workload through the C ABI
    on rotating buffer sets (inputs resident in HBM), then the backward's
    stages (msda_backward_profile events) and the roofline of the dominant
    kernel.  With extras: also the warm and graph-replay timings."""
    import torch
    from scale_deformable_attention_03_amd import _lib, ops

    bs, K, M, D = wl.value.shape
    Q, L, P = wl.sampling_locations.shape[1], wl.sampling_locations.shape[3], wl.sampling_locations.shape[4]
    rows = touched_rows(wl)
    ab = algorithmic_bytes(wl, rows)
    prob, keep = ops.problem_for(wl.value, wl.spatial_shapes, wl.level_start_index, wl.sampling_locations)

    # Rotating buffer sets: the sets together exceed twice the Infinity Cache.
    step_bytes = sum(t.numel() * t.element_size() for t in
                     (wl.value, wl.sampling_locations, wl.attention_weights, wl.grad_output)) * 2
    nsets = max(2, int(np.ceil(2 * MALL_BYTES / max(step_bytes, 1))) + 1)
    nsets = min(nsets, 8)
    sets = []
    need_ws = _lib.workspace_bytes(prob)
    for _ in range(nsets):
        s = dict(value=wl.value.to(dev), loc=wl.sampling_locations.to(dev), w=wl.attention_weights.to(dev),
                 g=wl.grad_output.to(dev))
        s["out"] = torch.empty(bs, Q, M * D, dtype=wl.value.dtype, device=dev)
        s["gv"] = torch.empty_like(s["value"])
        s["gl"] = torch.empty_like(s["loc"])
        s["gw"] = torch.empty_like(s["w"])
        s["ws"] = torch.empty(max(need_ws, 16), dtype=torch.uint8, device=dev)
        s["ptr"] = {k: v.data_ptr() for k, v in s.items() if isinstance(v, torch.Tensor)}
        sets.append(s)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    # the training pair: the forward also counts the backward's records
    def fwd(s):
        p = s["ptr"]
        _lib.forward_train(prob, p["value"], p["loc"], p["w"], p["out"], p["ws"] if need_ws else 0, need_ws, sp)

    def bwd(s):
        p = s["ptr"]
        _lib.backward_counted(prob, p["value"], p["loc"], p["w"], p["g"], p["gv"], p["gl"], p["gw"],
                              p["ws"] if need_ws else 0, need_ws, sp)

    log(f"[bench] {name}: bs {bs} K {K} Q {Q} M {M} D {D} L {L} P {P} {wl.dtype}; "
        f"{nsets} buffer sets; warmup {warmup} steps {steps}")
    for i in range(warmup):
        fwd(sets[i % nsets])
        bwd(sets[i % nsets])
    torch.cuda.synchronize()

    # The timed steps: the host enqueues nothing but the steps between the
    # two synchronizations.  (A timing event between a step's forward and
    # backward and around it cost 12-19 us per step of the encoder's ~330,
    # so the split below comes from a pass of its own.)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s = sets[i % nsets]
        fwd(s)
        bwd(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps

    # The forward / backward split and the per-step percentiles: the same
    # steps again, with HIP events around the forward and the backward (not
    # part of the timed region).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        s = sets[i % nsets]
        ev[i][0].record(stream)
        fwd(s)
        ev[i][1].record(stream)
        bwd(s)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    bwd_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    step_us = np.array([a.elapsed_time(c) for a, _, c in ev]) * 1e3
    fwd_us_all = np.array([a.elapsed_time(b) for a, b, _ in ev]) * 1e3
    bwd_us_all = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e3
    log(f"[bench] timed: {ms_per_step:.4f} ms/step wall; evented pass fwd {fwd_ms * 1e3:.1f} us, "
        f"bwd {bwd_ms * 1e3:.1f} us, step {float(np.mean(step_us)):.1f} us")

    out = {}
    if extras:
        # warm: the same steps back to back on one buffer set (its working set
        # may stay in the Infinity Cache between steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fwd(sets[0])
            bwd(sets[0])
        torch.cuda.synchronize()
        out["warm_ms_per_step"] = round((time.perf_counter() - t0) * 1e3 / steps, 5)

        # The same steps captured as HIP graphs (one per buffer set) and
        # replayed: the launches cost no host time, which matters for the
        # small problems.
        graphs = []
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for s_ in sets:
                fwd(s_)
                bwd(s_)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        for s_ in sets:
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_):
                gsp = torch.cuda.current_stream(dev).cuda_stream
                p_ = s_["ptr"]
                _lib.forward_train(prob, p_["value"], p_["loc"], p_["w"], p_["out"], p_["ws"] if need_ws else 0,
                                   need_ws, gsp)
                _lib.backward_counted(prob, p_["value"], p_["loc"], p_["w"], p_["g"], p_["gv"], p_["gl"],
                                      p_["gw"], p_["ws"] if need_ws else 0, need_ws, gsp)
            graphs.append(g_)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % nsets].replay()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for i in range(steps):
            graphs[i % nsets].replay()
        gb.record(stream)
        torch.cuda.synchronize()
        out["graph_replay_ms_per_step"] = round(ga.elapsed_time(gb) / steps, 5)
        log(f"[bench] graph replay: {out['graph_replay_ms_per_step'] * 1e3:.1f} us/step")
        del graphs

    # Per-stage times of the backward (HIP events recorded by the library
    # between its kernels, msda_backward_counted_profile), live, same rotation.
    hip = ctypes.CDLL("libamdhip64.so.7")     # PyTorch's runtime, already loaded
    nstage = len(_lib.BACKWARD_STAGES)
    nk = max(20, steps // 4)
    evs = []
    for _ in range(nk):
        arr = (ctypes.c_void_p * (nstage + 1))()
        for j in range(nstage + 1):
            if hip.hipEventCreate(ctypes.byref(arr, j * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")
        evs.append(arr)
    for i in range(nk):
        s = sets[i % nsets]
        p = s["ptr"]
        fwd(s)
        _lib.backward_counted_profile(prob, p["value"], p["loc"], p["w"], p["g"], p["gv"], p["gl"], p["gw"],
                                      p["ws"] if need_ws else 0, need_ws, evs[i], sp)
    torch.cuda.synchronize()
    stage_ms = np.zeros(nstage)
    f = ctypes.c_float()
    for arr in evs:
        for j in range(nstage):
            if hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(arr[j]), ctypes.c_void_p(arr[j + 1])) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            stage_ms[j] += f.value / nk
        for j in range(nstage + 1):
            hip.hipEventDestroy(ctypes.c_void_p(arr[j]))
    stages_us = {n_: round(float(v) * 1e3, 2) for n_, v in zip(_lib.BACKWARD_STAGES, stage_ms)}
    log(f"[bench] backward stages (us): {stages_us}")
    del sets

    digest = kernel_digest()
    kernels = {"msda_forward_kernel": (fwd_ms, ab["fwd"]),
               "msda_backward_kernel": (stage_ms[3], ab["grad"]),
               "msda_accumulate_kernel": (stage_ms[4], ab["accum"])}
    kname = max(kernels, key=lambda k: kernels[k][0])
    kms, kbytes = kernels[kname]
    achieved = kbytes / (kms * 1e-3) / 1e9
    traffic = load_traffic(digest, kname, name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kname,
                "kernel_us": round(kms * 1e3, 2), "algorithmic_bytes_per_launch": kbytes}
    eff_gbps = ab["total"] / (ms_per_step * 1e-3) / 1e9
    out.update({
        "workload": name,
        "dtype": wl.dtype + ("+" + wl.sample_dtype if wl.sample_dtype else ""),
        "shape": {"batch": bs, "num_queries": Q, "num_keys": K, "num_heads": M, "embed_dims": D,
                  "num_levels": L, "num_points": P},
        "ms_per_step": round(ms_per_step, 5),
        "queries_per_s": round(bs * Q / (ms_per_step * 1e-3), 1),
        "effective_gbps": round(eff_gbps, 1),
        "pct_hbm_roofline": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "step_us_percentiles": percentiles(step_us),
        "fwd_us_percentiles": percentiles(fwd_us_all),
        "bwd_us_percentiles": percentiles(bwd_us_all),
        "fwd_us": round(fwd_ms * 1e3, 2),
        "bwd_us": round(bwd_ms * 1e3, 2),
        "bwd_stages_us": stages_us,
        "algorithmic_bytes_total": ab["total"],
        "kernel_digest": digest,
        "roofline": roofline,
        "ab": ab, "rows": rows, "nsets": nsets,
    })
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="detr_encoder",
                    choices=["detr_encoder", "large_batch_encoder", "max_constraint", "detr_decoder",
                             "detr_decoder_f16", "tiny_single_level", "detr_encoder_bf16_f32"])
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-prologue comparison")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed-precision leg")
    ap.add_argument("--no-module", action="store_true", help="skip the module-step leg")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the large-batch, max-constraint, decoder and tiny workloads' lines")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the gather / atomic-scatter / copy ceiling measurements")
    ap.add_argument("--ingest-profiles", metavar="DIR",
                    help="summarise the rocprofv3 output of the profiling commands under DIR into profiles/ "
                         "(no GPU needed) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device-to-device copy of 512 MiB, 4 times (the reference "
                         "for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.ingest_profiles:
        ingest_profiles(args.ingest_profiles, args.workload)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MSDeformAttn core runs on a single MI355X here "
              "(batch or head sharding of this core needs no communication). "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported.", file=sys.stderr)
        return 2

    import torch
    from scale_deformable_attention_03_amd import _lib, ops
    from scale_deformable_attention_03_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    if args.calibrate_copy:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)     # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "copies": 4}), flush=True)
        return 0

    wl = W.NAMED[args.workload]()
    m = measure_workload(wl, args.workload, dev, args.steps, args.warmup, extras=True)
    bs, K, M, D = wl.value.shape
    Q, L, P = wl.sampling_locations.shape[1], wl.sampling_locations.shape[3], wl.sampling_locations.shape[4]
    ms_per_step, nsets, ab, rows = m["ms_per_step"], m["nsets"], m["ab"], m["rows"]
    fwd_ms = m["fwd_us"] * 1e-3
    result = {
        "metric": "MSDeformAttn fwd+bwd queries/s and achieved HBM GB/s (% roofline), DETR encoder",
        "value": m["queries_per_s"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": bs, "num_queries": Q, "num_keys": K,
                   "num_heads": M, "embed_dims": D, "num_levels": L, "num_points": P,
                   "spatial_shapes": [list(map(int, s_)) for s_ in wl.spatial_shapes],
                   "buffer_sets": nsets, "parallelism": "single GPU",
                   "step": "msda_forward_train + msda_backward_counted"},
        "effective_gbps": m["effective_gbps"],
        "pct_hbm_roofline": m["pct_hbm_roofline"],
        "graph_replay_ms_per_step": m["graph_replay_ms_per_step"],
        "warm_ms_per_step": m["warm_ms_per_step"],
        "step_us_percentiles": m["step_us_percentiles"],
        "fwd_us_percentiles": m["fwd_us_percentiles"],
        "bwd_us_percentiles": m["bwd_us_percentiles"],
        "fwd_us": m["fwd_us"],
        "bwd_us": m["bwd_us"],
        "bwd_stages_us": m["bwd_stages_us"],
        "algorithmic_bytes": ab,
        "touched_value_rows": rows,
        "device": device_info(props),
        "kernel_digest": m["kernel_digest"],
        "roofline": m["roofline"],
    }
    eff_gbps = m["effective_gbps"]
    del m
    if args.workload == "detr_encoder" and not args.no_other_workloads:
        # the large-batch bf16 encoder (the second encoder line, held to the
        # same target) and the other workloads, each with its own roofline
        others = {}
        for name in ("large_batch_encoder", "max_constraint", "detr_decoder", "detr_decoder_f16",
                     "tiny_single_level"):
            owl = W.NAMED[name]()
            om = measure_workload(owl, name, dev, max(10, args.steps), max(3, args.warmup), extras=False)
            for k in ("ab", "rows", "nsets"):
                om.pop(k, None)
            others[name] = om
            log(f"[bench] {name}: {om['ms_per_step'] * 1e3:.1f} us/step, {om['queries_per_s']:.4g} queries/s, "
                f"{om['pct_hbm_roofline']:.2f}% of HBM roofline; dominant {om['roofline']['kernel']} "
                f"frac {om['roofline']['frac']}")
            del owl
            torch.cuda.empty_cache()
        result["large_batch_encoder"] = others.pop("large_batch_encoder")
        result["other_workloads"] = others
    if not args.no_ceilings:
        result["ceilings"] = ceilings_leg(wl, dev, fwd_ms * 1e3, eff_gbps)
        log(f"[bench] ceilings: {result['ceilings']}")
    if not args.no_fused:
        result["fused_prologue"] = fused_prologue_leg(wl, dev, max(10, args.steps // 2), max(2, args.warmup // 2),
                                                      nsets)
    if not args.no_mixed and args.workload == "detr_encoder":
        result["mixed_precision"] = mixed_precision_leg(dev, max(10, args.steps // 2), max(2, args.warmup // 2),
                                                        nsets)
    if not args.no_module and args.workload == "detr_encoder":
        result["module_step"] = module_step_leg(dev, max(10, args.steps // 4), max(2, args.warmup // 2))
    if args.no_cpu_baseline:
        result["cpu_baseline"] = None
    else:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
