#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule layer core on one MI355X.

One step = one pass over the whole hot path on synthetic inputs already resident
in GPU memory:
  * a blockwise prefill of T = 4096 tokens (B = 1, 16 query/key heads shared 2:1 by
    32 value heads, dk = dv = 128, chunk 64, bf16 q/k/v/o, fp32 gates and state,
    zero starting state): one gdn_prefill call (both kernels back to back);
  * one decode token through 30 independent recurrent layers (fp32 states of
    32 x 128 x 128, N(0, 0.1^2), each layer's tensors in allocations of their own): one
    gdn_decode_step_layers launch over the layers' pointer table.
The K timed steps run back to back on one stream.  The inputs rotate over several buffer
sets whose total (~1.9 GB) is far larger than the 256 MB last-level cache, so every step
finds its data in HBM.

value = prefill tokens per second: T / the mean duration of one gdn_prefill call, measured
with HIP events on the stream around spans of K calls enqueued back to back over the same
rotation (so the figure is the calls' own average, not the cost of an event pair around a
single launch).  The decode figures are measured the same way: the pointer-table launch (the
decode roofline), one B = 30 launch over states stored back to back, 30 B = 1 launches, and
the 30 launches captured in a HIP graph.  Secondary: the same prefill call alone right after
a 1 GiB flush fill (one call between two events), the two kernels timed as the two stages
(gdn_prefill_prepare, then gdn_prefill_scan) with an event between them, warm-cache stages,
the fused-normalisation and all-fp32 calls, the 131072-token long-memory prompt (gdn_prefill,
which runs it in passes sized to the last-level cache, against one pass over the whole prompt),
and a plain device copy as the achievable-bandwidth reference.  The HBM bytes and the
matrix-core work per launch come from rocprofv3 counter runs of this script, summarised into
profiles/ (--summarize-counters, --summarize-mfma) and used while the kernel sources are unchanged.  The CPU oracle runs on the host on the same prefill workload,
alternating with cold GPU calls (its output doubles as a parity check of the GPU output).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
LAYERS = 30
CPU_BASELINE_S = 10.0           # seconds of oracle work timed for the CPU baseline

# Algorithmic bytes of the prefill per token at these head shapes: q and k (16 heads x 128 x
# bf16 each), v and o (32 heads x 128 x bf16 each), g and beta (32 heads x fp32 each).
PREFILL_BYTES_PER_TOKEN = 16 * 128 * 2 * 2 + 32 * 128 * 2 * 2 + 32 * 4 * 2     # 24,832
STATE_BYTES = 32 * 128 * 128 * 4                                               # 2 MiB
# Matrix-core FLOPs of the pages' blockwise form per token per value head (chunk C = 64,
# dk = dv = 128, the two Gram blocks shared by the two value heads of a key head):
#   2 * [C dk (Grams) + C dk (W) + 2 C dv (U~, P U) + 3 dk dv (W S^T, Q S^T, U^T K) + C^2 / 6 (inverse)]
# (the residual form the kernels use does about 8% fewer: no U~ product, P R diag(beta) added)
PREFILL_FLOP_PER_TOKEN_HEAD = 2 * (64 * 128 + 64 * 128 + 2 * 64 * 128 + 3 * 128 * 128 + 64 * 64 / 6)
# Decode: each fp32 state element read once and written once, plus q, k, v, g, beta, o.
DECODE_BYTES_PER_LAYER = 2 * STATE_BYTES + PREFILL_BYTES_PER_TOKEN                  # 4,219,136

SOURCES = ["linear_recurrent_attention_gated_amd/csrc/" + f for f in
           ("gdn_device.h", "gdn_prefill.h", "gdn_decode.h", "gdn_sequential.h", "gdn_launch.h",
            "gdn_api.cpp", "gdn_prefill_inst.hip", "gdn_decode.hip", "gdn_sequential.hip")]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
COPY_CALIBRATION_BYTES = 512 << 20
FLUSH_BYTES = 1 << 30


def load_traffic():
    """HBM bytes per launch measured with rocprofv3 counters (profiles/hbm_traffic.txt), used
    only while the kernel sources are unchanged since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            doc = dict(l.split(":", 1) for l in fh.read().splitlines() if ":" in l and not l.startswith("#"))
    except (OSError, ValueError):
        return None
    doc = {k.strip(): v.strip() for k, v in doc.items()}
    if doc.get("source_hash") != kernel_source_hash():
        return None
    out = {}
    for k, v in doc.items():
        try:
            out[k] = float(v)
        except ValueError:
            out[k] = v
    return out


def _kernel_key(name, grid_size):
    """The key under which a dispatch's counters are summarised.  The bench also runs the
    fused-normalisation and all-fp32 prefills: their kernels are other template instances, kept
    apart by name; decode launches by their number of layers (grid size)."""
    el = "f32" if "<float" in name else "bf16"
    if "copybuffer" in name.lower():
        return "copy"
    if "inter_chunk_kernel" in name:
        return "inter" if el == "bf16" else "inter_f32"
    if "intra_chunk_kernel" in name:
        return ("intra_qknorm" if ", true>" in name else "intra") + ("" if el == "bf16" else "_f32")
    if "decode_layers_kernel" in name:
        return "decode_layers_L%d" % (int(float(grid_size or "0")) // (256 * 256))
    if "decode_kernel" in name:
        return "decode_L%d" % (int(float(grid_size or "0")) // (256 * 256))
    return None


def _counter_rows(d, counters):
    """(key, counter, value) of every dispatch in the rocprofv3 CSV output under d."""
    import csv
    import glob
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") not in counters:
                    continue
                key = _kernel_key(row.get("Kernel_Name", ""), row.get("Grid_Size"))
                if key is not None:
                    yield key, row["Counter_Name"], float(row["Counter_Value"])


def summarize_counters(fetch_dir, write_dir):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from rocprofv3 CSV output,
    scaled by what the same counters read for a plain copy of COPY_CALIBRATION_BYTES."""

    def per_kernel(d, counter):
        sums = {}
        for key, _, value in _counter_rows(d, (counter,)):
            sums.setdefault(key, []).append(value * 1024.0)
        # the calibration copy is the largest copy; small copies are runtime housekeeping
        return {k: (max(v) if k == "copy" else sum(v) / len(v)) for k, v in sums.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    f_scale = fetch.get("copy", 0) / COPY_CALIBRATION_BYTES
    w_scale = write.get("copy", 0) / COPY_CALIBRATION_BYTES
    lines = ["# HBM bytes per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE counters), made by:",
             "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o fetch -- "
             "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration --skip-long" % fetch_dir,
             "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o write -- "
             "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration --skip-long" % write_dir,
             "#   python bench.py --summarize-counters %s %s" % (fetch_dir, write_dir),
             "# Raw counter bytes are divided by the factor the same counter reads for a plain",
             "# device-to-device copy of %d bytes (read and written once)." % COPY_CALIBRATION_BYTES,
             "# intra, inter: the bf16 prefill (the inter kernel also serves the fused-normalisation",
             "# prefill, intra_qknorm); *_f32: the all-fp32 prefill; prefill_bytes_per_launch = intra",
             "# + inter.  decode_L<n>: one decode launch over n layers (B = n).",
             "source_hash: %s" % kernel_source_hash(),
             "fetch_scale: %.4f" % f_scale, "write_scale: %.4f" % w_scale]
    for k in sorted(set(fetch) | set(write)):
        if k == "copy":
            continue
        fb = fetch.get(k, 0.0) / f_scale if f_scale else 0.0
        wb = write.get(k, 0.0) / w_scale if w_scale else 0.0
        lines += ["%s_fetch_bytes: %.0f" % (k, fb), "%s_write_bytes: %.0f" % (k, wb),
                  "%s_bytes: %.0f" % (k, fb + wb)]
    fb = fetch.get("intra", 0.0) / f_scale + fetch.get("inter", 0.0) / f_scale if f_scale else 0.0
    wb = write.get("intra", 0.0) / w_scale + write.get("inter", 0.0) / w_scale if w_scale else 0.0
    lines.append("prefill_bytes_per_launch: %.0f" % (fb + wb))
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.txt")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
MI355X_XCDS, MI355X_SIMDS = 8, 1024


def summarize_mfma(d):
    """Matrix-core work per dispatch and kernel from one rocprofv3 --pmc run of MFMA_COUNTERS:
    FLOPs = MOPS x 512 (rocprofv3's MfmaFlops metrics), and the busy fraction = MFMA busy cycles
    summed over the SIMDs / (active cycles x SIMDs) (its MfmaUtil metric).  GRBM_GUI_ACTIVE
    comes summed over the XCDs, each of which counts the dispatch's active cycles."""
    sums = {}
    for key, counter, value in _counter_rows(d, MFMA_COUNTERS):
        sums.setdefault((key, counter), []).append(value)
    avg = {k: sum(v) / len(v) for k, v in sums.items()}
    keys = sorted({k for k, _ in avg if k != "copy"})
    lines = ["# Matrix-core work per dispatch (rocprofv3 counters %s), made by:" % ", ".join(MFMA_COUNTERS),
             "#   rocprofv3 --pmc %s --output-format csv -d %s -o mfma -- "
             "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --skip-long" % (" ".join(MFMA_COUNTERS), d),
             "#   python bench.py --summarize-mfma %s" % d,
             "# *_flops_bf16 / *_flops_f32: MOPS x 512; *_busy_frac: MFMA busy cycles over (active",
             "# cycles per XCD x %d SIMDs); keys as in hbm_traffic.txt." % MI355X_SIMDS,
             "source_hash: %s" % kernel_source_hash()]
    for k in keys:
        fb = avg.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), 0.0) * 512
        ff = avg.get((k, "SQ_INSTS_VALU_MFMA_MOPS_F32"), 0.0) * 512
        busy = avg.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0)
        active = avg.get((k, "GRBM_GUI_ACTIVE"), 0.0) / MI355X_XCDS
        lines += ["%s_flops_bf16: %.0f" % (k, fb), "%s_flops_f32: %.0f" % (k, ff),
                  "%s_busy_frac: %.4f" % (k, busy / (active * MI355X_SIMDS) if active else 0.0)]
    pf = [avg.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), 0.0) * 512 for k in ("intra", "inter")]
    pf32 = [avg.get((k, "SQ_INSTS_VALU_MFMA_MOPS_F32"), 0.0) * 512 for k in ("intra", "inter")]
    lines += ["prefill_flops_bf16_per_launch: %.0f" % sum(pf),
              "prefill_flops_f32_per_launch: %.0f" % sum(pf32)]
    with open(MFMA_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_mfma():
    """The MFMA counter summary (profiles/mfma_counters.txt) while the kernel sources are
    unchanged since it was taken, else None."""
    try:
        with open(MFMA_FILE) as fh:
            doc = dict(l.split(":", 1) for l in fh.read().splitlines() if ":" in l and not l.startswith("#"))
    except (OSError, ValueError):
        return None
    doc = {k.strip(): v.strip() for k, v in doc.items()}
    if doc.get("source_hash") != kernel_source_hash():
        return None
    return {k: float(v) for k, v in doc.items() if k != "source_hash"}


def mfma_counter_fields(doc, call_us):
    """The prefill's matrix-core work as the counters measured it (profiles/mfma_counters.txt):
    FLOPs executed per call on the bf16 and fp32 matrix cores, their rate over the call's
    measured duration against the bf16 peak, and each kernel's matrix-core busy fraction."""
    if not doc:
        return None
    fb, ff = doc.get("prefill_flops_bf16_per_launch", 0.0), doc.get("prefill_flops_f32_per_launch", 0.0)
    tflops = (fb + ff) / (call_us * 1e-6) / 1e12
    return {"source": "profiles/mfma_counters.txt (SQ_INSTS_VALU_MFMA_MOPS_BF16/_F32 x 512, "
                      "SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE)",
            "gflop_bf16_per_call": round(fb / 1e9, 3), "gflop_f32_per_call": round(ff / 1e9, 3),
            "achieved_tflops": round(tflops, 2),
            "frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "busy_frac_intra": doc.get("intra_busy_frac"), "busy_frac_inter": doc.get("inter_busy_frac")}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=6, help="rotating input buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="accepted for older command lines: the plain device-to-device copy of "
                         "known size (the reference point for the HBM byte counters and the "
                         "achievable-bandwidth figure) now runs in every measurement")
    ap.add_argument("--skip-long", action="store_true",
                    help="leave out the 131072-token secondary (the HBM counter runs do: its launches "
                         "are the same kernels and would enter the per-launch averages)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script "
                         "with --copy-calibration into profiles/hbm_traffic.txt, then exit")
    ap.add_argument("--summarize-mfma", metavar="MFMA_DIR",
                    help="turn a rocprofv3 --pmc run of the MFMA counters (op counts, busy cycles, "
                         "active cycles) of this script into profiles/mfma_counters.txt, then exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace run of this script (with --no-cpu-baseline "
                         "and the same --steps / --warmup) into the per-phase kernel table in "
                         "profiles/, then exit")
    ap.add_argument("--trace-bench-out", metavar="FILE",
                    help="with --summarize-trace: the profiled run's stdout (its JSON line), to "
                         "set its event-timed figures beside the kernel times")
    ap.add_argument("--crossover", action="store_true",
                    help="time the token-sequential and the blockwise prefill on prefixes of the "
                         "128K long-memory draw (cold, 16/32 heads, d=128, bf16), print one JSON "
                         "line, then exit")
    ap.add_argument("--crossover-table", action="store_true",
                    help="time both prefill forms at short prompt lengths for several (dtype, d, "
                         "heads), print the measured crossovers as one JSON line, then exit")
    return ap.parse_args()


# short prompts around the crossover, then the 10-point doubling sweep 256 .. 128K
CROSSOVER_T = (1, 8, 16, 32, 48, 64, 96, 128, 192) + tuple(256 << i for i in range(10))


def crossover(args):
    """Both prefill forms on prefixes of one draw, each call cold (the flush fill first)."""
    import numpy as np
    import torch

    from linear_recurrent_attention_gated_amd import gdn
    from linear_recurrent_attention_gated_amd.inputs import LONG_128K, workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = LONG_128K
    host = workload_inputs(w, torch.bfloat16)
    full = {k: host[k].to(dev) for k in ("q", "k", "v", "g", "beta")}
    del host
    Hk, Hv, dk, dv, C = w.Hk, w.Hv, w.dk, w.dv, w.chunk
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, max(CROSSOVER_T), Hk, Hv, dk, dv, C,
                                                     torch.bfloat16), dtype=torch.uint8, device=dev)
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    s_out = torch.empty((1, Hv, dv, dk), dtype=torch.float32, device=dev)
    points = []
    for T in CROSSOVER_T:
        d = {k: v[:, :T].contiguous() for k, v in full.items()}
        o = torch.empty((1, T, Hv, dv), dtype=torch.bfloat16, device=dev)
        res = {"T": T}
        for name, flags in (("sequential", gdn.GDN_PATH_SEQUENTIAL), ("blockwise", 0)):
            reps = 5 if T <= 16384 else 2
            ts = []
            for r in range(reps + 1):
                scratch.fill_(r & 0xFF)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                gdn.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, o, s_out, C, ws,
                                   flags)
                e1.record()
                torch.cuda.synchronize()
                if r:
                    ts.append(e0.elapsed_time(e1) * 1e3)
            res[name + "_us"] = round(float(np.median(ts)), 2)
            res[name + "_mtok_s"] = round(T / float(np.median(ts)), 3)
        points.append(res)
        print("[crossover]", res, file=sys.stderr, flush=True)
    faster = [p["T"] for p in points if p["sequential_us"] < p["blockwise_us"]]
    print(json.dumps({"crossover": {
        "workload": w.name + " prefixes, zero start state, cold", "points": points,
        "sequential_faster_at": faster,
        "auto_max_tokens": gdn.gdn_prefill_sequential_max_tokens(1, Hk, Hv, dk, dv,
                                                                 torch.bfloat16)}}), flush=True)


# (dtype, d, Hk, Hv, B) of the crossover table; prompt lengths around the crossover
CROSSOVER_TABLE_CONFIGS = [("bf16", 128, 16, 32, 1), ("f32", 128, 16, 32, 1), ("bf16", 64, 16, 32, 1),
                           ("f32", 64, 16, 32, 1), ("bf16", 32, 16, 32, 1), ("f32", 32, 16, 32, 1),
                           ("bf16", 128, 2, 4, 1), ("f32", 128, 2, 4, 1), ("bf16", 128, 16, 32, 4),
                           ("f32", 128, 16, 32, 4), ("bf16", 64, 16, 32, 4)]
CROSSOVER_TABLE_T = (1, 8, 16, 24, 32, 40, 48, 56, 64, 80, 96, 128, 160, 192, 256)


def crossover_table(args):
    """The prompt length up to which the token-sequential form beats the blockwise one, per
    (dtype, d = dk = dv, heads): both forms timed cold on one seeded draw of each shape."""
    import numpy as np
    import torch

    from linear_recurrent_attention_gated_amd import gdn
    from linear_recurrent_attention_gated_amd.inputs import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    C = 64
    rows = []
    for name, d, Hk, Hv, Bt in CROSSOVER_TABLE_CONFIGS:
        dt = torch.bfloat16 if name == "bf16" else torch.float32
        Tm = max(CROSSOVER_TABLE_T)
        full = {k: v.to(dev) for k, v in make_inputs(Bt, Tm, Hk, Hv, d, d, 5, dt).items() if v is not None}
        ws = torch.empty(gdn.gdn_prefill_workspace_bytes(Bt, Tm, Hk, Hv, d, d, C, dt), dtype=torch.uint8,
                         device=dev)
        s_out = torch.empty((Bt, Hv, d, d), dtype=torch.float32, device=dev)
        points = []
        for T in CROSSOVER_TABLE_T:
            x = {k: v[:, :T].contiguous() for k, v in full.items()}
            o = torch.empty((Bt, T, Hv, d), dtype=dt, device=dev)
            res = {"T": T}
            for path, flags in (("sequential", gdn.GDN_PATH_SEQUENTIAL), ("blockwise", 0)):
                ts = []
                for r in range(8):
                    scratch.fill_(r & 0xFF)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    gdn.gdn_prefill_ex(x["q"], x["k"], x["v"], x["g"], x["beta"], None, o, s_out, C, ws,
                                       flags)
                    e1.record()
                    torch.cuda.synchronize()
                    if r:
                        ts.append(e0.elapsed_time(e1) * 1e3)
                res[path + "_us"] = round(float(np.median(ts)), 2)
            points.append(res)
        faster = [pt["T"] for pt in points if pt["sequential_us"] < pt["blockwise_us"]]
        # the crossover: the last length before the first one at which blockwise wins
        cross = 0
        for pt in points:
            if pt["sequential_us"] < pt["blockwise_us"]:
                cross = pt["T"]
            else:
                break
        # interpolated crossing of the two times between the last length the sequential form
        # wins and the next
        x = None
        for a, b in zip(points, points[1:]):
            da, db = a["sequential_us"] - a["blockwise_us"], b["sequential_us"] - b["blockwise_us"]
            if da < 0 <= db:
                x = round(a["T"] + (b["T"] - a["T"]) * (-da) / (db - da), 1)
                break
        row = {"dtype": name, "d": d, "Hk": Hk, "Hv": Hv, "B": Bt, "crossover_T": cross,
               "crossing_interpolated": x, "sequential_faster_at": faster, "points": points,
               "auto_max_tokens": gdn.gdn_prefill_sequential_max_tokens(Bt, Hk, Hv, d, d, dt)}
        rows.append(row)
        print("[crossover-table]", json.dumps({k: v for k, v in row.items() if k != "points"}),
              file=sys.stderr, flush=True)
        del full, ws
    print(json.dumps({"crossover_table": rows}), flush=True)


TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_stats_prefill_4k_decode_30layers.md")


def summarize_trace(trace_dir, warmup, steps, bench_out=None):
    """Per-kernel launch durations from a rocprofv3 --kernel-trace run of this script (made with
    --no-cpu-baseline and the given --warmup / --steps), written to TRACE_FILE.  The launches
    of each kernel are split into the script's phases by their order in the trace."""
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        sys.exit("no *kernel_trace.csv under " + trace_dir)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0

    def grid(r):
        return int(float(r.get("Grid_Size_X") or r.get("Grid_Size") or 0))

    def short(n):
        return n.split("(")[0]

    W, K = warmup, steps
    by_name, by_shape = {}, {}
    for r in rows:
        by_name.setdefault(short(r["Kernel_Name"]), []).append(dur(r))
        by_shape.setdefault((short(r["Kernel_Name"]), grid(r)), []).append(dur(r))
    total = sum(sum(v) for v in by_name.values())
    mean = lambda v: sum(v) / len(v) if v else float("nan")  # noqa: E731
    out = ["# Kernel time: prefill T=4096 (Hk=16, Hv=32, dk=dv=128, chunk 64) and a 30-layer decode",
           "",
           "Command (repo root):",
           "",
           "    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/stats -o bench -- \\",
           "        python bench.py --steps %d --warmup %d --no-cpu-baseline%s" % (
               K, W, " > " + bench_out if bench_out else ""),
           "    python bench.py --summarize-trace gpurun_out/stats --steps %d --warmup %d%s" % (
               K, W, " --trace-bench-out " + bench_out if bench_out else ""),
           "",
           "One bench step is one gdn_prefill call (intra_chunk_kernel then inter_chunk_kernel) and",
           "one gdn_decode_step_layers launch over 30 separately allocated layers, inputs rotating",
           "over buffer sets that do not fit the last-level cache.  After the steps the script runs,",
           "in this order: 3 spans of %d prefill calls back to back (the headline), 3 x %d layer" % (K, K),
           "launches, 3 x %d B=30 decode launches, 3 x %d x 30 B=1 decode launches, %d single cold" % (K, K, K + 1),
           "prefill calls (flush fill first), %d cold split-stage calls, 3 x %d replays of a HIP graph" % (K + 2, K),
           "of the 30 B=1 launches, %d warm split-stage calls, 11 cold fused-normalisation calls (their" % (K + 2),
           "scan is the bf16 inter kernel), 11 cold all-fp32 calls (`float` instances), 4 + 4 cold",
           "calls of the 131072-token prompt (in cache-sized passes, then in one pass) and a 512 MiB",
           "device copy.  Averages over all launches of a kernel therefore mix these phases; the",
           "phase tables below split them.",
           "",
           "| Kernel | Calls | Avg (us) | Min (us) | Max (us) | Share |",
           "|---|---|---|---|---|---|"]
    for k, v in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
        out.append("| %s | %d | %.2f | %.2f | %.2f | %.2f%% |" % (k, len(v), mean(v), min(v), max(v),
                                                                100 * sum(v) / total))
    out += ["", "Per launch shape (grid in work-items):", "",
            "| Kernel | Grid | Calls | Avg (us) | Min (us) | Max (us) |", "|---|---|---|---|---|---|"]
    for (k, gsz), v in sorted(by_shape.items(), key=lambda kv: -sum(kv[1])):
        out.append("| %s | %d | %d | %.2f | %.2f | %.2f |" % (k, gsz, len(v), mean(v), min(v), max(v)))

    def seq(pat):
        return [dur(r) for r in rows if pat in r["Kernel_Name"]]

    intra = seq("intra_chunk_kernel<unsigned short, 128, 128, 64, false>")
    inter = seq("inter_chunk_kernel<unsigned short, 128, 128, 64, true>")
    phases = [("timed steps (each call followed by a decode launch)", W, W + K),
              ("spans of back-to-back calls (headline)", W + K, W + 4 * K),
              ("single calls, cold", W + 4 * K + 1, W + 5 * K + 1),
              ("split stages, cold", W + 5 * K + 3, W + 6 * K + 3),
              ("split stages, warm", W + 6 * K + 5, W + 7 * K + 5)]
    out += ["", "bf16 prefill kernels by phase (average launch duration, us):", "",
            "| Phase | Calls | intra_chunk_kernel | inter_chunk_kernel | Sum |", "|---|---|---|---|---|"]
    for name, a, b in phases:
        i, j = intra[a:b], inter[a:b]
        out.append("| %s | %d | %.2f | %.2f | %.2f |" % (name, len(i), mean(i), mean(j), mean(i) + mean(j)))
    lay = seq("decode_layers_kernel")
    d30 = [dur(r) for r in rows if "decode_kernel<" in r["Kernel_Name"] and grid(r) == LAYERS * 32 * 8 * 256]
    d1 = [dur(r) for r in rows if "decode_kernel<" in r["Kernel_Name"] and grid(r) == 32 * 8 * 256]
    n1 = 3 * K * LAYERS
    f32i, f32s = seq("intra_chunk_kernel<float"), seq("inter_chunk_kernel<float")
    out += ["", "Decode and the other prefill builds (average launch duration, us):", "",
            "| Launch | Calls | Avg (us) |", "|---|---|---|",
            "| decode_layers_kernel, 30 layers, timed steps | %d | %.2f |" % (len(lay[W:W + K]), mean(lay[W:W + K])),
            "| decode_layers_kernel, 30 layers, back-to-back spans | %d | %.2f |" % (len(lay[W + K:W + 4 * K]),
                                                                                 mean(lay[W + K:W + 4 * K])),
            "| decode_kernel B=30, back-to-back spans | %d | %.2f |" % (len(d30), mean(d30)),
            "| decode_kernel B=1, eager (30 per token) | %d | %.2f |" % (len(d1[:n1]), mean(d1[:n1])),
            "| decode_kernel B=1, graph replays | %d | %.2f |" % (len(d1[n1:]), mean(d1[n1:])),
            "| intra_chunk_kernel, fused normalisation, cold | %d | %.2f |" % (
                len(seq("intra_chunk_kernel<unsigned short, 128, 128, 64, true>")),
                mean(seq("intra_chunk_kernel<unsigned short, 128, 128, 64, true>"))),
            "| intra_chunk_kernel fp32, cold | %d | %.2f |" % (len(f32i), mean(f32i)),
            "| inter_chunk_kernel fp32, cold | %d | %.2f |" % (len(f32s), mean(f32s))]
    if bench_out:
        # the profiled run's own HIP-event figures (its JSON line), against the kernel times
        doc = None
        with open(bench_out) as fh:
            for line in fh:
                if line.startswith("{") and '"metric"' in line:
                    doc = json.loads(line)
        if doc:
            pf, dec = doc["prefill"], doc["decode"]
            spans = phases[1]
            out += ["", "The same (profiled) run's HIP-event figures, from its JSON line: prefill call %.2f us "
                    "(spans %s) against %.2f us of kernel time in the spans phase above; decode "
                    "layers launch %.2f us against %.2f us.  Kernel-trace collection slows the "
                    "launches a little: the default bench run without the profiler is the "
                    "reference for the headline figures." % (
                        pf["us_mean"], pf["us_spans"], mean(intra[spans[1]:spans[2]]) + mean(inter[spans[1]:spans[2]]),
                        dec["us_per_token_layers"], mean(lay[W + K:W + 4 * K]))]
    with open(TRACE_FILE, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print(TRACE_FILE)


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.warmup, args.steps, args.trace_bench_out)
        return
    if args.crossover:
        crossover(args)
        return
    if args.crossover_table:
        crossover_table(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the gated-delta-rule core is built and measured "
              "on a single MI355X; runs on more than one GPU are not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_recurrent_attention_gated_amd import gdn
    from linear_recurrent_attention_gated_amd.inputs import (LONG_128K, PREFILL_4K, decode_inputs,
                                                             make_inputs, workload_inputs)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = gdn.lib()
    w = PREFILL_4K
    B, T, Hk, Hv, dk, dv, C = w.B, w.T, w.Hk, w.Hv, w.dk, w.dv, w.chunk
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # -- inputs: one seeded draw, copied into rotating buffer sets -----------------------------
    host = workload_inputs(w, torch.bfloat16)
    ws_bytes = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, C, torch.bfloat16)
    dec_host = [decode_inputs(l) for l in range(LAYERS)]
    dec_cat = {k: torch.cat([d[k] for d in dec_host]).contiguous() for k in dec_host[0]}
    sets = []
    for _ in range(args.sets):
        s = {k: host[k].to(dev) for k in ("q", "k", "v", "g", "beta")}
        s["o"] = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device=dev)
        s["state_out"] = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        dd = {k: v.to(dev) for k, v in dec_cat.items()}
        dd["o"] = torch.empty((LAYERS, Hv, dv), dtype=torch.bfloat16, device=dev)
        s["dec"] = dd
        # the same states again, each layer in an allocation of its own (not back to back)
        s["dec_states"] = [dd["state"][l].clone() for l in range(LAYERS)]
        sets.append(s)
    torch.cuda.synchronize()

    def pf_args(s):
        return (s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(), s["g"].data_ptr(),
                s["beta"].data_ptr(), None, s["o"].data_ptr(), s["state_out"].data_ptr(),
                B, T, Hk, Hv, dk, dv, C, gdn.GDN_BF16, s["ws"].data_ptr(), ws_bytes, sh)

    def dec_args(s, l0, nb):
        d = s["dec"]
        st = d["state"][l0].data_ptr()
        return (d["q"][l0].data_ptr(), d["k"][l0].data_ptr(), d["v"][l0].data_ptr(),
                d["g"][l0].data_ptr(), d["beta"][l0].data_ptr(), st, st, d["o"][l0].data_ptr(),
                nb, Hk, Hv, dk, dv, gdn.GDN_BF16, sh)

    def layer_table(s):
        d = s["dec"]
        t = (gdn.DecodeLayer * LAYERS)()
        for l in range(LAYERS):
            st = s["dec_states"][l].data_ptr()
            t[l] = gdn.DecodeLayer(d["q"][l].data_ptr(), d["k"][l].data_ptr(), d["v"][l].data_ptr(),
                                   d["g"][l].data_ptr(), d["beta"][l].data_ptr(), st, st,
                                   d["o"][l].data_ptr())
        return t

    PF = [pf_args(s) for s in sets]
    DEC_L = [layer_table(s) for s in sets]
    DEC = [[dec_args(s, l, 1) for l in range(LAYERS)] for s in sets]
    DEC_B = [dec_args(s, 0, LAYERS) for s in sets]

    def check(rc, fn):
        if rc != 0:
            raise gdn.GdnError(fn, rc)

    nsteps = args.warmup + args.steps
    # Written before the single-call cold measurements below (outside their timed spans): it
    # evicts the L2 and the 256 MB last-level cache.
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def prefill_call(i):
        check(lib.gdn_prefill(*PF[i % len(sets)]), "gdn_prefill")

    def decode_layers(i):
        check(lib.gdn_decode_step_layers(DEC_L[i % len(sets)], LAYERS, 1, Hk, Hv, dk, dv,
                                         gdn.GDN_BF16, 0, sh), "gdn_decode_step_layers")

    def decode_batched(i):
        check(lib.gdn_decode_step(*DEC_B[i % len(sets)]), "gdn_decode_step")

    def decode_looped(i):
        for a in DEC[i % len(sets)]:
            check(lib.gdn_decode_step(*a), "gdn_decode_step")

    def span_us(fn, n, start=0):
        """Mean device time of one fn(i), for n calls enqueued back to back on the stream between
        two events (i = start .. start + n - 1, rotating over the buffer sets), in us."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(start, start + n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    def step(i):
        prefill_call(i)
        decode_layers(i)

    # The K timed steps of the whole hot path -- one prefill call and one decode token through
    # the 30 layers each -- back to back on one stream.  The inputs rotate over `sets` buffer
    # sets (~180 MB of prefill data and ~130 MB of decode state each, ~1.9 GB in all), so every
    # step finds its data in HBM, not in the 256 MB last-level cache.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev_a.record(stream)
    for i in range(args.warmup, nsteps):
        step(i)
    ev_b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = ev_a.elapsed_time(ev_b) * 1e3 / args.steps

    # Each path's average launch duration, over the same rotation: the prefill call alone and
    # the decode token alone, n back to back (the headline figures)
    pf_spans = [span_us(prefill_call, args.steps, r * args.steps) for r in range(3)]
    t_dec_l = np.array([span_us(decode_layers, args.steps, r * args.steps) for r in range(3)])
    t_dec_b = np.array([span_us(decode_batched, args.steps, r * args.steps) for r in range(3)])
    t_dec = np.array([span_us(decode_looped, args.steps, r * args.steps) for r in range(3)])

    # The same prefill call on its own, cold: the flush fill, then one call between two events
    # (includes the event pair's own cost around a single launch; secondary)
    t_prefill_single = []
    for i in range(args.steps + 1):
        scratch.fill_(i & 0xFF)
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        prefill_call(i)
        b2.record(stream)
        torch.cuda.synchronize()
        if i:
            t_prefill_single.append(a.elapsed_time(b2) * 1e3)
    t_prefill_single = np.array(t_prefill_single)

    # -- the two prefill kernels on their own, cold: the stages with an event between them --
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps + 2):
        j = i % len(sets)
        scratch.fill_(i & 0xFF)
        if i >= 2:
            evs[i - 2][0].record(stream)
        check(lib.gdn_prefill_prepare(*PF[j]), "gdn_prefill_prepare")
        if i >= 2:
            evs[i - 2][1].record(stream)
        check(lib.gdn_prefill_scan(*PF[j]), "gdn_prefill_scan")
        if i >= 2:
            evs[i - 2][2].record(stream)
    torch.cuda.synchronize()
    t_intra = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    t_inter = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3

    # -- decode as a HIP graph: the 30 sequential launches captured once per buffer set and
    # replayed (no host launch gaps between layers); cold like the main steps ----------------
    cap = torch.cuda.Stream()
    graphs = []
    for j in range(len(sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            hs = cap.cuda_stream
            for a in DEC[j]:
                check(lib.gdn_decode_step(*(a[:-1] + (hs,))), "gdn_decode_step")
        graphs.append(g)
    torch.cuda.synchronize()
    t_dec_g = np.array([span_us(lambda i: graphs[i % len(sets)].replay(), args.steps, r * args.steps)
                        for r in range(3)])
    del graphs

    # -- warm-cache prefill (same buffers every time), secondary -------------------------------
    evw = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps + 2):
        if i >= 2:
            evw[i - 2][0].record(stream)
        check(lib.gdn_prefill_prepare(*PF[0]), "gdn_prefill_prepare")
        if i >= 2:
            evw[i - 2][1].record(stream)
        check(lib.gdn_prefill_scan(*PF[0]), "gdn_prefill_scan")
        if i >= 2:
            evw[i - 2][2].record(stream)
    torch.cuda.synchronize()
    tw_intra = np.array([e[0].elapsed_time(e[1]) for e in evw]) * 1e3
    tw_inter = np.array([e[1].elapsed_time(e[2]) for e in evw]) * 1e3

    # -- secondary variants of the same prefill, cold: fused q/k normalisation on raw q, k
    # (gdn_prefill_qknorm) and the all-fp32 build -------------------------------------------
    def cold_prefill_us(fn, args_, reps):
        ts = []
        for i in range(reps + 1):
            scratch.fill_(i & 0xFF)
            a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            check(fn(*args_), "gdn_prefill variant")
            b2.record(stream)
            torch.cuda.synchronize()
            if i:
                ts.append(a.elapsed_time(b2) * 1e3)
        return float(np.mean(ts))

    raw = make_inputs(B, T, Hk, Hv, dk, dv, w.seed, torch.bfloat16, unit_qk=False)
    rq, rk = raw["q"].to(dev), raw["k"].to(dev)
    o_v = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device=dev)   # own outputs: set 0's
    s_v = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=dev)   # feed the parity check
    a_qk = list(PF[0])
    a_qk[0], a_qk[1], a_qk[6], a_qk[7] = rq.data_ptr(), rk.data_ptr(), o_v.data_ptr(), s_v.data_ptr()
    qknorm_us = cold_prefill_us(lib.gdn_prefill_qknorm, tuple(a_qk), 10)
    del rq, rk, raw
    f32 = {k: host[k].float().to(dev) for k in ("q", "k", "v")}
    o32 = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    ws32 = torch.empty(gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, C, torch.float32),
                       dtype=torch.uint8, device=dev)
    a32 = (f32["q"].data_ptr(), f32["k"].data_ptr(), f32["v"].data_ptr(), sets[0]["g"].data_ptr(),
           sets[0]["beta"].data_ptr(), None, o32.data_ptr(), s_v.data_ptr(),
           B, T, Hk, Hv, dk, dv, C, gdn.GDN_F32, ws32.data_ptr(), ws32.numel(), sh)
    f32_us = cold_prefill_us(lib.gdn_prefill, a32, 10)
    del f32, o32, ws32, o_v, s_v

    long_passes_us = long_one_us = None
    if not args.skip_long:
        # -- the 128K long-memory prompt, cold: gdn_prefill (passes sized to the last-level cache)
        # against one pass over the whole prompt (the two stages called separately).  Its inputs are
        # drawn on the GPU (the same recipe as the oracle-checked CPU draw, another draw). --------
        Lw = LONG_128K
        lg = make_inputs(Lw.B, Lw.T, Lw.Hk, Lw.Hv, Lw.dk, Lw.dv, Lw.seed, torch.bfloat16, Lw.g_mean,
                         Lw.beta_mean, device=dev)
        lo = torch.empty((Lw.B, Lw.T, Lw.Hv, Lw.dv), dtype=torch.bfloat16, device=dev)
        ls = torch.empty((Lw.B, Lw.Hv, Lw.dv, Lw.dk), dtype=torch.float32, device=dev)
        lws_bytes = gdn.gdn_prefill_workspace_bytes(Lw.B, Lw.T, Lw.Hk, Lw.Hv, Lw.dk, Lw.dv, Lw.chunk,
                                                    torch.bfloat16)
        lws = torch.empty(lws_bytes, dtype=torch.uint8, device=dev)
        la = (lg["q"].data_ptr(), lg["k"].data_ptr(), lg["v"].data_ptr(), lg["g"].data_ptr(),
              lg["beta"].data_ptr(), None, lo.data_ptr(), ls.data_ptr(), Lw.B, Lw.T, Lw.Hk, Lw.Hv,
              Lw.dk, Lw.dv, Lw.chunk, gdn.GDN_BF16, lws.data_ptr(), lws_bytes, sh)

        def one_pass(*a):
            rc = lib.gdn_prefill_prepare(*a)
            return rc if rc else lib.gdn_prefill_scan(*a)

        long_passes_us = cold_prefill_us(lib.gdn_prefill, la, 3)
        long_one_us = cold_prefill_us(one_pass, la, 3)
        del lg, lo, ls, lws

    # -- achievable HBM bandwidth in the same run: a plain device-to-device copy of known
    # size, cold (it is also the reference point of the HBM byte counters) -----------------
    src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = []
    for r in range(4):
        scratch.fill_(r)
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b2.record(stream)
        torch.cuda.synchronize()
        if r:
            copy_ms.append(a.elapsed_time(b2))
    copy_gbs = 2 * COPY_CALIBRATION_BYTES / (min(copy_ms) * 1e-3) / 1e9
    del src, dst

    mean_pf = float(np.mean(pf_spans))
    value = T / (mean_pf * 1e-6)
    pf_bytes = T * PREFILL_BYTES_PER_TOKEN + STATE_BYTES        # zero start state: state_out only
    pf_flops = T * Hv * PREFILL_FLOP_PER_TOKEN_HEAD
    achieved = pf_bytes / (mean_pf * 1e-6) / 1e9
    traffic_doc = load_traffic()
    traffic = None
    if traffic_doc:
        traffic = traffic_doc.get("prefill_bytes_per_launch")

    dec_layer_us = float(t_dec.mean()) / LAYERS
    dec_b_us = float(t_dec_b.mean())
    dec_bytes_b = LAYERS * DECODE_BYTES_PER_LAYER
    dec_gbs_b = dec_bytes_b / (dec_b_us * 1e-6) / 1e9
    dec_gbs_loop = dec_bytes_b / (float(t_dec.mean()) * 1e-6) / 1e9
    dec_g_us = float(t_dec_g.mean())
    dec_l_us = float(t_dec_l.mean())
    dec_gbs_l = dec_bytes_b / (dec_l_us * 1e-6) / 1e9
    dec_gbs_g = dec_bytes_b / (dec_g_us * 1e-6) / 1e9

    out = {
        "metric": "GDN prefill tokens/s @T=4096 (MFMA %peak); decode-step us/token (HBM GB/s)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "Hk": Hk, "Hv": Hv, "dk": dk, "dv": dv,
                   "chunk": C, "state": "fp32, zero start", "decode_layers": LAYERS,
                   "input_sets": args.sets},
        "step_us": round(step_us, 2),
        "prefill": {
            "us_mean": round(mean_pf, 2),
            "us_spans": [round(x, 2) for x in pf_spans],
            "timing": f"mean over {len(pf_spans)} spans of {args.steps} calls enqueued back to back "
                      f"between two events on the stream, inputs rotating over {args.sets} buffer "
                      f"sets (each call finds its data in HBM)",
            "us_single_call_cold_mean": round(float(t_prefill_single.mean()), 2),
            "us_single_call_cold_p10": round(float(np.percentile(t_prefill_single, 10)), 2),
            "us_single_call_cold_p90": round(float(np.percentile(t_prefill_single, 90)), 2),
            "intra_chunk_us": round(float(t_intra.mean()), 2),
            "inter_chunk_us": round(float(t_inter.mean()), 2),
            "split_sum_us": round(float((t_intra + t_inter).mean()), 2),
            "warm_intra_chunk_us": round(float(tw_intra.mean()), 2),
            "warm_inter_chunk_us": round(float(tw_inter.mean()), 2),
            "qknorm_us": round(qknorm_us, 2),
            "f32_us": round(f32_us, 2),
            "long_131072": None if long_passes_us is None else {
                "workload": LONG_128K.name + ", bf16, zero start state, cold single calls",
                "us_cache_sized_passes": round(long_passes_us, 1),
                "mtok_s_cache_sized_passes": round(LONG_128K.T / long_passes_us, 2),
                "us_one_pass": round(long_one_us, 1),
                "mtok_s_one_pass": round(LONG_128K.T / long_one_us, 2)},
            "mfma_tflops": round(pf_flops / (mean_pf * 1e-6) / 1e12, 2),
            "mfma_frac": round(pf_flops / (mean_pf * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_counters": mfma_counter_fields(load_mfma(), mean_pf),
        },
        "roofline": {
            "kernel": "gdn_prefill = intra_chunk_kernel then inter_chunk_kernel (mean duration "
                      "of one call over back-to-back calls, HIP events on the stream)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": pf_bytes,
            "algorithmic_bytes_note": "q, k, v, g, beta read and o, state_out written once "
                                      "(24,832 B/token + 2 MiB); the zero start state is passed "
                                      "as NULL, so no state_in read is counted (a nonzero "
                                      "state_in adds 2 MiB)",
            "achievable_copy_gbs": round(copy_gbs, 1),
            "frac_of_copy": round(achieved / copy_gbs, 4),
        },
        "decode": {
            "us_per_token_looped": round(float(t_dec.mean()), 2),
            "us_per_layer_looped": round(dec_layer_us, 3),
            "hbm_gbs_looped": round(dec_gbs_loop, 1),
            "us_per_token_graph": round(dec_g_us, 2),
            "us_per_layer_graph": round(dec_g_us / LAYERS, 3),
            "hbm_gbs_graph": round(dec_gbs_g, 1),
            "us_per_token_batched": round(dec_b_us, 2),
            "hbm_gbs_batched": round(dec_gbs_b, 1),
            "us_per_token_layers": round(dec_l_us, 2),
            "hbm_gbs_layers": round(dec_gbs_l, 1),
            "roofline": {"kernel": "decode_layers_kernel, one launch over a pointer table of the 30 "
                                   "separately allocated layers (gdn_decode_step_layers)",
                         "bound": "hbm", "achieved": round(dec_gbs_l, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(dec_gbs_l / HBM_PEAK_GBS, 4),
                         "traffic": traffic_doc.get("decode_layers_L%d_bytes" % LAYERS) if traffic_doc else None,
                         "algorithmic_bytes_per_launch": dec_bytes_b},
            "roofline_batched": {"kernel": "decode_kernel, one launch over the 30 layers stored back "
                                           "to back (B=30)",
                                 "bound": "hbm", "achieved": round(dec_gbs_b, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(dec_gbs_b / HBM_PEAK_GBS, 4),
                                 "traffic": traffic_doc.get("decode_L%d_bytes" % LAYERS) if traffic_doc else None},
        },
    }

    if not args.no_cpu_baseline:
        # The oracle and the GPU prefill alternate within each round, in alternating order
        # (GPU then oracle in even rounds, oracle then GPU in odd ones), until about
        # CPU_BASELINE_S seconds of oracle work are done: background load and clock drift then
        # bias neither leg.
        from oracle import gdn_oracle as orc
        try:
            ncpu = len(os.sched_getaffinity(0))
        except AttributeError:
            ncpu = os.cpu_count() or 1
        threads = args.cpu_threads or ncpu
        f = lambda t: t.float().numpy()  # noqa: E731
        qa, ka, va, ga, ba = (f(host[k]) for k in ("q", "k", "v", "g", "beta"))
        cpu_runs, gpu_alt = [], []
        r = 0
        while sum(cpu_runs) < CPU_BASELINE_S or r < 2:
            legs = ("gpu", "cpu") if r % 2 == 0 else ("cpu", "gpu")
            for leg in legs:
                if leg == "cpu":
                    c0 = time.perf_counter()
                    o_ref, s_ref = orc.seq(qa, ka, va, ga, ba, nthreads=threads, rows_per_item=8)
                    cpu_runs.append(time.perf_counter() - c0)
                else:
                    scratch.fill_(r & 0xFF)
                    a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    check(lib.gdn_prefill(*PF[0]), "gdn_prefill")
                    b2.record(stream)
                    torch.cuda.synchronize()
                    gpu_alt.append(a.elapsed_time(b2) * 1e3)
            r += 1
        cpu_s = float(np.mean(cpu_runs))
        # one thread on a bounded sample: 2 of the 32 value heads, scaled to the workload
        c1 = time.perf_counter()
        orc.seq(qa, ka, va, ga, ba, pairs=[(0, 0), (0, 1)], nthreads=1, rows_per_item=8)
        one_s = (time.perf_counter() - c1) * Hv / 2
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as fh:
                cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
        except OSError:
            pass
        o_gpu = sets[0]["o"].float().cpu().numpy()
        s_gpu = sets[0]["state_out"].cpu().numpy()
        err = lambda x, r_: float(np.max(np.abs(x - r_)) / np.max(np.abs(r_)))  # noqa: E731
        out["cpu_baseline"] = {"value": round(T / cpu_s, 1), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the full prefill workload (T={T}, all {Hv} value heads), "
                                         f"fp64 token-by-token scan on {threads} threads, "
                                         f"{len(cpu_runs)} runs ({sum(cpu_runs):.1f} s) alternated "
                                         f"with {len(gpu_alt)} cold GPU prefill calls, the order "
                                         f"of the two legs swapped every round",
                               "gpu_us_alternated": round(float(np.mean(gpu_alt)), 2),
                               "single_thread_value": round(T / one_s, 1),
                               "single_thread_sample": f"value heads 0 and 1 of the same workload on "
                                                       f"1 thread, scaled by {Hv // 2}",
                               "cpu_model": cpu_model, "host_cpus": ncpu}
        out["parity_vs_oracle"] = {"o": err(o_gpu, o_ref), "state": err(s_gpu, s_ref),
                                   "tol_o": 2e-2, "tol_state": 1e-2}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
