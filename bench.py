"""Benchmark of the fused attention forward pass (fa_fwd) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

One step is one fa_fwd call over the whole workload (all query rows of all
heads) with Q, K, V already resident in device memory.  W untimed warm-up
steps are followed by K timed steps between two device synchronisations; the
kernel's own average duration is taken from HIP events recorded on the
stream the kernel is queued on.  Prints one JSON line.

Clock settling: an idle MI355X starts a burst of work at a low graphics
clock and needs a few tens of milliseconds of sustained load to reach the
clock its power limit allows (at C4 the first ~20 launches take 2.8 -> 2.03
ms, the rest 2.00 ms).  So after the W warm-up steps the same step keeps
running, untimed, until --settle-ms of wall time has passed since the first
warm-up step (default 1500 ms, 0 turns it off); the line reports how many
such steps ran ("settle").  The timed region is still exactly K steps.  The
graphics clock of each XCD and the socket power, read from the driver's
metrics table (amdsmi) right after the timed steps, go in "gpu_state".

Default workload: B=1, H=32, N=16384, d=128, bf16, causal, with 1% of the Q
and K rows amplified x8.  Throughput counts 4*B*H*N^2*d FLOPs, halved for
causal.  Also reported:
  roofline      achieved TFLOP/s of the kernel against the published bf16
                dense matrix-core peak of MI355X (2.5 PFLOP/s), and the HBM
                bytes per launch measured with rocprofv3 counters when the
                committed counter summary matches the current kernel source;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload's query rows, on this host's cores.

--splitkv runs the workload through fa_fwd_splitkv (keys cut into the
library's suggested number of chunks, then merged) instead of fa_fwd.
--decode NK times single-query decoding instead: B=1, H=32, d=128, one
query row against NK keys through fa_fwd_splitkv, reported as GB/s of K/V
read (the path is bound by HBM there).
--hkv HKV gives K/V only HKV heads (grouped-query attention through
fa_fwd_gqa; query head h reads K/V head h / (H/HKV)): with --decode the
K/V bytes shrink by H/HKV; with a workload its K/V keep their first HKV
heads (FLOPs unchanged).

--bwd times the backward pass (fa_bwd) of the workload instead, with O and
LSE from one fa_fwd call and dO drawn N(0,1) (seed 1000*cfg + 6); FLOPs are
counted as 2.5x the forward's (five N^2 d products, causal halved; the
kernels compute seven, recomputing S and dP for dQ).

--fp8 times the fp8 forward (fa_fwd_fp8) of the workload, with Q, K and V
quantized to the MX E4M3 block format beforehand (fa_quantize_qk_fp8,
fa_quantize_v_fp8; their time is reported as quantize_ms, outside the
step); FLOPs as for the bf16 forward, peak the dense fp8 matrix-core peak.

--copy-bytes S runs only a plain device-to-device copy of S bytes (used to
calibrate the FETCH_SIZE / WRITE_SIZE counters) and exits.

--summarize DIR turns the raw rocprofv3 output of one profiling session
(see PROFILE_STEPS below; no GPU needed) into the text summaries under
profiles/ that this script and the documentation quote.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix-core peak (published)
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 matrix-core peak (published)
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector peak (published)
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E bandwidth (published)
PEAK_CLOCK_MHZ = 2400.0         # the engine clock the published peaks assume
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_traffic.json")
# the sources that decide the forward kernels' code and launch (the entry
# points' argument checks in fa_api.cpp do not change what runs)
KERNEL_SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_device.h", "fa_internal.h"]
# the same for the backward and fp8 kernels, whose summaries carry the hash
# of their own sources
BWD_SOURCES = ["fa_bwd_bf16.hip", "fa_device.h", "fa_internal.h"]
FP8_SOURCES = ["fa_fp8.hip", "fa_device.h", "fa_internal.h"]


def kernel_source_hash(names=None):
    h = hashlib.sha256()
    for name in names or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "io_aware_softmax_fwd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _source_note(names):
    """'kernel source HASH of FILES' for a summary header."""
    return "kernel source %s of %s" % (kernel_source_hash(names), ", ".join(names))


def _traffic_table():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    return t if isinstance(t, dict) else {}


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed counter summary, or None if it
    is missing, has no entry for this workload, or was taken on different
    kernel source."""
    t = _traffic_table().get(workload_name)
    if not t or t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def io_models(w):
    """HBM bytes of one launch under the accounting of the IO argument:
    the algorithmic minimum (Q, K, V read once, O written once, LSE), the
    standard three-pass attention's 4N^2 + 4Nd elements per head (S written
    and read, P written and read, plus Q, K, V, O), the tiled pass's
    8 N^2 d^2 / M elements per head for an on-chip memory of M elements
    (aiqz.cc Flash Attention IO article, IO complexity section; notes page,
    sections 3.1 and 3.2), here M = 160 KB of LDS, and this kernel's own
    model: every 128-row query tile reads the K and V it needs once (only
    keys up to the diagonal when causal)."""
    e = w.elem_bytes
    heads = w.B * w.H
    m_elems = 160 * 1024 // e
    tiles = -(-w.N // 128)
    if w.causal:
        kv_keys = sum(min(w.N, 128 * (t + 1)) for t in range(tiles))
    else:
        kv_keys = tiles * w.N
    return {"algorithmic": w.algorithmic_bytes,
            "standard_4N2_4Nd": heads * (4 * w.N * w.N + 4 * w.N * w.d) * e,
            "tiled_8N2d2_over_M": heads * 8 * w.N * w.N * w.d * w.d / m_elems * e,
            "kv_per_query_tile": heads * (2 * kv_keys * w.d * e + 2 * w.N * w.d * e + 4 * w.N),
            "lds_bytes_M": 160 * 1024}


def cpu_baseline(x, w, target_s=15.0):
    """Time the fp64 oracle on sampled query rows of the workload (x holds
    its q, k, v; k and v may carry fewer heads than q)."""
    import oracle
    rng = np.random.default_rng(12345)
    total_rows = w.B * w.H * w.N
    n_keys = lambda r: (r % w.N) + 1 if w.causal else w.N   # noqa: E731
    # warm the thread pool, calibrate on a small sample, then size the timed
    # sample to about target_s seconds
    warm = np.arange(16, dtype=np.int64)
    oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal, rows=warm)
    rows = np.sort(rng.choice(total_rows, size=512, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal, rows=rows)
    t_cal = time.perf_counter() - t0
    n = int(min(total_rows, max(512, 512 * target_s / max(t_cal, 1e-6))))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attention_c(x["q"], x["k"], x["v"], w.scale, w.causal, rows=rows)
    dt = time.perf_counter() - t0
    flops = float(sum(4.0 * n_keys(int(r)) * w.d for r in rows))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "%d random query rows of the same workload (fp64 C oracle, %.1f s, "
                      "%.3g FLOPs counted as 4*keys*d per row)" % (n, dt, flops)}


def copy_calibration(nbytes):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 5}))


def run_untimed(step, sync, warmup, settle_ms):
    """W warm-up steps, then more untimed steps until settle_ms of wall time
    has passed since the first one; returns the number of settle steps."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    sync()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            step()
        n += 8
        sync()
    return n


def gpu_state():
    """Graphics clock of each XCD and socket power from the driver's metrics
    table (refreshed about once a second), or None where amdsmi is missing."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        clks = [int(c) for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 10000]
        pw = m.get("current_socket_power")
        amdsmi.amdsmi_shut_down()
        if not clks:
            return None
        return {"gfx_clock_mhz_per_xcd": clks, "gfx_clock_mhz_mean": round(float(np.mean(clks)), 1),
                "socket_power_w": pw if isinstance(pw, (int, float)) else None,
                "source": "amdsmi gpu metrics, read right after the timed steps"}
    except Exception:   # noqa: BLE001 - an absent or failing metrics reader leaves the field null
        return None


# The profiling session whose output --summarize reads.  Each step is run on
# the GPU host from the repository root with OUT set to an output folder and
# WL to the workload id (1..5); the steps whose command holds no --workload
# are the same for every workload (C4 shapes).
PROFILE_STEPS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/trace -o run "
             "-- python bench.py --workload $WL --settle-ms 0 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/fetch -o run "
             "-- python bench.py --workload $WL --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write -o run "
             "-- python bench.py --workload $WL --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/copy_fetch -o run "
                  "-- python bench.py --copy-bytes 268435456",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/copy_write -o run "
                  "-- python bench.py --copy-bytes 268435456",
    "sq": "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
          "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_WAIT_INST_LDS SQ_WAIT_ANY "
          "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d $OUT/sq -o run "
          "-- python bench.py --workload $WL --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline",
    "sq2": "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
           "SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE "
           "--output-format csv -d $OUT/sq2 -o run "
           "-- python bench.py --workload $WL --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline",
    "bwd_sq": "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
              "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_WAIT_INST_LDS SQ_WAIT_ANY "
              "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d $OUT/bwd_sq -o run "
              "-- python bench.py --bwd --steps 3 --warmup 1 --settle-ms 0",
    "bwd_sq2": "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
               "SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE "
               "--output-format csv -d $OUT/bwd_sq2 -o run "
               "-- python bench.py --bwd --steps 3 --warmup 1 --settle-ms 0",
    "fp8_sq": "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
              "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_WAIT_INST_LDS SQ_WAIT_ANY "
              "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d $OUT/fp8_sq -o run "
              "-- python bench.py --fp8 --steps 3 --warmup 1 --settle-ms 0",
    "fp8_sq2": "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
               "SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE "
               "--output-format csv -d $OUT/fp8_sq2 -o run "
               "-- python bench.py --fp8 --steps 3 --warmup 1 --settle-ms 0",
    "decode_gqa": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/decode_gqa -o run "
                  "-- python bench.py --decode 131072 --hkv 8",
    "decode_mha": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/decode_mha -o run "
                  "-- python bench.py --decode 131072",
    "decode_mqa": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/decode_mqa -o run "
                  "-- python bench.py --decode 131072 --hkv 1",
    "bwd": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/bwd -o run "
           "-- python bench.py --bwd",
    "fp8": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/fp8 -o run "
           "-- python bench.py --fp8",
    "gqa": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/gqa -o run "
           "-- python bench.py --hkv 8 --no-cpu-baseline",
}
# extra kernel-trace steps summarised kernel by kernel: step -> summary name
TRACE_ONLY = {"decode_gqa": "fa_fwd_gqa_decode_b1_h32_hkv8_nk131072_d128",
              "decode_mha": "fa_fwd_splitkv_decode_b1_h32_nk131072_d128",
              "decode_mqa": "fa_fwd_gqa_decode_b1_h32_hkv1_nk131072_d128",
              "bwd": "fa_bwd_bf16_n16k_d128_causal_amplified",
              "fp8": "fa_fwd_fp8_bf16_n16k_d128_causal_amplified",
              "gqa": "fa_fwd_gqa_hkv8_bf16_n16k_d128_causal_amplified"}
# sources whose hash a summary of another path carries (default: the
# forward kernels')
SUMMARY_SOURCES = {"fa_bwd_bf16_n16k_d128_causal_amplified": BWD_SOURCES,
                   "fa_fwd_fp8_bf16_n16k_d128_causal_amplified": FP8_SOURCES}
# counter steps of other paths, summarised kernel by kernel: summary name ->
# (steps, kernel-name key)
COUNTERS_ONLY = {"fa_bwd_bf16_n16k_d128_causal_amplified": (("bwd_sq", "bwd_sq2"), "fa::(anonymous namespace)::bwd_"),
                 "fa_fwd_fp8_bf16_n16k_d128_causal_amplified": (("fp8_sq", "fp8_sq2"), "fa::(anonymous namespace)::fwd_fp8")}
# the forward kernels of fa_fwd and fa_fwd_f32 (the summary's own kernel)
KERNEL_KEY = "fa::(anonymous namespace)::fwd_"
COPY_KEY = "copy"


def profile_command(step, wl):
    """The command of one profiling step for workload id wl, as run."""
    return PROFILE_STEPS[step].replace("$WL", str(wl))


def _counters(folder, key):
    """{counter: [per-dispatch totals]} for kernels whose name contains key."""
    per = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if key not in row["Kernel_Name"]:
                    continue
                d = per.setdefault(row["Counter_Name"], {})
                d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def _kernel_stats(folder, key):
    """Rows of the kernel-stats csv under folder whose kernel name contains key."""
    stats = glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        return []
    with open(stats[0]) as fh:
        return [row for row in csv.DictReader(fh) if key in row["Name"]]


def summarize(out_dir, workload_name, wl=4):
    """Write the profiles/ summaries of workload wl (named workload_name)
    from one profiling session's raw output; steps missing from out_dir are
    skipped.  The traffic entry is merged into TRAFFIC_FILE under the
    workload's name."""
    from io_aware_softmax_fwd_amd import workloads as W
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    src_hash = kernel_source_hash()
    avg_ns = None
    rows = _kernel_stats(os.path.join(out_dir, "trace"), KERNEL_KEY)
    if rows:
        lines = []
        for row in rows:
            if avg_ns is None:
                avg_ns = float(row["AverageNs"])
            lines.append("kernel: %s" % row["Name"])
            lines.append("calls=%s  average=%.1f us  min=%.1f us  max=%.1f us" % (
                row["Calls"], float(row["AverageNs"]) / 1e3, float(row["MinNs"]) / 1e3,
                float(row["MaxNs"]) / 1e3))
        with open(os.path.join(prof, "fa_fwd_bf16_%s_kernel_trace.txt" % workload_name), "w") as f:
            f.write("# rocprofv3 kernel trace, workload %s (kernel source %s)\n" % (workload_name, src_hash))
            f.write("# command: %s\n" % profile_command("trace", wl))
            f.write("\n".join(lines) + "\n")
    # HBM traffic, calibrated on a copy of known size
    rd = wr = None
    fetch = _counters(os.path.join(out_dir, "fetch"), KERNEL_KEY).get("FETCH_SIZE")
    write = _counters(os.path.join(out_dir, "write"), KERNEL_KEY).get("WRITE_SIZE")
    if fetch and write:
        cf = _counters(os.path.join(out_dir, "copy_fetch"), COPY_KEY)["FETCH_SIZE"]
        cw = _counters(os.path.join(out_dir, "copy_write"), COPY_KEY)["WRITE_SIZE"]
        copy_bytes = 268435456
        f_fetch = copy_bytes / (np.mean(cf) * 1024)
        f_write = copy_bytes / (np.mean(cw) * 1024)
        rd = float(np.mean(fetch)) * 1024 * f_fetch
        wr = float(np.mean(write)) * 1024 * f_write
        entry = {"workload": workload_name, "source_hash": src_hash,
                 "fetch_kib_per_launch": float(np.mean(fetch)), "write_kib_per_launch": float(np.mean(write)),
                 "copy_calibration": {"bytes": copy_bytes, "fetch_kib": float(np.mean(cf)),
                                      "write_kib": float(np.mean(cw)), "fetch_factor": f_fetch,
                                      "write_factor": f_write},
                 "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
                 "bytes_per_launch": rd + wr,
                 "commands": [profile_command(k, wl) for k in ("fetch", "write", "copy_fetch", "copy_write")]}
        w = W.WORKLOADS.get(wl)
        if w is not None and w.name == workload_name:
            models = io_models(w)
            entry["models_bytes_per_launch"] = models
            entry["measured_over_model"] = {k: (rd + wr) / v for k, v in models.items() if k != "lds_bytes_M"}
        if avg_ns:
            entry["kernel_avg_us"] = avg_ns / 1e3
            entry["measured_GBps"] = (rd + wr) / (avg_ns * 1e-9) / 1e9
        table = _traffic_table()
        table[workload_name] = entry
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
    # SQ counters
    sq = {}
    for part in ("sq", "sq2"):
        if os.path.isdir(os.path.join(out_dir, part)):
            for k, v in _counters(os.path.join(out_dir, part), KERNEL_KEY).items():
                sq[k] = float(np.mean(v))
    if sq:
        sq_lines = []
        gui = sq.get("GRBM_GUI_ACTIVE", 0.0) / 8.0          # summed over 8 XCDs
        for k in sorted(sq):
            sq_lines.append("%-28s %.4g" % (k, sq[k]))
        if gui:
            sq_lines.append("derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/XCD * 1024 SIMDs) = %.1f %%"
                            % (100 * sq.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (gui * 1024)))
            sq_lines.append("derived: VALU+MFMA co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / (GRBM_GUI_ACTIVE/XCD * 1024) = %.1f %%"
                            % (100 * sq.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / (gui * 1024)))
        if sq.get("SQ_INSTS_MFMA"):
            sq_lines.append("derived: non-MFMA VALU instructions per MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA = %.2f"
                            % ((sq.get("SQ_INSTS_VALU", 0) - sq["SQ_INSTS_MFMA"]) / sq["SQ_INSTS_MFMA"]))
        with open(os.path.join(prof, "fa_fwd_bf16_%s_counters.txt" % workload_name), "w") as f:
            f.write("# rocprofv3 counters per launch, workload %s (kernel source %s)\n" % (workload_name, src_hash))
            f.write("# commands:\n#   %s\n#   %s\n" % (profile_command("sq", wl), profile_command("sq2", wl)))
            f.write("\n".join(sq_lines) + "\n")
    # counters of other paths, per kernel
    for name, (steps_, key) in COUNTERS_ONLY.items():
        per_kernel = {}
        for part in steps_:
            for f in glob.glob(os.path.join(out_dir, part, "**", "*counter_collection.csv"), recursive=True):
                with open(f) as fh:
                    for row in csv.DictReader(fh):
                        if key not in row["Kernel_Name"]:
                            continue
                        kern = row["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
                        kern = kern.replace("void ", "")
                        # one reading per pass and dispatch (summed over the blocks
                        # it lists); a counter that both passes collect
                        # (GRBM_GUI_ACTIVE) is averaged over the passes
                        d = per_kernel.setdefault(kern, {}).setdefault(row["Counter_Name"], {})
                        at = (part, row["Dispatch_Id"])
                        d[at] = d.get(at, 0.0) + float(row["Counter_Value"])
        if not per_kernel:
            continue
        out = []
        for kern in sorted(per_kernel):
            c = {k: float(np.mean(list(v.values()))) for k, v in per_kernel[kern].items()}
            out.append("kernel: %s" % kern)
            out += ["  %-28s %.4g" % (k, c[k]) for k in sorted(c)]
            gui = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
            if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                out.append("  derived: MFMA busy = %.1f %%, VALU+MFMA co-issue = %.1f %%" % (
                    100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024),
                    100 * c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / (gui * 1024)))
            if c.get("SQ_INSTS_MFMA"):
                out.append("  derived: non-MFMA VALU instructions per MFMA = %.2f" % (
                    (c.get("SQ_INSTS_VALU", 0) - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"]))
        with open(os.path.join(prof, "%s_counters.txt" % name), "w") as f:
            f.write("# rocprofv3 counters per launch, per kernel, %s (%s)\n"
                    % (name, _source_note(SUMMARY_SOURCES.get(name, KERNEL_SOURCES))))
            f.write("# commands:\n" + "".join("#   %s\n" % PROFILE_STEPS[p] for p in steps_))
            f.write("\n".join(out) + "\n")
    # kernel-only traces of other calls (every kernel of the call)
    for step, name in TRACE_ONLY.items():
        st = _kernel_stats(os.path.join(out_dir, step), "fa::")
        if not st:
            continue
        out = ["kernel: %s\ncalls=%s  average=%.2f us  min=%.2f us  max=%.2f us" % (
            row["Name"], row["Calls"], float(row["AverageNs"]) / 1e3,
            float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3) for row in st]
        with open(os.path.join(prof, "%s_kernel_trace.txt" % name), "w") as f:
            f.write("# rocprofv3 kernel trace, %s (%s)\n" % (name, _source_note(SUMMARY_SOURCES.get(name, KERNEL_SOURCES))))
            f.write("# command: %s\n" % PROFILE_STEPS[step])
            f.write("\n".join(out) + "\n")
    print(json.dumps({"kernel_avg_us": avg_ns / 1e3 if avg_ns else None,
                      "traffic_bytes": (rd + wr) if rd is not None else None, "read": rd, "write": wr}))


def decode_bench(fa, args):
    """One query row per head against NK keys: the K/V read dominates."""
    import torch
    dev = torch.device("cuda:0")
    B, H, d, nk = 1, 32, 128, args.decode
    hkv = args.hkv or H
    g = torch.Generator(device=dev).manual_seed(5)
    q = torch.randn((B, H, 1, d), device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn((B, hkv, nk, d), device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn((B, hkv, nk, d), device=dev, generator=g).to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    scale = float(1 / np.sqrt(d))
    if args.hkv:
        f = fa.fa_fwd_gqa
        splits = fa.fa_fwd_gqa_num_splits(B, H, hkv, 1, nk, 1, cus)
    else:
        f = fa.fa_fwd_splitkv
        splits = fa.fa_fwd_splitkv_num_splits(B, H, 1, nk, cus)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, 1, d, splits), dtype=torch.uint8, device=dev)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    tail = (1, nk, d, scale, 1, splits, ws.data_ptr(), ws.numel(), stream.cuda_stream)
    a = ptrs + ((B, H, hkv) if args.hkv else (B, H)) + tail
    def step():
        st = f(*a)
        if st != 0:
            raise fa.FaError(st, f.__name__)

    settled = run_untimed(step, torch.cuda.synchronize, args.warmup, args.settle_ms)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        f(*a)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    kv_bytes = 2 * B * hkv * nk * d * 2
    print(json.dumps({"metric": "decode K/V read GB/s (1 query row, causal, %s)" % f.__name__,
                      "value": round(kv_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                      "ms_per_step": round(ms, 4), "steps": args.steps, "warmup": args.warmup,
                      "settle": {"ms": args.settle_ms, "steps": settled},
                      "config": {"workload": "decode", "B": B, "H": H, "Hkv": hkv, "Nq": 1,
                                 "Nk": nk, "d": d, "splits": splits},
                      "peak_hbm_GBps": 8000}), flush=True)


def bwd_bench(fa, args, w, x):
    """Time fa_bwd on the workload (fa_bwd_gqa with --hkv: K and V keep the
    workload's first HKV heads); returns the JSON line."""
    import torch
    dev = torch.device("cuda:0")

    from io_aware_softmax_fwd_amd import workloads as W

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    rng = np.random.default_rng(1000 * w.cfg + 6)
    g = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    hkv = args.hkv or w.H
    q, k, v = up(x["q_bits"]), up(x["k_bits"]), up(x["v_bits"])
    k, v = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
    dO = up(W.bf16_bits_rne(g))
    o, lse = fa.fwd_gqa(q, k, v, scale=w.scale, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_gqa_workspace_size(w.B, w.H, hkv, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    heads = (w.B, w.H, hkv) if args.hkv else (w.B, w.H)
    a = ((q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(), lse.data_ptr(),
          dq.data_ptr(), dk.data_ptr(), dv.data_ptr()) + heads +
         (w.N, w.d, w.scale, int(w.causal), ws.data_ptr(), ws.numel(), stream.cuda_stream))
    call = fa.fa_bwd_gqa if args.hkv else fa.fa_bwd

    def step():
        st = call(*a)
        if st != 0:
            raise fa.FaError(st, call.__name__)

    settled = run_untimed(step, torch.cuda.synchronize, args.warmup, args.settle_ms)
    for t in (dq, dk, dv):
        if not torch.isfinite(t.float()).all():
            raise RuntimeError("non-finite gradient")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call(*a)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = 2.5 * w.flops
    return {"metric": "attention backward TFLOP/s (2.5x forward FLOPs: 5 N^2 d products, causal halved)",
            "value": round(flops / (wall / args.steps) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
            "settle": {"ms": args.settle_ms, "steps": settled}, "gpu_state": gpu_state(),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) draws, bf16-rounded)",
            "config": {"workload": w.name + "_bwd" + ("_hkv%d" % hkv if args.hkv else ""), "B": w.B,
                       "H": w.H, "Hkv": hkv, "N": w.N, "d": w.d, "causal": w.causal, "flops": flops,
                       "entry_point": "fa_bwd_gqa" if args.hkv else "fa_bwd"},
            "roofline": {"bound": "mfma", "achieved": round(flops / (ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": None, "kernel_ms": round(ms, 4),
                         "executed_flops": 3.5 * w.flops}}


def fp8_bench(fa, args, w, x):
    """Time fa_fwd_fp8 on the workload's quantized inputs (fa_fwd_fp8_gqa with
    --hkv: K and V keep the workload's first HKV heads); returns the JSON line."""
    import torch
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    hkv = args.hkv or w.H
    q, k, v = up(x["q_bits"]), up(x["k_bits"]), up(x["v_bits"])
    k, v = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    q8, qs = fa.quantize_qk_fp8(q)
    k8, ks = fa.quantize_qk_fp8(k)
    v8t, vs = fa.quantize_v_fp8(v)
    ev[1].record(stream)
    torch.cuda.synchronize()
    quant_ms = ev[0].elapsed_time(ev[1])
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    heads = (w.B, w.H, hkv) if args.hkv else (w.B, w.H)
    a = ((q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(), v8t.data_ptr(), vs.data_ptr(),
          o.data_ptr(), lse.data_ptr()) + heads + (w.N, w.d, w.scale, int(w.causal), stream.cuda_stream))
    call = fa.fa_fwd_fp8_gqa if args.hkv else fa.fa_fwd_fp8

    def step():
        st = call(*a)
        if st != 0:
            raise fa.FaError(st, call.__name__)

    settled = run_untimed(step, torch.cuda.synchronize, args.warmup, args.settle_ms)
    if not (torch.isfinite(lse).all() and torch.isfinite(o.float()).all()):
        raise RuntimeError("non-finite output")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call(*a)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    ach = w.flops / (ms * 1e-3) / 1e12
    return {"metric": "fp8 fwd attention TFLOP/s (4BHN^2d, causal halved), MX E4M3 inputs resident",
            "value": round(w.flops / (wall / args.steps) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
            "settle": {"ms": args.settle_ms, "steps": settled}, "gpu_state": gpu_state(),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
            "data": "synthetic (seeded N(0,1) draws, bf16-rounded, then MX E4M3 block-quantized)",
            "config": {"workload": w.name + "_fp8" + ("_hkv%d" % hkv if args.hkv else ""), "B": w.B,
                       "H": w.H, "Hkv": hkv, "N": w.N, "d": w.d, "causal": w.causal, "flops": w.flops,
                       "entry_point": "fa_fwd_fp8_gqa" if args.hkv else "fa_fwd_fp8",
                       "quantize_ms": round(quant_ms, 4)},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None,
                         "kernel_ms": round(ms, 4)}}


def launch_distribution(step, stream, n):
    """Median and minimum of n single launches, each bracketed by events on
    the launch stream (after the timed steps, so they do not perturb them).
    No L2 flush between launches: the large workloads' inputs exceed the L2."""
    import torch
    if n < 1:
        return None
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    return {"n": n, "median": round(t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), 4),
            "min": round(t[0], 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", type=int, default=4, help="workload id 1..5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--summarize", metavar="DIR", default=None)
    ap.add_argument("--splitkv", action="store_true")
    ap.add_argument("--decode", type=int, default=0, metavar="NK")
    ap.add_argument("--hkv", type=int, default=0, metavar="HKV")
    ap.add_argument("--bwd", action="store_true")
    ap.add_argument("--fp8", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="keep running untimed steps after the warm-up until this much wall time "
                         "has passed since the first warm-up step (0: off)")
    args = ap.parse_args()

    if args.summarize:
        from io_aware_softmax_fwd_amd import workloads as W
        summarize(args.summarize, W.WORKLOADS[args.workload].name, args.workload)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only; the forward pass shards by "
              "(batch, head) with no communication, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return

    import io_aware_softmax_fwd_amd as fa
    from io_aware_softmax_fwd_amd import workloads as W

    if args.decode:
        decode_bench(fa, args)
        return

    w = W.WORKLOADS[args.workload]
    x = W.make_inputs(w)
    dev = torch.device("cuda:0")
    if args.bwd:
        if w.dtype != "bf16":
            raise SystemExit("--bwd needs a bf16 workload")
        print(json.dumps(bwd_bench(fa, args, w, x)), flush=True)
        return
    if args.fp8:
        if w.dtype != "bf16":
            raise SystemExit("--fp8 needs a bf16 workload")
        print(json.dumps(fp8_bench(fa, args, w, x)), flush=True)
        return
    hkv = args.hkv or w.H
    if args.hkv:
        if w.dtype != "bf16" or w.H % hkv != 0:
            raise SystemExit("--hkv needs a bf16 workload and HKV dividing its H")
        for name in ("k", "v"):
            x[name] = np.ascontiguousarray(x[name][:, :hkv])
            x[name + "_bits"] = np.ascontiguousarray(x[name + "_bits"][:, :hkv])

    def up(name):
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    q, k, v = up("q"), up("k"), up("v")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    f = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32
    call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 w.B, w.H, w.N, w.d, w.scale, int(w.causal), stream.cuda_stream)

    if args.hkv:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        splits = (fa.fa_fwd_gqa_num_splits(w.B, w.H, hkv, w.N, w.N, int(w.causal), cus)
                  if args.splitkv else 1)
        ws = torch.empty(max(1, fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.N, w.d, splits)),
                         dtype=torch.uint8, device=dev)
        f = fa.fa_fwd_gqa
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, hkv, w.N, w.N, w.d, w.scale, int(w.causal), splits, ws.data_ptr(),
                     ws.numel(), stream.cuda_stream)
    elif args.splitkv:
        if w.dtype != "bf16":
            raise SystemExit("--splitkv needs a bf16 workload")
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        splits = fa.fa_fwd_splitkv_num_splits(w.B, w.H, w.N, w.N, cus)
        ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.N, w.d, splits),
                         dtype=torch.uint8, device=dev)
        f = fa.fa_fwd_splitkv
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.N, w.N, w.d, w.scale, int(w.causal), splits, ws.data_ptr(),
                     ws.numel(), stream.cuda_stream)

    # the library's own ctypes entry point, without the wrapper's lookup: at
    # C2's ~10 us per launch the Python side of a call is not negligible
    raw = getattr(fa.load(), f.__name__)

    def step():
        st = raw(*call_args)
        if st != 0:
            raise fa.FaError(st, f.__name__)

    settled = run_untimed(step, torch.cuda.synchronize, args.warmup, args.settle_ms)
    if not (torch.isfinite(lse).all() and torch.isfinite(o.float()).all()):
        raise RuntimeError("non-finite output")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    state = gpu_state()
    per_launch = launch_distribution(step, stream, min(args.steps, 100))

    ms_per_step = wall * 1e3 / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (kernel_ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name) if not (args.hkv or args.splitkv) else None
    n_rows = w.B * w.H * w.N
    alg_bytes = (w.algorithmic_bytes if not args.hkv else
                 2 * n_rows * w.d * 2 + 2 * w.B * hkv * w.N * w.d * 2 + 4 * n_rows)
    # C1 (fp32) runs on the vector ALUs: its roof is the fp32 vector peak
    bound, peak = ("mfma", PEAK_BF16_TFLOPS) if w.dtype == "bf16" else ("alu", PEAK_FP32_VECTOR_TFLOPS)
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel_ms": round(kernel_ms, 4),
            "algorithmic_bytes": alg_bytes, "per_launch_ms": per_launch, "l2_flush": False}
    if state and state.get("gfx_clock_mhz_mean"):
        # the same fraction against the peak scaled to the clock the run had
        roof["frac_at_measured_clock"] = round(achieved / (peak * state["gfx_clock_mhz_mean"] / PEAK_CLOCK_MHZ), 4)
    hbm = {"algorithmic_bytes": alg_bytes,
           "algorithmic_GBps": round(alg_bytes / (kernel_ms * 1e-3) / 1e9, 1),
           "measured_bytes": traffic,
           "measured_GBps": round(traffic / (kernel_ms * 1e-3) / 1e9, 1) if traffic else None,
           "peak_GBps": PEAK_HBM_GBPS}
    line = {
        "metric": "fwd attention TFLOP/s (4BHN^2d, causal halved) + % bf16 MFMA peak, N=16K d=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settled},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) draws, bf16-rounded)",
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name + ("_hkv%d" % hkv if args.hkv else ""), "B": w.B, "H": w.H,
                   "Hkv": hkv, "N": w.N, "d": w.d, "causal": w.causal,
                   "amplified_rows": w.amplify, "flops": w.flops, "entry_point": f.__name__},
        "roofline": roof,
        "hbm": hbm,
        "gpu_state": state,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
