"""Throughput of causal attention forward + backward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of synthetic input
already resident in HBM: attn_fwd then attn_bwd, on one HIP stream. W untimed
steps, then K timed steps between two device synchronisations (HIP events on
that stream bracket the K steps). A second timed pass launches each kernel
of the step K times back to back between two HIP events, in five blocks
interleaved across the kernels, through attn_fwd and the backward's two
stage entry points (attn_bwd_dq_preprocess then attn_bwd_dkdv: exactly what
attn_bwd launches), which gives each kernel's average duration without
slowing the first pass.

Prints one JSON line. ``value`` is the counted causal FLOP rate of the whole
step (forward 2*B*H*T^2*d, backward 2.5 times that); ``roofline`` describes
the kernel with the longest average duration; ``cpu_baseline`` is the float64
CPU oracle timed on a bounded sample of heads of the same workload;
``unfused`` times the materialising path (attn_fwd_unfused + attn_bwd_unfused,
the T x T matrices through HBM) on the same inputs, after the timed region,
and gives its ratio to the flash-attention step; ``decode`` times attn_decode
over a K/V cache larger than the Infinity Cache and reports its HBM rate
against the 8 TB/s roofline; ``block`` times the whole attention layer
(attn_block_fwd + attn_block_bwd: c_attn, attention, c_proj and their
gradients) at the same shape; ``fp8`` times the FP8 forward (attn_quantize_fp8
then attn_fwd_fp8) on the same qkv, against the FP8 MFMA peak, and reports
how far its output lies from the bf16 forward's. ``split_us`` gives the
median forward, backward and step times of the kernel-timing pass; ``cold``
times single steps after a 512 MiB scratch write (inputs out of every
cache); ``hbm`` is the step's algorithmic HBM rate; ``b64`` times the same
step at batch 64 and ``other_shapes`` at the 16-head and T = 2048 shapes;
``peaks`` measures the chip's sustained bf16 MFMA rate (and
the clock it ran at) and its HBM copy rate with the library's probes, next to
the specification peaks the roofline uses; they run before the warm-up steps,
so the chip has reached its sustained clocks when the timed region starts.
``tiny_f32`` times the float32 workload (launch-bound; reported only), and
``cpu_baseline.per_workload`` times the float64 oracle on every workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attention fwd+bwd TFLOP/s at GPT-2 124M shape; % of bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, AMD specification
FP8_PEAK_TFLOPS = 5033.2    # MI355X dense FP8 MFMA, AMD specification (twice bf16)
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, AMD specification
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "causal_flash_attention_amd", "csrc")

# Kernel -> (source file, bound, algorithmic FLOPs per launch in units of one
# causal T x T x d product per head, i.e. B*H*T^2*d), in launch order. The
# forward does two products (S = QK^T, O = PV); the backward's five counted
# products are credited one to dQ (dQ) and four to dK/dV (S, dP, dV, dK); the
# dQ kernel's recomputation of S and dP is executed but not credited, and so
# is its row-sum D = rowsum(dO * O) (the backward preprocess, done there).
KERNELS = {
    "attn_fwd": ("attn_fwd_bf16.hip", "mfma", 2.0),
    "attn_bwd_dq_preprocess": ("attn_bwd_bf16.hip", "mfma", 1.0),
    "attn_bwd_dkdv": ("attn_bwd_bf16.hip", "mfma", 4.0),
}
STAGES = list(KERNELS)
# Kernels outside the step whose HBM traffic is also recorded: the decode pass.
EXTRA_TRAFFIC = {"decode_partial": ("attn_decode_bf16.hip",),
                 "attn_quantize_fp8": ("attn_fp8.hip",),
                 "attn_fwd_fp8": ("attn_fp8.hip",),
                 "attn_quantize_bwd_fp8": ("attn_fp8_bwd.hip",),
                 "attn_bwd_fp8_dkdv": ("attn_fp8_bwd.hip",),
                 "attn_bwd_fp8_dq": ("attn_fp8_bwd.hip",)}


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # About 35 ms of warm-up at the headline shape: after an idle period the
    # first tens of milliseconds of load run at lower clocks.
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default=None, help="workload name (default: the headline)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true",
                   help="skip timing the materialising path")
    p.add_argument("--no-decode", action="store_true", help="skip timing decode")
    p.add_argument("--no-fp8", action="store_true", help="skip timing the FP8 forward")
    p.add_argument("--no-block", action="store_true", help="skip timing the attention layer")
    p.add_argument("--no-b64", action="store_true",
                   help="skip the step at batch 64 and at the other workload shapes")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the steps after a cache-clearing scratch write")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the MFMA and HBM peak probes")
    p.add_argument("--cpu-seconds-each", type=float, default=8.0,
                   help="seconds of the float64 oracle per workload in cpu_baseline.per_workload")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, run a plain 256 MiB device copy (for counter scaling)")
    p.add_argument("--write-profiles", action="store_true",
                   help="summarise rocprofv3 CSV output (--trace-dir, --fetch-dir, --write-dir) "
                        "into profiles/ and exit")
    p.add_argument("--trace-dir", default=None)
    p.add_argument("--fetch-dir", default=None)
    p.add_argument("--write-dir", default=None)
    p.add_argument("--mfma-dir", default=None,
                   help="rocprofv3 --pmc output with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, "
                        "SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE")
    p.add_argument("--mfma-command", default="", help="the command that produced --mfma-dir")
    p.add_argument("--wave-dirs", nargs="*", default=[],
                   help="rocprofv3 --pmc outputs that together hold the SQ_WAVE_CYCLES, "
                        "SQ_ACTIVE_INST_*, SQ_WAIT_*, SQ_WAVES and SQ_INSTS_* counters")
    p.add_argument("--wave-command", default="", help="the commands that produced --wave-dirs")
    p.add_argument("--profile-command", default="",
                   help="the commands that produced the CSVs, recorded in the summaries")
    return p.parse_args(argv)


# The generated programs the step's kernels run (their code is in these
# includes, so a change to one changes the kernel).
GENERATED = {"attn_fwd": ["attn_fwd_asm.inc"], "attn_bwd_dq_preprocess": ["attn_dq_asm.inc"],
             "attn_bwd_dkdv": ["attn_dkdv_asm.inc"]}


def kernel_digest(kernel: str) -> str:
    src = (KERNELS.get(kernel) or EXTRA_TRAFFIC[kernel])[0]
    return source_digest(os.path.join(CSRC, src),
                         [os.path.join(CSRC, f) for f in GENERATED.get(kernel, [])])


def source_digest(path: str, extra=()) -> str:
    h = hashlib.sha256()
    for f in sorted({os.path.join(CSRC, "attn_common.h"), path, *extra}):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none or the kernel's source changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_sha256_16:\s*(\w+)", text, re.M)
    m_val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not (m_src and m_val):
        return None
    if m_src.group(1) != kernel_digest(kernel):
        return None
    return float(m_val.group(1))


COPY_BYTES = 256 << 20  # the --copy-calibration copy


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _kernel_of(name: str):
    if "attn_bwd_dq_pre_bf16_asm_kernel" in name:  # what attn_bwd launches for dQ
        return "attn_bwd_dq_preprocess"
    if "attn_bwd_dq_bf16_kernel" in name:  # <true>: the fused form attn_bwd launches
        return "attn_bwd_dq_preprocess" if ("<true>" in name or "ILb1E" in name) else "attn_bwd_dq"
    m = re.search(r"gemm_bf16_kernel<(\d), (\d), (\d+), (true|false)>", name)
    if m:  # materialising path and attention block: orientations, tile width, output type
        ori = "".join("r" if x == "0" else "t" for x in m.group(1, 2))
        return f"gemm_{ori}{m.group(3)}_{'f32' if m.group(4) == 'true' else 'bf16'}"
    for k, tag in (("block_colsum", "colsum_partial_kernel"),
                   ("block_colsum_final", "colsum_final_kernel"),
                   ("block_sum_slabs", "sum_slabs_kernel"),
                   ("unfused_softmax_bwd", "softmax_bwd_rows_kernel"),
                   ("unfused_softmax", "softmax_rows_kernel"),
                   ("decode_partial", "decode_partial_kernel"),
                   ("decode_combine", "decode_combine_kernel"),
                   ("attn_fwd_fp8", "attn_fwd_fp8_kernel"),
                   ("attn_bwd_fp8_dq", "attn_bwd_fp8_dq_kernel"),
                   ("attn_bwd_fp8_dkdv", "attn_bwd_fp8_dkdv_kernel"),
                   ("attn_quantize_bwd_fp8", "attn_quantize_bwd_fp8_kernel"),
                   ("attn_quantize_fp8", "attn_quantize_fp8_kernel"),
                   ("peak_mfma", "peak_mfma_kernel"),
                   ("peak_copy", "peak_copy_kernel"),
                   ("peak_read", "peak_read_kernel")):
        if tag in name:
            return k
    for k, tag in (("attn_fwd", "attn_fwd_bf16_asm_kernel"), ("attn_fwd", "attn_fwd_bf16_kernel"),
                   ("attn_bwd_preprocess", "attn_bwd_pre_bf16_kernel"),
                   ("attn_bwd_dkdv", "attn_bwd_dkdv_bf16_asm_kernel"),
                   ("attn_bwd_dkdv", "attn_bwd_dkdv_bf16_kernel")):
        if tag in name:
            return k
    if "copyBuffer" in name:  # the runtime's device copy of --copy-calibration
        return "copy"
    return None


def _counter_means(d: str, counter: str):
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        k = _kernel_of(r.get("Kernel_Name", ""))
        if k:
            per.setdefault(k, []).append(float(r["Counter_Value"]))
    # The calibration is the 256 MiB copy, the largest runtime copy of the run
    # (small runtime copies, such as a scalar staged for the host, also occur).
    return {k: (max(v) if k == "copy" else sum(v) / len(v)) for k, v in per.items()}


N_SIMD = 1024  # 256 CUs x 4 SIMDs
N_XCD = 8


def write_mfma_profile(args, w) -> None:
    """MFMA utilisation per kernel from a counter pass: busy cycles summed
    over all SIMDs over (GPU-active cycles of one XCD x SIMDs), the derived
    MfmaUtil of rocprofv3, and the share of LDS-active cycles lost to bank
    conflicts. GRBM_GUI_ACTIVE comes summed over the eight XCDs."""
    per = {}
    for r in _csv_rows(args.mfma_dir, "counter_collection.csv"):
        k = _kernel_of(r["Kernel_Name"])
        if k is None:
            continue
        per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# MFMA utilisation per kernel, workload {w.name}, from rocprofv3 counters",
             f"# command: {args.mfma_command or '(see the bench.py --write-profiles invocation)'}",
             "# mfma_util = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs);",
             "# lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; means over the dispatches",
             "# kernel, dispatches, mfma_busy_cycles_per_simd, gui_active_cycles, mfma_util_percent, "
             "lds_conflict_percent"]
    order = list(KERNELS) + [k for k in sorted(per) if k not in KERNELS]
    for k in order:
        d = per.get(k)
        if not d or "SQ_VALU_MFMA_BUSY_CYCLES" not in d or "GRBM_GUI_ACTIVE" not in d:
            continue
        busy = statistics.mean(d["SQ_VALU_MFMA_BUSY_CYCLES"]) / N_SIMD
        active = statistics.mean(d["GRBM_GUI_ACTIVE"]) / N_XCD
        lds = statistics.mean(d.get("SQ_LDS_IDX_ACTIVE", [0.0]))
        conf = statistics.mean(d.get("SQ_LDS_BANK_CONFLICT", [0.0]))
        lines.append(f"{k}, {len(d['GRBM_GUI_ACTIVE'])}, {busy:.0f}, {active:.0f}, "
                     f"{100.0 * busy / active:.1f}, {100.0 * conf / lds if lds else 0.0:.1f}")
    path = os.path.join(PROFILE_DIR, f"mfma_util_{w.name}.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)


WAVE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                 "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
                 "SQ_ACTIVE_INST_MISC", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAVES",
                 "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS")


def write_wave_profile(args, w) -> None:
    """Where the waves of each kernel spend their cycles, from two counter
    passes: the share of wave-cycles spent issuing (by instruction type),
    waiting on a dependency (s_waitcnt, barrier) and ready but not issued
    (another wave held the unit), and the instructions issued per wave."""
    per = {}  # kernel -> counter -> per-dispatch totals
    for d in args.wave_dirs:
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            k = _kernel_of(r["Kernel_Name"])
            if k is None or r["Counter_Name"] not in WAVE_COUNTERS:
                continue
            key = (k, r["Dispatch_Id"], r["Counter_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (k, _, c), v in acc.items():
            per.setdefault(k, {}).setdefault(c, []).append(v)
    lines = [f"# Wave cycles per kernel, workload {w.name}, from rocprofv3 counters",
             f"# command: {args.wave_command or '(see the bench.py --write-profiles invocation)'}",
             "# shares of SQ_WAVE_CYCLES (medians over the dispatches): issuing = SQ_ACTIVE_INST_ANY "
             "(valu, salu, lds, vmem, misc: SQ_ACTIVE_INST_*), waiting = SQ_WAIT_ANY (s_waitcnt, "
             "barrier), not_issued = SQ_WAIT_INST_ANY (ready, another wave held the unit);",
             "# per_wave = SQ_INSTS_* / SQ_WAVES",
             "# kernel, dispatches, issuing, valu, salu, lds, vmem, misc, waiting, not_issued, "
             "valu_per_wave, mfma_per_wave, salu_per_wave, lds_per_wave"]
    order = list(KERNELS) + [k for k in sorted(per) if k not in KERNELS]
    for k in order:
        d = per.get(k)
        if not d or any(c not in d for c in WAVE_COUNTERS):
            continue
        m = {c: statistics.median(v) for c, v in d.items()}
        wc, nw = m["SQ_WAVE_CYCLES"], m["SQ_WAVES"]
        share = [m[c] / wc for c in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                                     "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS",
                                     "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_MISC", "SQ_WAIT_ANY",
                                     "SQ_WAIT_INST_ANY")]
        insts = [m[c] / nw for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
                                     "SQ_INSTS_LDS")]
        lines.append(f"{k}, {len(d['SQ_WAVES'])}, " + ", ".join(f"{x:.3f}" for x in share) + ", " +
                     ", ".join(f"{x:.0f}" for x in insts))
    path = os.path.join(PROFILE_DIR, f"wave_cycles_{w.name}.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)


def write_profiles(args, w) -> int:
    """Turn rocprofv3 CSV output into the text summaries under profiles/."""
    os.makedirs(PROFILE_DIR, exist_ok=True)
    cmd = args.profile_command or "(see the bench.py --write-profiles invocation)"
    if args.trace_dir:
        rows = _csv_rows(args.trace_dir, "kernel_stats.csv")
        trace = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                        for r in _csv_rows(args.trace_dir, "kernel_trace.csv")))
        per, b2b = {}, {}  # name -> dispatch durations (us): all, and back to back
        for i, (t0, t1, name) in enumerate(trace):
            dur = (t1 - t0) / 1e3
            per.setdefault(name, []).append(dur)
            if ((i > 0 and trace[i - 1][2] == name) or
                    (i + 1 < len(trace) and trace[i + 1][2] == name)):
                b2b.setdefault(name, []).append(dur)
        lines = [f"# rocprofv3 kernel-trace statistics, workload {w.name}",
                 f"# command: {cmd}",
                 "# back_to_back_avg_us: mean over the dispatches that directly follow or precede "
                 "a dispatch of the same kernel (bench.py's per-kernel pass, the regime of its "
                 "kernels_us and roofline)",
                 "# kernel, calls, average_us, median_us, min_us, max_us, share_percent, "
                 "back_to_back_calls, back_to_back_avg_us"]
        for r in rows:
            k = _kernel_of(r["Name"]) or r["Name"][:60]
            med = statistics.median(per[r["Name"]]) if per.get(r["Name"]) else float("nan")
            bb = b2b.get(r["Name"], [])
            bb_avg = f"{sum(bb) / len(bb):.2f}" if bb else "-"
            lines.append(f"{k}, {r['Calls']}, {float(r['AverageNs']) / 1e3:.2f}, {med:.2f}, "
                         f"{float(r['MinNs']) / 1e3:.2f}, {float(r['MaxNs']) / 1e3:.2f}, "
                         f"{float(r['Percentage']):.2f}, {len(bb)}, {bb_avg}")
        path = os.path.join(PROFILE_DIR, f"kernel_stats_{w.name}.txt")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(path)
    if args.mfma_dir:
        write_mfma_profile(args, w)
    if args.wave_dirs:
        write_wave_profile(args, w)
    if args.fetch_dir and args.write_dir:
        fetch = _counter_means(args.fetch_dir, "FETCH_SIZE")
        write = _counter_means(args.write_dir, "WRITE_SIZE")
        if "copy" not in fetch or "copy" not in write:
            raise SystemExit("the counter runs need --copy-calibration (a plain copy of known size)")
        f_fetch = COPY_BYTES / (fetch["copy"] * 1024.0)
        f_write = COPY_BYTES / (write["copy"] * 1024.0)
        for k in list(KERNELS) + list(EXTRA_TRAFFIC):
            if k not in fetch or k not in write:
                continue
            traffic = fetch[k] * 1024.0 * f_fetch + write[k] * 1024.0 * f_write
            text = "\n".join([
                f"# HBM traffic of {k} on workload {w.name}, from rocprofv3 counters",
                f"# command: {cmd}",
                f"source_sha256_16: {kernel_digest(k)}",
                f"fetch_kib_per_dispatch: {fetch[k]:.1f}",
                f"write_kib_per_dispatch: {write[k]:.1f}",
                f"copy_calibration: a {COPY_BYTES >> 20} MiB device copy reads FETCH_SIZE "
                f"{fetch['copy']:.1f} KiB and WRITE_SIZE {write['copy']:.1f} KiB per dispatch; "
                f"scale factors fetch {f_fetch:.4f}, write {f_write:.4f}",
                f"traffic_bytes_per_launch: {traffic:.6e}",
            ]) + "\n"
            path = os.path.join(PROFILE_DIR, f"{k}_{w.name}_hbm_traffic.txt")
            with open(path, "w") as fh:
                fh.write(text)
            print(path)
    return 0


def cpu_baseline(w, target_s: float):
    """Time the float64 oracle (forward + backward) on whole heads of the
    workload until about target_s seconds have passed."""
    import numpy as np

    import oracle
    from causal_flash_attention_amd import inputs as I

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    # inputs of batch row 0 only (the heads timed come from it)
    qkv, dout = I.attention_inputs(1, w.T, w.n_head, w.head_dim, w.dtype, w.qkv_std, w.dout_std, seed=0)
    q64, g64 = I.to_float64(qkv, w.dtype), I.to_float64(dout, w.dtype)
    D = w.head_dim
    done = 0
    t0 = time.perf_counter()
    while True:
        h = done % w.n_head
        q, k, v = oracle.split_packed_head(q64, 0, h, w.n_head, D)
        g = g64[0, :, h * D:(h + 1) * D]
        oracle.head_forward(q, k, v)
        oracle.head_backward(q, k, v, g)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s or done >= w.B * w.n_head:
            break
    flops = 7.0 * done * w.T * w.T * D
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} head passes of {w.name} (T={w.T}, d={D}; the {w.n_head} heads of batch "
                  f"row 0 in turn, {w.B * w.n_head} passes being the whole workload's count), "
                  f"float64 forward+backward materialising T x T per head, {el:.1f} s wall, "
                  f"counted 7*T^2*d FLOPs per head",
        "wall_s": el,
        "heads_timed": done,
        "cpu_model": model,
        "cpu_count": os.cpu_count(),
        "affinity_cpus": affinity,
    }


def cpu_baseline_all(target_s: float):
    """The float64 oracle on every workload: whole heads of each, up to about
    target_s seconds per workload (the whole workload when it fits)."""
    from causal_flash_attention_amd.workloads import WORKLOADS

    res = {}
    for wl in WORKLOADS:
        r = cpu_baseline(wl, target_s)
        heads_total = wl.B * wl.n_head
        heads_done = r["heads_timed"]
        res[wl.name] = {"dtype": wl.dtype, "heads_timed": heads_done, "heads_total": heads_total,
                        "wall_s": r["wall_s"], "counted_gflops": 1000.0 * r["value"],
                        "est_whole_workload_s": r["wall_s"] * heads_total / heads_done,
                        "blas_threads": r["cores"]}
    return res


def time_tiny_f32(stream, dev, n=200):
    """The float32 workload (B 1, T 64, 2 heads): attn_fwd_f32 + attn_bwd_f32
    per step, n steps between HIP events. At this size a step is a few
    launches' worth of latency, so the time is reported, not judged."""
    import numpy as np
    import torch

    from causal_flash_attention_amd import binding
    from causal_flash_attention_amd import inputs as I
    from causal_flash_attention_amd.workloads import BY_NAME

    w = BY_NAME["tiny_f32_b1_h2_t64"]
    B, T, H, D = w.B, w.T, w.n_head, w.head_dim
    qh, gh = I.attention_inputs(B, T, H, D, "f32", w.qkv_std, w.dout_std, seed=0)
    qkv = torch.from_numpy(np.ascontiguousarray(qh, dtype=np.float32)).to(dev)
    dout = torch.from_numpy(np.ascontiguousarray(gh, dtype=np.float32)).to(dev)
    out = torch.empty((B, T, H * D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dqkv = torch.empty_like(qkv)
    delta = torch.empty(binding.workspace_floats(B, T, H), dtype=torch.float32, device=dev)

    def step():
        binding.attn_fwd(qkv, out, lse, H, D, stream)
        binding.attn_bwd(dout, qkv, out, lse, dqkv, delta, H, D, stream)

    for _ in range(20):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / n
    return {"workload": w.name, "dtype": "f32", "us_per_step": us, "steps": n,
            "counted_gflops": w.counted_flops()["total"] / (us * 1e-6) / 1e9,
            "what": "launch-bound: time reported only, not judged against a roofline"}


def step_hbm_bytes(w) -> float:
    """Bytes the three kernels of a step must move at least once, with
    X = B*H*T*d elements and R = B*H*T rows: forward qkv + out + lse
    (8X + 4R); dQ with the preprocess q, k, v, dout, out, lse in and dQ plus
    the 40-byte workspace rows out (12X + 44R); dK/dV q, k, v, dout and the
    32-byte workspace terms in, dK and dV out (12X + 32R)."""
    X = float(w.B) * w.n_head * w.T * w.head_dim
    R = float(w.B) * w.n_head * w.T
    return 32.0 * X + 80.0 * R


def time_cold(step, stream, dev, n):
    """Steps timed one by one after a 512 MiB scratch write, which evicts the
    inputs from the caches (the 256 MB Infinity Cache included)."""
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    times = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(1000.0 * e0.elapsed_time(e1))
    del scratch
    return {"us_per_step": statistics.median(times), "steps": n, "scratch_mib": 512,
            "what": "median of single steps, each after a 512 MiB scratch write"}


def time_other_batch(w, stream, dev, K):
    """The same step on another workload: the GPT-2 124M layer at B = 64, and
    the 16-head (350M) and T = 2048, 25-head shapes."""
    import numpy as np
    import torch
    from causal_flash_attention_amd import binding
    from causal_flash_attention_amd import inputs as I
    B, T, H, D = w.B, w.T, w.n_head, w.head_dim
    qh, gh = I.attention_inputs(B, T, H, D, w.dtype, w.qkv_std, w.dout_std, seed=0)
    qkv = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).to(dev)
    dout = torch.from_numpy(gh.view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty((B, T, H * D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dqkv = torch.empty_like(qkv)
    delta = torch.empty(binding.workspace_floats(B, T, H), dtype=torch.float32, device=dev)

    def step():
        binding.attn_fwd(qkv, out, lse, H, D, stream)
        binding.attn_bwd(dout, qkv, out, lse, dqkv, delta, H, D, stream)

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / K
    tflops = w.counted_flops()["total"] / (us * 1e-6) / 1e12
    return {"workload": w.name, "us_per_step": us, "steps": K, "tflops": tflops,
            "pct_of_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS}


def measure_peaks(stream, dev):
    """The chip's sustained bf16 MFMA rate (attn_peak_mfma: register-only
    MFMA chains on every SIMD) with the clock it ran at, and its HBM copy
    rate (attn_peak_copy over 1 GiB, read + write bytes counted) and read rate
    (attn_peak_read over the same 1 GiB)."""
    import torch
    from causal_flash_attention_amd import binding
    n_wg, iters = 2048, 4096
    flops = binding.attn_peak_mfma_flops(n_wg, iters)
    out = torch.empty(256 * n_wg, dtype=torch.float32, device=dev)
    ticks = torch.empty(2 * n_wg, dtype=torch.int64, device=dev)
    # Sustained means after the clock has settled: the first milliseconds of
    # load after idle run at a lower clock (about 1.3 GHz within 3 ms against
    # about 1.9 GHz after 0.2 s under the attention kernels), so the probe
    # repeats for 0.2 s before the calls it times. This also puts the timed
    # steps, which follow, on a settled clock.
    t_end = time.time() + 0.2
    while True:
        binding.attn_peak_mfma(out, ticks, n_wg, iters, stream)
        torch.cuda.synchronize()
        if time.time() >= t_end:
            break
    rates = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        binding.attn_peak_mfma(out, ticks, n_wg, iters, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    t = ticks.view(n_wg, 2).cpu().double()
    clock_ghz = float((t[:, 0] / t[:, 1]).median()) * 0.1  # constant clock: 100 MHz
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        binding.attn_peak_copy(src, dst, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        binding.attn_peak_copy(src, dst, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    slots = torch.zeros(binding.lib().attn_peak_read_slots(), dtype=torch.int32, device=dev)
    for _ in range(3):
        binding.attn_peak_read(src, slots, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        binding.attn_peak_read(src, slots, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    read_gbs = float(nbytes) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, slots
    return {"mfma_bf16_tflops": max(rates), "mfma_clock_ghz": clock_ghz,
            "mfma_spec_tflops": BF16_PEAK_TFLOPS, "hbm_copy_gbs": copy_gbs,
            "hbm_read_gbs": read_gbs, "hbm_spec_gbs": HBM_PEAK_GBS,
            "what": "attn_peak_mfma (register-only bf16 32x32x16 MFMA chains, every SIMD), "
                    "attn_peak_copy (1 GiB device copy, read + write bytes) and attn_peak_read "
                    "(1 GiB read)"}


def time_unfused(w, qkv, dout, stream, K):
    """The materialising path on the same inputs: 5 untimed steps, then
    min(K, 20) steps between HIP events (fwd and bwd timed separately too)."""
    import torch

    from causal_flash_attention_amd import binding

    B, T, H, D = w.B, w.T, w.n_head, w.head_dim
    C = H * D
    dev = qkv.device
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    probs = torch.empty((B, H, T, binding.unfused_row_stride(T)), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.unfused_workspace_bytes(B, T, H), dtype=torch.uint8, device=dev)
    dqkv = torch.empty_like(qkv)

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        binding.attn_fwd_unfused(qkv, out, lse, probs, ws, H, D, stream)
        if evs:
            evs[1].record(stream)
        binding.attn_bwd_unfused(dout, qkv, probs, dqkv, ws, H, D, stream)
        if evs:
            evs[2].record(stream)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    n = min(K, 20)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for i in range(n):
        step(ev[i])
    torch.cuda.synchronize()
    total = sum(ev[i][0].elapsed_time(ev[i][2]) for i in range(n)) / n
    fwd = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(n)) / n
    flops = w.counted_flops()["total"]
    return {"ms_per_step": total, "fwd_ms": fwd, "bwd_ms": total - fwd, "steps": n,
            "counted_tflops": flops / (total * 1e-3) / 1e12,
            "what": "attn_fwd_unfused + attn_bwd_unfused: full T x T products, fp32 scores "
                    "and dP, bf16 P and dS through HBM"}


# Decode workload: GPT-2 124M heads, batch 64, 4096 cached positions in
# separate (B, T, C) caches: 805 MB of K and V per call, three times the
# 256 MB Infinity Cache, so repeated calls stream from HBM.
DECODE_B, DECODE_T, DECODE_H = 64, 4096, 12


def time_decode(stream, calls=50):
    import torch

    from causal_flash_attention_amd import binding

    B, T, H, D = DECODE_B, DECODE_T, DECODE_H, 64
    C = H * D
    g = torch.Generator(device="cuda").manual_seed(0)  # synthetic, seeded
    k = torch.randn((B, T, C), generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((B, T, C), generator=g, device="cuda", dtype=torch.bfloat16)
    q = torch.randn((B, C), generator=g, device="cuda", dtype=torch.bfloat16)
    out = torch.empty((B, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(binding.decode_workspace_floats(B, T, H), device="cuda")
    for _ in range(10):
        binding.attn_decode(q, k, v, out, lse, ws, T, H, D, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        binding.attn_decode(q, k, v, out, lse, ws, T, H, D, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / calls
    nbytes = 2.0 * B * T * C * 2  # K and V read once
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"decode B={B} T={T} n_head={H} head_dim={D}, separate K/V caches",
            "us_per_call": us, "calls": calls, "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS}}


def time_block(w, attn_step_us, stream, calls=50):
    """The attention layer around the fused attention, forward + backward,
    GPT-2 initialisation scale (weights and biases N(0, 0.02^2)), seeded."""
    import torch

    from causal_flash_attention_amd import binding

    B, T, H, D = w.B, w.T, w.n_head, w.head_dim
    C = H * D
    bf, dev = torch.bfloat16, "cuda"
    g = torch.Generator(device=dev).manual_seed(0)
    rnd = lambda *s, std=1.0: (torch.randn(s, generator=g, device=dev, dtype=torch.float32) * std).to(bf)  # noqa: E731
    x, dy = rnd(B, T, C), rnd(B, T, C)
    wa, ba, wp, bp = rnd(C, 3 * C, std=0.02), rnd(3 * C, std=0.02), rnd(C, C, std=0.02), rnd(C, std=0.02)
    qkv = torch.empty((B, T, 3 * C), dtype=bf, device=dev)
    att = torch.empty((B, T, C), dtype=bf, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    y = torch.empty((B, T, C), dtype=bf, device=dev)
    datt, dx = torch.empty_like(att), torch.empty_like(att)
    dqkv = torch.empty_like(qkv)
    dwa, dba = torch.empty((C, 3 * C), device=dev), torch.empty(3 * C, device=dev)
    dwp, dbp = torch.empty((C, C), device=dev), torch.empty(C, device=dev)
    ws = torch.empty(binding.block_workspace_bytes(B, T, H), dtype=torch.uint8, device=dev)

    def fwd():
        binding.attn_block_fwd(x, wa, ba, wp, bp, qkv, att, lse, y, H, D, stream)

    def bwd():
        binding.attn_block_bwd(dy, x, wa, wp, qkv, att, lse, datt, dqkv, dx, dwa, dba, dwp, dbp,
                               ws, H, D, stream)

    for _ in range(20):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    f_ms = b_ms = 0.0
    for _ in range(calls):
        ev[0].record(stream)
        fwd()
        ev[1].record(stream)
        bwd()
        ev[2].record(stream)
        torch.cuda.synchronize()
        f_ms += ev[0].elapsed_time(ev[1])
        b_ms += ev[1].elapsed_time(ev[2])
    f_us, b_us = 1000.0 * f_ms / calls, 1000.0 * b_ms / calls
    R = B * T
    lin = 2.0 * R * C * 3 * C + 2.0 * R * C * C     # c_attn + c_proj, forward
    attn = w.counted_flops()["total"]
    total = 3.0 * lin + attn                         # backward: data and weight gradients
    step_us = f_us + b_us
    lin_us = max(step_us - attn_step_us, 1e-3)       # linear maps and gradient sums
    lin_tf = 3.0 * lin / (lin_us * 1e-6) / 1e12
    return {"workload": f"{w.name} attention layer (c_attn, attention, c_proj), weights N(0, 0.02^2)",
            "fwd_us": f_us, "bwd_us": b_us, "step_us": step_us, "calls": calls,
            "counted_gflop": total / 1e9, "tflops": total / (step_us * 1e-6) / 1e12,
            "linear_us": lin_us, "linear_tflops": lin_tf,
            "linear_roofline": {"bound": "mfma", "achieved": lin_tf, "peak": BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": lin_tf / BF16_PEAK_TFLOPS,
                                "what": "the six products of c_attn and c_proj (forward, data and "
                                        "weight gradients) with the bias sums, timed as the layer "
                                        "step minus the attention step"}}


def time_fp8(w, qkv, out_bf16, fwd_bf16_us, stream, dout=None, dqkv_bf16=None, step_bf16_us=None,
             calls=100):
    """The FP8 forward on the step's qkv: quantize and forward timed apart and
    together; the forward's FLOP rate against the FP8 MFMA peak, the
    quantization's HBM rate (bf16 qkv read, FP8 buffer written)."""
    import torch

    from causal_flash_attention_amd import binding

    B, T, H, D = w.B, w.T, w.n_head, w.head_dim
    C = H * D
    nbuf = binding.fp8_buffer_bytes(B, T, H)
    buf = torch.empty(nbuf, dtype=torch.uint8, device="cuda")
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")

    def quant():
        binding.attn_quantize_fp8(qkv, buf, H, D, stream)

    def fwd():
        binding.attn_fwd_fp8(buf, out, lse, H, D, stream)

    def both():
        quant()
        fwd()

    def timed(fn):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / calls

    q_us, f_us, p_us = timed(quant), timed(fwd), timed(both)
    bwd_part = None
    if dout is not None:
        b8 = torch.empty(binding.fp8_bwd_buffer_bytes(B, T, H), dtype=torch.uint8, device="cuda")
        dqkv = torch.empty_like(qkv)

        def qbwd():
            binding.attn_quantize_bwd_fp8(dout, qkv, out, lse, b8, H, D, stream)

        def bwd():
            binding.attn_bwd_fp8(buf, b8, dqkv, H, D, stream)

        def step():
            quant()
            fwd()
            qbwd()
            bwd()

        qb_us, b_us, s_us = timed(qbwd), timed(bwd), timed(step)
        ref = dqkv_bf16.float()
        rel_g = float(torch.linalg.vector_norm(dqkv.float() - ref) / torch.linalg.vector_norm(ref))
        counted = w.counted_flops()
        bwd_part = {"quantize_bwd_us": qb_us, "bwd_us": b_us, "bwd_tflops": counted["bwd"] / (b_us * 1e-6) / 1e12,
                    "step_us": s_us, "step_tflops": counted["total"] / (s_us * 1e-6) / 1e12,
                    "step_speedup_vs_bf16": (step_bf16_us / s_us) if step_bf16_us else None,
                    "rel_l2_dqkv_vs_bf16": rel_g}
    fwd_flops = 2.0 * B * H * T * T * D  # S = QK^T and O = PV, causal halves counted
    tf = fwd_flops / (f_us * 1e-6) / 1e12
    qbytes = 3.0 * B * T * C * 2 + nbuf
    gbs = qbytes / (q_us * 1e-6) / 1e9
    ref = out_bf16.float()
    rel = float(torch.linalg.vector_norm(out.float() - ref) / torch.linalg.vector_norm(ref))
    res = {"workload": w.name, "quantize_us": q_us, "fwd_us": f_us, "pass_us": p_us,
            "calls": calls, "fwd_tflops": tf, "pass_tflops": fwd_flops / (p_us * 1e-6) / 1e12,
            "fwd_speedup_vs_bf16_fwd": fwd_bf16_us / f_us,
            "rel_l2_vs_bf16_fwd": rel,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / FP8_PEAK_TFLOPS,
                         "traffic": traffic_from_profile("attn_fwd_fp8", w.name),
                         "kernel": "attn_fwd_fp8"},
            "quantize_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                  "bytes_per_call": qbytes,
                                  "traffic": traffic_from_profile("attn_quantize_fp8", w.name)}}
    if bwd_part is not None:
        res["backward"] = bwd_part
    return res


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every (batch, head) is independent, so more GPUs would split the batch or the heads with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    from causal_flash_attention_amd.workloads import BY_NAME, HEADLINE

    w = BY_NAME[args.workload] if args.workload else HEADLINE
    if args.write_profiles:
        return write_profiles(args, w)

    import numpy as np
    import torch

    from causal_flash_attention_amd import binding
    from causal_flash_attention_amd import inputs as I

    if w.dtype != "bf16":
        raise SystemExit("the bench times the bf16 path")
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    B, T, H, D = w.B, w.T, w.n_head, w.head_dim
    C = H * D
    qkv_h, dout_h = I.attention_inputs(B, T, H, D, w.dtype, w.qkv_std, w.dout_std, seed=0)
    qkv = torch.from_numpy(qkv_h.view(np.int16)).view(torch.bfloat16).to(dev)
    dout = torch.from_numpy(dout_h.view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dqkv = torch.empty((B, T, 3 * C), dtype=torch.bfloat16, device=dev)
    delta = torch.empty(binding.workspace_floats(B, T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        binding.attn_fwd(qkv, out, lse, H, D, stream)
        binding.attn_bwd(dout, qkv, out, lse, dqkv, delta, H, D, stream)

    # The step's kernels one by one, through the stage entry points (exactly
    # what attn_fwd and attn_bwd launch); each call is idempotent.
    stages = {"attn_fwd": lambda: binding.attn_fwd(qkv, out, lse, H, D, stream),
              "attn_bwd_dq_preprocess": lambda: binding.attn_bwd_dq_preprocess(
                  dout, qkv, out, lse, dqkv, delta, H, D, stream),
              "attn_bwd_dkdv": lambda: binding.attn_bwd_dkdv(dout, qkv, delta, dqkv, H, D, stream)}
    assert list(stages) == STAGES

    # The chip's sustained peaks are measured first: about a second of full
    # load, which also brings the clocks to where they stay under sustained
    # load. After idle, the first tens of milliseconds of load run up to 25%
    # slower (measured: 203.8 against 162.9 us per step on one box with 5
    # and 200 warm-up steps), which would otherwise leak into a short timed
    # region.
    peaks = None if args.no_peaks else measure_peaks(stream, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps.
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / K

    # Kernel-timing region: each kernel of the step K times back to back
    # between two HIP events on the step's stream, in 5 blocks of K/5 with the
    # kernels interleaved block by block; the mean over all K launches and
    # the median over the blocks. (Events recorded between the kernels of
    # every step slow the kernels themselves by up to 10%, as rocprofv3's
    # per-dispatch durations show, so they are not used.)
    n_blk = 5
    per_blk = max(1, K // n_blk)
    blk_us = {name: [] for name in STAGES}
    torch.cuda.synchronize()
    for _ in range(n_blk):
        for name, fn in stages.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per_blk):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            blk_us[name].append(1000.0 * e0.elapsed_time(e1) / per_blk)
    kernel_us = {name: sum(v) / len(v) for name, v in blk_us.items()}
    split_us = {"fwd": statistics.median(blk_us["attn_fwd"]),
                "bwd": statistics.median(a + b for a, b in zip(blk_us["attn_bwd_dq_preprocess"],
                                                               blk_us["attn_bwd_dkdv"])),
                "kernels_sum": sum(statistics.median(v) for v in blk_us.values())}
    cold = None if args.no_cold else time_cold(step, stream, dev, min(K, 20))

    flops = w.counted_flops()
    tflops = flops["total"] / (ms_per_step * 1e-3) / 1e12
    unit_flops = float(B) * H * T * T * D  # one causal T x T x d product over all heads

    dom = max(STAGES, key=lambda n: kernel_us[n])
    _src, bound, units = KERNELS[dom]
    dur_s = kernel_us[dom] * 1e-6
    traffic = traffic_from_profile(dom, w.name)
    assert bound == "mfma"  # every kernel of the step is a causal contraction
    achieved = units * unit_flops / dur_s / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic,
            "kernel": dom}

    step_bytes = step_hbm_bytes(w)
    hbm = {"algorithmic_bytes": step_bytes, "gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
           "peak": HBM_PEAK_GBS,
           "what": "bytes each kernel of the step must read and write once (qkv, out, lse, dout, "
                   "dqkv and the backward workspace), over the step time"}
    hbm["frac"] = hbm["gbs"] / HBM_PEAK_GBS
    b64 = None if args.no_b64 else time_other_batch(BY_NAME["gpt2_124m_b64_t1024"], stream, dev,
                                                     min(K, 50))
    others = None if args.no_b64 else {
        n: time_other_batch(BY_NAME[n], stream, dev, min(K, 50))
        for n in ("gpt2_350m_b16_t1024", "gpt2_1p5b_style_b4_t2048_h25")}
    tiny = None if args.no_b64 else time_tiny_f32(stream, dev)

    unfused = None if args.no_unfused else time_unfused(w, qkv, dout, stream, K)
    decode = None if args.no_decode else time_decode(stream)
    block = None if args.no_block else time_block(w, ms_per_step * 1000.0, stream)
    if not args.no_fp8:
        attn_fwd_out = torch.empty((B, T, H * D), dtype=torch.bfloat16, device=dev)
        attn_fwd_lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        binding.attn_fwd(qkv, attn_fwd_out, attn_fwd_lse, H, D, stream)
        attn_dqkv = torch.empty_like(qkv)
        attn_delta = torch.empty_like(delta)
        binding.attn_bwd(dout, qkv, attn_fwd_out, attn_fwd_lse, attn_dqkv, attn_delta, H, D, stream)
        fp8 = time_fp8(w, qkv, attn_fwd_out, kernel_us["attn_fwd"], stream, dout=dout,
                       dqkv_bf16=attn_dqkv, step_bf16_us=ms_per_step * 1000.0)
    else:
        fp8 = None

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "n_head": H, "head_dim": D,
                   "causal": True, "qkv_std": w.qkv_std, "dout_std": w.dout_std,
                   "counted_gflop_per_step": flops["total"] / 1e9},
        "pct_of_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS,
        "kernels_us": kernel_us,
        "split_us": split_us,
        "hbm": hbm,
        "host_wall_s": wall,
        "roofline": roof,
    }
    if cold is not None:
        result["cold"] = cold
    if peaks is not None:
        result["peaks"] = peaks
        result["pct_of_measured_bf16_peak"] = 100.0 * tflops / peaks["mfma_bf16_tflops"]
    if b64 is not None:
        result["b64"] = b64
    if others is not None:
        result["other_shapes"] = others
    if tiny is not None:
        result["tiny_f32"] = tiny
    if unfused is not None:
        unfused["fa_speedup"] = unfused["ms_per_step"] / ms_per_step
        result["unfused"] = unfused
    if decode is not None:
        result["decode"] = decode
    if fp8 is not None:
        result["fp8"] = fp8
    if block is not None:
        result["block"] = block
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        result["cpu_baseline"]["per_workload"] = cpu_baseline_all(args.cpu_seconds_each)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
