#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * kda_prefill_cp over the long-context varlen batch (8 sequences, lengths
    drawn log-uniform over [1K, 256K] and rescaled to 1,048,576 tokens, 16
    heads, dk = dv = 128, bf16 q/k/v, fp32 g/beta/state, zero initial state;
    sequences split into segments that run side by side), then
  * 64 consecutive in-place kda_decode_step calls on the decode batch
    (512 sequences x 32 heads, 1 GiB fp32 state).
Inputs are generated on the device before timing (resident in HBM).

Prints ONE JSON line.  `value` is prefill tokens/s (sequence tokens, all 16
heads each); the decode figures sit under "decode".  Kernel durations come from
HIP events recorded on the stream the kernels run on, inside the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--prefill cp|plain] [--seg-len L]

Counter runs (rocprofv3 --pmc around one workload at a time) and the summaries
under profiles/ that the JSON line reads while their kernel-source hash matches:

    python bench.py --pmc-workload NAME           # 2 kda_prefill_cp calls + a 1 GiB negation
    python bench.py --traffic-from FETCH.csv WRITE.csv --workload NAME
    python bench.py --mfma-from MFMA.csv --workload NAME
    python bench.py --stats-from TRACE_DIR --workload NAME
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode tokens/s + % HBM peak (1 GPU)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA, TFLOP/s
DK = DV = 128
# algorithmic bytes per head-token of prefill: q, k, v, out (bf16) + g (fp32) + beta (fp32)
PREFILL_BYTES_PER_HT = 3 * 2 * DK + 4 * DK + 4 + 2 * DV
# reference chunk-form flops per head-token (three dk x dv contractions + chunk terms at C = 64)
PREFILL_FREF_PER_HT = 6 * DK * DV + 2 * 64 * (DK + DV)
# minimal flops per head-token: the three dk x dv contractions alone
PREFILL_FALG_PER_HT = 6 * DK * DV
# decode bytes per (sequence, head): state read + write, q/k/v/out bf16, g fp32, beta fp32
DECODE_BYTES_PER_UNIT = 2 * DK * DV * 4 + 3 * 2 * DK + 4 * DK + 4 + 2 * DV
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, TFLOP/s
# backward, per head-token: q, k, v, dout in bf16, g fp32, beta in; dq, dk, dg,
# dv fp32 and dbeta out
BWD_BYTES_PER_HT = 4 * 2 * DK + 4 * DK + 4 + 4 * (3 * DK + DV) + 4
# backward, chunk form: the dk x dv contractions per head-token (2 flops per
# multiply-add) -- states at chunk starts (U = V - K+ S, S' = gamma S + K^T W: 2),
# the state-gradient chain (K^ G, K+^T Z, Q+^T dO: 3), the chunk gradients
# (dO S^T, dX S^T, W G^T: 3); 8 contractions x 2 dk dv flops
BWD_FLOP_PER_HT = 16 * DK * DV
PREFILL_KERNELS = {
    "cp": "kda_prefill_cp call: kda_prefill_kernel<bf16,32,4,MODE_PREP> (chunk operands; with at most 256 sequences its last two workgroups build the two plans, else kda_cp_plan_kernel runs first), "
          "kda_chain_kernel<bf16,32,8 waves,2 tiles,summary> (a segment's last 36 chunks when its transition over them is zero), kda_cp_combine_kernel, "
          "kda_chain_kernel<bf16,32,4 waves,2 tiles,output,single buffer,pieces> (one workgroup per (piece, head))",
    "plain": "kda_prefill call: kda_prefill_kernel<bf16,32,4,MODE_FUSED>",
}
PREFILL_SRC = os.path.join(ROOT, "gated_delta_rule_40_amd", "csrc", "kda_prefill.hip")
BACKWARD_SRC = os.path.join(ROOT, "gated_delta_rule_40_amd", "csrc", "kda_backward.hip")
PREFILL_WORKLOADS = ("prefill_t4096_h8", "prefill_4x16384_h32", "prefill_varlen_1m_h16")


def profile_path(workload, kind):
    """profiles/kda_prefill_<workload without its prefill_ prefix>_<kind>.json"""
    short = workload[len("prefill_"):] if workload.startswith("prefill_") else workload
    return os.path.join(ROOT, "profiles", "kda_prefill_%s_%s.json" % (short, kind))


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_traffic(workload):
    """HBM bytes per kda_prefill_cp call on `workload` from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    try:
        with open(profile_path(workload, "traffic")) as f:
            d = json.load(f)
        if d.get("kernel_source_sha256_16") != source_hash(PREFILL_SRC):
            return None
        return float(d["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


# the launches of one kda_prefill_cp call, by kernel name
CP_KINDS = {"plan": lambda n: "kda_cp_plan_kernel" in n,
            "chunk_operands": lambda n: "kda_prefill_kernel" in n and "Li1EEE" in n,
            # kda_chain_kernel<TIn, C, NW, NCT, SUMMARY, SB, SNAP>: the 5th argument
            "summaries": lambda n: "kda_chain_kernel" in n and n.split("ELb", 1)[1][:1] == "1",
            "combine": lambda n: "kda_cp_combine_kernel" in n,
            "outputs": lambda n: "kda_chain_kernel" in n and n.split("ELb", 1)[1][:1] == "0"}
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")


def write_mfma(path, workload):
    """Executed MFMA work per kda_prefill_cp call on `workload` from one
    rocprofv3 --pmc run of the MFMA_COUNTERS over ``--pmc-workload``:
    fp16, bf16 and fp32 MFMA flops (each MOPS unit is 512 flops) per kernel
    kind and per call, and the share of cycles the MFMA units were busy."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            name, vals = rows.setdefault(d, (r["Kernel_Name"], {}))
            vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    first_extra = min((d for d, (n, _) in rows.items() if "kda_decode_tokens_kernel" in n), default=None)
    rows = {d: v for d, v in rows.items() if first_extra is None or d < first_extra}
    out = {"kernel_source_sha256_16": source_hash(PREFILL_SRC), "workload": workload,
           "commands": ["cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --output-format csv -d <dir> -o run "
                        "-- python <repo>/bench.py --pmc-workload %s" % (" ".join(MFMA_COUNTERS), workload),
                        "python bench.py --mfma-from <dir>/run_counter_collection.csv --workload %s" % workload],
           "unit": "flops executed by MFMA instructions per kda_prefill_cp call (MOPS x 512); 'raw' holds "
                   "each counter's average per launch as rocprofv3 reports it"}
    per_kind, f16, bf16, f32 = {}, 0.0, 0.0, 0.0
    for kind, match in CP_KINDS.items():
        ks = [v for n, v in rows.values() if match(n)]
        avg = lambda c: sum(k.get(c, 0.0) for k in ks) / max(len(ks), 1)
        per_kind[kind] = {"launches": len(ks), "f16_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_F16") * 512,
                          "bf16_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512,
                          "f32_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_F32") * 512,
                          "raw": {c: avg(c) for c in MFMA_COUNTERS}}
        f16 += per_kind[kind]["f16_flops"]
        bf16 += per_kind[kind]["bf16_flops"]
        f32 += per_kind[kind]["f32_flops"]
    out.update(per_kernel=per_kind, f16_flops_per_call=f16, bf16_flops_per_call=bf16, f32_flops_per_call=f32)
    with open(profile_path(workload, "mfma"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def pmc_mfma(workload):
    """(fp16 + bf16, fp32) MFMA flops per kda_prefill_cp call on `workload`
    from the committed counter summary, if it was taken on the current kernel
    source (else None)."""
    try:
        with open(profile_path(workload, "mfma")) as f:
            d = json.load(f)
        if d.get("kernel_source_sha256_16") != source_hash(PREFILL_SRC):
            return None
        return float(d["f16_flops_per_call"]) + float(d.get("bf16_flops_per_call", 0.0)), float(d["f32_flops_per_call"])
    except (OSError, ValueError, KeyError):
        return None


def _pmc_rows(path):
    """{dispatch id: (kernel name, counter value in KiB)} from a rocprofv3 counter
    CSV, for the timed steps only: the dispatches before the first replay
    kernel (the replay and backward measurements, which follow the steps, reuse
    some of the prefill kernels)."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            name, val = rows.get(d, (r["Kernel_Name"], 0.0))
            rows[d] = (name, val + float(r["Counter_Value"]))
    first_extra = min((d for d, (n, _) in rows.items() if "kda_decode_tokens_kernel" in n), default=None)
    return {d: v for d, v in rows.items()
            if first_extra is None or d < first_extra or "kda" not in v[0]}


def write_traffic(fetch_csv, write_csv, workload):
    """HBM bytes per kda_prefill_cp call on `workload` from two rocprofv3 --pmc
    runs of ``bench.py --pmc-workload`` (FETCH_SIZE, then WRITE_SIZE), each
    scaled by what the same counter reads for the 1 GiB-in / 1 GiB-out
    negation in the same run."""
    out = {"kernel_source_sha256_16": source_hash(PREFILL_SRC), "workload": workload,
           "commands": ["cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --output-format csv -d <dir> -o run "
                        "-- python <repo>/bench.py --pmc-workload %s" % (c, workload)
                        for c in ("FETCH_SIZE", "WRITE_SIZE")]
                       + ["python bench.py --traffic-from <fetch dir>/run_counter_collection.csv "
                          "<write dir>/run_counter_collection.csv --workload %s" % workload],
           "unit": "bytes per kda_prefill_cp call (all five launches), counters scaled by the 1 GiB negation"}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path)
        calib = max(v for n, v in rows.values() if "neg" in n.lower())
        factor = float(1 << 30) / (calib * 1024.0)
        # one kda_prefill_cp call = one launch of each kind (each kind is
        # averaged over its own launches: the plan and combine kernels also
        # serve the backward)
        per_kind = {}
        for kind, match in CP_KINDS.items():
            vals = [v for n, v in rows.values() if match(n)]
            per_kind[kind] = {"launches": len(vals), "kib_avg_raw": sum(vals) / max(len(vals), 1),
                              "bytes_avg": sum(vals) / max(len(vals), 1) * 1024.0 * factor}
        per_call = sum(k["kib_avg_raw"] for k in per_kind.values()) * 1024.0
        out[counter] = {"calibration_kib": calib, "scale": factor, "per_kernel": per_kind,
                        "kib_per_call_raw": per_call / 1024.0, "bytes_per_call": per_call * factor}
        total += per_call * factor
    out["hbm_bytes_per_launch"] = total
    with open(profile_path(workload, "traffic"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def kernel_label(name):
    """Short label of a libkda kernel from its (possibly mangled) name."""
    for key, label in (("kda_cp_plan_kernel", "kda_cp_plan_kernel"), ("kda_cp_combine_kernel", "kda_cp_combine_kernel"),
                       ("kda_decode_tokens_kernel", "kda_decode_tokens_kernel"), ("kda_decode_kernel", "kda_decode_kernel")):
        if key in name:
            return label
    dt = "bf16" if "DF16b" in name else "fp32"
    if "kda_prefill_kernel" in name:
        # (up to 256 sequences the same launch also builds the segment plans)
        kind = "chunk operands" if "Li1EEE" in name else ("chunk and gradient images" if "Li3EEE" in name else "fused")
        return "kda_prefill_kernel<%s> (%s)" % (dt, kind)
    if "kda_chain_kernel" in name:
        # kda_chain_kernel<TIn, C, NW, NCT, SUMMARY, SB, SNAP>
        flags = [f[:1] for f in name.split("ELb")[1:4]]
        kind = "segment summaries" if flags[0] == "1" else (
            "chunk-start states, U, W" if len(flags) > 2 and flags[2] == "1" else "segment outputs")
        return "kda_chain_kernel<%s> (%s)" % (dt, kind)
    if "kda_grad_chain_kernel" in name:
        kind = "gradient summaries" if name.split("ELb", 1)[1][:1] == "1" else "state gradients at chunk ends, dX"
        return "kda_grad_chain_kernel<%s> (%s)" % (dt, kind)
    if "kda_bwd_chunk_kernel" in name:
        return "kda_bwd_chunk_kernel<%s> (chunk gradients)" % dt
    return name.split("(")[0][:60]


def call_starts(ks):
    """Indices of the first launch of each kda_prefill_cp / kda_backward call
    in a time-sorted kernel list: the plan kernel, or (up to 256 sequences,
    where the plans are built inside it) the chunk-operand launch."""
    is_plan = lambda n: "kda_cp_plan_kernel" in n
    is_prep = lambda n: "kda_prefill_kernel" in n and ("Li1EEE" in n or "Li3EEE" in n)
    return [i for i, k in enumerate(ks)
            if is_plan(k[2]) or (is_prep(k[2]) and (i == 0 or not is_plan(ks[i - 1][2])))]


def write_stats(trace_dir, workload):
    """Per-kernel durations of the kda_prefill_cp calls of a rocprofv3
    --kernel-trace run of ``bench.py --pmc-workload`` (the last call: the
    first one pays first-use costs), written as a text summary."""
    import csv
    rows = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
            if "kda" in r["Kernel_Name"]]
    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    starts = call_starts(ks)
    calls = len(starts)
    last = ks[starts[-1]:]
    short = workload[len("prefill_"):] if workload.startswith("prefill_") else workload
    path = os.path.join(ROOT, "profiles", "kda_prefill_cp_%s_kernel_stats.txt" % short)
    lines = ["# rocprofv3 kernel trace: one kda_prefill_cp call on %s (automatic seg_len), MI355X (gfx950)" % workload,
             "# kernel source sha256/16: %s" % source_hash(PREFILL_SRC),
             "#",
             "# command (repo at <repo>):",
             "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run \\",
             "#       -- python <repo>/bench.py --pmc-workload %s" % workload,
             "#   python bench.py --stats-from <dir> --workload %s" % workload,
             "# source: <dir>/run_kernel_trace.csv, the last of the run's %d calls" % calls,
             "#",
             "%-52s %12s" % ("kernel", "duration_us")]
    for s0, e0, name in last:
        lines.append("%-52s %12.1f" % (kernel_label(name), (e0 - s0) / 1e3))
    lines.append("")
    lines.append("# kernel time per call: %.1f us; first launch start to last launch end: %.1f us"
                 % (sum(e0 - s0 for s0, e0, _ in last) / 1e3, (last[-1][1] - last[0][0]) / 1e3))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def backward_run(workload, calls=5):
    """Profiling run: kda_backward on this workload `calls` times after one
    warm-up call (nothing else), printing the time per call."""
    import torch
    from gated_delta_rule_40_amd import inputs as I
    from gated_delta_rule_40_amd import libkda as K
    K.load()
    dev = torch.device("cuda:0")
    b = I.make_prefill(I.WORKLOADS[workload], device=dev)
    T_, H_ = b["q"].shape[0], b["q"].shape[1]
    N_ = b["cu_seqlens"].shape[0] - 1
    gen = torch.Generator(device=dev).manual_seed(7)
    dout = torch.randn(T_, H_, DV, generator=gen, device=dev).to(torch.bfloat16)
    ws = torch.empty(K.kda_backward_workspace_size(N_, T_, H_, DK, DV, torch.bfloat16), dtype=torch.uint8, device=dev)
    grads = K.kda_backward(b["q"], b["k"], b["v"], b["g"], b["beta"], b["initial_state"], b["cu_seqlens"], dout,
                           None, workspace=ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(calls):
        K.kda_backward(b["q"], b["k"], b["v"], b["g"], b["beta"], b["initial_state"], b["cu_seqlens"], dout, None,
                       grads=grads, workspace=ws)
    ev[1].record()
    torch.cuda.synchronize()
    print(json.dumps({"backward_workload": workload, "calls": calls,
                      "ms_per_call": ev[0].elapsed_time(ev[1]) / calls}), flush=True)


def write_backward_stats(trace_dir, workload):
    """Kernel timeline of the last kda_backward call of a rocprofv3
    --kernel-trace run of ``bench.py --backward-workload``: start and end of
    every launch relative to the call's first, so that the two strands that
    run side by side show as overlapping intervals."""
    import csv
    rows = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
            if "kda" in r["Kernel_Name"]]
    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    starts = call_starts(ks)
    last = ks[starts[-1]:]
    t0 = last[0][0]
    short = workload[len("prefill_"):] if workload.startswith("prefill_") else workload
    path = os.path.join(ROOT, "profiles", "kda_backward_%s_kernel_stats.txt" % short)
    lines = ["# rocprofv3 kernel trace: one kda_backward call on %s (bf16), MI355X (gfx950)" % workload,
             "# kernel source sha256/16 (kda_prefill.hip): %s, (kda_backward.hip): %s"
             % (source_hash(PREFILL_SRC), source_hash(BACKWARD_SRC)),
             "#",
             "# command (repo at <repo>):",
             "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run \\",
             "#       -- python <repo>/bench.py --backward-workload %s" % workload,
             "#   python bench.py --backward-stats-from <dir> --backward-workload %s" % workload,
             "# source: <dir>/run_kernel_trace.csv, the last of the run's %d calls; times in us from the" % len(starts),
             "# call's first launch (the two strands after the chunk images run on two streams)",
             "#",
             "%-64s %9s %9s %9s" % ("kernel", "start", "end", "duration")]
    for s0, e0, name in last:
        lines.append("%-64s %9.1f %9.1f %9.1f" % (kernel_label(name), (s0 - t0) / 1e3, (e0 - t0) / 1e3, (e0 - s0) / 1e3))
    lines.append("")
    lines.append("# first launch start to last launch end: %.1f us; sum of kernel durations: %.1f us"
                 % ((last[-1][1] - t0) / 1e3, sum(e0 - s0 for s0, e0, _ in last) / 1e3))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_kernel_summary(trace_dir, name):
    """Average duration of every libkda kernel in a rocprofv3 --kernel-trace
    run of the default bench step (``bench.py --steps 2 --warmup 1
    --no-cpu-baseline``), written as a text summary: the decode, replay and
    backward kernels that the JSON line times with HIP events."""
    import csv
    rows = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
            if "kda" in r["Kernel_Name"]]
    agg = {}
    for r in rows:
        lab = kernel_label(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg.setdefault(lab, []).append(d)
    path = os.path.join(ROOT, "profiles", "%s_kernel_stats.txt" % name)
    lines = ["# rocprofv3 kernel trace of the default bench step, MI355X (gfx950)",
             "# kernel source sha256/16 (kda_prefill.hip): %s" % source_hash(PREFILL_SRC),
             "#",
             "# command (repo at <repo>):",
             "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run \\",
             "#       -- python <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline",
             "#   python bench.py --kernel-summary-from <dir> --summary-name %s" % name,
             "# every libkda kernel of the run (prefill calls of all workloads, 64 decode steps per",
             "# bench step, the replay and backward measurements), averaged over its launches",
             "#",
             "%-60s %7s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    for lab, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%-60s %7d %12.1f %12.1f %12.1f" % (lab, len(ds), sum(ds) / len(ds), min(ds), max(ds)))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def host_cores():
    """(cores used, cores available): the cores this process may run on
    (sched_getaffinity), at most OMP_NUM_THREADS when the environment sets it."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    used = min(avail, int(env)) if env.isdigit() and int(env) > 0 else avail
    return max(1, used), avail


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pre, H, small, target_s=20.0):
    """Time the fp64 oracle (as it stands) on host cores on a bounded sample:
    the first Ls tokens of every sequence of the same prefill inputs, all
    heads; plus single-thread runs of the oracle on the small workloads
    (`small`: {name: host input dict}) for a per-core rate."""
    import numpy as np
    import torch
    from oracle import kda_oracle as O

    cores, avail = host_cores()
    cu = pre["cu_seqlens"].cpu().tolist()
    N = len(cu) - 1

    def run(Ls):
        rows = [torch.arange(cu[n], cu[n] + min(Ls, cu[n + 1] - cu[n])) for n in range(N)]
        lens = [len(r) for r in rows]
        idx = torch.cat(rows).to(pre["q"].device)
        sub = {k_: pre[k_].index_select(0, idx).float().cpu().numpy() for k_ in ("q", "k", "v", "g", "beta")}
        scu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        t0 = time.perf_counter()
        O.prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], None, scu, num_threads=cores)
        return time.perf_counter() - t0, sum(lens)

    O.build()
    t, tok = run(2048)                     # calibration (long enough that setup does not dominate)
    rate = tok / max(t, 1e-6)
    # the sample's tokens are sum_n min(Ls, L_n): the smallest Ls that reaches
    # rate * target_s (or the whole input)
    lens = [cu[n + 1] - cu[n] for n in range(N)]
    want = rate * target_s
    lo, hi = 2048, max(max(lens), 2048)
    while lo < hi:
        mid = (lo + hi) // 2
        if sum(min(mid, L) for L in lens) >= want:
            hi = mid
        else:
            lo = mid + 1
    Ls = lo
    t, tok = run(Ls)
    what = ("all tokens of the %d sequences" % N if Ls >= max(lens)
            else "the first %d tokens of each of the %d sequences" % (Ls, N))
    single = {}
    for name, inp in small.items():
        T1, H1 = inp["q"].shape[0], inp["q"].shape[1]
        init = inp["initial_state"]
        t0 = time.perf_counter()
        O.prefill(inp["q"].float().numpy(), inp["k"].float().numpy(), inp["v"].float().numpy(), inp["g"].numpy(),
                  inp["beta"].numpy(), None if init is None else init.double().numpy(), inp["cu_seqlens"].numpy(),
                  num_threads=1)
        dt = time.perf_counter() - t0
        single[name] = {"tokens_per_s": T1 / dt, "head_tokens_per_s": T1 * H1 / dt, "s": dt,
                        "fp64_gflops": T1 * H1 * 7 * DK * DV / dt / 1e9}
    return {"value": tok / t, "unit": "tokens/s", "cores": cores, "cores_available": avail, "cpu_model": cpu_model(),
            "kind": "oracle", "head_tokens_per_s": tok * H / t, "fp64_gflops": tok * H * 7 * DK * DV / t / 1e9,
            "sample": "%s x %d heads of the same prefill inputs "
                      "(%d tokens, %d head-tokens, %.1f s, fp64 token loop, OpenMP over (sequence, head))"
                      % (what, H, tok, tok * H, t),
            "single_thread": single}


def pmc_workload_run(name):
    """One workload under a counter run: a 1 GiB negation (the reference for
    the HBM counters: torch's elementwise negation reads 1 GiB and writes
    1 GiB, its kernel name holds "neg"), then two kda_prefill_cp calls."""
    import torch
    from gated_delta_rule_40_amd import inputs as I
    from gated_delta_rule_40_amd import libkda as K

    assert torch.cuda.is_available(), "needs a GPU"
    K.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    inp = I.make_prefill(I.WORKLOADS[name], device=dev)
    T, H = inp["q"].shape[0], inp["q"].shape[1]
    N = inp["cu_seqlens"].shape[0] - 1
    out = torch.empty(T, H, DV, dtype=inp["q"].dtype, device=dev)
    fin = torch.empty(N, H, DK, DV, dtype=torch.float32, device=dev)
    ws = torch.empty(K.kda_prefill_cp_workspace_size(N, T, H, DK, DV, inp["q"].dtype, 0), dtype=torch.uint8,
                     device=dev)
    for i in range(2):
        K.kda_prefill_cp(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
                         inp["cu_seqlens"], out, fin, seg_len=0, workspace=ws)
        torch.cuda.synchronize()
        print("pmc workload %s: kda_prefill_cp call %d done" % (name, i + 1), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", choices=("cp", "plain"), default="cp",
                    help="cp: kda_prefill_cp (segments side by side); plain: kda_prefill")
    ap.add_argument("--seg-len", type=int, default=0, help="kda_prefill_cp segment length (0 = automatic)")
    ap.add_argument("--pmc-workload", choices=PREFILL_WORKLOADS,
                    help="counter run: a 1 GiB negation then two kda_prefill_cp calls on this workload, and exit")
    ap.add_argument("--workload", choices=PREFILL_WORKLOADS, default="prefill_varlen_1m_h16",
                    help="workload of --mfma-from / --traffic-from")
    ap.add_argument("--mfma-from", metavar="PMC_CSV",
                    help="write the executed-MFMA summary from a rocprofv3 --pmc run of the MFMA counters and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic summary from two rocprofv3 counter CSVs and exit (no GPU)")
    ap.add_argument("--stats-from", metavar="TRACE_DIR",
                    help="write the per-kernel duration summary of a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--kernel-summary-from", metavar="TRACE_DIR",
                    help="write the average duration of every libkda kernel of a bench trace and exit")
    ap.add_argument("--summary-name", default="kda_bench_step",
                    help="file name stem under profiles/ for --kernel-summary-from")
    ap.add_argument("--backward-workload", choices=PREFILL_WORKLOADS,
                    help="profiling run: kda_backward on this workload only, and exit")
    ap.add_argument("--backward-stats-from", metavar="TRACE_DIR",
                    help="write the kernel timeline of a --backward-workload trace and exit")
    args = ap.parse_args()
    if args.backward_stats_from:
        write_backward_stats(args.backward_stats_from, args.backward_workload or "prefill_t4096_h8")
        return
    if args.backward_workload:
        backward_run(args.backward_workload)
        return
    if args.kernel_summary_from:
        write_kernel_summary(args.kernel_summary_from, args.summary_name)
        return
    if args.stats_from:
        write_stats(args.stats_from, args.workload)
        return
    if args.mfma_from:
        write_mfma(args.mfma_from, args.workload)
        return
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.workload)
        return
    if args.pmc_workload:
        pmc_workload_run(args.pmc_workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libkda runs the KDA path on a single MI355X "
              "(heads and sequences would shard across GPUs with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_40_amd import inputs as I
    from gated_delta_rule_40_amd import libkda as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl_p = I.WORKLOADS["prefill_varlen_1m_h16"]
    wl_d = I.WORKLOADS["decode_512x32"]
    pre = I.make_prefill(wl_p, device=dev)
    dec = I.make_decode(wl_d, device=dev, steps=args.decode_steps)
    T, H = pre["q"].shape[0], pre["q"].shape[1]
    N = pre["cu_seqlens"].shape[0] - 1
    out = torch.empty(T, H, DV, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(N, H, DK, DV, dtype=torch.float32, device=dev)
    Nd, Hd = wl_d.num_seqs, wl_d.heads
    state = dec["state"]
    dout = torch.empty(args.decode_steps, Nd, Hd, DV, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    ws = None
    if args.prefill == "cp":
        ws_bytes = K.kda_prefill_cp_workspace_size(N, T, H, DK, DV, torch.bfloat16, args.seg_len)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def prefill():
        if args.prefill == "cp":
            K.kda_prefill_cp(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], None, pre["cu_seqlens"], out,
                             fin, seg_len=args.seg_len, workspace=ws)
        else:
            K.kda_prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], None, pre["cu_seqlens"], out, fin)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        prefill()
        if ev is not None:
            ev[1].record(stream)
        for s in range(args.decode_steps):
            K.kda_decode_step(dec["q"][s], dec["k"][s], dec["v"][s], dec["g"][s], dec["beta"][s], state, dout[s])
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    head_tokens = T * H
    pre_bytes = head_tokens * PREFILL_BYTES_PER_HT + N * H * DK * DV * 4      # + final state write
    pre_gbs = pre_bytes / (pre_avg * 1e-3) / 1e9
    pre_tflops = head_tokens * PREFILL_FREF_PER_HT / (pre_avg * 1e-3) / 1e12
    dec_step_ms = dec_avg / args.decode_steps
    dec_bytes = Nd * Hd * DECODE_BYTES_PER_UNIT
    dec_gbs = dec_bytes / (dec_step_ms * 1e-3) / 1e9
    traffic = pmc_traffic("prefill_varlen_1m_h16")
    mfma = pmc_mfma("prefill_varlen_1m_h16")

    # speculative-decoding replay: 4 draft tokens per (sequence, head) of the
    # decode batch, outputs for all of them and the state committed, one call
    # (its own measurement, outside the timed steps)
    RT = min(4, dec["q"].shape[0])
    perm = lambda x: x[:RT].transpose(0, 1).reshape(Nd * RT, *x.shape[2:]).contiguous()
    rq, rk, rv, rg, rb = (perm(dec[key]) for key in ("q", "k", "v", "g", "beta"))
    rcu = torch.arange(Nd + 1, dtype=torch.int32, device=dev) * RT
    rout = torch.empty(Nd * RT, Hd, DV, dtype=torch.bfloat16, device=dev)

    def replay():
        K.kda_decode_tokens(rq, rk, rv, rg, rb, rcu, state, state_out=state, out=rout)

    for _ in range(2):
        replay()
    r_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    r_ev[0].record(stream)
    for _ in range(5):
        replay()
    r_ev[1].record(stream)
    torch.cuda.synchronize()
    rep_ms = r_ev[0].elapsed_time(r_ev[1]) / 5
    rep_bytes = Nd * Hd * (2 * DK * DV * 4 + RT * (DECODE_BYTES_PER_UNIT - 2 * DK * DV * 4))
    rep_gbs = rep_bytes / (rep_ms * 1e-3) / 1e9

    # backward (training): its own measurement, outside the timed steps, on
    # the 4,096-token, 8-head workload and on 4 x 16,384 tokens x 32 heads
    def time_backward(wl_name, calls):
        b = I.make_prefill(I.WORKLOADS[wl_name], device=dev)
        T_, H_ = b["q"].shape[0], b["q"].shape[1]
        N_ = b["cu_seqlens"].shape[0] - 1
        gen = torch.Generator(device=dev).manual_seed(7)
        dout_ = torch.randn(T_, H_, DV, generator=gen, device=dev).to(torch.bfloat16)
        ws_ = torch.empty(K.kda_backward_workspace_size(N_, T_, H_, DK, DV, torch.bfloat16), dtype=torch.uint8,
                          device=dev)
        grads = K.kda_backward(b["q"], b["k"], b["v"], b["g"], b["beta"], b["initial_state"], b["cu_seqlens"],
                               dout_, None, workspace=ws_)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(calls):
            K.kda_backward(b["q"], b["k"], b["v"], b["g"], b["beta"], b["initial_state"], b["cu_seqlens"], dout_,
                           None, grads=grads, workspace=ws_)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / calls
        del b, dout_, ws_, grads
        tflops = T_ * H_ * BWD_FLOP_PER_HT / (ms * 1e-3) / 1e12
        nbytes = T_ * H_ * BWD_BYTES_PER_HT + 3 * N_ * H_ * DK * DV * 4      # + initial state, dfinal, dinit
        return {"workload": wl_name, "total_tokens": T_, "heads": H_, "num_seqs": N_, "ms_per_call": ms,
                "tokens_per_s": T_ / (ms * 1e-3), "head_tokens_per_s": T_ * H_ / (ms * 1e-3),
                "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": tflops / BF16_PEAK_TFLOPS, "flop_per_head_token": BWD_FLOP_PER_HT,
                             "hbm_achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
                             "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes_per_launch": nbytes}}

    bwd_small = time_backward("prefill_t4096_h8", 5)
    bwd_large = time_backward("prefill_4x16384_h32", 3)

    def flop_fields(head_tokens_c, ms):
        fref = head_tokens_c * PREFILL_FREF_PER_HT / (ms * 1e-3) / 1e12
        falg = head_tokens_c * PREFILL_FALG_PER_HT / (ms * 1e-3) / 1e12
        return {"fref_tflops": fref, "mfma_frac_fref": fref / BF16_PEAK_TFLOPS,
                "falg_tflops": falg, "mfma_frac_falg": falg / BF16_PEAK_TFLOPS}

    def counter_fields(name, ms):
        """HBM bytes and executed MFMA flops of one kda_prefill_cp call, from the
        committed counter summaries while they match the kernel source."""
        tr, mf = pmc_traffic(name), pmc_mfma(name)
        return {"counter_hbm_bytes": tr,
                "counter_hbm_gbs": None if tr is None else tr / (ms * 1e-3) / 1e9,
                "mfma_executed": None if mf is None else {
                    "f16_bf16_tflops": mf[0] / (ms * 1e-3) / 1e12, "f32_tflops": mf[1] / (ms * 1e-3) / 1e12,
                    "f16_bf16_frac_of_peak": mf[0] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
                "counter_source": "rocprofv3 counters: %s, %s" % (
                    os.path.relpath(profile_path(name, "traffic"), ROOT),
                    os.path.relpath(profile_path(name, "mfma"), ROOT))}

    def time_calls(calls, reps=5):
        res = {}
        for key, fn in calls.items():
            for _ in range(2):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(reps):
                fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            res[key] = ev[0].elapsed_time(ev[1]) / reps
        return res

    # the other prefill configurations (parity cases of their own), timed the
    # same way for reference: context-parallel and plain entry points
    def time_prefill_config(name, inp=None, entries=("kda_prefill_cp", "kda_prefill")):
        wl = I.WORKLOADS[name]
        own = inp is None
        if own:
            inp = I.make_prefill(wl, device=dev)
        Tc, Hc = inp["q"].shape[0], inp["q"].shape[1]
        Nc = inp["cu_seqlens"].shape[0] - 1
        o = torch.empty(Tc, Hc, DV, dtype=inp["q"].dtype, device=dev)
        f = torch.empty(Nc, Hc, DK, DV, dtype=torch.float32, device=dev)
        w = None
        if "kda_prefill_cp" in entries:
            w = torch.empty(K.kda_prefill_cp_workspace_size(Nc, Tc, Hc, DK, DV, inp["q"].dtype, 0),
                            dtype=torch.uint8, device=dev)
        calls = {"kda_prefill_cp": lambda: K.kda_prefill_cp(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                            inp["initial_state"], inp["cu_seqlens"], o, f,
                                                            seg_len=0, workspace=w),
                 "kda_prefill": lambda: K.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                      inp["initial_state"], inp["cu_seqlens"], o, f)}
        entry = {"total_tokens": Tc, "heads": Hc, "num_seqs": Nc}
        init_bytes = 0 if inp["initial_state"] is None else Nc * Hc * DK * DV * 4
        nbytes = Tc * Hc * PREFILL_BYTES_PER_HT + Nc * Hc * DK * DV * 4 + init_bytes   # + final (initial) state
        for key, ms in time_calls({k_: calls[k_] for k_ in entries}).items():
            entry[key] = {"ms": ms, "tokens_per_s": Tc / (ms * 1e-3), "head_tokens_per_s": Tc * Hc / (ms * 1e-3),
                          "hbm_algorithmic_gbs": nbytes / (ms * 1e-3) / 1e9,
                          "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "algorithmic_bytes_per_call": nbytes}
            entry[key].update(flop_fields(Tc * Hc, ms))
            if key == "kda_prefill_cp":
                entry[key].update(counter_fields(name, ms))
        if name == "prefill_t4096_h8":
            # state snapshots every 512 tokens (kda_prefill_snapshots, 32-token
            # chunks, 64-column blocks) against kda_prefill at the same tiling
            every = 512
            snaps = torch.empty(Nc, Tc // every, Hc, DK, DV, dtype=torch.float32, device=dev)
            ms_s = time_calls({
                "snapshots": lambda: K.kda_prefill_snapshots(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                             inp["initial_state"], inp["cu_seqlens"], o, f,
                                                             snaps, every),
                "same_tiling": lambda: K.kda_prefill_ex(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                        inp["initial_state"], inp["cu_seqlens"], o, f,
                                                        chunk=32, dv_block=64)})
            entry["kda_prefill_snapshots"] = {"snap_every": every, "snapshots_per_seq": Tc // every,
                                              "ms": ms_s["snapshots"], "kda_prefill_same_tiling_ms": ms_s["same_tiling"],
                                              "overhead": ms_s["snapshots"] / ms_s["same_tiling"] - 1.0}
            del snaps
        small_host = {k_: (v_.cpu() if torch.is_tensor(v_) else v_) for k_, v_ in inp.items()} \
            if name == "prefill_t4096_h8" else None
        del o, f, w
        if own:
            del inp
        return entry, small_host

    other_prefill, small_inputs = {}, {}
    for name in ("prefill_t4096_h8", "prefill_4x16384_h32"):
        other_prefill[name], host_inp = time_prefill_config(name)
        if host_inp is not None:
            small_inputs[name] = host_inp
    # plain kda_prefill on the bench's own 1M-token input (the longest
    # sequence then runs as one chain)
    other_prefill["prefill_varlen_1m_h16"], _ = time_prefill_config("prefill_varlen_1m_h16", inp=pre,
                                                                    entries=("kda_prefill",))
    small_inputs = dict({"parity_t128_fp32": I.make_prefill(I.WORKLOADS["parity_t128_fp32"])}, **small_inputs)

    result = {
        "metric": METRIC,
        "value": T / (pre_avg * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill_varlen_1m_h16 + decode_512x32",
            "prefill": {"entry": "kda_prefill_cp" if args.prefill == "cp" else "kda_prefill",
                        "seg_len": args.seg_len if args.prefill == "cp" else None,
                        "num_seqs": N, "lengths": pre["lengths"], "total_tokens": T, "heads": H,
                        "dk": DK, "dv": DV, "io": "bf16 q/k/v/out, fp32 g/beta/state",
                        "initial_state": "zero", "ms": pre_avg, "head_tokens_per_s": head_tokens / (pre_avg * 1e-3),
                        "fref_tflops": pre_tflops, "mfma_frac_fref": pre_tflops / BF16_PEAK_TFLOPS,
                        "falg_tflops": head_tokens * PREFILL_FALG_PER_HT / (pre_avg * 1e-3) / 1e12,
                        "mfma_frac_falg": head_tokens * PREFILL_FALG_PER_HT / (pre_avg * 1e-3) / 1e12
                        / BF16_PEAK_TFLOPS,
                        "counter_hbm_bytes": traffic,
                        "counter_hbm_gbs": None if traffic is None else traffic / (pre_avg * 1e-3) / 1e9,
                        "mfma_executed": None if mfma is None else {
                            "f16_bf16_tflops": mfma[0] / (pre_avg * 1e-3) / 1e12,
                            "f32_tflops": mfma[1] / (pre_avg * 1e-3) / 1e12,
                            "f16_bf16_frac_of_peak": mfma[0] / (pre_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                            "source": "rocprofv3 MFMA counters (profiles/kda_prefill_varlen_1m_h16_mfma.json)"},
                        "compute": "fp16 MFMA operands (exact power-of-two column scaling), fp32 accumulate and state"},
            "decode": {"num_seqs": Nd, "heads": Hd, "steps": args.decode_steps, "state_bytes": Nd * Hd * DK * DV * 4},
        },
        "roofline": {"bound": "hbm", "achieved": pre_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pre_gbs / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": PREFILL_KERNELS[args.prefill], "algorithmic_bytes_per_launch": pre_bytes,
                     "avg_launch_ms": pre_avg},
        "decode": {"tokens_per_s": Nd / (dec_step_ms * 1e-3), "ms_per_decode_step": dec_step_ms,
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_gbs / HBM_PEAK_GBS, "kernel": "kda_decode_kernel<bf16>",
                                "algorithmic_bytes_per_launch": dec_bytes}},
        "decode_tokens": {"draft_tokens": RT, "ms_per_call": rep_ms, "tokens_per_s": Nd * RT / (rep_ms * 1e-3),
                          "roofline": {"bound": "hbm", "achieved": rep_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": rep_gbs / HBM_PEAK_GBS, "kernel": "kda_decode_tokens_kernel<bf16>",
                                       "algorithmic_bytes_per_launch": rep_bytes}},
        "backward": dict(bwd_small, larger=bwd_large,
                         kernels="kda_cp_plan_kernel; kda_prefill_kernel<bf16,32,4,MODE_PREPG> (chunk and "
                                 "gradient images); then side by side: kda_chain_kernel summaries, "
                                 "kda_cp_combine_kernel, kda_chain_kernel with state stores | "
                                 "kda_grad_chain_kernel summaries, kda_cp_combine_kernel<transposed>, "
                                 "kda_grad_chain_kernel; then kda_bwd_chunk_kernel<bf16>"),
        "other_prefill_configs": other_prefill,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pre, H, small_inputs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
