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
# decode bytes per (sequence, head): state read + write, q/k/v/out bf16, g fp32, beta fp32
DECODE_BYTES_PER_UNIT = 2 * DK * DV * 4 + 3 * 2 * DK + 4 * DK + 4 + 2 * DV
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, TFLOP/s
# backward, per head-token: q, k, v, dout in bf16, g fp32, beta in; dq, dk, dg,
# dv fp32 and dbeta out
BWD_BYTES_PER_HT = 4 * 2 * DK + 4 * DK + 4 + 4 * (3 * DK + DV) + 4
# backward token form, flops per state element and token: recompute
# (decay 1, S^T k 2, rank-1 update 2) + reverse (decay 1, S^T k 2, q do^T 2,
# dS^T k 2, S do with the update 4, dk 4, dSbar 2, dg 2, decay 1) = 25
BWD_FLOP_PER_HT = 25 * DK * DV
PREFILL_KERNELS = {
    "cp": "kda_prefill_cp call: kda_cp_plan_kernel (two plans), kda_prefill_kernel<bf16,32,4,MODE_PREP> (chunk operands), "
          "kda_chain_kernel<bf16,32,8 waves,2 tiles,summary>, kda_cp_combine_kernel, "
          "kda_chain_kernel<bf16,32,4 waves,2 tiles,output,single buffer>",
    "plain": "kda_prefill call: kda_prefill_kernel<bf16,32,4,MODE_FUSED>",
}
PMC_SUMMARY = os.path.join(ROOT, "profiles", "kda_prefill_varlen_1m_h16_traffic.json")
PREFILL_SRC = os.path.join(ROOT, "gated_delta_rule_40_amd", "csrc", "kda_prefill.hip")


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_traffic():
    """HBM bytes per prefill launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    try:
        with open(PMC_SUMMARY) as f:
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
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "kda_prefill_varlen_1m_h16_mfma.json")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")


def write_mfma(path):
    """Executed MFMA work per kda_prefill_cp call from one rocprofv3 --pmc run of
    the four MFMA_COUNTERS (timed steps only): fp16 and fp32 MFMA flops (each
    MOPS unit is 512 flops) per kernel kind and per call, and the share of
    cycles the MFMA units were busy."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            name, vals = rows.setdefault(d, (r["Kernel_Name"], {}))
            vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    first_extra = min((d for d, (n, _) in rows.items() if "kda_decode_tokens_kernel" in n), default=None)
    rows = {d: v for d, v in rows.items() if first_extra is None or d < first_extra}
    out = {"kernel_source_sha256_16": source_hash(PREFILL_SRC),
           "commands": ["cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --output-format csv -d <dir> -o run "
                        "-- python <repo>/bench.py --steps 1 --warmup 1 --decode-steps 2 --no-cpu-baseline"
                        % " ".join(MFMA_COUNTERS),
                        "python bench.py --mfma-from <dir>/run_counter_collection.csv"],
           "unit": "flops executed by MFMA instructions per kda_prefill_cp call (MOPS x 512); 'raw' holds "
                   "each counter's average per launch as rocprofv3 reports it"}
    per_kind, f16, f32 = {}, 0.0, 0.0
    for kind, match in CP_KINDS.items():
        ks = [v for n, v in rows.values() if match(n)]
        avg = lambda c: sum(k.get(c, 0.0) for k in ks) / max(len(ks), 1)
        per_kind[kind] = {"launches": len(ks), "f16_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_F16") * 512,
                          "f32_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_F32") * 512,
                          "raw": {c: avg(c) for c in MFMA_COUNTERS}}
        f16 += per_kind[kind]["f16_flops"]
        f32 += per_kind[kind]["f32_flops"]
    out.update(per_kernel=per_kind, f16_flops_per_call=f16, f32_flops_per_call=f32)
    with open(MFMA_SUMMARY, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def pmc_mfma():
    """(fp16, fp32) MFMA flops per prefill call from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    try:
        with open(MFMA_SUMMARY) as f:
            d = json.load(f)
        if d.get("kernel_source_sha256_16") != source_hash(PREFILL_SRC):
            return None
        return float(d["f16_flops_per_call"]), float(d["f32_flops_per_call"])
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


def write_traffic(fetch_csv, write_csv):
    """HBM bytes per kda_prefill_cp call from two rocprofv3 --pmc runs of
    ``bench.py --copy-calibration`` (FETCH_SIZE, then WRITE_SIZE), each scaled
    by what the same counter reads for the 1 GiB-in / 1 GiB-out negation."""
    out = {"kernel_source_sha256_16": source_hash(PREFILL_SRC),
           "commands": ["cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --output-format csv -d <dir> -o run "
                        "-- python <repo>/bench.py --steps 1 --warmup 1 --decode-steps 2 --no-cpu-baseline "
                        "--copy-calibration" % c for c in ("FETCH_SIZE", "WRITE_SIZE")]
                       + ["python bench.py --traffic-from <fetch dir>/run_counter_collection.csv "
                          "<write dir>/run_counter_collection.csv"],
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
    with open(PMC_SUMMARY, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def cpu_baseline(pre, H, target_s=20.0):
    """Time the fp64 oracle (as it stands) on host cores on a bounded sample:
    the first Ls tokens of every sequence of the same prefill inputs, all heads."""
    import numpy as np
    import torch
    from oracle import kda_oracle as O

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = max(1, min(cores, 16))
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
    return {"value": tok / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%s x %d heads of the same prefill inputs "
                      "(%d tokens, %d head-tokens, %.1f s, fp64 token loop, OpenMP over (sequence, head))"
                      % (what, H, tok, tok * H, t)}


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--mfma-from", metavar="PMC_CSV",
                    help="write the executed-MFMA summary from a rocprofv3 --pmc run of the MFMA counters and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic summary from two rocprofv3 counter CSVs and exit (no GPU)")
    args = ap.parse_args()
    if args.mfma_from:
        write_mfma(args.mfma_from)
        return
    if args.traffic_from:
        write_traffic(*args.traffic_from)
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
    if args.copy_calibration:
        # a plain streaming kernel of known size for the HBM counters: torch's
        # elementwise negation reads 1 GiB and writes 1 GiB (kernel name holds "neg")
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
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
    traffic = pmc_traffic()
    mfma = pmc_mfma()

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

    # backward (training) on the 4,096-token, 8-head workload: its own
    # measurement, outside the timed steps
    wl_b = I.WORKLOADS["prefill_t4096_h8"]
    bwd = I.make_prefill(wl_b, device=dev)
    Tb, Hb = bwd["q"].shape[0], bwd["q"].shape[1]
    gen = torch.Generator(device=dev).manual_seed(7)
    b_dout = torch.randn(Tb, Hb, DV, generator=gen, device=dev).to(torch.bfloat16)
    b_ws = torch.empty(K.kda_backward_workspace_size(1, Tb, Hb, DK, DV, torch.bfloat16), dtype=torch.uint8, device=dev)
    b_grads = None

    def backward():
        return K.kda_backward(bwd["q"], bwd["k"], bwd["v"], bwd["g"], bwd["beta"], bwd["initial_state"],
                              bwd["cu_seqlens"], b_dout, None, grads=b_grads, workspace=b_ws)

    b_grads = backward()
    torch.cuda.synchronize()
    b_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b_ev[0].record(stream)
    for _ in range(3):
        backward()
    b_ev[1].record(stream)
    torch.cuda.synchronize()
    bwd_ms = b_ev[0].elapsed_time(b_ev[1]) / 3
    bwd_tflops = Tb * Hb * BWD_FLOP_PER_HT / (bwd_ms * 1e-3) / 1e12
    bwd_bytes = Tb * Hb * BWD_BYTES_PER_HT + 3 * Hb * DK * DV * 4      # + initial state, dfinal, dinit

    # the other prefill configurations (parity cases of their own), timed the
    # same way for reference: context-parallel and plain entry points
    def time_prefill_config(name):
        wl = I.WORKLOADS[name]
        inp = I.make_prefill(wl, device=dev)
        Tc, Hc = inp["q"].shape[0], inp["q"].shape[1]
        Nc = inp["cu_seqlens"].shape[0] - 1
        o = torch.empty(Tc, Hc, DV, dtype=inp["q"].dtype, device=dev)
        f = torch.empty(Nc, Hc, DK, DV, dtype=torch.float32, device=dev)
        w = torch.empty(K.kda_prefill_cp_workspace_size(Nc, Tc, Hc, DK, DV, inp["q"].dtype, 0), dtype=torch.uint8,
                        device=dev)
        calls = {"kda_prefill_cp": lambda: K.kda_prefill_cp(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                            inp["initial_state"], inp["cu_seqlens"], o, f,
                                                            seg_len=0, workspace=w),
                 "kda_prefill": lambda: K.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                      inp["initial_state"], inp["cu_seqlens"], o, f)}
        entry = {"total_tokens": Tc, "heads": Hc, "num_seqs": Nc}
        nbytes = Tc * Hc * PREFILL_BYTES_PER_HT + 2 * Nc * Hc * DK * DV * 4   # + initial and final states
        for key, fn in calls.items():
            for _ in range(2):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(5):
                fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / 5
            entry[key] = {"ms": ms, "tokens_per_s": Tc / (ms * 1e-3), "head_tokens_per_s": Tc * Hc / (ms * 1e-3),
                          "hbm_algorithmic_gbs": nbytes / (ms * 1e-3) / 1e9,
                          "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del inp, o, f, w
        return entry

    other_prefill = {name: time_prefill_config(name) for name in ("prefill_t4096_h8", "prefill_4x16384_h32")}

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
                        "mfma_executed": None if mfma is None else {
                            "f16_tflops": mfma[0] / (pre_avg * 1e-3) / 1e12,
                            "f32_tflops": mfma[1] / (pre_avg * 1e-3) / 1e12,
                            "f16_frac_of_peak": mfma[0] / (pre_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
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
        "backward": {"workload": "prefill_t4096_h8", "ms_per_call": bwd_ms, "tokens_per_s": Tb / (bwd_ms * 1e-3),
                     "head_tokens_per_s": Tb * Hb / (bwd_ms * 1e-3),
                     "roofline": {"bound": "alu", "achieved": bwd_tflops, "peak": FP32_VALU_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": bwd_tflops / FP32_VALU_PEAK_TFLOPS,
                                  "flop_per_head_token": BWD_FLOP_PER_HT,
                                  "hbm_achieved_gbs": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
                                  "algorithmic_bytes_per_launch": bwd_bytes},
                     "kernels": "kda_cp_plan_kernel, chunk operands, kda_chain_kernel summary and output with "
                                "state stores, kda_cp_combine_kernel x2, kda_backward_summary_kernel<bf16>, "
                                "kda_backward_kernel<bf16>, kda_backward_reduce_kernel"},
        "other_prefill_configs": other_prefill,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pre, H)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
