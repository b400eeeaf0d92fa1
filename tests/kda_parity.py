"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run
the fp64 oracle on the very same (host-copied) inputs, compare.

Tolerance rule: for every compared element,
    |gpu - oracle| <= tol * RMS(oracle) + ulp_out(x) / 2,
RMS taken over the same compared elements, for `out` and for the final state
separately; tol = 1e-4 when q/k/v are fp32 and 2e-2 when they are bf16 (state
and accumulation fp32 in both cases).  ulp_out(x) / 2 is the rounding of the
stored result: half a unit in the last place of the tensor's own dtype (bf16
for a bf16 `out`, fp32 for states), at x = max(|gpu|, |oracle|).  Storing the
exact result in bf16 already moves it by up to that much, which for heavy-tailed
outputs (max|o| ~ 10-20 RMS) alone exceeds 2e-2 RMS, so the rounding of the
stored dtype is allowed on top of the stated bound.
"""
import sys

import numpy as np
import torch

from gated_delta_rule_40_amd import libkda as K
from oracle import kda_oracle as O

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}


def host(x):
    return None if x is None else x.detach().float().cpu().numpy()


def run_prefill(inp, chunk=0, dv_block=0, final=True, out=None, fin=None, use_init=True):
    q = inp["q"]
    T, H, dk = q.shape
    dv = inp["v"].shape[-1]
    N = inp["cu_seqlens"].shape[0] - 1
    if out is None:
        out = torch.empty(T, H, dv, dtype=q.dtype, device=q.device)
    if final and fin is None:
        fin = torch.empty(N, H, dk, dv, dtype=torch.float32, device=q.device)
    init = inp["initial_state"] if use_init else None
    K.kda_prefill_ex(q, inp["k"], inp["v"], inp["g"], inp["beta"], init, inp["cu_seqlens"], out,
                     fin if final else None, chunk=chunk, dv_block=dv_block)
    torch.cuda.synchronize()
    return out, fin


def run_prefill_cp(inp, seg_len=0, final=True, out=None, fin=None, use_init=True, workspace=None):
    q = inp["q"]
    T, H, dk = q.shape
    dv = inp["v"].shape[-1]
    N = inp["cu_seqlens"].shape[0] - 1
    if out is None:
        out = torch.empty(T, H, dv, dtype=q.dtype, device=q.device)
    if final and fin is None:
        fin = torch.empty(N, H, dk, dv, dtype=torch.float32, device=q.device)
    init = inp["initial_state"] if use_init else None
    K.kda_prefill_cp(q, inp["k"], inp["v"], inp["g"], inp["beta"], init, inp["cu_seqlens"], out,
                     fin if final else None, seg_len=seg_len, workspace=workspace)
    torch.cuda.synchronize()
    return out, fin


def oracle_prefill(inp, use_init=True, threads=0):
    init = inp["initial_state"] if use_init else None
    return O.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]), host(inp["beta"]),
                     None if init is None else init.detach().double().cpu().numpy(),
                     inp["cu_seqlens"].cpu().numpy(), num_threads=threads)


MANT_BITS = {torch.bfloat16: 8, torch.float32: 24, torch.float16: 11}


def half_ulp(x, dtype):
    """Half a unit in the last place of |x| in `dtype` (0 for x = 0)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - MANT_BITS[dtype]), 0.0)


def max_rel_err(got, ref, dtype=torch.float32, ulps=0.5):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0, 0.0, 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(got - ref)
    excess = d - 2 * ulps * half_ulp(np.maximum(np.abs(got), np.abs(ref)), dtype)
    err = float(d.max())
    rel = float(np.maximum(excess, 0).max()) / rms if rms > 0 else float(excess.max())
    return rel, err, rms


def assert_close(got, ref, tol, what, dtype=torch.float32, ulps=0.5):
    """`dtype`: the dtype `got` was stored in (its rounding is allowed on top);
    ulps = 1 when both sides are device results stored in that dtype."""
    rel, err, rms = max_rel_err(got, ref, dtype, ulps)
    log("  %-30s max|d|=%.3e rms=%.3e raw max|d|/rms=%.3e (|d|-ulp/2)/rms=%.3e (tol %.0e)"
        % (what, err, rms, err / rms if rms > 0 else err, rel, tol))
    assert np.all(np.isfinite(np.asarray(got))), "%s has non-finite values" % what
    assert rel <= tol, "%s: (|d| - ulp/2) / rms = %.3e > %.0e" % (what, rel, tol)


class StreamingCompare:
    """The rule of assert_close over a tensor too large to hold twice in fp64:
    blocks of (got, ref) are added one by one, keeping max|d|, the largest
    excess |d| - ulps * ulp(x) / 2 and the sum of ref^2; check() then applies
    tol * RMS with the RMS over every element added (the whole tensor)."""

    def __init__(self, what, tol, dtype=torch.float32, ulps=0.5):
        self.what, self.tol, self.dtype, self.ulps = what, tol, dtype, ulps
        self.sq, self.n, self.maxd, self.maxex, self.finite = 0.0, 0, 0.0, -np.inf, True

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        if not ref.size:
            return
        self.finite &= bool(np.all(np.isfinite(got)))
        d = np.abs(got - ref)
        ex = d - 2 * self.ulps * half_ulp(np.maximum(np.abs(got), np.abs(ref)), self.dtype)
        self.sq += float(np.sum(ref * ref))
        self.n += ref.size
        self.maxd = max(self.maxd, float(d.max()))
        self.maxex = max(self.maxex, float(ex.max()))

    def check(self):
        rms = float(np.sqrt(self.sq / max(self.n, 1)))
        rel = max(self.maxex, 0.0) / rms if rms > 0 else max(self.maxex, 0.0)
        log("  %-30s %d elements max|d|=%.3e rms=%.3e raw max|d|/rms=%.3e (|d|-ulp/2)/rms=%.3e (tol %.0e)"
            % (self.what, self.n, self.maxd, rms, self.maxd / rms if rms > 0 else self.maxd, rel, self.tol))
        assert self.finite, "%s has non-finite values" % self.what
        assert rel <= self.tol, "%s: (|d| - ulp/2) / rms = %.3e > %.0e" % (self.what, rel, self.tol)
        return rel


def oracle_threads():
    """Host threads for the oracle: the cores this process may use, at most
    OMP_NUM_THREADS when that is set."""
    import os
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)
