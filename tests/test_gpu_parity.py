"""GPU parity of libkda (HIP, gfx950) against the fp64 oracle, through the C ABI.

Every comparison with the oracle uses the rule in tests/kda_parity.py:
|gpu - oracle| <= tol * RMS(oracle) + half an ulp of the stored dtype, on `out`
and on the final state, tol = 1e-4 for fp32 q/k/v and 2e-2 for bf16 q/k/v.
Device-vs-device comparisons (two tilings, split vs whole, decode vs prefill)
allow 2 * tol and one ulp, since both sides carry their own error.  Inputs come
from gated_delta_rule_40_amd.inputs (seeded); the oracle reads host copies of
exactly the tensors the GPU read.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_40_amd import inputs as I
from gated_delta_rule_40_amd import libkda as K
from kda_parity import TOL, assert_close, host, log, oracle_prefill, run_prefill, to_dev
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    K.load()


def _check_prefill(inp, tol, label, chunk=0, dv_block=0, use_init=True):
    log("[prefill] %s chunk=%d dv_block=%d T=%d H=%d N=%d dtype=%s" % (
        label, chunk, dv_block, inp["q"].shape[0], inp["q"].shape[1], inp["cu_seqlens"].shape[0] - 1,
        inp["q"].dtype))
    out, fin = run_prefill(inp, chunk=chunk, dv_block=dv_block, use_init=use_init)
    ref_out, ref_fin = oracle_prefill(inp, use_init=use_init)
    cu = inp["cu_seqlens"].cpu().numpy()
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]) if len(cu) > 1 else []
    assert_close(host(out)[rows], ref_out[rows], tol, label + " out", out.dtype)
    assert_close(host(fin), ref_fin, tol, label + " final_state")
    return out, fin


# ------------------------------------------------------------ named workloads
def test_parity_t128_fp32():
    """B=1, H=1, T=128, fp32 q/k/v, zero initial state (all tilings)."""
    wl = I.WORKLOADS["parity_t128_fp32"]
    inp = to_dev(I.make_prefill(wl))
    for chunk in (0, 16, 32):
        for bv in (0, 16, 32, 64, 128):
            _check_prefill(inp, TOL[torch.float32], "t128_fp32", chunk, bv)


def test_parity_t4096_h8_bf16():
    """B=1, H=8, T=4096, bf16 q/k/v, N(0, 0.1) initial state; full size, every output."""
    wl = I.WORKLOADS["prefill_t4096_h8"]
    inp = to_dev(I.make_prefill(wl))
    _check_prefill(inp, TOL[torch.bfloat16], "t4096_h8", 0, 0)
    _check_prefill(inp, TOL[torch.bfloat16], "t4096_h8", 32, 64)


# ------------------------------------------------------------ ragged / varlen
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_varlen(dtype):
    lengths = [1, 17, 64, 0, 100, 63, 65, 130, 200]
    inp = to_dev(I.random_prefill(lengths, H=3, dtype=dtype, seed=7))
    for chunk in ((32, 64) if dtype == torch.bfloat16 else (16, 32)):
        for bv in ((32, 64, 128) if chunk == 64 else (16, 64, 128)):
            _check_prefill(inp, TOL[dtype], "ragged", chunk, bv)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_page_gate_range(dtype):
    """g drawn over the pages' whole range (-5, 0): decay factors up to e^80."""
    inp = to_dev(I.random_prefill([300, 47], H=2, dtype=dtype, seed=8, g_lo=-5.0))
    _check_prefill(inp, TOL[dtype], "g_in_(-5,0)")
    # closed end of the range: g = -5 exactly on every channel, and g = 0
    for gval in (-5.0, 0.0):
        inp2 = dict(inp)
        inp2["g"] = torch.full_like(inp["g"], gval)
        _check_prefill(inp2, TOL[dtype], "g=%g" % gval)


@pytest.mark.parametrize("bval", [0.0, 1.0])
def test_beta_extremes(bval):
    inp = to_dev(I.random_prefill([150, 33], H=2, dtype=torch.bfloat16, seed=9))
    inp["beta"] = torch.full_like(inp["beta"], bval)
    _check_prefill(inp, TOL[torch.bfloat16], "beta=%g" % bval)


def test_null_initial_state_and_null_final():
    inp = to_dev(I.random_prefill([90, 40], H=2, dtype=torch.bfloat16, seed=10))
    _check_prefill(inp, TOL[torch.bfloat16], "null_init", use_init=False)
    out_a, _ = run_prefill(inp, final=False)
    out_b, _ = run_prefill(inp, final=True)
    assert torch.equal(out_a, out_b)


def test_final_state_may_alias_initial_state():
    inp = to_dev(I.random_prefill([130, 64, 5], H=4, dtype=torch.bfloat16, seed=11))
    _, fin = run_prefill(inp)
    state = inp["initial_state"].clone()
    inp2 = dict(inp)
    inp2["initial_state"] = state
    run_prefill(inp2, fin=state)
    assert torch.equal(state, fin)


def test_empty_sequences_and_untouched_rows():
    """Empty sequences keep their state; rows not owned by any sequence are untouched."""
    inp = to_dev(I.random_prefill([0, 40, 0, 25], H=2, dtype=torch.bfloat16, seed=12))
    T = inp["q"].shape[0]
    # add 7 padding rows after the last sequence
    pad = lambda x: torch.cat([x, torch.zeros((7,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)])
    for key in ("q", "k", "v", "g", "beta"):
        inp[key] = pad(inp[key]).contiguous()
    out = torch.full((T + 7, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out, fin = run_prefill(inp, out=out)
    assert torch.isnan(out[T:].float()).all()
    assert torch.equal(fin[0], inp["initial_state"][0]) and torch.equal(fin[2], inp["initial_state"][2])
    ref_out, ref_fin = oracle_prefill(inp)
    assert_close(host(out)[:T], ref_out[:T], TOL[torch.bfloat16], "untouched out", torch.bfloat16)
    assert_close(host(fin), ref_fin, TOL[torch.bfloat16], "untouched final_state")


# ------------------------------------------------------------ invariances
def test_dv_blocks_are_bitwise_identical():
    """Value columns are independent; every value-block size runs the same
    per-column arithmetic, so all tilings agree bit for bit."""
    inp = to_dev(I.random_prefill([77, 256, 3], H=3, dtype=torch.bfloat16, seed=13))
    outs = [run_prefill(inp, chunk=32, dv_block=bv) for bv in (16, 32, 64, 128)]
    outs64 = [run_prefill(inp, chunk=64, dv_block=bv) for bv in (32, 64, 128)]
    for o, f in outs64[1:]:
        assert torch.equal(o, outs64[0][0]) and torch.equal(f, outs64[0][1])
    for o, f in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(f, outs[0][1])


def test_chunk_size_invariance():
    inp = to_dev(I.random_prefill([500, 129], H=2, dtype=torch.bfloat16, seed=14))
    o32, f32 = run_prefill(inp, chunk=32)
    o64, f64 = run_prefill(inp, chunk=64)
    ref_o, ref_f = oracle_prefill(inp)
    for o, f, c in ((o32, f32, 32), (o64, f64, 64)):
        assert_close(host(o), ref_o, TOL[torch.bfloat16], "chunk %d out" % c, torch.bfloat16)
        assert_close(host(f), ref_f, TOL[torch.bfloat16], "chunk %d final" % c)
    assert_close(host(o32), host(o64), 2 * TOL[torch.bfloat16], "chunk 32 vs 64", torch.bfloat16, ulps=1.0)


def test_varlen_packing_equals_separate_runs():
    lengths = [45, 200, 1, 96]
    inp = to_dev(I.random_prefill(lengths, H=2, dtype=torch.bfloat16, seed=15))
    out, fin = run_prefill(inp, dv_block=32)
    cu = inp["cu_seqlens"].cpu().tolist()
    for n, L in enumerate(lengths):
        s, e = cu[n], cu[n + 1]
        sub = {k: inp[k][s:e].contiguous() for k in ("q", "k", "v", "g", "beta")}
        sub["initial_state"] = inp["initial_state"][n:n + 1].contiguous()
        sub["cu_seqlens"] = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        o, f = run_prefill(sub, dv_block=32)
        assert torch.equal(o, out[s:e]) and torch.equal(f[0], fin[n])


def test_continuation_split_equals_whole():
    inp = to_dev(I.random_prefill([700], H=2, dtype=torch.bfloat16, seed=16))
    out, fin = run_prefill(inp)
    for split in (64, 333):
        a = {k: inp[k][:split].contiguous() for k in ("q", "k", "v", "g", "beta")}
        a["initial_state"] = inp["initial_state"]
        a["cu_seqlens"] = torch.tensor([0, split], dtype=torch.int32, device="cuda")
        oa, fa = run_prefill(a)
        b = {k: inp[k][split:].contiguous() for k in ("q", "k", "v", "g", "beta")}
        b["initial_state"] = fa
        b["cu_seqlens"] = torch.tensor([0, 700 - split], dtype=torch.int32, device="cuda")
        ob, fb = run_prefill(b)
        assert_close(host(torch.cat([oa, ob])), host(out), 2 * TOL[torch.bfloat16], "split %d out" % split,
                     torch.bfloat16, ulps=1.0)
        assert_close(host(fb), host(fin), 2 * TOL[torch.bfloat16], "split %d final" % split)


def test_run_to_run_bitwise_determinism():
    inp = to_dev(I.random_prefill([333, 64, 17], H=4, dtype=torch.bfloat16, seed=17))
    o1, f1 = run_prefill(inp)
    o2, f2 = run_prefill(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_nonzero_stream():
    inp = to_dev(I.random_prefill([100], H=2, dtype=torch.bfloat16, seed=18))
    ref, _ = run_prefill(inp)
    s = torch.cuda.Stream()
    out = torch.empty_like(ref)
    with torch.cuda.stream(s):
        K.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
                      inp["cu_seqlens"], out, None)
    s.synchronize()
    assert torch.equal(out, ref)


# ------------------------------------------------------------ decode
def _decode_inputs(N, H, steps, dtype, seed, g_lo=-5 / 16):
    wl = I.Workload("dec", "decode", heads=H, dtype=dtype, num_seqs=N, steps=steps, seed=seed, g_lo=g_lo)
    return I.make_decode(wl, device="cuda")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_steps_vs_oracle(dtype):
    d = _decode_inputs(N=37, H=3, steps=8, dtype=dtype, seed=20, g_lo=-5.0)
    S = d["state"].clone()
    S_ref = d["state"].double().cpu().numpy()
    out = torch.empty(37, 3, 128, dtype=dtype, device="cuda")
    for s in range(8):
        log("[decode] step %d dtype=%s" % (s, dtype))
        K.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, out)
        torch.cuda.synchronize()
        ref_o, S_ref = O.decode_step(host(d["q"][s]), host(d["k"][s]), host(d["v"][s]), host(d["g"][s]),
                                     host(d["beta"][s]), S_ref)
        assert_close(host(out), ref_o, TOL[dtype], "decode out step %d" % s, dtype)
    assert_close(host(S), S_ref, TOL[dtype], "decode state")


def test_decode_equals_prefill_of_one_token():
    d = _decode_inputs(N=16, H=4, steps=1, dtype=torch.bfloat16, seed=21)
    S = d["state"].clone()
    out = torch.empty(16, 4, 128, dtype=torch.bfloat16, device="cuda")
    K.kda_decode_step(d["q"][0], d["k"][0], d["v"][0], d["g"][0], d["beta"][0], S, out)
    inp = dict(q=d["q"][0], k=d["k"][0], v=d["v"][0], g=d["g"][0], beta=d["beta"][0],
               initial_state=d["state"], cu_seqlens=torch.arange(17, dtype=torch.int32, device="cuda"))
    po, pf = run_prefill(inp)
    assert_close(host(out), host(po), 2 * TOL[torch.bfloat16], "decode vs prefill T=1 out", torch.bfloat16, ulps=1.0)
    assert_close(host(S), host(pf), 2 * TOL[torch.bfloat16], "decode vs prefill T=1 state")


def test_64_decode_steps_equal_64_token_prefill():
    N, H, steps = 8, 2, 64
    d = _decode_inputs(N=N, H=H, steps=steps, dtype=torch.bfloat16, seed=22)
    S = d["state"].clone()
    outs = []
    for s in range(steps):
        o = torch.empty(N, H, 128, dtype=torch.bfloat16, device="cuda")
        K.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, o)
        outs.append(o)
    dec = torch.stack(outs)                                   # [steps, N, H, dv]
    perm = lambda x: x.transpose(0, 1).reshape(N * steps, *x.shape[2:]).contiguous()
    inp = dict(q=perm(d["q"]), k=perm(d["k"]), v=perm(d["v"]), g=perm(d["g"]), beta=perm(d["beta"]),
               initial_state=d["state"], cu_seqlens=torch.arange(N + 1, dtype=torch.int32, device="cuda") * steps)
    po, pf = run_prefill(inp)
    assert_close(host(dec.transpose(0, 1).reshape(N * steps, H, 128)), host(po), 2 * TOL[torch.bfloat16],
                 "64 decode vs prefill out", torch.bfloat16, ulps=1.0)
    assert_close(host(S), host(pf), 2 * TOL[torch.bfloat16], "64 decode vs prefill state")
