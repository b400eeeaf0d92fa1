"""Parity at full size on every output: the 4 x 16,384-token x 32-head and the
1,048,576-token x 16-head prefill workloads (every (sequence, head) unit, for
kda_prefill and for kda_prefill_cp at its automatic segment length, which is
what bench.py times), the 512 x 32 decode workload (every unit, all 64
in-place steps), and the backward on the two workloads bench.py times it on
(every unit of both).

The result being checked is the recurrence of card "KDA 单头递归" (page
ailearn.mscapital.top/kimi-k3.html), computed by the fp64 oracle on host
copies of the very tensors the GPU read.  Host memory stays bounded: the
1M-token workload is checked eight heads at a time and the decode workload
128 sequences at a time, with StreamingCompare applying the tolerance rule of
tests/kda_parity.py (RMS over the whole tensor) across the pieces.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_40_amd import inputs as I
from gated_delta_rule_40_amd import libkda as K
from kda_parity import (TOL, StreamingCompare, host, log, oracle_threads, run_prefill, run_prefill_cp)
from oracle import kda_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOK_BLOCK = 1 << 16          # tokens per host comparison block


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    K.load()


def _prefill_every_unit(wl_name, head_group):
    wl = I.WORKLOADS[wl_name]
    inp = I.make_prefill(wl, device="cuda")
    T, H = inp["q"].shape[0], inp["q"].shape[1]
    N = inp["cu_seqlens"].shape[0] - 1
    log("[%s] T=%d H=%d N=%d lengths=%s oracle threads=%d" % (wl_name, T, H, N, inp["lengths"], oracle_threads()))
    runs = {}
    log("[%s] kda_prefill" % wl_name)
    runs["kda_prefill"] = run_prefill(inp)
    log("[%s] kda_prefill_cp (automatic seg_len)" % wl_name)
    runs["kda_prefill_cp"] = run_prefill_cp(inp, seg_len=0)
    tol = TOL[torch.bfloat16]
    cmp_out = {name: StreamingCompare("%s %s out" % (name, wl_name), tol, torch.bfloat16) for name in runs}
    cmp_fin = {name: StreamingCompare("%s %s final" % (name, wl_name), tol) for name in runs}
    cu = inp["cu_seqlens"].cpu().numpy()
    init = inp["initial_state"]
    for h0 in range(0, H, head_group):
        h1 = min(H, h0 + head_group)
        sub = {key: inp[key][:, h0:h1].float().cpu().numpy() for key in ("q", "k", "v", "g", "beta")}
        log("[%s] oracle heads %d..%d" % (wl_name, h0, h1 - 1))
        ref_out, ref_fin = O.prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                                     None if init is None else init[:, h0:h1].double().cpu().numpy(), cu,
                                     num_threads=oracle_threads())
        del sub
        for name, (out, fin) in runs.items():
            for t0 in range(0, T, TOK_BLOCK):
                t1 = min(T, t0 + TOK_BLOCK)
                cmp_out[name].add(out[t0:t1, h0:h1].float().cpu().numpy(), ref_out[t0:t1])
            cmp_fin[name].add(fin[:, h0:h1].cpu().numpy(), ref_fin)
        del ref_out, ref_fin
    for name in runs:
        cmp_out[name].check()
        cmp_fin[name].check()


@pytest.mark.timeout(900)
def test_parity_4x16384_h32_every_unit():
    """B=4 x 16,384 tokens, H=32, bf16, N(0, 0.1) initial state: all 128 units."""
    _prefill_every_unit("prefill_4x16384_h32", head_group=32)


@pytest.mark.timeout(900)
def test_parity_varlen_1m_h16_every_unit():
    """8 sequences, 1,048,576 tokens, H=16, bf16, zero initial state: all 128 units."""
    _prefill_every_unit("prefill_varlen_1m_h16", head_group=8)


@pytest.mark.timeout(900)
def test_decode_512x32_64_steps_every_unit():
    """512 sequences x 32 heads, 1 GiB fp32 state, 64 in-place steps: every
    output of every step and the state after the last step."""
    wl = I.WORKLOADS["decode_512x32"]
    d = I.make_decode(wl, device="cuda")
    N, H, steps = wl.num_seqs, wl.heads, wl.steps
    init = d["state"].cpu()                    # the GPU updates d["state"] in place
    S = d["state"]
    out = torch.empty(steps, N, H, 128, dtype=torch.bfloat16, device="cuda")
    log("[decode_512x32] %d steps on the GPU" % steps)
    for s in range(steps):
        K.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, out[s])
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    cmp_out = StreamingCompare("decode_512x32 out (64 steps)", tol, torch.bfloat16)
    cmp_S = StreamingCompare("decode_512x32 state after 64 steps", tol)
    threads = oracle_threads()
    SB = 128
    for n0 in range(0, N, SB):
        n1 = min(N, n0 + SB)
        log("[decode_512x32] oracle sequences %d..%d" % (n0, n1 - 1))
        S_ref = init[n0:n1].double().numpy()
        for s in range(steps):
            o, S_ref = O.decode_step(host(d["q"][s, n0:n1]), host(d["k"][s, n0:n1]), host(d["v"][s, n0:n1]),
                                     host(d["g"][s, n0:n1]), host(d["beta"][s, n0:n1]), S_ref, num_threads=threads)
            cmp_out.add(host(out[s, n0:n1]), o)
        cmp_S.add(host(S[n0:n1]), S_ref)
    cmp_out.check()
    cmp_S.check()


def _backward_vs_oracle(wl_name, head_group, threads):
    """kda_backward on the whole workload, as bench.py times it (dout ~ N(0, 1)
    in bf16 from a generator seeded with 7 on the device, no final-state
    gradient), against the fp64 oracle backward on every unit, head_group
    heads at a time (the oracle keeps every state of a unit in host memory,
    so each group runs with few threads)."""
    wl = I.WORKLOADS[wl_name]
    inp = I.make_prefill(wl, device="cuda")
    T, H = inp["q"].shape[0], inp["q"].shape[1]
    gen = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(T, H, 128, generator=gen, device="cuda").to(torch.bfloat16)
    log("[%s backward] T=%d H=%d lengths=%s, oracle %d heads at a time with %d threads" %
        (wl_name, T, H, inp["lengths"], head_group, threads))
    gr = K.kda_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
                        inp["cu_seqlens"], dout, None)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    keys = ("dq", "dk", "dv", "dg", "dbeta", "dinit")
    cmp = {key: StreamingCompare("%s backward %s" % (wl_name, key), tol) for key in keys}
    init = inp["initial_state"]
    for h0 in range(0, H, head_group):
        h1 = min(H, h0 + head_group)
        sel = lambda x: x[:, h0:h1].contiguous()
        ref = O.backward(host(sel(inp["q"])), host(sel(inp["k"])), host(sel(inp["v"])), host(sel(inp["g"])),
                         host(sel(inp["beta"])), None if init is None else sel(init).double().cpu().numpy(),
                         inp["cu_seqlens"].cpu().numpy(), sel(dout).double().cpu().numpy(), None,
                         num_threads=threads)
        for key in keys:
            got = sel(gr[key]).cpu().numpy()
            for t0 in range(0, got.shape[0], TOK_BLOCK):
                cmp[key].add(got[t0:t0 + TOK_BLOCK], ref[key][t0:t0 + TOK_BLOCK])
        del ref
    for key in keys:
        cmp[key].check()


@pytest.mark.timeout(600)
def test_backward_t4096_h8_every_unit():
    """kda_backward on the 4,096-token x 8-head workload: every gradient of every unit."""
    _backward_vs_oracle("prefill_t4096_h8", 8, min(oracle_threads(), 8))


@pytest.mark.timeout(900)
def test_backward_4x16384_h32_every_unit():
    """kda_backward on 4 x 16,384 tokens x 32 heads (segments of 256 chunks, the
    gradient summaries' head walk): every gradient of all 128 units, four
    heads at a time."""
    _backward_vs_oracle("prefill_4x16384_h32", 4, min(oracle_threads(), 4))
