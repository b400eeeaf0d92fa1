"""Operand range of the 16-bit path (bf16 q/k/v: fp16 MFMA operands).

The recurrence of card "KDA 单头递归" (page ailearn.mscapital.top/kimi-k3.html)
gives beta no range and does not normalise keys, so these cases leave the
synthetic workloads' unit keys and beta in (0, 1):

* keys of norm 8, 32 and 64 (beta scaled so that beta |k|^2 stays in (0, 2),
  where the step is non-expansive), with queries of norm about 16;
* spike keys (one channel = 64) under a constant gate of -10.9/32 per token,
  so that a 32-token chunk decays by e^-10.9, just inside the e^-11 span of
  the chunk-start reference: the column operand k e^-Gamma / 32 of such a
  chunk would reach 1.1e5, beyond fp16 range, and the chunk must take the
  sub-tile references instead;
* constant beta of 2, 4 and -0.5 with unit keys;
* gates spread so that about half the chunks take either reference.

Each case runs kda_prefill (default tiling and 64-token chunks) and
kda_prefill_cp (automatic and short segments) against the fp64 oracle, to
the bf16 tolerance rule of tests/kda_parity.py.
"""
import pytest
import torch

from gated_delta_rule_40_amd import inputs as I
from gated_delta_rule_40_amd import libkda as K
from kda_parity import TOL, assert_close, host, log, oracle_prefill, run_prefill, run_prefill_cp, to_dev

pytestmark = pytest.mark.gpu

LENGTHS = [300, 77, 1, 160]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    K.load()


def _inputs(seed, knorm=1.0, beta_scale=None, beta_const=None, qscale=1.0, spike_every=0, g_const=None,
            g_lo=-5.0 / 16.0):
    inp = I.random_prefill(LENGTHS, H=2, dtype=torch.bfloat16, seed=seed, g_lo=g_lo)
    k = inp["k"].float() * knorm
    if spike_every:
        rows = torch.arange(0, k.shape[0], spike_every)
        k[rows] = 0.0
        k[rows, :, 5] = knorm
    inp["k"] = k.to(torch.bfloat16)
    inp["q"] = (inp["q"].float() * qscale).to(torch.bfloat16)
    if beta_scale is not None:
        inp["beta"] = (inp["beta"] * beta_scale).contiguous()
    if beta_const is not None:
        inp["beta"] = torch.full_like(inp["beta"], beta_const)
    if g_const is not None:
        inp["g"] = torch.full_like(inp["g"], g_const)
    return to_dev(inp)


def _check_all_entries(inp, label):
    ref_out, ref_fin = oracle_prefill(inp)
    tol = TOL[torch.bfloat16]
    runs = (("prefill", lambda: run_prefill(inp)),
            ("prefill chunk 64", lambda: run_prefill(inp, chunk=64, dv_block=64)),
            ("prefill_cp", lambda: run_prefill_cp(inp)),
            ("prefill_cp seg 64", lambda: run_prefill_cp(inp, seg_len=64)))
    for name, run in runs:
        log("[range] %s: %s" % (label, name))
        out, fin = run()
        assert_close(host(out), ref_out, tol, "%s %s out" % (label, name), torch.bfloat16)
        assert_close(host(fin), ref_fin, tol, "%s %s final" % (label, name))


@pytest.mark.parametrize("knorm", [8.0, 32.0, 64.0])
def test_unnormalised_keys(knorm):
    _check_all_entries(_inputs(40, knorm=knorm, beta_scale=2.0 / knorm ** 2, qscale=16.0), "|k|=%g" % knorm)


@pytest.mark.parametrize("knorm", [32.0, 64.0])
def test_spike_keys_at_the_edge_of_the_chunk_span(knorm):
    # k_c = knorm on one channel every third token; every chunk decays by
    # e^-10.9 on every channel (fast-path span), so k e^-Gamma / 32 would
    # reach knorm * 1700 for the chunk's last tokens
    inp = _inputs(41, knorm=knorm, beta_scale=1.0 / knorm ** 2, spike_every=3, g_const=-10.9 / 32)
    _check_all_entries(inp, "spike %g, g=-10.9/32" % knorm)


@pytest.mark.parametrize("beta", [2.0, 4.0, -0.5])
def test_constant_beta_outside_unit_interval(beta):
    _check_all_entries(_inputs(42, beta_const=beta), "beta=%g" % beta)


def test_mixed_chunk_references_with_large_keys():
    # g ~ U(-0.69, 0): chunk spans scatter around e^-11, so neighbouring
    # chunks take different references; keys of norm 16
    inp = _inputs(43, knorm=16.0, beta_scale=1.0 / 256, g_lo=-0.69)
    _check_all_entries(inp, "mixed spans |k|=16")
