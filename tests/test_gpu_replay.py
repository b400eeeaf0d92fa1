"""GPU parity of kda_decode_tokens (a few tokens per sequence with the state
kept on chip: speculative-decoding verification and replay of the accepted
prefix) against the fp64 oracle, through the C ABI.  The oracle runs the plain
token recurrence over exactly the tokens the call processes."""
import numpy as np
import pytest
import torch

from gated_delta_rule_40_amd import inputs as I
from gated_delta_rule_40_amd import libkda as K
from kda_parity import TOL, assert_close, host, log
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    K.load()


def _draft(lengths, H, dtype, seed, g_lo=-5 / 16):
    inp = I.random_prefill(lengths, H=H, dtype=dtype, seed=seed, init="normal", g_lo=g_lo, device="cuda")
    return inp


def _oracle(inp, counts):
    """Oracle over the first counts[n] tokens of each sequence."""
    cu = inp["cu_seqlens"].cpu().numpy()
    rows = np.concatenate([np.arange(cu[n], cu[n] + counts[n]) for n in range(len(counts))]).astype(np.int64)
    sub = {key: host(inp[key])[rows] for key in ("q", "k", "v", "g", "beta")}
    scu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out, fin = O.prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                         inp["initial_state"].double().cpu().numpy(), scu)
    return rows, out, fin


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tokens_vs_oracle(dtype):
    rng = np.random.default_rng(40)
    lengths = [int(x) for x in rng.integers(0, 9, 24)]
    inp = _draft(lengths, H=3, dtype=dtype, seed=41)
    req = [int(x) for x in rng.integers(-1, 11, 24)]          # clamped to [0, length]
    counts = [min(max(r, 0), L) for r, L in zip(req, lengths)]
    log("[decode_tokens] lengths %s requested %s" % (lengths, req))
    T, H = inp["q"].shape[:2]
    out = torch.full((T, H, 128), float("nan"), dtype=dtype, device="cuda")
    state_out = torch.empty_like(inp["initial_state"])
    nt = torch.tensor(req, dtype=torch.int32, device="cuda")
    K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                        inp["initial_state"], state_out=state_out, out=out, num_tokens=nt)
    torch.cuda.synchronize()
    rows, ref_out, ref_fin = _oracle(inp, counts)
    got = host(out)
    assert_close(got[rows], ref_out, TOL[dtype], "decode_tokens out", dtype)
    assert_close(host(state_out), ref_fin, TOL[dtype], "decode_tokens state")
    untouched = np.setdiff1d(np.arange(T), rows)
    assert np.isnan(got[untouched]).all()


def test_tokens_equal_decode_steps_bitwise():
    """Each token's arithmetic is that of kda_decode_step."""
    N, H, steps = 16, 4, 5
    inp = _draft([steps] * N, H=H, dtype=torch.bfloat16, seed=42, g_lo=-5.0)
    state = inp["initial_state"].clone()
    out_t = torch.empty(N * steps, H, 128, dtype=torch.bfloat16, device="cuda")
    K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                        inp["initial_state"], state_out=state, out=out_t)
    S = inp["initial_state"].clone()
    for j in range(steps):
        idx = torch.arange(N, device="cuda") * steps + j
        o = torch.empty(N, H, 128, dtype=torch.bfloat16, device="cuda")
        K.kda_decode_step(*(inp[key][idx].contiguous() for key in ("q", "k", "v", "g", "beta")), S, o)
        assert torch.equal(o, out_t[idx])
    torch.cuda.synchronize()
    assert torch.equal(S, state)


def test_verify_then_replay_accepted_prefix():
    N, H, draft = 32, 4, 6
    rng = np.random.default_rng(43)
    inp = _draft([draft] * N, H=H, dtype=torch.bfloat16, seed=44)
    committed = inp["initial_state"].clone()
    # verify: outputs for every draft token, nothing committed
    out_v = torch.empty(N * draft, H, 128, dtype=torch.bfloat16, device="cuda")
    K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], committed,
                        state_out=None, out=out_v)
    torch.cuda.synchronize()
    assert torch.equal(committed, inp["initial_state"])
    _, ref_v, _ = _oracle(inp, [draft] * N)
    assert_close(host(out_v), ref_v, TOL[torch.bfloat16], "verify out", torch.bfloat16)
    # replay the accepted prefix in place, no outputs
    accepted = [int(x) for x in rng.integers(0, draft + 1, N)]
    nt = torch.tensor(accepted, dtype=torch.int32, device="cuda")
    K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], committed,
                        state_out=committed, out=None, num_tokens=nt)
    torch.cuda.synchronize()
    _, _, ref_fin = _oracle(inp, accepted)
    assert_close(host(committed), ref_fin, TOL[torch.bfloat16], "replayed state")
    # a sequence that accepted nothing keeps its state bit for bit
    for n, a in enumerate(accepted):
        if a == 0:
            assert torch.equal(committed[n], inp["initial_state"][n])


def test_replay_512x32_four_tokens():
    """512 sequences x 32 heads, 4 draft tokens each, every unit against the oracle."""
    N, H, draft = 512, 32, 4
    inp = _draft([draft] * N, H=H, dtype=torch.bfloat16, seed=45)
    state = torch.empty_like(inp["initial_state"])
    out = torch.empty(N * draft, H, 128, dtype=torch.bfloat16, device="cuda")
    K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                        inp["initial_state"], state_out=state, out=out)
    torch.cuda.synchronize()
    log("[decode_tokens] oracle on 512 x 32 units, 4 tokens each")
    _, ref_out, ref_fin = _oracle(inp, [draft] * N)
    assert_close(host(out), ref_out, TOL[torch.bfloat16], "512x32 out", torch.bfloat16)
    assert_close(host(state), ref_fin, TOL[torch.bfloat16], "512x32 state")


def test_odd_pair_count_and_runs_past_the_staged_tokens():
    """An odd number of (sequence, head) pairs (a workgroup takes two: the last
    one has a single pair) and sequences longer than the tokens whose vectors
    are read up front (four), against the oracle."""
    lengths = [9, 1, 0, 13, 5]                                 # 3 heads: 15 pairs
    inp = _draft(lengths, H=3, dtype=torch.bfloat16, seed=46)
    T, H = inp["q"].shape[:2]
    out = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    state_out = torch.empty_like(inp["initial_state"])
    K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                        inp["initial_state"], state_out=state_out, out=out)
    torch.cuda.synchronize()
    rows, ref_out, ref_fin = _oracle(inp, lengths)
    assert_close(host(out)[rows], ref_out, TOL[torch.bfloat16], "odd pairs out", torch.bfloat16)
    assert_close(host(state_out), ref_fin, TOL[torch.bfloat16], "odd pairs state")


def test_no_tokens_commits_the_state_unchanged():
    """total_tokens = 0: no token is processed; state_out receives state_in
    bit for bit (and in place it stays as it is)."""
    N, H = 3, 2
    lib = K.load()
    dummy = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")   # never read
    gdummy = torch.zeros(4, 128, dtype=torch.float32, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    state_in = torch.randn(N, H, 128, 128, dtype=torch.float32, device="cuda")
    keep = state_in.clone()
    state_out = torch.full_like(state_in, float("nan"))
    p = dummy.data_ptr()
    for so in (state_out, state_in):
        st = lib.kda_decode_tokens(p, p, p, gdummy.data_ptr(), gdummy.data_ptr(), cu.data_ptr(), None,
                                   state_in.data_ptr(), so.data_ptr(), N, 0, H, 128, 128, K.KDA_BF16, p,
                                   K._stream(None))
        assert st == K.KDA_OK, K.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(state_out, keep)
    assert torch.equal(state_in, keep)
