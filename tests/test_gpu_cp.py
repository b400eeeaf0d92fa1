"""GPU parity of the context-parallel prefill (kda_prefill_cp) against the
fp64 oracle, through the C ABI.

kda_prefill_cp splits every sequence into segments, summarises each segment
by its end state from zero and its transition (the recurrence is affine in
the entering state), chains the summaries into entering states and reruns the
segments for the outputs.  The oracle knows nothing of segments: it runs the
token recurrence straight through, so these tests check the whole scheme.
Comparisons use the rule of tests/kda_parity.py (tol * RMS + half an ulp of
the stored dtype).  Small seg_len values force many segments per sequence,
one-chunk segments and ragged last segments; negative seg_len values cut the
packed chunk order into pieces that span sequence boundaries.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_40_amd import inputs as I
from gated_delta_rule_40_amd import libkda as K
from kda_parity import TOL, assert_close, host, log, oracle_prefill, run_prefill, run_prefill_cp, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    K.load()


def _check_cp(inp, tol, label, seg_len, use_init=True):
    N = inp["cu_seqlens"].shape[0] - 1
    log("[prefill_cp] %s seg_len=%d T=%d H=%d N=%d dtype=%s init=%s" % (
        label, seg_len, inp["q"].shape[0], inp["q"].shape[1], N, inp["q"].dtype, use_init))
    out, fin = run_prefill_cp(inp, seg_len=seg_len, use_init=use_init)
    ref_out, ref_fin = oracle_prefill(inp, use_init=use_init)
    cu = inp["cu_seqlens"].cpu().numpy()
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in range(N)])
    assert_close(host(out)[rows], ref_out[rows], tol, label + " out", out.dtype)
    assert_close(host(fin), ref_fin, tol, label + " final_state")
    return out, fin


LENGTHS = [1, 17, 64, 0, 100, 63, 65, 130, 200, 333]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("seg_len", [32, 64, 96, 128])
def test_cp_ragged_vs_oracle(dtype, seg_len):
    inp = to_dev(I.random_prefill(LENGTHS, H=3, dtype=dtype, seed=30))
    _check_cp(inp, TOL[dtype], "cp_ragged", seg_len)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("seg_len", [-32, -64, -96, -160])
def test_cp_pieces_ragged_vs_oracle(dtype, seg_len):
    # pieces (negative seg_len): the packed chunk order is cut into pieces of
    # -seg_len / 32 chunks and each sequence into its parts in them, so a
    # workgroup's piece holds the end of one sequence, whole short ones,
    # empty ones and the start of the next, and runs them in turn
    inp = to_dev(I.random_prefill(LENGTHS, H=3, dtype=dtype, seed=30))
    _check_cp(inp, TOL[dtype], "cp_pieces", seg_len)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cp_pieces_null_initial_state(dtype):
    inp = to_dev(I.random_prefill([250, 0, 77, 5], H=2, dtype=dtype, seed=31))
    _check_cp(inp, TOL[dtype], "cp_pieces_null_init", -64, use_init=False)


@pytest.mark.parametrize("g_lo", [-5.0 / 16.0, -0.002])
def test_cp_pieces_tail_vs_oracle(g_lo):
    # pieces of 48 chunks with 32 heads: more (segment, head) pairs than
    # compute units, so the summaries run in the 256-column form and walk a
    # segment's last 36 chunks first (in full again when the transition over
    # them is not exactly zero, g in (-0.002, 0]), and the outputs run in
    # two-tile workgroups, one per (piece, head)
    inp = to_dev(I.random_prefill([4000, 100, 6000, 3333, 3067], H=32, dtype=torch.bfloat16, seed=44, g_lo=g_lo))
    _check_cp(inp, TOL[torch.bfloat16], "cp_pieces_tail_g_lo=%g" % g_lo, -1536)


@pytest.mark.parametrize("lengths,seg_len", [
    ([64, 64, 0, 128, 0], -64),         # piece ends on sequence ends; empty sequences between and last
    ([64, 64, 0, 128, 0], -99968),      # one piece holds every sequence: one workgroup per head walks them all
    ([0, 0, 31, 0], -32),               # a single ragged chunk among empty sequences
    ([700, 1, 1, 1, 900], -96),         # one-token sequences sharing a piece with the ends of long ones
])
def test_cp_pieces_edges_vs_oracle(lengths, seg_len):
    inp = to_dev(I.random_prefill(lengths, H=2, dtype=torch.bfloat16, seed=46))
    _check_cp(inp, TOL[torch.bfloat16], "cp_pieces_edges", seg_len)


def test_cp_pieces_run_to_run_bitwise_determinism():
    inp = to_dev(I.random_prefill([333, 640, 17, 0, 2000], H=4, dtype=torch.bfloat16, seed=45))
    o1, f1 = run_prefill_cp(inp, seg_len=-256)
    o2, f2 = run_prefill_cp(inp, seg_len=-256)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cp_null_initial_state(dtype):
    inp = to_dev(I.random_prefill([250, 0, 77], H=2, dtype=dtype, seed=31))
    _check_cp(inp, TOL[dtype], "cp_null_init", 64, use_init=False)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cp_page_gate_range(dtype):
    """g over the whole range (-5, 0), and its closed ends g = -5 and g = 0."""
    inp = to_dev(I.random_prefill([300, 47], H=2, dtype=dtype, seed=32, g_lo=-5.0))
    _check_cp(inp, TOL[dtype], "cp_g_in_(-5,0)", 64)
    for gval in (-5.0, 0.0):
        inp2 = dict(inp)
        inp2["g"] = torch.full_like(inp["g"], gval)
        _check_cp(inp2, TOL[dtype], "cp_g=%g" % gval, 64)


@pytest.mark.parametrize("seg_len", [0, 512])
def test_cp_t4096_h8_vs_oracle(seg_len):
    """B=1, H=8, T=4096, bf16, N(0, 0.1) initial state, every output: the
    automatic segment length (the one bench.py times) and 8 segments of 512."""
    inp = to_dev(I.make_prefill(I.WORKLOADS["prefill_t4096_h8"]))
    _check_cp(inp, TOL[torch.bfloat16], "cp_t4096_h8", seg_len)


def test_cp_single_segment_equals_plain_prefill_bitwise():
    """With one segment per sequence the segmented pass runs the plain kernel's
    arithmetic (32-token chunks, 64-column value blocks) from the same state."""
    inp = to_dev(I.random_prefill([45, 200, 1, 0, 96], H=2, dtype=torch.bfloat16, seed=33))
    o_ref, f_ref = run_prefill(inp, chunk=32, dv_block=64)
    o, f = run_prefill_cp(inp, seg_len=256)
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)


def test_cp_equals_plain_prefill_within_tolerance():
    inp = to_dev(I.random_prefill([1000, 517, 3], H=4, dtype=torch.bfloat16, seed=34))
    o_ref, f_ref = run_prefill(inp)
    for seg_len in (32, 128, 0, -64, -1024):
        o, f = run_prefill_cp(inp, seg_len=seg_len)
        assert_close(host(o), host(o_ref), 2 * TOL[torch.bfloat16], "cp(%d) vs plain out" % seg_len,
                     torch.bfloat16, ulps=1.0)
        assert_close(host(f), host(f_ref), 2 * TOL[torch.bfloat16], "cp(%d) vs plain final" % seg_len)


def test_cp_final_state_may_alias_initial_state():
    inp = to_dev(I.random_prefill([130, 640, 5], H=4, dtype=torch.bfloat16, seed=35))
    _, fin = run_prefill_cp(inp, seg_len=64)
    state = inp["initial_state"].clone()
    inp2 = dict(inp)
    inp2["initial_state"] = state
    run_prefill_cp(inp2, seg_len=64, fin=state)
    assert torch.equal(state, fin)


def test_cp_workspace_contents_are_ignored_and_reusable():
    big = to_dev(I.random_prefill([700, 300], H=3, dtype=torch.bfloat16, seed=36))
    small = to_dev(I.random_prefill([90, 200, 31], H=3, dtype=torch.bfloat16, seed=37))
    need = max(K.kda_prefill_cp_workspace_size(2, 1000, 3, 128, 128, torch.bfloat16, 32),
               K.kda_prefill_cp_workspace_size(3, 321, 3, 128, 128, torch.bfloat16, 32))
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    o_fresh, f_fresh = run_prefill_cp(small, seg_len=32)
    run_prefill_cp(big, seg_len=32, workspace=ws)
    o, f = run_prefill_cp(small, seg_len=32, workspace=ws)
    assert torch.equal(o, o_fresh) and torch.equal(f, f_fresh)


def test_cp_empty_sequences_and_untouched_rows():
    inp = to_dev(I.random_prefill([0, 140, 0, 25], H=2, dtype=torch.bfloat16, seed=38))
    T = inp["q"].shape[0]
    pad = lambda x: torch.cat([x, torch.zeros((7,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)])
    for key in ("q", "k", "v", "g", "beta"):
        inp[key] = pad(inp[key]).contiguous()
    out = torch.full((T + 7, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out, fin = run_prefill_cp(inp, seg_len=32, out=out)
    assert torch.isnan(out[T:].float()).all()
    assert torch.equal(fin[0], inp["initial_state"][0]) and torch.equal(fin[2], inp["initial_state"][2])
    ref_out, ref_fin = oracle_prefill(inp)
    assert_close(host(out)[:T], ref_out[:T], TOL[torch.bfloat16], "cp untouched out", torch.bfloat16)
    assert_close(host(fin), ref_fin, TOL[torch.bfloat16], "cp untouched final_state")


@pytest.mark.parametrize("dtype,seg_len", [(torch.float32, 1024), (torch.float32, 1088), (torch.bfloat16, 1024)])
def test_cp_summary_units_vs_oracle(dtype, seg_len):
    # (total_tokens / seg_len) x heads >= 256 and segments of 1,024 tokens or
    # more: for fp32 the summaries and the combine run on units, four (1,024:
    # 32 chunks) or two (1,088: 34 chunks) per segment, and every segment's
    # output run starts from its first unit's state; bf16 keeps whole
    # segments (its summaries take the tail walk, 32 chunks < 36 here: in full)
    inp = to_dev(I.random_prefill([2200, 0, 1500, 700, 1], H=64, dtype=dtype, seed=41))
    assert (inp["q"].shape[0] // seg_len) * 64 >= 256
    _check_cp(inp, TOL[dtype], "cp_units", seg_len)


@pytest.mark.parametrize("g_lo", [-5.0 / 16.0, -0.002])
def test_cp_summary_tail_vs_oracle(g_lo):
    # units of 256 chunks (seg_len 8,192; H = 64 puts the summaries in the
    # 256-column form that holds every transition column).  Under the
    # workloads' decay (g in (-5/16, 0]) the transition over a unit's last 36
    # chunks is exactly zero, and each unit is summarised from those chunks
    # alone; with g in (-0.002, 0] it is not, and each unit is walked again
    # in full.  Both against the oracle's straight token walk.
    inp = to_dev(I.random_prefill([20000, 9000, 300], H=64, dtype=torch.bfloat16, seed=43, g_lo=g_lo))
    _check_cp(inp, TOL[torch.bfloat16], "cp_tail_g_lo=%g" % g_lo, 8192)


@pytest.mark.parametrize("dtype,nseq,seg_len", [(torch.float32, 300, 64), (torch.bfloat16, 300, 64),
                                                (torch.bfloat16, 256, 64), (torch.bfloat16, 257, 64),
                                                (torch.bfloat16, 300, -64), (torch.float32, 300, -96),
                                                (torch.bfloat16, 600, -160), (torch.bfloat16, 256, -64)])
def test_cp_many_sequences_vs_oracle(dtype, nseq, seg_len):
    # more than 256 sequences: the plan kernel walks them in several blocks of
    # 256 (segment and chunk numbering, the order of sequences by unit count;
    # with pieces, the total chunk count first and each block's last piece
    # passed on to the next); up to 256 the plans are built inside the
    # chunk-operand launch
    rng = np.random.default_rng(40)
    lengths = [int(x) for x in rng.integers(0, 90, size=nseq)]
    lengths[7], lengths[123], lengths[nseq - 1] = 0, 257, 300
    inp = to_dev(I.random_prefill(lengths, H=2, dtype=dtype, seed=40))
    _check_cp(inp, TOL[dtype], "cp_many_seqs_%d" % nseq, seg_len)


def test_cp_run_to_run_bitwise_determinism():
    inp = to_dev(I.random_prefill([333, 640, 17], H=4, dtype=torch.bfloat16, seed=39))
    o1, f1 = run_prefill_cp(inp, seg_len=64)
    o2, f2 = run_prefill_cp(inp, seg_len=64)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cp_every_image_slot_but_the_spare_one_used(dtype):
    # every length is 1 mod 32, so the chunk count reaches its bound less one:
    # the chunk-operand pass's placeholder stores go to the one image slot
    # past the last chunk, next to images the passes after it read
    lengths = [33, 1, 97, 65, 129]
    total = sum(lengths)
    chunks = sum((n + 31) // 32 for n in lengths)
    assert chunks == total // 32 + len(lengths)                # = the slots the workspace holds, less one
    inp = to_dev(I.random_prefill(lengths, H=3, dtype=dtype, seed=42))
    for seg_len in (32, 64):
        _check_cp(inp, TOL[dtype], "cp_tight_slots", seg_len)
