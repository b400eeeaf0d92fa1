"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked example, the page's product form written with explicit
matrices, closed forms (beta = 0, alpha = 1 with orthonormal keys),
structural identities (continuation, varlen packing, segment composition,
linearity), a contraction bound, and a second independent implementation.
The last test plants plausible mistakes in a copy of the recurrence and
checks that the pins reject every one of them.

Method source: page "Kimi K3 把 3T 级模型、百万上下文和 Agent 训练接成一套系统"
(ailearn.mscapital.top/kimi-k3.html), cards "KDA 单头递归" (the recurrence),
"g ∈ (-5, 0)" (gate range) and "传固定状态片段" (fixed-size state fragments
composed by a prefix combination).
"""
import os

import numpy as np
import pytest

from oracle import kda_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example_dk2.txt")


def _rand_inputs(rng, lengths, H, dk, dv, g_lo=-5 / 16, beta=None, unit_k=True, init=True):
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, dk)).astype(np.float32) * dk ** -0.5
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    g = (rng.random((T, H, dk)) * g_lo).astype(np.float32)
    b = (1 / (1 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32) if beta is None \
        else np.full((T, H), beta, np.float32)
    S0 = rng.standard_normal((len(lengths), H, dk, dv)) * 0.1 if init else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, g, b, S0, cu


def _parse_golden():
    data = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            data[key.strip()] = [[float(x) for x in grp.split()] for grp in val.split("|")]
    return {k: np.array(v) for k, v in data.items()}


# ---------------------------------------------------------------- hand example
@pytest.mark.parametrize("impl", ["c", "numpy"])
def test_hand_worked_example(impl):
    d = _parse_golden()
    T = d["k"].shape[0]
    k = d["k"].reshape(T, 1, 2)
    v = d["v"].reshape(T, 1, 2)
    q = d["q"].reshape(T, 1, 2)
    g = np.log(d["alpha"]).reshape(T, 1, 2)
    beta = d["beta"].reshape(T, 1)
    cu = [0, T]
    fn = O.prefill if impl == "c" else O.numpy_prefill
    out, fin = fn(q, k, v, g, beta, None, cu)
    np.testing.assert_allclose(out[:, 0, :], d["out"], atol=1e-6)
    np.testing.assert_allclose(fin[0, 0], d["final_state"].reshape(2, 2), atol=1e-6)


# ---------------------------------------------------------- product form (P1)
def _product_form(q, k, v, g, beta, S0):
    """S_t = A_t S_{t-1} + beta_t k_t v_t^T with A_t = (I - beta k k^T) Diag(alpha),
    unrolled as S_T = A_T..A_1 S_0 + sum_t A_T..A_{t+1} beta_t k_t v_t^T, using
    explicit dk x dk matrices; o_t = S_t^T q_t on every prefix."""
    T, dk = k.shape
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    A = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    outs = []
    S_t = None
    for t_end in range(1, T + 1):
        prod = np.eye(dk)
        for t in range(t_end):
            prod = A[t] @ prod
        S_t = prod @ S0
        for t in range(t_end):
            tail = np.eye(dk)
            for s in range(t + 1, t_end):
                tail = A[s] @ tail
            S_t = S_t + tail @ (beta[t] * np.outer(k[t], v[t]))
        outs.append(S_t.T @ q[t_end - 1])
    return np.array(outs), S_t


@pytest.mark.parametrize("seed,dk,dv,T,g_lo,unit_k", [
    (0, 5, 3, 8, -5 / 16, True),
    (1, 4, 6, 7, -5.0, True),      # the pages' full gate range
    (2, 3, 3, 6, -1.0, False),     # keys not normalised: the recurrence does not assume it
    (3, 8, 2, 5, -0.1, True),
])
def test_product_form(seed, dk, dv, T, g_lo, unit_k):
    rng = np.random.default_rng(seed)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [T], 1, dk, dv, g_lo=g_lo, unit_k=unit_k)
    out, fin = O.prefill(q, k, v, g, b, S0, cu)
    ref_out, ref_S = _product_form(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], S0[0, 0])
    np.testing.assert_allclose(out[:, 0], ref_out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], ref_S, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------- beta = 0 (P2)
def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(5)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [50], 2, 16, 12, g_lo=-5.0, beta=0.0)
    out, fin = O.prefill(q, k, v, g, b, S0, cu)
    G = np.cumsum(g.astype(np.float64), axis=0)          # [T, H, dk]
    for h in range(2):
        np.testing.assert_allclose(fin[0, h], np.exp(G[-1, h])[:, None] * S0[0, h], rtol=1e-12, atol=1e-300)
        ref = np.einsum("tc,cj->tj", q[:, h].astype(np.float64) * np.exp(G[:, h]), S0[0, h])
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-10, atol=1e-14)


# ---------------------------------- alpha = 1 with orthonormal keys (P3)
def test_alpha_one_orthonormal_overwrite():
    rng = np.random.default_rng(6)
    dk, dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T.astype(np.float32)                      # rows orthonormal (to fp32 rounding)
    k = keys[rng.permutation(dk)][:T].reshape(T, 1, dk)
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    q = rng.standard_normal((T, 1, dk)).astype(np.float32)
    g = np.zeros((T, 1, dk), np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv))
    kk = k[:, 0].astype(np.float64)
    # beta = 1: each key reads back exactly its value; other keys are untouched
    _, fin = O.prefill(q, k, v, g, np.ones((T, 1), np.float32), S0, [0, T])
    for t in range(T):
        np.testing.assert_allclose(fin[0, 0].T @ kk[t], v[t, 0], atol=1e-6)
    # general beta: S_t^T k_t = (1 - beta) S_{t-1}^T k_t + beta v_t  (one token)
    for beta in (0.0, 0.3, 0.75, 1.0):
        _, f1 = O.prefill(q[:1], k[:1], v[:1], g[:1], np.full((1, 1), beta, np.float32), S0, [0, 1])
        lhs = f1[0, 0].T @ kk[0]
        rhs = (1 - beta) * (S0[0, 0].T @ kk[0]) + beta * v[0, 0]
        np.testing.assert_allclose(lhs, rhs, atol=1e-6)
        # directions orthogonal to k_0 keep their read-out
        np.testing.assert_allclose(f1[0, 0].T @ kk[1], S0[0, 0].T @ kk[1], atol=1e-6)


# ------------------------------------------------- continuation (P4)
def test_continuation_split_equals_whole():
    rng = np.random.default_rng(7)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [90], 3, 16, 16, g_lo=-2.0)
    out, fin = O.prefill(q, k, v, g, b, S0, cu)
    for split in (1, 37, 89):
        o1, f1 = O.prefill(q[:split], k[:split], v[:split], g[:split], b[:split], S0, [0, split])
        o2, f2 = O.prefill(q[split:], k[split:], v[split:], g[split:], b[split:], f1, [0, 90 - split])
        np.testing.assert_allclose(np.concatenate([o1, o2]), out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(f2, fin, rtol=1e-12, atol=1e-12)


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(8)
    N, H, dk, dv, steps = 3, 2, 16, 8, 10
    q, k, v, g, b, _, _ = _rand_inputs(rng, [steps * N], H, dk, dv, g_lo=-1.0)
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.1
    # token s of sequence n lives at row s*N + n (decode step-major layout)
    S = S0.copy()
    dec_out = np.zeros((steps, N, H, dv))
    for s in range(steps):
        sl = slice(s * N, (s + 1) * N)
        dec_out[s], S = O.decode_step(q[sl], k[sl], v[sl], g[sl], b[sl], S)
    # same tokens packed sequence-major for prefill
    perm = np.array([s * N + n for n in range(N) for s in range(steps)])
    cu = np.arange(N + 1) * steps
    out, fin = O.prefill(q[perm], k[perm], v[perm], g[perm], b[perm], S0, cu)
    np.testing.assert_allclose(out.reshape(N, steps, H, dv).transpose(1, 0, 2, 3), dec_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fin, S, rtol=1e-12, atol=1e-13)


# ------------------------------------------------- varlen packing (P5)
def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(9)
    lengths = [5, 0, 33, 1, 17]
    q, k, v, g, b, S0, cu = _rand_inputs(rng, lengths, 2, 8, 8, g_lo=-5.0)
    out, fin = O.prefill(q, k, v, g, b, S0, cu)
    for n, L in enumerate(lengths):
        s, e = cu[n], cu[n + 1]
        o, f = O.prefill(q[s:e], k[s:e], v[s:e], g[s:e], b[s:e], S0[n:n + 1], [0, L])
        np.testing.assert_allclose(out[s:e], o, rtol=0, atol=0)
        np.testing.assert_allclose(fin[n], f[0], rtol=0, atol=0)
    # empty sequence: final state equals the initial state
    np.testing.assert_array_equal(fin[1], S0[1])


def test_null_initial_state_is_zero():
    rng = np.random.default_rng(10)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [20, 7], 2, 8, 4)
    o1, f1 = O.prefill(q, k, v, g, b, None, cu)
    o2, f2 = O.prefill(q, k, v, g, b, np.zeros_like(S0), cu)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


# ------------------------------------ segment composition / CP identity (P7)
def test_segment_composition_identity():
    """A run is affine in its entering state: S_T = M S_0 + S_T|_{S_0=0}, where the
    segment transition M is the run of the same segment with v = 0 from S_0 = I.
    Two segments compose as S = M_2 (M_1 S_0 + S_1^0) + S_2^0 (fixed-size state
    fragments combined by a prefix combination)."""
    rng = np.random.default_rng(11)
    dk, dv, T1, T2 = 12, 7, 40, 25
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [T1 + T2], 1, dk, dv, g_lo=-1.0)
    _, fin = O.prefill(q, k, v, g, b, S0, cu)
    eye = np.eye(dk)[None, None]
    zv = np.zeros((T1 + T2, 1, dk), np.float32)
    s1, s2 = slice(0, T1), slice(T1, T1 + T2)
    _, M1 = O.prefill(q[s1], k[s1], zv[s1], g[s1], b[s1], eye, [0, T1])
    _, M2 = O.prefill(q[s2], k[s2], zv[s2], g[s2], b[s2], eye, [0, T2])
    _, Z1 = O.prefill(q[s1], k[s1], v[s1], g[s1], b[s1], None, [0, T1])
    _, Z2 = O.prefill(q[s2], k[s2], v[s2], g[s2], b[s2], None, [0, T2])
    comb = M2[0, 0] @ (M1[0, 0] @ S0[0, 0] + Z1[0, 0]) + Z2[0, 0]
    np.testing.assert_allclose(comb, fin[0, 0], rtol=1e-11, atol=1e-12)


# ----------------------------------------------------- linearity (P8)
def test_linear_in_values_and_state():
    rng = np.random.default_rng(12)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [30], 2, 8, 6)
    v2 = rng.standard_normal(v.shape).astype(np.float32)
    S02 = rng.standard_normal(S0.shape)
    a1, a2 = 0.75, -1.5
    o1, f1 = O.prefill(q, k, v, g, b, S0, cu)
    o2, f2 = O.prefill(q, k, v2, g, b, S02, cu)
    vc = (a1 * v.astype(np.float64) + a2 * v2.astype(np.float64)).astype(np.float32)
    oc, fc = O.prefill(q, k, vc, g, b, a1 * S0 + a2 * S02, cu)
    # vc is rounded to fp32 once; allow that rounding
    np.testing.assert_allclose(oc, a1 * o1 + a2 * o2, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(fc, a1 * f1 + a2 * f2, rtol=1e-5, atol=1e-5)


# ----------------------------------------------------- contraction (P9)
def test_transition_is_a_contraction():
    """With unit keys, beta in [0, 1] and alpha <= 1, (I - beta k k^T) Diag(alpha)
    has spectral norm <= 1, so with v = 0 the state norm never grows, and with
    v != 0 it grows by at most beta |v| per token."""
    rng = np.random.default_rng(13)
    dk, dv, T = 16, 16, 60
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [T], 1, dk, dv, g_lo=-0.05)
    S = S0
    for t in range(T):
        _, S_new = O.prefill(q[t:t + 1], k[t:t + 1], np.zeros_like(v[t:t + 1]), g[t:t + 1], b[t:t + 1], S, [0, 1])
        assert np.linalg.norm(S_new) <= np.linalg.norm(S) * (1 + 1e-12)
        _, S_v = O.prefill(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], S, [0, 1])
        assert np.linalg.norm(S_v) <= np.linalg.norm(S) + b[t, 0] * np.linalg.norm(v[t, 0]) + 1e-9
        S = S_v


# ---------------------------------------------- two implementations (P11)
@pytest.mark.parametrize("lengths,H,dk,dv,g_lo", [
    ([128], 1, 128, 128, -5 / 16),
    ([3, 40, 0, 17], 3, 32, 16, -5.0),
    ([64, 64], 2, 128, 64, -1.0),
])
def test_c_oracle_matches_numpy(lengths, H, dk, dv, g_lo):
    rng = np.random.default_rng(sum(lengths) + H)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, lengths, H, dk, dv, g_lo=g_lo)
    o1, f1 = O.prefill(q, k, v, g, b, S0, cu)
    o2, f2 = O.numpy_prefill(q, k, v, g, b, S0, cu)
    scale = max(np.abs(o2).max(), 1e-30)
    assert np.abs(o1 - o2).max() <= 1e-12 * scale
    assert np.abs(f1 - f2).max() <= 1e-12 * max(np.abs(f2).max(), 1e-30)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(14)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [30, 50, 20], 4, 16, 16)
    o1, f1 = O.prefill(q, k, v, g, b, S0, cu, num_threads=1)
    o2, f2 = O.prefill(q, k, v, g, b, S0, cu, num_threads=4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_invalid_arguments_rejected():
    rng = np.random.default_rng(15)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [4, 4], 1, 4, 4)
    with pytest.raises(ValueError):
        O.prefill(q, k, v, g, b, S0, np.array([0, 5, 4], np.int32))  # decreasing cu_seqlens


# ------------------------------------------- planted mistakes are caught
def _mutant(kind):
    """A copy of the token loop with one plausible mistake planted."""
    def run(q, k, v, g, beta, S0, cu):
        q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
        T, H, dk = q.shape
        dv = v.shape[2]
        out = np.zeros((T, H, dv))
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0[0, 0], np.float64)
        for t in range(T):
            a = np.exp(g[t, 0])
            kt, bt = k[t, 0], beta[t, 0]
            if kind == "read_before_update":
                o = S.T @ q[t, 0]
            if kind == "decay_after_write":
                S = S + bt * np.outer(kt, v[t, 0] - S.T @ kt)
                S = a[:, None] * S
            elif kind == "decay_columns":
                S = S * a[None, :dv] if dv == dk else S * a[:dv][None, :]
                S = S + bt * np.outer(kt, v[t, 0] - S.T @ kt)
            elif kind == "plus_sign":
                S = a[:, None] * S
                S = S + bt * np.outer(kt, v[t, 0] + S.T @ kt)
            elif kind == "no_beta_on_read":
                S = a[:, None] * S
                S = S + np.outer(kt, bt * v[t, 0] - S.T @ kt)
            elif kind == "exp2_gate":
                S = np.exp2(g[t, 0])[:, None] * S
                S = S + bt * np.outer(kt, v[t, 0] - S.T @ kt)
            else:
                S = a[:, None] * S
                S = S + bt * np.outer(kt, v[t, 0] - S.T @ kt)
            if kind == "transposed_output":
                o = S @ q[t, 0][:dv]
            elif kind != "read_before_update":
                o = S.T @ q[t, 0]
            out[t, 0] = o
        return out, S[None, None]
    return run


@pytest.mark.parametrize("kind", ["read_before_update", "decay_after_write", "decay_columns",
                                  "plus_sign", "no_beta_on_read", "exp2_gate", "transposed_output"])
def test_pins_reject_planted_mistakes(kind):
    """Each planted mistake must fail the hand example or the product form."""
    bad = _mutant(kind)
    # sanity: the unmutated copy passes both
    good = _mutant("none")
    d = _parse_golden()
    T = d["k"].shape[0]
    args = (d["q"].reshape(T, 1, 2), d["k"].reshape(T, 1, 2), d["v"].reshape(T, 1, 2),
            np.log(d["alpha"]).reshape(T, 1, 2), d["beta"].reshape(T, 1), None, [0, T])
    o, f = good(*args)
    assert np.allclose(o[:, 0], d["out"], atol=1e-6) and np.allclose(f[0, 0], d["final_state"].reshape(2, 2), atol=1e-6)
    o, f = bad(*args)
    fails_golden = not (np.allclose(o[:, 0], d["out"], atol=1e-6)
                        and np.allclose(f[0, 0], d["final_state"].reshape(2, 2), atol=1e-6))
    rng = np.random.default_rng(21)
    q, k, v, g, b, S0, cu = _rand_inputs(rng, [6], 1, 4, 4, g_lo=-1.0)
    ref_out, ref_S = _product_form(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], S0[0, 0])
    o, f = bad(q, k, v, g, b, S0, cu)
    fails_product = not (np.allclose(o[:, 0], ref_out, atol=1e-9) and np.allclose(f[0, 0], ref_S, atol=1e-9))
    assert fails_golden and fails_product
