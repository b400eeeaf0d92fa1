"""Pins for the fp64 backward of the oracle (oracle/kda_oracle.c,
kda_oracle_backward): gradients of a scalar loss
L = <dout, out> + <dfinal, final_state> with respect to q, k, v, g, beta and
the initial state.

* torch fp64 autograd of a token loop written here from the page's product
  form (page ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"):
  S_t = (I - b k k^T) Diag(exp(g)) S_{t-1} + b k v^T, o_t = S_t^T q_t;
* central finite differences of the C forward oracle, on inputs and steps
  exactly representable in fp32 (so the fp64 forward sees exact perturbations);
* the closed form at beta = 0 (pure decay);
* a planted sign error is caught by the finite-difference check;
* the gradient transition of a stretch of tokens is the transpose of its
  forward transition (which the GPU backward takes from the forward pass).
"""
import numpy as np
import pytest
import torch

from oracle import kda_oracle as O


def _inputs(lengths, H, dk, dv, seed, grid=None):
    rng = np.random.default_rng(seed)
    T, N = sum(lengths), len(lengths)
    def draw(*shape, scale=1.0, lo=None):
        x = rng.standard_normal(shape) * scale if lo is None else rng.uniform(lo, 0.0, shape)
        if grid:   # multiples of 2^-grid: exactly representable, and so are x +- 2^-(grid+2)
            x = np.round(x * 2.0 ** grid) / 2.0 ** grid
        return x.astype(np.float32)
    inp = dict(q=draw(T, H, dk, scale=0.5), k=draw(T, H, dk, scale=0.5), v=draw(T, H, dv),
               g=draw(T, H, dk, lo=-1.0), beta=(draw(T, H, scale=0.3) + 0.5).astype(np.float32),
               init=rng.standard_normal((N, H, dk, dv)) * 0.3,
               cu=np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32),
               dout=rng.standard_normal((T, H, dv)), dfinal=rng.standard_normal((N, H, dk, dv)))
    return inp


def _loss(inp, **override):
    x = dict(inp)
    x.update(override)
    out, fin = O.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["init"], x["cu"])
    return float(np.sum(out * x["dout"]) + np.sum(fin * x["dfinal"]))


def _torch_grads(inp):
    """Autograd of the page's product form, fp64, one token at a time."""
    t = {key: torch.tensor(np.asarray(inp[key], np.float64), requires_grad=True)
         for key in ("q", "k", "v", "g", "beta", "init")}
    cu = inp["cu"]
    N, H, dk, dv = inp["init"].shape
    outs = [[None] * H for _ in range(int(cu[-1]))]      # outs[token][head]
    fins = []
    for n in range(N):
        per_head = []
        for h in range(H):
            S = t["init"][n, h]
            for tok in range(int(cu[n]), int(cu[n + 1])):
                kt, b = t["k"][tok, h], t["beta"][tok, h]
                A = (torch.eye(dk, dtype=torch.float64) - b * torch.outer(kt, kt)) @ torch.diag(torch.exp(t["g"][tok, h]))
                S = A @ S + b * torch.outer(kt, t["v"][tok, h])
                outs[tok][h] = S.T @ t["q"][tok, h]
            per_head.append(S)
        fins.append(torch.stack(per_head))
    out = torch.stack([torch.stack(o) for o in outs])
    fin = torch.stack(fins)
    L = (out * torch.tensor(inp["dout"])).sum() + (fin * torch.tensor(inp["dfinal"])).sum()
    L.backward()
    return {"dq": t["q"].grad.numpy(), "dk": t["k"].grad.numpy(), "dv": t["v"].grad.numpy(),
            "dg": t["g"].grad.numpy(), "dbeta": t["beta"].grad.numpy(), "dinit": t["init"].grad.numpy()}


def _oracle_grads(inp):
    return O.backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["init"], inp["cu"],
                      inp["dout"], inp["dfinal"])


def test_backward_matches_torch_autograd_of_product_form():
    inp = _inputs([5, 3, 0, 4], H=2, dk=6, dv=5, seed=1)
    got = _oracle_grads(inp)
    ref = _torch_grads(inp)
    for key in ref:
        scale = max(np.abs(ref[key]).max(), 1e-30)
        assert np.abs(got[key] - ref[key]).max() <= 1e-11 * scale, key


def _fd_check(inp, grads, key, picks, h):
    """Central differences of the C forward oracle at the picked elements."""
    src = {"dinit": "init"}.get(key, key[1:])
    base = inp[src]
    ok = True
    for idx in picks:
        plus, minus = base.copy(), base.copy()
        plus[idx] += h
        minus[idx] -= h
        fd = (_loss(inp, **{src: plus}) - _loss(inp, **{src: minus})) / (2 * h)
        g = grads[key][idx]
        ok &= abs(fd - g) <= 1e-6 * max(1.0, abs(g))
    return ok


@pytest.mark.parametrize("key", ["dq", "dk", "dv", "dg", "dbeta", "dinit"])
def test_backward_finite_differences(key):
    inp = _inputs([4, 3], H=1, dk=3, dv=2, seed=2, grid=10)
    grads = _oracle_grads(inp)
    rng = np.random.default_rng(3)
    shape = grads[key].shape
    picks = [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(6)]
    assert _fd_check(inp, grads, key, picks, h=2.0 ** -12)


def test_finite_differences_catch_a_planted_sign_error():
    inp = _inputs([4, 3], H=1, dk=3, dv=2, seed=2, grid=10)
    grads = _oracle_grads(inp)
    grads["dg"] = -grads["dg"]
    picks = [(t, 0, c) for t in range(2) for c in range(3)]
    assert not _fd_check(inp, grads, "dg", picks, h=2.0 ** -12)


def test_backward_beta_zero_closed_form():
    """beta = 0: S_t = Diag(exp(Gamma_t)) S_0 with Gamma_t = sum_{i<=t} g_i, so
    dq_t = S_t do_t, dv = dk = 0, and dS_0 = sum_t Diag(e^Gamma_t) q_t do_t^T
    + Diag(e^Gamma_T) dfinal."""
    inp = _inputs([6], H=1, dk=4, dv=3, seed=4)
    inp["beta"] = np.zeros_like(inp["beta"])
    got = _oracle_grads(inp)
    S0 = inp["init"][0, 0]
    Gam = np.cumsum(inp["g"][:, 0].astype(np.float64), axis=0)
    dS0 = np.exp(Gam[-1])[:, None] * inp["dfinal"][0, 0]
    for t in range(6):
        St = np.exp(Gam[t])[:, None] * S0
        assert np.allclose(got["dq"][t, 0], St @ inp["dout"][t, 0], atol=1e-12)
        dS0 += np.exp(Gam[t])[:, None] * np.outer(inp["q"][t, 0], inp["dout"][t, 0])
    assert np.allclose(got["dinit"][0, 0], dS0, atol=1e-12)
    assert np.abs(got["dv"]).max() == 0 and np.abs(got["dk"]).max() == 0


def test_gradient_transition_is_transpose_of_forward_transition():
    """With v = 0 and dout = 0 the forward map init -> final_state is the
    segment transition M (per value column) and the backward map
    dfinal -> dinit is the gradient transition R.  R = M^T: the gradient step
    Diag(alpha)(I - beta k k^T) is the transpose of the forward step
    (I - beta k k^T) Diag(alpha), and the steps run in the opposite order.
    M is built column by column from unit initial states and compared with
    the R the backward oracle applies to unit dfinal matrices."""
    inp = _inputs([37], H=1, dk=6, dv=6, seed=91)
    inp["g"] = (inp["g"] * np.float32(0.05)).astype(np.float32)   # weak decay: M stays well above rounding
    zero_v = np.zeros_like(inp["v"])
    dk = 6
    M = np.zeros((dk, dk))
    R = np.zeros((dk, dk))
    for j in range(dk):
        e = np.zeros((1, 1, dk, 6))
        e[0, 0, j, 0] = 1.0                               # value column 0 carries unit vector e_j
        _, fin = O.prefill(inp["q"], inp["k"], zero_v, inp["g"], inp["beta"], e, inp["cu"])
        M[:, j] = fin[0, 0, :, 0]
        gr = O.backward(inp["q"], inp["k"], zero_v, inp["g"], inp["beta"], e * 0.0, inp["cu"],
                        np.zeros_like(inp["dout"][:, :, :6]), e)
        R[:, j] = gr["dinit"][0, 0, :, 0]
    assert np.abs(M).max() > 1e-2                          # a nontrivial transition
    assert np.abs(M - M.T).max() > 1e-3                    # and not symmetric: the transpose matters
    np.testing.assert_allclose(R, M.T, rtol=1e-12, atol=1e-14)
