"""fp64 check of the chunked form that the device kernels evaluate (CPU only).

The device prefill does not run the token loop: it processes C-token chunks
with dense contractions.  This test restates that chunked algebra in plain
numpy fp64 and checks it against the oracle, so that the derivation itself
is verified independently of any kernel (it shares no code with the HIP
path and does not replace the oracle).

Derivation (from the recurrence on page ailearn.mscapital.top/kimi-k3.html,
card "KDA 单头递归"): inside a chunk with entering state S0 and cumulative
log-decay Gamma_r = sum_{i<=r} g_i,
    S_r = Diag(e^Gamma_r) S0 + sum_{i<=r} Diag(e^(Gamma_r - Gamma_i)) k_i w_i^T
    (I + Diag(beta) A) W = Diag(beta) (V - K+ S0),  A_ri = sum_c k_rc k_ic e^(Gamma_rc - Gamma_ic), i<r
    O = Q+ S0 + P W,  P_ri = sum_c q_rc k_ic e^(Gamma_rc - Gamma_ic), i<=r
    S_C = Diag(e^Gamma_C) S0 + K^T W,  K^ = K (.) e^(Gamma_C - Gamma)
The decay factors are referenced to 16-token sub-tile boundaries (the
"g ∈ (-5, 0)" card: cumulative scaling inside a 16-token tile stays within
the bf16 range), so every factor except the diagonal sub-tile's column factor
is <= 1 and that one is <= e^80 for g >= -5.
"""
import numpy as np
import pytest

from oracle import kda_oracle as O

SUB = 16


def chunked_prefill(q, k, v, g, beta, S0, cu, C):
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    nsub = C // SUB
    out = np.zeros((T, H, dv))
    fin = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[n, h].astype(np.float64).copy()
            for c0 in range(cu[n], cu[n + 1], C):
                L = min(C, cu[n + 1] - c0)
                # zero-padded ragged tail: k = q = v = 0, g = 0, beta = 0
                K = np.zeros((C, dk)); Q = np.zeros((C, dk)); V = np.zeros((C, dv))
                G = np.zeros((C, dk)); B = np.zeros(C)
                K[:L] = k[c0:c0 + L, h]; Q[:L] = q[c0:c0 + L, h]; V[:L] = v[c0:c0 + L, h]
                G[:L] = g[c0:c0 + L, h]; B[:L] = beta[c0:c0 + L, h]
                al = np.exp(G)
                R = np.zeros((C, dk)); D = np.zeros((C, dk)); F = np.zeros((nsub, dk))
                for a in range(nsub):
                    p = np.ones(dk)
                    for rr in range(SUB):
                        p = p * al[a * SUB + rr]
                        R[a * SUB + rr] = p                 # e^(Gamma_r - rho_a), includes token r
                    F[a] = p
                    p = np.ones(dk)
                    for rr in reversed(range(SUB)):
                        D[a * SUB + rr] = p                 # e^(rho_{a+1} - Gamma_r), excludes token r
                        p = p * al[a * SUB + rr]
                erho = np.array([np.prod(F[:a], axis=0) for a in range(nsub)])
                suff = np.array([np.prod(F[a + 1:], axis=0) for a in range(nsub)])
                gam = np.prod(F, axis=0)
                Hs = np.zeros((nsub, nsub, dk))
                for a in range(nsub):
                    for b in range(a):
                        Hs[a, b] = np.prod(F[b + 1:a], axis=0)
                    Hs[a, a] = 1.0 / F[a]
                Kr, Qr, KD = K * R, Q * R, K * D
                A = np.zeros((C, C)); P = np.zeros((C, C))
                for a in range(nsub):
                    ra = slice(a * SUB, (a + 1) * SUB)
                    for b in range(a + 1):
                        cb = slice(b * SUB, (b + 1) * SUB)
                        col = KD[cb] * Hs[a, b]
                        At = Kr[ra] @ col.T
                        Pt = Qr[ra] @ col.T
                        if a == b:
                            At = np.tril(At, -1)
                            Pt = np.tril(Pt, 0)
                        A[ra, cb] = At
                        P[ra, cb] = Pt
                Nm = B[:, None] * A
                Kp = np.concatenate([Kr[a * SUB:(a + 1) * SUB] * erho[a] for a in range(nsub)])
                Qp = np.concatenate([Qr[a * SUB:(a + 1) * SUB] * erho[a] for a in range(nsub)])
                Kh = np.concatenate([KD[a * SUB:(a + 1) * SUB] * suff[a] for a in range(nsub)])
                # state-dependent chain
                X = B[:, None] * (V - Kp @ S)
                W = np.zeros((C, dv))
                for a in range(nsub):
                    ra = slice(a * SUB, (a + 1) * SUB)
                    rhs = X[ra].copy()
                    for b in range(a):
                        cb = slice(b * SUB, (b + 1) * SUB)
                        rhs -= Nm[ra, cb] @ W[cb]
                    inv = np.linalg.inv(np.eye(SUB) + Nm[ra, ra])
                    W[ra] = inv @ rhs
                Oc = Qp @ S + P @ W
                S = gam[:, None] * S + Kh.T @ W
                out[c0:c0 + L, h] = Oc[:L]
            fin[n, h] = S
    return out, fin


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("g_lo", [-5 / 16, -5.0])
def test_chunked_form_matches_oracle(C, g_lo):
    rng = np.random.default_rng(100 + C)
    lengths = [200, 1, 64, 0, 77]
    H, dk, dv = 2, 32, 24
    T = sum(lengths)
    q = rng.standard_normal((T, H, dk)) * dk ** -0.5
    k = rng.standard_normal((T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.random((T, H, dk)) * g_lo
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((len(lengths), H, dk, dv)) * 0.1
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    f32 = lambda x: x.astype(np.float32)
    q, k, v, g, beta = map(f32, (q, k, v, g, beta))
    ref_o, ref_f = O.prefill(q, k, v, g, beta, S0, cu)
    o, f = chunked_prefill(q, k, v, g, beta, S0, cu, C)
    assert np.abs(o - ref_o).max() <= 1e-11 * np.abs(ref_o).max()
    assert np.abs(f - ref_f).max() <= 1e-11 * np.abs(ref_f).max()


def test_factor_ranges_stay_in_bf16_range():
    """With g in [-5, 0] no factor used by the chunked form leaves bf16's range:
    every factor is <= 1 except the diagonal column factor, bounded by e^80."""
    g = np.full((64, 4), -5.0)
    al = np.exp(g)
    F = np.prod(al[:16], axis=0)
    assert np.all(1.0 / F <= np.exp(80.0) * (1 + 1e-12))
    assert np.exp(80.0) < 3.38e38      # largest finite bf16 / fp32 is ~3.39e38
    assert np.all(F >= np.float32(1.1754944e-38))   # smallest normal fp32 / bf16
