"""fp64 CPU oracle for the Kimi Delta Attention (KDA) per-head recurrence.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``gated_delta_rule_40_amd``) never imports it and shares no code with it.

Method source: page "Kimi K3 把 3T 级模型、百万上下文和 Agent 训练接成一套系统"
(ailearn.mscapital.top/kimi-k3.html), card "KDA 单头递归": the state update
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, decay per
channel first, then delta-rule correction and write; the query reads the
updated S_t.  Readings: alpha_t = exp(g_t); S is dk x dv; o_t = S_t^T q_t; no
internal scaling or normalisation; NULL initial state = zeros.

Two independent implementations live here:

* ``prefill`` / ``decode_step``: the C library ``kda_oracle.c`` (fp64 token
  loop, OpenMP over (sequence, head) units);
* ``numpy_prefill``: a numpy fp64 token loop written in the page's grouping
  (apply ``I - beta k k^T`` to the decayed state, then add ``beta k v^T``).

``backward`` gives fp64 gradients through the recurrence (pinned in
``tests/test_oracle_backward.py`` against torch fp64 autograd of a token loop
written from the page's product form, central finite differences, and closed
forms).

Parity status: pinned by the tests in ``tests/test_oracle.py`` (hand-worked
example, the page's product form with explicit matrices, beta = 0 and
alpha = 1 closed forms, continuation, varlen, linearity, contraction, and the
two implementations against each other).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``kda_oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
             _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i32 = ctypes.c_int32
        lib.kda_oracle_prefill.argtypes = [fp, fp, fp, fp, fp, dp, ip, i32, i32, i32, i32, dp, dp, i32]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = [fp, fp, fp, fp, fp, dp, i32, i32, i32, i32, dp, i32]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [fp, fp, fp, fp, fp, dp, ip, i32, i32, i32, i32, dp, dp,
                                            dp, dp, dp, dp, dp, dp, i32]
        lib.kda_oracle_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor -> numpy without importing torch here
        x = x.detach().float().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().double().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def prefill(q, k, v, g, beta, initial_state, cu_seqlens, num_threads: int = 0):
    """Token-by-token fp64 prefill over packed sequences (C implementation).

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; initial_state:
    [N, H, dk, dv] or None; cu_seqlens: [N+1] host integers.
    Returns (out [T, H, dv] fp64, final_state [N, H, dk, dv] fp64).
    """
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk) and v.shape[:2] == (T, H)
    assert beta.shape == (T, H) and int(cu[-1]) <= T
    init = None if initial_state is None else _f64(initial_state)
    if init is not None:
        assert init.shape == (N, H, dk, dv)
    out = np.zeros((T, H, dv), dtype=np.float64)
    final = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = lib.kda_oracle_prefill(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float),
        None if init is None else _ptr(init, ctypes.c_double), _ptr(cu, ctypes.c_int32),
        N, H, dk, dv, _ptr(out, ctypes.c_double), _ptr(final, ctypes.c_double), int(num_threads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill failed with code %d" % rc)
    return out, final


def decode_step(q, k, v, g, beta, state, num_threads: int = 0):
    """One token per (sequence, head) from ``state`` (fp64 copy; input untouched).

    q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; state: [N, H, dk, dv].
    Returns (out [N, H, dv] fp64, new_state fp64).
    """
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    S = _f64(state).copy()
    N, H, dk = q.shape
    dv = v.shape[2]
    assert S.shape == (N, H, dk, dv)
    out = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.kda_oracle_decode_step(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float), _ptr(S, ctypes.c_double),
        N, H, dk, dv, _ptr(out, ctypes.c_double), int(num_threads))
    if rc != 0:
        raise ValueError("kda_oracle_decode_step failed with code %d" % rc)
    return out, S


def backward(q, k, v, g, beta, initial_state, cu_seqlens, dout, dfinal=None, num_threads: int = 0):
    """fp64 gradients of a scalar loss through the recurrence (C implementation):
    given dL/d(out) ``dout`` [T, H, dv] and dL/d(final_state) ``dfinal``
    [N, H, dk, dv] (None = zero), returns a dict with dq, dk, dv, dg [T, H, *],
    dbeta [T, H] and dinit [N, H, dk, dv], all fp64.  Keeps every state of a
    sequence in memory: test-sized inputs."""
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    init = None if initial_state is None else _f64(initial_state)
    dout = _f64(dout)
    assert dout.shape == (T, H, dv)
    dfin = None if dfinal is None else _f64(dfinal)
    if dfin is not None:
        assert dfin.shape == (N, H, dk, dv)
    res = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
           "dg": np.zeros((T, H, dk)), "dbeta": np.zeros((T, H)), "dinit": np.zeros((N, H, dk, dv))}
    d = lambda key: _ptr(res[key], ctypes.c_double)
    rc = lib.kda_oracle_backward(
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float),
        None if init is None else _ptr(init, ctypes.c_double), _ptr(cu, ctypes.c_int32),
        N, H, dk, dv, _ptr(dout, ctypes.c_double), None if dfin is None else _ptr(dfin, ctypes.c_double),
        d("dq"), d("dk"), d("dv"), d("dg"), d("dbeta"), d("dinit"), int(num_threads))
    if rc != 0:
        raise ValueError("kda_oracle_backward failed with code %d" % rc)
    return res


def numpy_prefill(q, k, v, g, beta, initial_state, cu_seqlens):
    """Second, independent fp64 implementation in the page's grouping.

    Per token: Sbar = Diag(exp(g_t)) S; S = Sbar - beta k (k^T Sbar) + beta k v^T;
    o_t = S^T q_t.  Pure numpy, one Python iteration per (sequence, head, token):
    for small cases only.
    """
    q, k, v, g, beta = (_f32(x).astype(np.float64) for x in (q, k, v, g, beta))
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    init = None if initial_state is None else _f64(initial_state)
    out = np.zeros((T, H, dv))
    final = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if init is None else init[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                kt, b = k[t, h], beta[t, h]
                Sbar = np.exp(g[t, h])[:, None] * S
                S = Sbar - b * np.outer(kt, kt @ Sbar) + b * np.outer(kt, v[t, h])
                out[t, h] = S.T @ q[t, h]
            final[n, h] = S
    return out, final
