"""ctypes binding over libkda.so (C ABI declared in include/kda.h).

Argument marshalling only: shapes and dtypes are read off torch tensors,
device pointers and the current HIP stream are passed to the C entry points,
and every step of the computation runs in libkda's HIP kernels.  There is no
fallback: if the library is missing the calls raise.

    kda_prefill(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    kda_prefill_ex(..., chunk=0, dv_block=0)
    kda_prefill_snapshots(..., snapshots, snap_every)
    kda_prefill_cp(..., seg_len=0, workspace=None)
    kda_prefill_cp_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, seg_len)
    kda_prefill_cp_noalloc(..., seg_len=0)
    kda_decode_step(q, k, v, g, beta, state_inout, out)
    kda_decode_tokens(q, k, v, g, beta, cu_seqlens, state_in, state_out=None, out=None, num_tokens=None)
    kda_backward(q, k, v, g, beta, initial_state, cu_seqlens, dout, dfinal=None, ...) -> gradients
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_LAUNCH, KDA_ERR_SCRATCH = 0, 1, 2, 3, 4
KDA_STATIC_SCRATCH_BYTES = 256 * 1024 * 1024      # include/kda.h
KDA_F32, KDA_BF16 = 0, 1

EXPORTS = ("kda_prefill", "kda_prefill_ex", "kda_prefill_snapshots", "kda_prefill_cp",
           "kda_prefill_cp_workspace_size", "kda_prefill_cp_noalloc", "kda_decode_step", "kda_decode_tokens", "kda_backward",
           "kda_backward_workspace_size", "kda_status_string", "kda_version")

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libkda.so (built by ``python -m gated_delta_rule_40_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError("libkda.so not built at %s; run python -m gated_delta_rule_40_amd.build" % p)
    lib = ctypes.CDLL(p)
    vp, fp, ip, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32
    lib.kda_prefill.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, ctypes.c_int, vp, fp, vp]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill_ex.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, ctypes.c_int, vp, fp,
                                   i32, i32, vp]
    lib.kda_prefill_ex.restype = ctypes.c_int
    lib.kda_prefill_snapshots.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, ctypes.c_int, vp,
                                          fp, i32, i32, fp, vp]
    lib.kda_prefill_snapshots.restype = ctypes.c_int
    lib.kda_prefill_cp.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, ctypes.c_int, vp, fp,
                                   i32, vp, ctypes.c_size_t, vp]
    lib.kda_prefill_cp.restype = ctypes.c_int
    lib.kda_prefill_cp_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, ctypes.c_int, vp,
                                           fp, i32, vp]
    lib.kda_prefill_cp_noalloc.restype = ctypes.c_int
    lib.kda_prefill_cp_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, i32]
    lib.kda_prefill_cp_workspace_size.restype = ctypes.c_size_t
    lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, i32, i32, i32, i32, ctypes.c_int, vp, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_tokens.argtypes = [vp, vp, vp, fp, fp, ip, ip, fp, fp, i32, i32, i32, i32, i32, ctypes.c_int,
                                      vp, vp]
    lib.kda_decode_tokens.restype = ctypes.c_int
    lib.kda_backward.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, ctypes.c_int, vp, fp,
                                 fp, fp, fp, fp, fp, fp, vp, ctypes.c_size_t, vp]
    lib.kda_backward.restype = ctypes.c_int
    lib.kda_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_backward_workspace_size.restype = ctypes.c_size_t
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(status).decode()


def _check(status: int) -> None:
    if status != KDA_OK:
        raise KdaError(status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_device(ref: torch.Tensor, **tensors) -> None:
    """Every given tensor (None entries skipped) must be a device tensor on
    ref's device: the library dereferences the pointers on the GPU, so a host
    pointer or another device's memory would fault there."""
    _require(torch.is_tensor(ref) and ref.is_cuda, "q must be a device tensor")
    for name, t in tensors.items():
        if t is None:
            continue
        _require(torch.is_tensor(t) and t.is_cuda and t.device == ref.device,
                 "%s must be a tensor on %s" % (name, ref.device))


def _check_prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state):
    _on_device(q, k=k, v=v, g=g, beta=beta, initial_state=initial_state, cu_seqlens=cu_seqlens, out=out,
               final_state=final_state)
    _require(q.dim() == 3 and v.dim() == 3 and cu_seqlens.dim() == 1 and cu_seqlens.shape[0] >= 1,
             "q, k, g, v, out must be [T, H, d] and cu_seqlens [N + 1]")
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.shape[0] - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out),
                    ("cu_seqlens", cu_seqlens)):
        _require(t.is_contiguous(), "%s must be contiguous" % name)
    _require(cu_seqlens.dtype == torch.int32, "cu_seqlens must be int32")
    _require(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be float32")
    _require(k.shape == q.shape and g.shape == q.shape and v.shape[:2] == (T, H) and out.shape == v.shape,
             "shape mismatch")
    _require(tuple(beta.shape) == (T, H), "beta must be [T, H]")
    _require(k.dtype == q.dtype and v.dtype == q.dtype and out.dtype == q.dtype, "q/k/v/out dtypes differ")
    for name, s in (("initial_state", initial_state), ("final_state", final_state)):
        if s is not None:
            _require(s.dtype == torch.float32 and s.is_contiguous() and tuple(s.shape) == (N, H, dk, dv),
                     "%s must be contiguous float32 [N, H, dk, dv]" % name)
    return N, T, H, dk, dv


def kda_prefill_ex(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                   chunk: int = 0, dv_block: int = 0, stream=None) -> None:
    """Packed varlen prefill.  q, k, g: [T, H, dk]; v, out: [T, H, dv];
    beta: [T, H] fp32; initial_state/final_state: [N, H, dk, dv] fp32 or None;
    cu_seqlens: [N+1] int32 on the device."""
    N, T, H, dk, dv = _check_prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    lib = load()
    _check(lib.kda_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                              _ptr(cu_seqlens), N, T, H, dk, dv, _dtype_code(q), _ptr(out),
                              _ptr(final_state), int(chunk), int(dv_block), _stream(stream)))


def kda_prefill_snapshots(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, snapshots,
                          snap_every: int, stream=None) -> None:
    """kda_prefill plus the state after every snap_every tokens of each
    sequence: snapshots [N, max_snaps, H, dk, dv] fp32 (max_snaps from its shape)."""
    N, T, H, dk, dv = _check_prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    _on_device(q, snapshots=snapshots)
    _require(snapshots.dtype == torch.float32 and snapshots.is_contiguous() and snapshots.dim() == 5 and
             snapshots.shape[0] == N and tuple(snapshots.shape[2:]) == (H, dk, dv),
             "snapshots must be contiguous float32 [N, max_snaps, H, dk, dv]")
    lib = load()
    _check(lib.kda_prefill_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                     _ptr(cu_seqlens), N, T, H, dk, dv, _dtype_code(q), _ptr(out),
                                     _ptr(final_state), int(snap_every), int(snapshots.shape[1]),
                                     _ptr(snapshots), _stream(stream)))


def kda_prefill_cp_workspace_size(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int,
                                  dtype=torch.bfloat16, seg_len: int = 0) -> int:
    """Bytes of device workspace kda_prefill_cp needs (0 = unsupported sizes);
    dtype is that of q/k/v (torch.bfloat16 or torch.float32)."""
    code = {torch.bfloat16: KDA_BF16, torch.float32: KDA_F32}.get(dtype)
    if code is None:
        raise TypeError("dtype must be torch.bfloat16 or torch.float32, got %s" % dtype)
    return int(load().kda_prefill_cp_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, code, seg_len))


def kda_prefill_cp(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                   seg_len: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Context-parallel prefill (same arguments and result as kda_prefill):
    sequences are split into seg_len-token segments that run side by side
    (seg_len < 0: pieces of -seg_len tokens over the packed chunk order;
    0: automatic, see include/kda.h).
    ``workspace`` is a uint8 device tensor of at least
    kda_prefill_cp_workspace_size(...) bytes; if None, one is allocated."""
    N, T, H, dk, dv = _check_prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    need = kda_prefill_cp_workspace_size(N, T, H, dk, dv, q.dtype, seg_len)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _on_device(q, workspace=workspace)
    _require(workspace.is_contiguous(), "workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    lib = load()
    _check(lib.kda_prefill_cp(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                              _ptr(cu_seqlens), N, T, H, dk, dv, _dtype_code(q), _ptr(out),
                              _ptr(final_state), int(seg_len), _ptr(workspace), nbytes, _stream(stream)))


def kda_prefill_cp_noalloc(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                           seg_len: int = 0, stream=None) -> None:
    """kda_prefill_cp in the library's static device scratch: no workspace
    argument and no allocation.  Raises KdaError(KDA_ERR_SCRATCH) when the
    problem needs more than KDA_STATIC_SCRATCH_BYTES; calls overlapping in
    time on one GPU race on the shared scratch."""
    N, T, H, dk, dv = _check_prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    lib = load()
    _check(lib.kda_prefill_cp_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                      _ptr(cu_seqlens), N, T, H, dk, dv, _dtype_code(q), _ptr(out),
                                      _ptr(final_state), int(seg_len), _stream(stream)))


def kda_prefill(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, stream=None) -> None:
    """kda_prefill with the library's default tiling."""
    kda_prefill_ex(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, 0, 0, stream)


def kda_decode_step(q, k, v, g, beta, state_inout, out, stream=None) -> None:
    """One decode step, state updated in place.  q, k, g: [N, H, dk];
    v, out: [N, H, dv]; beta: [N, H]; state_inout: [N, H, dk, dv] fp32."""
    _on_device(q, k=k, v=v, g=g, beta=beta, state_inout=state_inout, out=out)
    _require(q.dim() == 3 and v.dim() == 3, "q, k, g, v, out must be [N, H, d]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state_inout),
                    ("out", out)):
        _require(t.is_contiguous(), "%s must be contiguous" % name)
    _require(k.dtype == q.dtype and v.dtype == q.dtype and out.dtype == q.dtype, "q/k/v/out dtypes differ")
    _require(k.shape == q.shape and g.shape == q.shape and v.shape[:2] == (N, H) and out.shape == v.shape,
             "shape mismatch")
    _require(tuple(beta.shape) == (N, H) and tuple(state_inout.shape) == (N, H, dk, dv), "shape mismatch")
    _require(state_inout.dtype == torch.float32 and g.dtype == torch.float32 and beta.dtype == torch.float32,
             "g, beta and state must be float32")
    lib = load()
    _check(lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_inout), N, H, dk,
                               dv, _dtype_code(q), _ptr(out), _stream(stream)))


def kda_decode_tokens(q, k, v, g, beta, cu_seqlens, state_in, state_out=None, out=None, num_tokens=None,
                      stream=None) -> None:
    """A few consecutive tokens per (sequence, head), state kept on chip.
    q, k, g: [T, H, dk]; v, out: [T, H, dv]; beta: [T, H]; cu_seqlens: [N+1]
    int32 on the device; num_tokens: [N] int32 on the device or None;
    state_in / state_out: [N, H, dk, dv] fp32 (state_out None: not written)."""
    _on_device(q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu_seqlens, state_in=state_in, state_out=state_out,
               out=out, num_tokens=num_tokens)
    _require(q.dim() == 3 and v.dim() == 3 and cu_seqlens.dim() == 1 and cu_seqlens.shape[0] >= 1,
             "q, k, g, v, out must be [T, H, d] and cu_seqlens [N + 1]")
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.shape[0] - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state_in", state_in),
                    ("cu_seqlens", cu_seqlens)):
        _require(t.is_contiguous(), "%s must be contiguous" % name)
    _require(cu_seqlens.dtype == torch.int32, "cu_seqlens must be int32")
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q/k/v dtypes differ")
    _require(k.shape == q.shape and g.shape == q.shape and v.shape[:2] == (T, H) and tuple(beta.shape) == (T, H),
             "shape mismatch")
    _require(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be float32")
    for name, st in (("state_in", state_in), ("state_out", state_out)):
        if st is not None:
            _require(st.dtype == torch.float32 and st.is_contiguous() and tuple(st.shape) == (N, H, dk, dv),
                     "%s must be contiguous float32 [N, H, dk, dv]" % name)
    if out is not None:
        _require(out.is_contiguous() and out.shape == v.shape and out.dtype == q.dtype, "out must match v")
    if num_tokens is not None:
        _require(num_tokens.dtype == torch.int32 and num_tokens.is_contiguous() and tuple(num_tokens.shape) == (N,),
                 "num_tokens must be int32 [N] on the device")
    lib = load()
    _check(lib.kda_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                 _ptr(num_tokens), _ptr(state_in), _ptr(state_out), N, T, H, dk, dv,
                                 _dtype_code(q), _ptr(out), _stream(stream)))


def kda_backward_workspace_size(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int,
                                dtype=torch.bfloat16) -> int:
    code = {torch.bfloat16: KDA_BF16, torch.float32: KDA_F32}.get(dtype)
    if code is None:
        raise TypeError("dtype must be torch.bfloat16 or torch.float32, got %s" % dtype)
    return int(load().kda_backward_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, code))


def kda_backward(q, k, v, g, beta, initial_state, cu_seqlens, dout, dfinal=None, grads=None, want_dinit=True,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of a scalar loss given dout = dL/d(out) [T, H, dv] (q's dtype)
    and dfinal = dL/d(final_state) [N, H, dk, dv] fp32 or None.  Returns a dict
    of fp32 tensors dq, dk, dv, dg [T, H, *], dbeta [T, H] and dinit
    [N, H, dk, dv] (None unless want_dinit); ``grads`` may supply them."""
    N, T, H, dk, dv = _check_prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, dout, None)
    _on_device(q, dfinal=dfinal, workspace=workspace)
    if dfinal is not None:
        _require(dfinal.dtype == torch.float32 and dfinal.is_contiguous() and tuple(dfinal.shape) == (N, H, dk, dv),
                 "dfinal must be contiguous float32 [N, H, dk, dv]")
    dev = q.device
    shapes = {"dq": (T, H, dk), "dk": (T, H, dk), "dv": (T, H, dv), "dg": (T, H, dk), "dbeta": (T, H),
              "dinit": (N, H, dk, dv)}
    if grads is None:
        f = lambda *shape: torch.empty(*shape, dtype=torch.float32, device=dev)
        grads = {key: f(*shape) for key, shape in shapes.items() if key != "dinit"}
        grads["dinit"] = f(*shapes["dinit"]) if want_dinit else None
    for key, shape in shapes.items():
        t = grads.get(key)
        if t is None and key == "dinit":
            continue
        _require(t is not None, "grads[%r] is missing" % key)
        _on_device(q, **{key: t})
        _require(t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shape,
                 "grads[%r] must be contiguous float32 %s" % (key, list(shape)))
    need = kda_backward_workspace_size(N, T, H, dk, dv, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _require(workspace.is_contiguous(), "workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    lib = load()
    _check(lib.kda_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
                            N, T, H, dk, dv, _dtype_code(q), _ptr(dout), _ptr(dfinal), _ptr(grads["dq"]),
                            _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["dbeta"]),
                            _ptr(grads.get("dinit")), _ptr(workspace), nbytes, _stream(stream)))
    return grads
