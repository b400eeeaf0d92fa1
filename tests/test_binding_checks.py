"""The Python binding rejects, with ValueError and before any call into
libkda, tensors that the kernels would dereference wrongly: host (CPU)
tensors, for every tensor argument of every entry point.  These run on a
CPU-only host; the dtype and shape mismatches that need device tensors are
checked in tests/test_gpu_binding_checks.py."""
import pytest
import torch

from gated_delta_rule_40_amd import libkda as K

T, H, D, N = 8, 2, 128, 1


def _prefill_inputs(dtype=torch.bfloat16):
    f = lambda *s: torch.zeros(*s, dtype=torch.float32)
    return dict(q=torch.zeros(T, H, D, dtype=dtype), k=torch.zeros(T, H, D, dtype=dtype),
                v=torch.zeros(T, H, D, dtype=dtype), g=f(T, H, D), beta=f(T, H), initial_state=f(N, H, D, D),
                cu_seqlens=torch.tensor([0, T], dtype=torch.int32), out=torch.zeros(T, H, D, dtype=dtype),
                final_state=f(N, H, D, D))


PREFILL_ARGS = ("q", "k", "v", "g", "beta", "initial_state", "cu_seqlens", "out", "final_state")


@pytest.mark.parametrize("entry", ["kda_prefill", "kda_prefill_ex", "kda_prefill_cp"])
def test_prefill_rejects_host_tensors(entry):
    a = _prefill_inputs()
    with pytest.raises(ValueError, match="device tensor|tensor on"):
        getattr(K, entry)(*(a[n] for n in PREFILL_ARGS))


def test_prefill_snapshots_rejects_host_tensors():
    a = _prefill_inputs()
    snaps = torch.zeros(N, 1, H, D, D)
    with pytest.raises(ValueError):
        K.kda_prefill_snapshots(*(a[n] for n in PREFILL_ARGS), snaps, 32)


def test_decode_step_rejects_host_tensors():
    f = lambda *s: torch.zeros(*s, dtype=torch.float32)
    b = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        K.kda_decode_step(b(N, H, D), b(N, H, D), b(N, H, D), f(N, H, D), f(N, H), f(N, H, D, D), b(N, H, D))


def test_decode_tokens_rejects_host_tensors():
    a = _prefill_inputs()
    with pytest.raises(ValueError):
        K.kda_decode_tokens(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"], a["initial_state"])


def test_backward_rejects_host_tensors():
    a = _prefill_inputs()
    with pytest.raises(ValueError):
        K.kda_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"], a["cu_seqlens"], a["out"])


def test_workspace_size_rejects_unknown_dtype():
    with pytest.raises(TypeError):
        K.kda_prefill_cp_workspace_size(1, 16, 1, 128, 128, torch.float16)
    with pytest.raises(TypeError):
        K.kda_backward_workspace_size(1, 16, 1, 128, 128, torch.float16)
