"""Binding checks that need device tensors: dtype, shape and device
mismatches raise ValueError before any kernel is launched (a mismatched
dtype would make a kernel write past the end of a buffer)."""
import pytest
import torch

from gated_delta_rule_40_amd import libkda as K

pytestmark = pytest.mark.gpu

T, H, D, N = 8, 2, 128, 1


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    K.load()


def _dev(*s, dtype=torch.float32):
    return torch.zeros(*s, dtype=dtype, device="cuda")


def test_decode_step_rejects_mismatched_dtypes():
    q = _dev(N, H, D, dtype=torch.float32)
    bf = _dev(N, H, D, dtype=torch.bfloat16)
    args = [q, q.clone(), q.clone(), _dev(N, H, D), _dev(N, H), _dev(N, H, D, D), q.clone()]
    for pos in (1, 2, 6):                      # k, v, out in bf16 with fp32 q
        bad = list(args)
        bad[pos] = bf
        with pytest.raises(ValueError, match="dtypes differ"):
            K.kda_decode_step(*bad)


def test_decode_tokens_rejects_mismatched_dtypes():
    q = _dev(T, H, D)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="dtypes differ"):
        K.kda_decode_tokens(q, _dev(T, H, D, dtype=torch.bfloat16), q.clone(), _dev(T, H, D), _dev(T, H), cu,
                            _dev(N, H, D, D))


def test_prefill_rejects_host_state_with_device_inputs():
    b = lambda: _dev(T, H, D, dtype=torch.bfloat16)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="initial_state"):
        K.kda_prefill(b(), b(), b(), _dev(T, H, D), _dev(T, H), torch.zeros(N, H, D, D), cu, b(), None)


def test_backward_rejects_bad_grads():
    b = lambda: _dev(T, H, D, dtype=torch.bfloat16)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    grads = {"dq": _dev(T, H, D), "dk": _dev(T, H, D), "dv": _dev(T, H, D), "dg": _dev(T, H, D),
             "dbeta": _dev(T, H), "dinit": None}
    bad = dict(grads, dv=_dev(T, H, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dv"):
        K.kda_backward(b(), b(), b(), _dev(T, H, D), _dev(T, H), None, cu, b(), grads=bad)
    bad = dict(grads, dq=torch.zeros(T, H, D))
    with pytest.raises(ValueError, match="dq"):
        K.kda_backward(b(), b(), b(), _dev(T, H, D), _dev(T, H), None, cu, b(), grads=bad)
    bad = dict(grads, dbeta=_dev(T, H + 1))
    with pytest.raises(ValueError, match="dbeta"):
        K.kda_backward(b(), b(), b(), _dev(T, H, D), _dev(T, H), None, cu, b(), grads=bad)
