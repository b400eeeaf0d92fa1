"""KDA_VALIDATE=1: the entry points that take cu_seqlens copy it to the host
and reject contents that break cu[0] = 0, non-decreasing, cu[N] <= T with
KDA_ERR_INVALID_ARG, launching nothing.  The variable is read at the first
call, so each case runs in a child process with its own environment."""
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, torch
sys.path.insert(0, %(root)r)
from gated_delta_rule_40_amd import inputs as I
from gated_delta_rule_40_amd import libkda as K
inp = I.random_prefill([40, 30], H=2, dtype=torch.bfloat16, seed=70, device="cuda")
T = inp["q"].shape[0]
out = torch.empty(T, 2, 128, dtype=torch.bfloat16, device="cuda")
fin = torch.empty(2, 2, 128, 128, device="cuda")
args = lambda cu: (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"], cu, out, fin)
calls = {"kda_prefill": lambda cu: K.kda_prefill(*args(cu)),
         "kda_prefill_cp": lambda cu: K.kda_prefill_cp(*args(cu)),
         "kda_prefill_cp pieces": lambda cu: K.kda_prefill_cp(*args(cu), seg_len=-64),
         "kda_decode_tokens": lambda cu: K.kda_decode_tokens(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu,
                                                             inp["initial_state"], state_out=fin, out=out),
         "kda_backward": lambda cu: K.kda_backward(*args(cu)[:7], out)}
bad = {"decreasing": [0, 50, 40], "past_the_end": [0, 40, T + 1], "nonzero_start": [1, 40, 70]}
results = []
for name, fn in calls.items():
    fn(torch.tensor([0, 40, 70], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for label, cu in bad.items():
        try:
            fn(torch.tensor(cu, dtype=torch.int32, device="cuda"))
            results.append("%%s %%s: accepted" %% (name, label))
        except K.KdaError as e:
            results.append("%%s %%s: %%d" %% (name, label, e.status))
print("\n".join(results), flush=True)
'''


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _run(validate):
    # (bad contents are only ever passed with validation on: they are then
    # rejected on the host and no kernel sees them)
    env = dict(os.environ, KDA_VALIDATE="1" if validate else "0")
    res = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT}], env=env, capture_output=True, text=True,
                         timeout=300)
    print(res.stdout, res.stderr[-2000:], flush=True)
    assert res.returncode == 0
    return [line for line in res.stdout.splitlines() if ": " in line]


def test_validate_rejects_bad_cu_seqlens():
    lines = _run(True)
    assert len(lines) == 15
    assert all(line.endswith(": 1") for line in lines), lines

