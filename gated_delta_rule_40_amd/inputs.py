"""Seeded synthetic inputs for the KDA recurrence.

This module only draws random tensors: it holds none of the recurrence's
arithmetic, and both the device path and the fp64 oracle consume what it
returns.  Shapes follow the Kimi K3 notes (head dim 128 and up to 1,048,576
context tokens, page ailearn.mscapital.top/kimi-k3.html, spec grid and the
"百万上下文的关键" section); the gate range follows the "g ∈ (-5, 0)" card.

Layout (row-major, contiguous):
    q, k, g : [T_tot, H, dk]     v, out : [T_tot, H, dv]     beta : [T_tot, H]
    initial_state / final_state : [N, H, dk, dv] fp32
    cu_seqlens : [N+1] int32, cu[0] = 0, cu[N] = T_tot

Recipe (identical for every workload; the draw order is fixed):
    q    ~ N(0, 1) * dk^-1/2
    k    ~ N(0, 1), then L2-normalised over dk per (token, head)
    v    ~ N(0, 1)
    g    = u * g_lo with u ~ U[0, 1), i.e. g in (g_lo, 0]   (g_lo = -5/16)
    beta = sigmoid(N(0, 1))
    initial_state ~ N(0, 0.1^2) or zeros
q, k, v (and the output) are rounded to the workload dtype (bf16 or fp32)
with round-to-nearest-even; g, beta and the state are fp32.  The oracle reads
the rounded values widened to fp32, so parity measures the kernels alone.
Values depend on the generator's device (CPU or GPU): each test feeds the
very same tensors to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

DK = 128
DV = 128


@dataclass
class Workload:
    """One of the five synthetic workloads (sizes fixed, dtype, state init)."""
    name: str
    kind: str                      # "prefill" or "decode"
    heads: int
    dtype: torch.dtype
    lengths: Optional[List[int]] = None   # prefill: per-sequence lengths (None -> drawn)
    num_seqs: int = 1
    total_tokens: int = 0
    init: str = "zero"             # "zero" or "normal"
    steps: int = 1                 # decode: consecutive steps
    seed: int = 0
    g_lo: float = -5.0 / 16.0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "parity_t128_fp32": Workload("parity_t128_fp32", "prefill", heads=1, dtype=torch.float32,
                                 lengths=[128], num_seqs=1, total_tokens=128, init="zero", seed=1000),
    "prefill_t4096_h8": Workload("prefill_t4096_h8", "prefill", heads=8, dtype=torch.bfloat16,
                                 lengths=[4096], num_seqs=1, total_tokens=4096, init="normal", seed=1001),
    "prefill_4x16384_h32": Workload("prefill_4x16384_h32", "prefill", heads=32, dtype=torch.bfloat16,
                                    lengths=[16384] * 4, num_seqs=4, total_tokens=65536, init="normal",
                                    seed=1002),
    "prefill_varlen_1m_h16": Workload("prefill_varlen_1m_h16", "prefill", heads=16, dtype=torch.bfloat16,
                                      lengths=None, num_seqs=8, total_tokens=1 << 20, init="zero",
                                      seed=1003, extra={"len_lo": 1024, "len_hi": 262144}),
    "decode_512x32": Workload("decode_512x32", "decode", heads=32, dtype=torch.bfloat16,
                              num_seqs=512, steps=64, init="normal", seed=1004),
}


def loguniform_lengths(n: int, total: int, lo: int, hi: int, gen: torch.Generator) -> List[int]:
    """n lengths exp(U(ln lo, ln hi)), rescaled to sum to ``total``, floored,
    with the rounding remainder added to the longest sequence."""
    u = torch.rand(n, generator=gen, dtype=torch.float64, device=gen.device).cpu()
    raw = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    scaled = torch.floor(raw / raw.sum() * total).to(torch.int64)
    lens = [int(x) for x in scaled]
    lens[max(range(n), key=lambda i: lens[i])] += total - sum(lens)
    return lens


def cu_from_lengths(lengths: List[int], device="cpu") -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_tokens(T: int, H: int, dtype: torch.dtype, gen: torch.Generator, device,
                dk: int = DK, dv: int = DV, g_lo: float = -5.0 / 16.0):
    """Draw q, k, v, g, beta for T tokens x H heads in the fixed order."""
    q = torch.randn(T, H, dk, generator=gen, device=device) * (dk ** -0.5)
    k = torch.randn(T, H, dk, generator=gen, device=device)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    v = torch.randn(T, H, dv, generator=gen, device=device)
    g = torch.rand(T, H, dk, generator=gen, device=device) * g_lo
    beta = torch.sigmoid(torch.randn(T, H, generator=gen, device=device))
    return q.to(dtype), k.to(dtype), v.to(dtype), g.float().contiguous(), beta.float().contiguous()


def make_prefill(wl: Workload, device="cpu", dk: int = DK, dv: int = DV):
    """Inputs of a prefill workload as a dict of tensors on ``device``."""
    gen = _gen(wl.seed, device)
    T = wl.total_tokens
    q, k, v, g, beta = make_tokens(T, wl.heads, wl.dtype, gen, device, dk, dv, wl.g_lo)
    N = wl.num_seqs
    init = None
    if wl.init == "normal":
        init = (torch.randn(N, wl.heads, dk, dv, generator=gen, device=device) * 0.1).float()
    lengths = wl.lengths
    if lengths is None:
        lengths = loguniform_lengths(N, T, wl.extra["len_lo"], wl.extra["len_hi"], gen)
    assert sum(lengths) == T
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=init,
                cu_seqlens=cu_from_lengths(lengths, device), lengths=list(lengths))


def make_decode(wl: Workload, device="cpu", dk: int = DK, dv: int = DV, steps: Optional[int] = None):
    """Inputs of a decode workload: per-step q, k, v, g, beta stacked on a
    leading step axis ([steps, N, H, d]) plus the fp32 state [N, H, dk, dv]."""
    steps = wl.steps if steps is None else steps
    gen = _gen(wl.seed, device)
    N, H = wl.num_seqs, wl.heads
    q, k, v, g, beta = make_tokens(steps * N, H, wl.dtype, gen, device, dk, dv, wl.g_lo)
    state = (torch.randn(N, H, dk, dv, generator=gen, device=device) * 0.1).float()
    rs = lambda x: x.reshape(steps, N, H, *x.shape[2:]).contiguous()
    return dict(q=rs(q), k=rs(k), v=rs(v), g=rs(g), beta=beta.reshape(steps, N, H).contiguous(),
                state=state)


def random_prefill(lengths: List[int], H: int, dtype: torch.dtype, seed: int, device="cpu",
                   init: str = "normal", g_lo: float = -5.0 / 16.0, dk: int = DK, dv: int = DV):
    """Ad-hoc prefill inputs (tests): same recipe, arbitrary lengths/heads/gate range."""
    wl = Workload("adhoc", "prefill", heads=H, dtype=dtype, lengths=list(lengths),
                  num_seqs=len(lengths), total_tokens=int(sum(lengths)), init=init, seed=seed,
                  g_lo=g_lo)
    return make_prefill(wl, device, dk, dv)
