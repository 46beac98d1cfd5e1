"""Seeded synthetic inputs for the Gated DeltaNet recurrence.

This module is shared by the GPU tests, the oracle tests, the smoke check and the
benchmark. It only draws random numbers and shapes them; it contains none of the
recurrence's arithmetic, and neither the GPU library nor the oracle imports it.

Recipe (one seed per case; draws in a fixed order q, k, v, beta, g, state):
  q, k   standard normal, each (token, QK head) row scaled to unit length, i.e. a
         uniformly random direction; then cast to the input dtype (round to nearest even)
  v      standard normal, cast to the input dtype
  beta   sigmoid(N(0, 1))                                    (fp32)
  g      log(sigmoid(N(2, 1))), evaluated as -log1p(exp(-x)) (fp32, a log-decay <= 0)
  state  zeros, or N(0, s0_std^2) when s0_std > 0            (fp32)
Retrieval inputs replace g by 0 and beta by 1.

Draws are fp64 on the CPU and fp32 on a GPU (torch's generator on that device), so a CPU
case and a GPU case with the same seed are different, equally distributed, draws.
"""
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Shape:
    n: int       # independent sequences (or stacked layers for decode)
    t: int       # tokens per call
    h_qk: int    # QK heads
    h_v: int     # V heads (a multiple of h_qk)
    d: int       # d_k = d_v
    dtype: torch.dtype = torch.bfloat16  # q, k, v dtype


# The five workloads.
TINY = Shape(n=1, t=64, h_qk=1, h_v=2, d=16, dtype=torch.float32)
PREFILL_4K = Shape(n=1, t=4096, h_qk=16, h_v=32, d=128)
DECODE_30L = Shape(n=30, t=1, h_qk=16, h_v=32, d=128)
LONG_SEGMENT = Shape(n=1, t=4096, h_qk=16, h_v=32, d=128)  # 32 segments = 131072 tokens
ABLATION_2K = Shape(n=1, t=2048, h_qk=16, h_v=32, d=128)   # the state-residency ablation prompt
LONG_SEGMENTS = 32
SWEEP_T = (256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)
SWEEP_CHUNKS = (32, 64, 128)


def make_case(shape: Shape, seed: int, device="cpu", s0_std: float = 0.0,
              retrieval: bool = False, zero_state_as_none: bool = True):
    """Return dict(q, k, v, g, beta, state_in) on `device`.

    state_in is None when s0_std == 0 and zero_state_as_none (the "S0 = 0" cases).
    """
    dev = torch.device(device)
    draw = torch.float64 if dev.type == "cpu" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    n, t, hq, hv, d = shape.n, shape.t, shape.h_qk, shape.h_v, shape.d

    def normal(*size, mean=0.0, std=1.0):
        x = torch.randn(*size, generator=gen, device=dev, dtype=draw)
        return x * std + mean if (std != 1.0 or mean != 0.0) else x

    def direction(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)

    q = direction(normal(n, t, hq, d)).to(shape.dtype)
    k = direction(normal(n, t, hq, d)).to(shape.dtype)
    v = normal(n, t, hv, d).to(shape.dtype)
    beta = torch.sigmoid(normal(n, t, hv)).to(torch.float32)
    g = (-torch.log1p(torch.exp(-normal(n, t, hv, mean=2.0)))).to(torch.float32)
    state = None
    if s0_std > 0:
        state = normal(n, hv, d, d, std=s0_std).to(torch.float32)
    elif not zero_state_as_none:
        state = torch.zeros(n, hv, d, d, device=dev, dtype=torch.float32)
    if retrieval:
        g = torch.zeros_like(g)
        beta = torch.ones_like(beta)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g.contiguous(),
                beta=beta.contiguous(), state_in=state)
