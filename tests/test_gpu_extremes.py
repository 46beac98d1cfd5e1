"""GPU parity under extreme gates and write strengths, against the fp64 oracle: decays strong
enough that exp(gamma) underflows fp32 inside a chunk (g down to -60 per token), no decay,
a mix of both, and write strengths of exactly 0 and 1. The chunked form applies decays as
pairwise exp(gamma_r - gamma_s) <= 1, so none of these may overflow or produce NaN."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(kind, seed):
    c = gdn_inputs.make_case(Shape(n=2, t=150, h_qk=2, h_v=4, d=128), seed=seed, device=DEV,
                             s0_std=0.05)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    shape = c["g"].shape
    if kind == "strong_decay":
        g = -torch.rand(shape, generator=gen, dtype=torch.float64) * 60.0
    elif kind == "no_decay":
        g = torch.zeros(shape, dtype=torch.float64)
    else:  # mixed: mostly mild, with occasional resets
        g = -torch.rand(shape, generator=gen, dtype=torch.float64) * 0.1
        g[torch.rand(shape, generator=gen) < 0.05] = -50.0
    beta = torch.rand(shape, generator=gen, dtype=torch.float64)
    beta[torch.rand(shape, generator=gen) < 0.2] = 0.0
    beta[torch.rand(shape, generator=gen) < 0.2] = 1.0
    c["g"] = g.to(torch.float32).to(DEV)
    c["beta"] = beta.to(torch.float32).to(DEV)
    return c


def ref(c):
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"])


@pytest.mark.parametrize("kind", ["strong_decay", "no_decay", "mixed"])
@pytest.mark.parametrize("method", ["C16", "C32", "C64", "C128", "scan"])
def test_extreme_gates(kind, method):
    c = case(kind, seed=1300 + len(kind) + len(method))
    if method == "scan":
        out, st = gdn.gdn_prefill_scan(**c)
    else:
        out, st = gdn.gdn_prefill_chunked(**c, chunk=int(method[1:]))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(st).all()
    o_ref, s_ref = ref(c)
    assert_parity(out, st, o_ref, s_ref, f"{method} {kind}")


@pytest.mark.parametrize("kind", ["strong_decay", "no_decay", "mixed"])
def test_extreme_gates_decode(kind):
    c = case(kind, seed=1400 + len(kind))
    d1 = {key: (val[:, :1].contiguous() if key != "state_in" else val) for key, val in c.items()}
    out, st = gdn.gdn_decode_step(**d1)
    torch.cuda.synchronize()
    o_ref, s_ref = ref(d1)
    assert_parity(out, st, o_ref, s_ref, f"decode {kind}")


@pytest.mark.parametrize("method", ["C16", "C32", "C64", "C128", "scan", "decode"])
def test_extreme_input_scales(method):
    """q rows scaled by 1000, k rows exactly zero (they normalise to zero with l2_eps > 0,
    so their token writes nothing) and k rows of norm 1e-3 (where l2_eps matters): the
    normalisation inside every method matches the oracle's."""
    c = gdn_inputs.make_case(Shape(n=1, t=130, h_qk=2, h_v=4, d=128), seed=1500, device=DEV,
                             s0_std=0.05)
    gen = torch.Generator(device="cpu").manual_seed(1501)
    t = c["q"].shape[1]
    big = torch.rand(t, generator=gen) < 0.2
    zero = torch.rand(t, generator=gen) < 0.1
    tiny = (torch.rand(t, generator=gen) < 0.1) & ~zero
    q = c["q"].float().cpu()
    k = c["k"].float().cpu()
    q[:, big] *= 1000.0
    k[:, zero] = 0.0
    k[:, tiny] *= 1e-3
    c["q"] = q.to(c["v"].dtype).to(DEV)
    c["k"] = k.to(c["v"].dtype).to(DEV)
    if method == "decode":
        c = {key: (val[:, :1].contiguous() if key != "state_in" else val) for key, val in c.items()}
        out, st = gdn.gdn_decode_step(**c)
    elif method == "scan":
        out, st = gdn.gdn_prefill_scan(**c)
    else:
        out, st = gdn.gdn_prefill_chunked(**c, chunk=int(method[1:]))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(st).all()
    o_ref, s_ref = ref(c)
    assert_parity(out, st, o_ref, s_ref, f"{method} input scales")


@pytest.mark.parametrize("kind", ["spread_59", "spread_61", "some_positive"])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_decay_product_threshold(kind, chunk):
    """The chunked form takes the pairwise decays of a chunk as products of two exponentials
    when no gate is positive and the gate sum over the chunk's tokens after the first spans at
    most 60, and one exponential per element otherwise. Gates just inside (59) and just
    outside (61) that bound, and gates of both signs, against the oracle, over two full
    chunks and a ragged one."""
    shape = Shape(n=1, t=2 * chunk + 5, h_qk=2, h_v=4, d=128)
    c = gdn_inputs.make_case(shape, seed=1600 + chunk + len(kind), device=DEV, s0_std=0.05)
    gen = torch.Generator(device="cpu").manual_seed(1610 + chunk)
    if kind == "some_positive":
        g = torch.rand(c["g"].shape, generator=gen, dtype=torch.float64) * 0.25 - 0.2
    else:
        span = 59.0 if kind == "spread_59" else 61.0
        g = torch.full(c["g"].shape, -span / (chunk - 1), dtype=torch.float64)
    c["g"] = g.to(torch.float32).to(DEV)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(st).all()
    o_ref, s_ref = ref(c)
    assert_parity(out, st, o_ref, s_ref, f"C={chunk} {kind}")
