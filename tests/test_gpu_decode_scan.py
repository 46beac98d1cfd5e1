"""GPU parity: gdn_decode_step and gdn_prefill_scan against the fp64 oracle.

Every case draws seeded synthetic inputs on the GPU (gdn_inputs), runs the HIP library
through its C ABI, copies inputs and results to the host and compares them with the
oracle at the tolerances in parity.py.
"""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cpu(c):
    return {key: (None if val is None else val.cpu()) for key, val in c.items()}


def run_oracle(c, eps=1e-6, heads=None):
    h = cpu(c)
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"], l2_eps=eps,
                      heads=heads)


# ----------------------------------------------------------------------------- decode
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_one_step(d, dtype):
    shape = Shape(n=3, t=1, h_qk=2, h_v=4, d=d, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=100 + d, device=DEV, s0_std=0.5)
    out, st = gdn.gdn_decode_step(**c)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"decode d={d} {dtype}")


def test_decode_in_place_and_zero_state():
    shape = Shape(n=2, t=1, h_qk=2, h_v=4, d=64)
    c = gdn_inputs.make_case(shape, seed=7, device=DEV, s0_std=0.3)
    o_ref, s_ref = run_oracle(c)
    st = c["state_in"].clone()
    out, st2 = gdn.gdn_decode_step(c["q"], c["k"], c["v"], c["g"], c["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr()
    assert_parity(out, st, o_ref, s_ref, "decode in place")
    c0 = dict(c, state_in=None)
    o_ref, s_ref = run_oracle(c0)
    out, st = gdn.gdn_decode_step(**c0)
    torch.cuda.synchronize()
    assert_parity(out, st, o_ref, s_ref, "decode zero state")


def test_decode_tiny_as_64_steps():
    """The tiny fp32 workload (T=64, 1 QK + 2 V heads, d=16) as 64 decode calls."""
    c = gdn_inputs.make_case(gdn_inputs.TINY, seed=1, device=DEV)
    o_ref, s_ref = run_oracle(c)
    st = torch.zeros(1, 2, 16, 16, device=DEV)
    outs = []
    for t in range(64):
        out, _ = gdn.gdn_decode_step(c["q"][:, t:t + 1].contiguous(), c["k"][:, t:t + 1].contiguous(),
                                     c["v"][:, t:t + 1].contiguous(), c["g"][:, t:t + 1].contiguous(),
                                     c["beta"][:, t:t + 1].contiguous(), st, state_out=st)
        outs.append(out)
    torch.cuda.synchronize()
    assert_parity(torch.cat(outs, dim=1), st, o_ref, s_ref, "decode tiny x64")


# ----------------------------------------------------------------------------- scan
def test_scan_tiny():
    c = gdn_inputs.make_case(gdn_inputs.TINY, seed=1, device=DEV)
    out, st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, "scan tiny")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("t", [1, 37, 100])
def test_scan_shapes(d, dtype, t):
    shape = Shape(n=2, t=t, h_qk=2, h_v=4, d=d, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=200 + t + d, device=DEV, s0_std=0.1)
    out, st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"scan d={d} t={t} {dtype}")


def test_scan_in_place_empty_and_deterministic():
    shape = Shape(n=1, t=50, h_qk=2, h_v=4, d=32)
    c = gdn_inputs.make_case(shape, seed=9, device=DEV, s0_std=0.2)
    o1, s1 = gdn.gdn_prefill_scan(**c)
    st = c["state_in"].clone()
    o2, _ = gdn.gdn_prefill_scan(c["q"], c["k"], c["v"], c["g"], c["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, st)  # bitwise run to run
    # t == 0: the state passes through (or is zeroed when state_in is None)
    e = {key: (val[:, :0].contiguous() if key != "state_in" else val) for key, val in c.items()}
    _, s0 = gdn.gdn_prefill_scan(**e)
    _, z0 = gdn.gdn_prefill_scan(**dict(e, state_in=None))
    torch.cuda.synchronize()
    assert torch.equal(s0, c["state_in"]) and torch.count_nonzero(z0) == 0


def test_scan_retrieval_and_column_independence():
    shape = Shape(n=1, t=64, h_qk=2, h_v=4, d=64)
    c = gdn_inputs.make_case(shape, seed=11, device=DEV, retrieval=True)
    # g = 0, beta = 1 and q = k: every output returns its own value vector
    out, _ = gdn.gdn_prefill_scan(c["k"], c["k"], c["v"], c["g"], c["beta"], l2_eps=0.0)
    v = c["v"].float()
    torch.cuda.synchronize()
    err = (out - v).abs().max().item() / v.pow(2).mean().sqrt().item()
    assert err < 2e-3, err
    # a zero value channel with a zero state column stays exactly zero
    c = gdn_inputs.make_case(shape, seed=12, device=DEV, s0_std=0.1)
    c["v"][..., 5] = 0
    c["state_in"][..., 5] = 0
    out, st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[..., 5]) == 0 and torch.count_nonzero(st[..., 5]) == 0
