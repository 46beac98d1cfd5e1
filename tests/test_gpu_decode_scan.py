"""GPU parity: gdn_decode_step and gdn_prefill_scan against the fp64 oracle.

Every case draws seeded synthetic inputs on the GPU (gdn_inputs), runs the HIP library
through its C ABI, copies inputs and results to the host and compares them with the
oracle at the tolerances in parity.py.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cpu(c):
    return {key: (None if val is None else val.cpu()) for key, val in c.items()}


def run_oracle(c, eps=1e-6, heads=None):
    h = cpu(c)
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"], l2_eps=eps,
                      heads=heads)


def heads_of(out, st, heads, h_v):
    """Select flattened (seq * h_v + head) heads from [n, t, h_v, d] and [n, h_v, d, d]."""
    o = np.stack([to64(out)[hid // h_v, :, hid % h_v] for hid in heads])
    s = np.stack([to64(st)[hid // h_v, hid % h_v] for hid in heads])
    return o, s


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


def test_decode_30_layers_4096_steps():
    """The stacked decode workload: 30 layers x 32 V heads x 128x128 fp32 state,
    S0 ~ N(0, 0.02^2), 4096 consecutive steps with the state carried in place. The oracle
    follows a sample of (layer, head) pairs; outputs of every step and the state every
    512 steps are compared for them."""
    L, steps, snap = 30, 4096, 512
    per_step = Shape(n=L * steps, t=1, h_qk=16, h_v=32, d=128)
    c = gdn_inputs.make_case(per_step, seed=3, device=DEV)
    x = {key: c[key].view(steps, L, *c[key].shape[1:]) for key in ("q", "k", "v", "g", "beta")}
    s0 = gdn_inputs.make_case(Shape(n=L, t=1, h_qk=16, h_v=32, d=128), seed=33, device=DEV,
                              s0_std=0.02)["state_in"]
    st = s0.clone()
    outs = torch.empty(steps, L, 1, 32, 128, device=DEV)
    snaps = []
    for s in range(steps):
        gdn.gdn_decode_step(x["q"][s], x["k"][s], x["v"][s], x["g"][s], x["beta"][s], st,
                            out=outs[s], state_out=st)
        if (s + 1) % snap == 0:
            snaps.append(st.clone())
    torch.cuda.synchronize()
    assert torch.isfinite(outs).all() and torch.isfinite(st).all()
    sample = [(0, 0), (7, 13), (15, 31), (29, 30)]  # (layer, V head)
    for layer in sorted({l for l, _ in sample}):
        hs = [h for l, h in sample if l == layer]
        seq = {key: x[key][:, layer].reshape(1, steps, *x[key].shape[3:]).cpu()
               for key in ("q", "k", "v", "g", "beta")}
        state = s0[layer:layer + 1].cpu()
        for seg in range(steps // snap):
            sl = slice(seg * snap, (seg + 1) * snap)
            o_ref, s_ref = oracle.run(seq["q"][:, sl], seq["k"][:, sl], seq["v"][:, sl],
                                      seq["g"][:, sl], seq["beta"][:, sl], state, heads=hs)
            for h in hs:
                got_o = outs[sl, layer, 0, h].cpu()
                got_s = snaps[seg][layer, h].cpu()
                assert_parity(got_o, got_s, o_ref[0, :, h], s_ref[0, h],
                              f"decode layer {layer} head {h} steps {sl}")
            state = torch.from_numpy(s_ref)


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


def test_scan_prefill_4k_sampled_heads():
    """The 4096-token prefill workload (16 QK / 32 V heads, d=128, bf16, S0=0), every
    output of a sample of V heads against the oracle."""
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=2, device=DEV)
    out, st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    heads = [0, 1, 17, 31]
    o_ref, s_ref = run_oracle(c, heads=heads)
    got = heads_of(out, st, heads, 32)
    ref = heads_of(o_ref, s_ref, heads, 32)
    assert_parity(got[0], got[1], ref[0], ref[1], "scan 4k")


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
