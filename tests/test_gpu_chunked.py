"""GPU parity: gdn_prefill_chunked against the fp64 oracle on small and ragged shapes, every
chunk size, head dimension and input dtype (the workloads' full sizes are in
test_gpu_fullsize.py).
"""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity, out_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cpu(c):
    return {key: (None if val is None else val.cpu()) for key, val in c.items()}


def run_oracle(c, eps=1e-6):
    h = cpu(c)
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"], l2_eps=eps)


# ------------------------------------------------------------------------ small cases
def test_chunked_tiny():
    """The tiny fp32 workload: T=64, 1 QK + 2 V heads, d=16, chunk 16; scan and chunked
    against the oracle."""
    c = gdn_inputs.make_case(gdn_inputs.TINY, seed=1, device=DEV)
    o_ref, s_ref = run_oracle(c)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=16)
    out2, st2 = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    assert_parity(out, st, o_ref, s_ref, "chunked tiny C=16")
    assert_parity(out2, st2, o_ref, s_ref, "scan tiny")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_chunked_shapes(d, dtype, chunk):
    """Several chunks plus a ragged tail (T mod C != 0), non-zero initial state, two V
    heads per QK head, two sequences."""
    t = 3 * chunk + 7
    shape = Shape(n=2, t=t, h_qk=2, h_v=4, d=d, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=300 + d + chunk, device=DEV, s0_std=0.1)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"chunked d={d} C={chunk} t={t} {dtype}")


@pytest.mark.parametrize("t,chunk", [(1, 64), (5, 64), (63, 64), (64, 64), (65, 64),
                                     (100, 32), (127, 128), (129, 128), (17, 16)])
def test_chunked_tails(t, chunk):
    shape = Shape(n=1, t=t, h_qk=4, h_v=8, d=128)
    c = gdn_inputs.make_case(shape, seed=400 + t, device=DEV, s0_std=0.05)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"chunked tail t={t} C={chunk}")


@pytest.mark.parametrize("n,t", [(1, 150), (2, 300), (2, 192)])
def test_chunked64_odd_chunk_counts(n, t):
    """The 64-token kernel (d = 128, bf16) with an odd number of chunks greater than one
    (3, 5 and 3 full ones): its two-window loop ends in a padding window that must leave
    each sequence's state unchanged."""
    shape = Shape(n=n, t=t, h_qk=2, h_v=4, d=128)
    c = gdn_inputs.make_case(shape, seed=460 + t + n, device=DEV, s0_std=0.1)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=64)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"chunked C=64 n={n} t={t}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("t,chunk", [(16, 16), (31, 16), (20, 32), (32, 32)])
def test_chunked_single_chunk(t, chunk, dtype):
    """Prompts of one chunk (a full one and a short one at C = 16 and 32): the pipelined
    scan runs its first and last windows on the same chunk."""
    shape = Shape(n=1, t=t, h_qk=2, h_v=4, d=128, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=450 + t + chunk, device=DEV, s0_std=0.1)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"chunked single chunk t={t} C={chunk} {dtype}")
    out2, st2 = gdn.gdn_prefill(**c)
    torch.cuda.synchronize()
    assert_parity(out2, st2, o_ref, s_ref, f"dispatched t={t} {dtype}")


def test_chunked_head_groups():
    """h_v / h_qk = 1 and 4 (the mapping V head h -> QK head h // group)."""
    for h_qk, h_v in ((4, 4), (2, 8)):
        shape = Shape(n=1, t=80, h_qk=h_qk, h_v=h_v, d=64)
        c = gdn_inputs.make_case(shape, seed=500 + h_v, device=DEV, s0_std=0.1)
        out, st = gdn.gdn_prefill_chunked(**c, chunk=32)
        torch.cuda.synchronize()
        o_ref, s_ref = run_oracle(c)
        assert_parity(out, st, o_ref, s_ref, f"chunked h_qk={h_qk} h_v={h_v}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunked_in_place_empty_deterministic(chunk):
    shape = Shape(n=1, t=200, h_qk=2, h_v=4, d=128)
    c = gdn_inputs.make_case(shape, seed=9, device=DEV, s0_std=0.2)
    o1, s1 = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    st = c["state_in"].clone()
    o2, _ = gdn.gdn_prefill_chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], st, state_out=st,
                                    chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, st)  # bitwise run to run, in place
    e = {key: (val[:, :0].contiguous() if key != "state_in" else val) for key, val in c.items()}
    _, s0 = gdn.gdn_prefill_chunked(**e, chunk=chunk)
    _, z0 = gdn.gdn_prefill_chunked(**dict(e, state_in=None), chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(s0, c["state_in"]) and torch.count_nonzero(z0) == 0


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunked_retrieval_and_column_independence(chunk):
    shape = Shape(n=1, t=256, h_qk=2, h_v=4, d=128)
    c = gdn_inputs.make_case(shape, seed=11, device=DEV, retrieval=True)
    out, _ = gdn.gdn_prefill_chunked(c["k"], c["k"], c["v"], c["g"], c["beta"], l2_eps=0.0,
                                     chunk=chunk)
    torch.cuda.synchronize()
    assert out_error(out, c["v"]) < 2e-3
    c = gdn_inputs.make_case(shape, seed=12, device=DEV, s0_std=0.1)
    c["v"][..., 77] = 0
    c["state_in"][..., 77] = 0
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[..., 77]) == 0 and torch.count_nonzero(st[..., 77]) == 0
