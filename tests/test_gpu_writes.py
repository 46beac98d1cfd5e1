"""Every output element is written, by every entry point: out and state_out are filled with
NaN before the call and must come back finite and bit-identical to a call into zero-filled
buffers (a missed store or a read of an unwritten output would show as NaN or a difference).
The same pair of calls also checks that each result is the same run to run."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
from gdn_inputs import Shape

pytestmark = pytest.mark.gpu
DEV = "cuda"


def outputs(c, fill):
    n, t, h_v, d = c["v"].shape
    out = torch.full((n, t, h_v, d), fill, device=DEV)
    st = torch.full((n, h_v, d, d), fill, device=DEV)
    return out, st


def check(call, c):
    nan_out, nan_st = outputs(c, float("nan"))
    zero_out, zero_st = outputs(c, 0.0)
    call(nan_out, nan_st)
    call(zero_out, zero_st)
    torch.cuda.synchronize()
    assert torch.isfinite(nan_out).all() and torch.isfinite(nan_st).all()
    assert torch.equal(nan_out, zero_out) and torch.equal(nan_st, zero_st)


# ragged lengths (partial last chunk, shorter than one chunk) and every head size
CASES = [(1, 100, 128), (2, 37, 64), (1, 16, 32), (1, 45, 16), (3, 250, 128)]


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("n,t,d", CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_chunked_writes_every_output(chunk, n, t, d, dtype):
    c = gdn_inputs.make_case(Shape(n=n, t=t, h_qk=2, h_v=4, d=d, dtype=dtype), seed=900 + t,
                             device=DEV, s0_std=0.05)
    check(lambda o, s: gdn.gdn_prefill_chunked(**c, chunk=chunk, out=o, state_out=s), c)


@pytest.mark.parametrize("n,t,d", CASES)
def test_scan_and_blockwise_write_every_output(n, t, d):
    c = gdn_inputs.make_case(Shape(n=n, t=t, h_qk=2, h_v=4, d=d), seed=910 + t, device=DEV,
                             s0_std=0.05)
    check(lambda o, s: gdn.gdn_prefill_scan(**c, out=o, state_out=s), c)
    check(lambda o, s: gdn.gdn_prefill_scan_blockwise(**c, block_t=7, out=o, state_out=s), c)


@pytest.mark.parametrize("overlapped", [False, True], ids=["in_order", "overlapped"])
def test_segmented_writes_every_output(overlapped):
    c = gdn_inputs.make_case(Shape(n=2, t=600, h_qk=2, h_v=4, d=128), seed=920, device=DEV,
                             s0_std=0.05)
    check(lambda o, s: gdn.gdn_prefill_segmented(**c, seg_t=250, overlapped=overlapped,
                                                 out=o, state_out=s), c)


@pytest.mark.parametrize("n", [1, 30])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_decode_writes_every_output(n, d):
    c = gdn_inputs.make_case(Shape(n=n, t=1, h_qk=16, h_v=32, d=d), seed=930 + n, device=DEV,
                             s0_std=0.05)
    check(lambda o, s: gdn.gdn_decode_step(**c, out=o, state_out=s), c)


def test_prefill_4k_writes_every_output():
    """The bench workload through the chosen method (chunk 32)."""
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=940, device=DEV)
    check(lambda o, s: gdn.gdn_prefill(**c, out=o, state_out=s), c)
