"""GPU parity with every CU's LDS filled with NaN right before each call.

A kernel that reads LDS it never wrote (a padding slot, a row past a short chunk) takes
whatever the previous kernel left there; finite leftovers can hide such a read behind a
zero coefficient, NaN cannot (0 * NaN = NaN). Each case here first fills the LDS of every CU
with quiet NaNs, then runs the prefill and compares it with the oracle; non-finite outputs
or states fail. The cases are single chunks and short ragged tails of every chunk size,
in bf16 and fp32, where padding is most of the chunk.
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
NAN_BITS = 0x7FC00000


def run_oracle(c):
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"])


def filled(call):
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.debug_fill_lds(sink, NAN_BITS, blocks=4 * 256)
    res = call()
    torch.cuda.synchronize()
    assert int(sink.item()) == 0, "LDS fill failed"
    return res


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("t,chunk", [(16, 16), (31, 16), (20, 32), (32, 32), (1, 64), (5, 64),
                                     (64, 64), (65, 64), (100, 128), (128, 128), (129, 64)])
def test_chunked_single_and_tail_chunks(t, chunk, dtype):
    shape = Shape(n=1, t=t, h_qk=2, h_v=4, d=128, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=700 + t + chunk, device=DEV, s0_std=0.05)
    out, st = filled(lambda: gdn.gdn_prefill_chunked(**c, chunk=chunk))
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"LDS filled: chunked t={t} C={chunk} {dtype}")


@pytest.mark.parametrize("t", [1, 7, 16, 17, 23, 31, 32, 33])
def test_prefill_short(t):
    """gdn_prefill (the dispatching entry point) on short sequences, t = 16 .. 31 among
    them, at the full head layout."""
    shape = Shape(n=1, t=t, h_qk=16, h_v=32, d=128)
    c = gdn_inputs.make_case(shape, seed=800 + t, device=DEV, s0_std=0.05)
    out, st = filled(lambda: gdn.gdn_prefill(**c))
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"LDS filled: gdn_prefill t={t}")


@pytest.mark.parametrize("t", [1, 5, 64, 77])
def test_scan_short(t):
    shape = Shape(n=1, t=t, h_qk=2, h_v=4, d=128)
    c = gdn_inputs.make_case(shape, seed=900 + t, device=DEV, s0_std=0.05)
    out, st = filled(lambda: gdn.gdn_prefill_scan(**c))
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"LDS filled: scan t={t}")


@pytest.mark.parametrize("d", [16, 128])
def test_decode_step(d):
    shape = Shape(n=2, t=1, h_qk=2, h_v=4, d=d)
    c = gdn_inputs.make_case(shape, seed=950 + d, device=DEV, s0_std=0.3)
    out, st = filled(lambda: gdn.gdn_decode_step(**c))
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"LDS filled: decode d={d}")
