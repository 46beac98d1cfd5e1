"""GPU parity for V-head to QK-head ratios other than 2 (1, 3, 4 and 8 V heads per QK head):
the chunked kernels (which take the V heads of a QK head in pairs, repeating the last one
when the count is odd), the direct scan, the decode step and the ablation, against the fp64
oracle."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"

RATIOS = [(3, 3), (2, 6), (1, 4), (1, 8)]  # (h_qk, h_v)


def ref(c):
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"])


@pytest.mark.parametrize("h_qk,h_v", RATIOS)
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("d", [64, 128])
def test_chunked_gqa(h_qk, h_v, chunk, d):
    c = gdn_inputs.make_case(Shape(n=2, t=100, h_qk=h_qk, h_v=h_v, d=d), seed=1000 + h_v + d,
                             device=DEV, s0_std=0.05)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref = ref(c)
    assert_parity(out, st, o_ref, s_ref, f"chunked C={chunk} h_qk={h_qk} h_v={h_v} d={d}")


@pytest.mark.parametrize("h_qk,h_v", RATIOS)
def test_scan_decode_blockwise_gqa(h_qk, h_v):
    c = gdn_inputs.make_case(Shape(n=2, t=40, h_qk=h_qk, h_v=h_v, d=128), seed=1100 + h_v,
                             device=DEV, s0_std=0.05)
    o_ref, s_ref = ref(c)
    out, st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    assert_parity(out, st, o_ref, s_ref, f"scan h_qk={h_qk} h_v={h_v}")
    out_b, st_b = gdn.gdn_prefill_scan_blockwise(**c, block_t=9)
    torch.cuda.synchronize()
    assert torch.equal(out_b, out) and torch.equal(st_b, st)
    d1 = {key: (val[:, :1].contiguous() if key != "state_in" else val) for key, val in c.items()}
    o1_ref, s1_ref = ref(d1)
    o1, s1 = gdn.gdn_decode_step(**d1)
    torch.cuda.synchronize()
    assert_parity(o1, s1, o1_ref, s1_ref, f"decode h_qk={h_qk} h_v={h_v}")


def test_chunked64_one_v_head_per_qk_head_staggered():
    """One V head per QK head at 4096 tokens (16 heads, 1,024 (chunk, head) items): the
    64-token preparation then runs one workgroup per V head with the staggered start; every
    head's outputs and state against the oracle."""
    c = gdn_inputs.make_case(Shape(n=1, t=4096, h_qk=16, h_v=16, d=128), seed=1150, device=DEV,
                             s0_std=0.02)
    out, st = gdn.gdn_prefill_chunked(**c, chunk=64)
    torch.cuda.synchronize()
    o_ref, s_ref = ref(c)
    assert_parity(out, st, o_ref, s_ref, "chunked C=64 h_qk=h_v=16 t=4096")
