"""GPU parity: the state-residency ablation (gdn_prefill_scan_blockwise) gives the bits of the
resident direct scan for every block length, and matches the fp64 oracle."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("block_t", [1, 7, 32, 300, 1000])
def test_blockwise_small(dtype, block_t):
    """Two sequences, ragged blocks, non-zero initial state."""
    shape = Shape(n=2, t=300, h_qk=2, h_v=4, d=64, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=800 + block_t, device=DEV, s0_std=0.1)
    out, st = gdn.gdn_prefill_scan_blockwise(**c, block_t=block_t)
    ref_out, ref_st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    o_ref, s_ref = oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"])
    assert_parity(out, st, o_ref, s_ref, f"blockwise block_t={block_t} {dtype}")


def test_blockwise_empty():
    shape = Shape(n=1, t=40, h_qk=1, h_v=2, d=32)
    c = gdn_inputs.make_case(shape, seed=810, device=DEV, s0_std=0.1)
    e = {key: (val[:, :0].contiguous() if key != "state_in" else val) for key, val in c.items()}
    _, s0 = gdn.gdn_prefill_scan_blockwise(**e, block_t=8)
    torch.cuda.synchronize()
    assert torch.equal(s0, c["state_in"])


def test_blockwise_ablation_2k():
    """The ablation workload (2048 tokens, 16 QK / 32 V heads, d = 128, bf16) in 32-token
    blocks: the resident scan's bits, and sampled V heads against the oracle."""
    c = gdn_inputs.make_case(gdn_inputs.ABLATION_2K, seed=300, device=DEV)
    out, st = gdn.gdn_prefill_scan_blockwise(**c, block_t=32)
    ref_out, ref_st = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    for hv in (5, 30):
        hq = hv // 2
        o_ref, s_ref = oracle.run(h["q"][:, :, hq:hq + 1].contiguous(), h["k"][:, :, hq:hq + 1].contiguous(),
                                  h["v"][:, :, hv:hv + 1].contiguous(), h["g"][:, :, hv:hv + 1].contiguous(),
                                  h["beta"][:, :, hv:hv + 1].contiguous())
        assert_parity(out[:, :, hv], st[:, hv], o_ref[:, :, 0], s_ref[:, 0], f"blockwise 2K head {hv}")
