"""GPU: the allocation-free segmented prefill (gdn_prefill_segmented_noalloc, its workspace in
the library's static per-GPU array) gives the same bits as gdn_prefill_segmented with a
caller workspace and the in-order schedule, on two calls in a row (the second smaller, so
it runs on the array as the first call left it), and rejects segments whose workspace
exceeds the array."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(shape, seed, seg_t, s0_std):
    c = gdn_inputs.make_case(shape, seed=seed, device=DEV, s0_std=s0_std)
    n, t, hv, d = shape.n, shape.t, shape.h_v, shape.d
    out = torch.full((n, t, hv, d), float("nan"), device=DEV)
    st = torch.full((n, hv, d, d), float("nan"), device=DEV)
    gdn.gdn_prefill_segmented_noalloc(**c, seg_t=seg_t, out=out, state_out=st)
    ref_out, ref_st = gdn.gdn_prefill_segmented(**c, seg_t=seg_t, overlapped=False)
    torch.cuda.synchronize()
    return out, st, ref_out, ref_st


def test_noalloc_matches_segmented_twice():
    # 1: the 4K layout, two sequences, ragged last segment (3000 = 2 x 1024 + 952), S0 != 0
    big = Shape(n=2, t=3000, h_qk=16, h_v=32, d=128)
    out, st, ref_out, ref_st = _pair(big, seed=910, seg_t=1024, s0_std=0.02)
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    assert_parity(out, st, ref_out.double(), ref_st.double(), "noalloc 1")
    # 2: smaller, other heads and dtype, segments of other lengths (chunked and direct scan)
    small = Shape(n=1, t=500, h_qk=2, h_v=4, d=64, dtype=torch.float32)
    out, st, ref_out, ref_st = _pair(small, seed=911, seg_t=203, s0_std=0.1)
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    assert_parity(out, st, ref_out.double(), ref_st.double(), "noalloc 2")


def test_noalloc_rejects_oversized_segments():
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=912, device=DEV)
    out = torch.full((1, 4096, 32, 128), 7.0, device=DEV)
    st = torch.full((1, 32, 128, 128), 7.0, device=DEV)
    with pytest.raises(gdn.GdnError, match="WORKSPACE"):
        gdn.gdn_prefill_segmented_noalloc(**c, seg_t=2048, out=out, state_out=st)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((st == 7.0).all())
