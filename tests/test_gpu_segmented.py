"""GPU parity: gdn_prefill_segmented (bounded-workspace prompt chunking) against the fp64
oracle and against one gdn_prefill call over the whole prompt."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_oracle(c):
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("seg_t", [1, 7, 64, 100, 290, 1000])
def test_segmented_small(dtype, seg_t):
    """Two sequences, ragged segments (one token at a time, a chunked segment followed by a
    direct-scan remainder, one segment longer than the prompt), non-zero initial state: every
    output and state against the oracle; the overlapped schedule gives the same bits."""
    shape = Shape(n=2, t=300, h_qk=2, h_v=4, d=64, dtype=dtype)
    c = gdn_inputs.make_case(shape, seed=700 + seg_t, device=DEV, s0_std=0.1)
    out, st = gdn.gdn_prefill_segmented(**c, seg_t=seg_t)
    o2, s2 = gdn.gdn_prefill_segmented(**c, seg_t=seg_t, overlapped=True)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(c)
    assert_parity(out, st, o_ref, s_ref, f"segmented seg_t={seg_t} {dtype}")
    assert torch.equal(out, o2) and torch.equal(st, s2)


def test_segmented_in_place_and_empty():
    shape = Shape(n=1, t=130, h_qk=1, h_v=2, d=32)
    c = gdn_inputs.make_case(shape, seed=710, device=DEV, s0_std=0.1)
    o1, s1 = gdn.gdn_prefill_segmented(**c, seg_t=50)
    st = c["state_in"].clone()
    o2, _ = gdn.gdn_prefill_segmented(c["q"], c["k"], c["v"], c["g"], c["beta"], st,
                                      state_out=st, seg_t=50)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, st)
    e = {key: (val[:, :0].contiguous() if key != "state_in" else val) for key, val in c.items()}
    _, s0 = gdn.gdn_prefill_segmented(**e, seg_t=50)
    torch.cuda.synchronize()
    assert torch.equal(s0, c["state_in"])


@pytest.mark.parametrize("overlapped", [False, True], ids=["in_order", "overlapped"])
@pytest.mark.parametrize("seg_t", [1000, 1024, 8192])
def test_segmented_prefill_4k(seg_t, overlapped):
    """The 4096-token workload in segments (the chosen method per segment length): sampled
    V heads against the oracle, every head against one whole-prompt gdn_prefill call.
    q and k are written on the caller's stream right before the call, behind a long matrix
    product, after being filled with NaN: a segment that read them before the caller's
    earlier work had finished would produce NaN."""
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=2, device=DEV)
    src = {key: c[key] for key in ("q", "k")}
    seg_in = dict(c)
    for key in ("q", "k"):
        seg_in[key] = torch.full_like(src[key], float("nan"))
    torch.cuda.synchronize()
    a = torch.randn(8192, 8192, device=DEV)
    busy = a @ a  # several milliseconds on the caller's stream
    for key in ("q", "k"):
        seg_in[key].copy_(src[key])
    ws = torch.empty(gdn.gdn_prefill_segmented_workspace_bytes(1, 4096, 16, 32, 128, seg_t,
                                                               overlapped),
                     device=DEV, dtype=torch.uint8)
    ws.fill_(0xFF)  # stale slot contents must not leak into any segment
    out, st = gdn.gdn_prefill_segmented(**seg_in, seg_t=seg_t, workspace=ws, overlapped=overlapped)
    del busy
    whole_out, whole_st = gdn.gdn_prefill(**c)
    torch.cuda.synchronize()
    assert_parity(out, st, whole_out, whole_st, f"segmented {seg_t} vs whole call")
    heads = [4, 27]
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    for hv in heads:
        hq = hv // 2
        o_ref, s_ref = oracle.run(h["q"][:, :, hq:hq + 1].contiguous(), h["k"][:, :, hq:hq + 1].contiguous(),
                                  h["v"][:, :, hv:hv + 1].contiguous(), h["g"][:, :, hv:hv + 1].contiguous(),
                                  h["beta"][:, :, hv:hv + 1].contiguous())
        assert_parity(out[:, :, hv], st[:, hv], o_ref[:, :, 0], s_ref[:, 0], f"segmented {seg_t} head {hv}")


def test_single_token_prefill_is_the_decode_step():
    """gdn_prefill with t == 1 gives the decode step's bits (it runs that kernel)."""
    c = gdn_inputs.make_case(Shape(n=3, t=1, h_qk=16, h_v=32, d=128), seed=730, device=DEV,
                             s0_std=0.05)
    o1, s1 = gdn.gdn_prefill(**c)
    o2, s2 = gdn.gdn_decode_step(**c)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = run_oracle(c)
    assert_parity(o1, s1, o_ref, s_ref, "prefill t=1")
