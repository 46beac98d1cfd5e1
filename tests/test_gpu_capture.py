"""The compute calls may be recorded under HIP stream capture (they enqueue kernels only, no
memset or copy): prefill (chunked, scan, an empty call), the decode step and in-order
segmented prefill recorded into one graph, replayed three times with the outputs cleared by
eager work between replays, every replay checked bit for bit against the eager results. The
overlapped segmented schedule refuses a capturing stream without disturbing the capture."""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
from gdn_inputs import Shape

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_calls_replay_from_a_graph():
    pre = gdn_inputs.make_case(Shape(n=2, t=700, h_qk=4, h_v=8, d=128), seed=1200, device=DEV,
                               s0_std=0.05)
    short = gdn_inputs.make_case(Shape(n=1, t=9, h_qk=4, h_v=8, d=64), seed=1201, device=DEV)
    dec = gdn_inputs.make_case(Shape(n=3, t=1, h_qk=4, h_v=8, d=128), seed=1202, device=DEV,
                               s0_std=0.05)
    empty = {key: (val[:, :0].contiguous() if key != "state_in" else val) for key, val in pre.items()}

    def buffers(c):
        n, t, h_v, d = c["v"].shape
        return torch.empty(n, t, h_v, d, device=DEV), torch.empty(n, h_v, d, d, device=DEV)

    outs = {name: buffers(c) for name, c in (("chunked", pre), ("scan", short), ("decode", dec),
                                             ("segmented", pre), ("empty", empty))}
    ws_c = torch.empty(gdn.gdn_workspace_bytes(2, 700, 4, 8, 128, chunk=32), device=DEV,
                       dtype=torch.uint8)
    ws_s = torch.empty(gdn.gdn_workspace_bytes(1, 9, 4, 8, 64, chunk=0), device=DEV,
                       dtype=torch.uint8)
    ws_g = torch.empty(gdn.gdn_prefill_segmented_workspace_bytes(2, 700, 4, 8, 128, 256),
                       device=DEV, dtype=torch.uint8)
    ws_o = torch.empty(gdn.gdn_prefill_segmented_workspace_bytes(2, 700, 4, 8, 128, 256, True),
                       device=DEV, dtype=torch.uint8)

    def run_all():
        gdn.gdn_prefill_chunked(**pre, chunk=32, out=outs["chunked"][0],
                                state_out=outs["chunked"][1], workspace=ws_c)
        gdn.gdn_prefill_scan(**short, out=outs["scan"][0], state_out=outs["scan"][1],
                             workspace=ws_s)
        gdn.gdn_decode_step(**dec, out=outs["decode"][0], state_out=outs["decode"][1])
        gdn.gdn_prefill_segmented(**pre, seg_t=256, out=outs["segmented"][0],
                                  state_out=outs["segmented"][1], workspace=ws_g)
        gdn.gdn_prefill_chunked(**empty, chunk=32, out=outs["empty"][0],
                                state_out=outs["empty"][1], workspace=ws_c)

    run_all()
    torch.cuda.synchronize()
    eager = {name: (o.clone(), s.clone()) for name, (o, s) in outs.items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        with pytest.raises(gdn.GdnError, match="UNSUPPORTED"):
            gdn.gdn_prefill_segmented(**pre, seg_t=256, overlapped=True, workspace=ws_o)
        run_all()
    torch.cuda.synchronize()

    for replay in range(3):
        for o, s in outs.values():
            o.fill_(float("nan"))
            s.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, (o, s) in outs.items():
            assert torch.equal(o, eager[name][0]) and torch.equal(s, eager[name][1]), (replay, name)


def test_mfma_calibration_loop_runs():
    """gdn_calib_mfma_bf16 (measurement only): the launch completes, the reported flops follow
    its shape, and every lane writes a finite sum."""
    sink = torch.full((16 * 256,), float("nan"), device=DEV)
    flops = gdn.calib_mfma_bf16(5, 16, sink)
    torch.cuda.synchronize()
    assert flops == 16 * 4 * 5 * 4 * 32 * 32 * 16 * 2
    assert torch.isfinite(sink).all()
