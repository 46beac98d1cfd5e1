"""The Python binding rejects tensors that do not match the call before anything is
launched: a wrong shape, dtype, device or layout of any tensor would otherwise reach the
kernels as a raw pointer and read or write out of bounds.

The CPU tests use CPU tensors (rejected as not on the GPU). The GPU tests build one valid
call per entry point, spoil one tensor at a time, and check that ValueError is raised and
that the caller's output buffers were not touched.
"""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs

SHAPE = gdn_inputs.Shape(n=2, t=40, h_qk=2, h_v=4, d=32)


def _case(device):
    return gdn_inputs.make_case(SHAPE, seed=11, device=device, s0_std=0.05)


def test_cpu_tensors_are_rejected():
    c = _case("cpu")
    for fn in (gdn.gdn_prefill_chunked, gdn.gdn_prefill_scan, gdn.gdn_prefill):
        with pytest.raises(ValueError, match="CUDA"):
            fn(**c)
    d1 = {key: (val[:, :1].contiguous() if key != "state_in" else val) for key, val in c.items()}
    with pytest.raises(ValueError, match="CUDA"):
        gdn.gdn_decode_step(**d1)


def test_non_tensor_arguments_are_rejected():
    c = _case("cpu")
    c["k"] = c["k"].float().numpy()
    with pytest.raises(ValueError):
        gdn.gdn_prefill_chunked(**c)


def _spoilers(c):
    """(name, kwargs-override) pairs, each one wrong in exactly one way."""
    n, t, hq, hv, d = SHAPE.n, SHAPE.t, SHAPE.h_qk, SHAPE.h_v, SHAPE.d
    dev = c["q"].device
    f32 = torch.float32
    bad = [
        ("k short", dict(k=c["k"][:, :-1].contiguous())),
        ("k other heads", dict(k=torch.zeros(n, t, hq * 2, d, device=dev, dtype=c["k"].dtype))),
        ("k fp32", dict(k=c["k"].float())),
        ("v short", dict(v=c["v"][:, :-1].contiguous())),
        ("v other d", dict(v=torch.zeros(n, t, hv, d // 2, device=dev, dtype=c["v"].dtype))),
        ("g short", dict(g=c["g"][:, :-1].contiguous())),
        ("g bf16", dict(g=c["g"].to(torch.bfloat16))),
        ("beta short", dict(beta=c["beta"][:, :, :-1].contiguous())),
        ("beta 4-d", dict(beta=c["beta"].unsqueeze(-1))),
        ("state_in short", dict(state_in=c["state_in"][:-1].contiguous())),
        ("state_in bf16", dict(state_in=c["state_in"].to(torch.bfloat16))),
        ("state_in transposed view", dict(state_in=c["state_in"].transpose(2, 3))),
        ("k on cpu", dict(k=c["k"].cpu())),
        ("q non-contiguous", dict(q=c["q"].transpose(0, 1).contiguous().transpose(0, 1))
         if n > 1 else dict(q=c["q"][:, ::2])),
        ("out too small", dict(out=torch.zeros(n, t - 1, hv, d, device=dev, dtype=f32))),
        ("out bf16", dict(out=torch.zeros(n, t, hv, d, device=dev, dtype=torch.bfloat16))),
        ("out on cpu", dict(out=torch.zeros(n, t, hv, d, dtype=f32))),
        ("state_out too small", dict(state_out=torch.zeros(n, hv, d, d - 1, device=dev, dtype=f32))),
        ("state_out bf16", dict(state_out=torch.zeros(n, hv, d, d, device=dev, dtype=torch.bfloat16))),
        ("state_out strided", dict(state_out=torch.zeros(n, hv, d, 2 * d, device=dev, dtype=f32)[..., ::2])),
    ]
    return bad


@pytest.mark.gpu
@pytest.mark.parametrize("entry", ["chunked", "scan", "prefill", "segmented"])
def test_spoiled_prefill_calls_raise_before_launch(entry):
    dev = "cuda:0"
    c = _case(dev)
    fn = {"chunked": lambda **kw: gdn.gdn_prefill_chunked(chunk=32, **kw),
          "scan": gdn.gdn_prefill_scan, "prefill": gdn.gdn_prefill,
          "segmented": lambda **kw: gdn.gdn_prefill_segmented(seg_t=16, **kw)}[entry]
    n, t, hv, d = SHAPE.n, SHAPE.t, SHAPE.h_v, SHAPE.d
    for name, over in _spoilers(c):
        out = torch.full((n, t, hv, d), 7.0, device=dev)
        st = torch.full((n, hv, d, d), 7.0, device=dev)
        kw = dict(c, out=out, state_out=st)
        kw.update(over)
        with pytest.raises(ValueError):
            fn(**kw)
        torch.cuda.synchronize()
        if "out" not in over:
            assert bool((out == 7.0).all()), f"{entry}/{name}: out was written"
        if "state_out" not in over:
            assert bool((st == 7.0).all()), f"{entry}/{name}: state_out was written"


@pytest.mark.gpu
def test_spoiled_workspace_is_rejected():
    dev = "cuda:0"
    c = _case(dev)
    need = gdn.gdn_workspace_bytes(SHAPE.n, SHAPE.t, SHAPE.h_qk, SHAPE.h_v, SHAPE.d, chunk=32)
    for ws in (torch.zeros(need // 4 + 1, device=dev, dtype=torch.float32),
               torch.zeros(need, dtype=torch.uint8),
               torch.zeros(2 * need, device=dev, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError, match="workspace"):
            gdn.gdn_prefill_chunked(chunk=32, workspace=ws, **c)


@pytest.mark.gpu
def test_spoiled_decode_calls_raise_before_launch():
    dev = "cuda:0"
    c = _case(dev)
    d1 = {key: (val[:, :1].contiguous() if key != "state_in" else val) for key, val in c.items()}
    n, hv, d = SHAPE.n, SHAPE.h_v, SHAPE.d
    for name, over in [("k short", dict(k=d1["k"][:1].contiguous())),
                       ("g 2 tokens", dict(g=c["g"][:, :2].contiguous())),
                       ("beta fp64", dict(beta=d1["beta"].double())),
                       ("state_out bf16", dict(state_out=torch.zeros(n, hv, d, d, device=dev,
                                                                     dtype=torch.bfloat16)))]:
        out = torch.full((n, 1, hv, d), 7.0, device=dev)
        kw = dict(d1, out=out)
        kw.update(over)
        with pytest.raises(ValueError):
            gdn.gdn_decode_step(**kw)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all()), name


@pytest.mark.gpu
def test_decode_graph_rejects_layers_of_other_shapes():
    dev = "cuda:0"
    mk = lambda hq, hv: gdn_inputs.make_case(gdn_inputs.Shape(1, 1, hq, hv, 32), seed=3,
                                             device=dev, s0_std=0.02)
    a, b = mk(2, 4), mk(1, 2)
    layers = [a, b]
    s = torch.cuda.Stream()
    with pytest.raises(ValueError, match="layer 1"):
        gdn.DecodeGraph([x["q"] for x in layers], [x["k"] for x in layers],
                        [x["v"] for x in layers], [x["g"] for x in layers],
                        [x["beta"] for x in layers], [x["state_in"] for x in layers], stream=s)
