"""GPU: the recorded per-layer decode (gdn_decode_graph_create / gdn_graph_launch) against
the same steps called one by one, and the per-layer steps against the fp64 oracle.

Thirty layers of the decode workload (16 QK / 32 V heads, d = 128, bf16, one sequence per
layer, initial states with standard deviation 0.02), each with its own inputs. The graph is
replayed three times with new inputs written in place between replays, with eager work and
synchronisation in between, and every replay must match the eager steps bitwise (same
kernels on the same inputs); the first token is also checked against the oracle.
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
LAYERS = 30
SHAPE = Shape(n=1, t=1, h_qk=16, h_v=32, d=128)


def token_inputs(seed):
    """One decode token's inputs for every layer (list of dicts of CUDA tensors)."""
    return [gdn_inputs.make_case(SHAPE, seed=seed * 100 + i, device=DEV, s0_std=0.02,
                                 zero_state_as_none=False) for i in range(LAYERS)]


def test_decode_graph_matches_eager_steps_and_oracle():
    first = token_inputs(1)
    keys = ("q", "k", "v", "g", "beta")
    # graph buffers (written in place per token) and an eager copy of everything
    buf = {key: [c[key].clone() for c in first] for key in keys}
    st_graph = [c["state_in"].clone() for c in first]
    st_eager = [c["state_in"].clone() for c in first]
    stream = torch.cuda.Stream()
    graph = gdn.DecodeGraph(buf["q"], buf["k"], buf["v"], buf["g"], buf["beta"], st_graph,
                            stream=stream)
    try:
        for token in range(3):
            cases = first if token == 0 else token_inputs(10 + token)
            for key in keys:
                for i in range(LAYERS):
                    buf[key][i].copy_(cases[i][key])
            torch.cuda.synchronize()
            graph.launch()
            eager_out = []
            for i in range(LAYERS):
                o, _ = gdn.gdn_decode_step(cases[i]["q"], cases[i]["k"], cases[i]["v"],
                                           cases[i]["g"], cases[i]["beta"], st_eager[i],
                                           state_out=st_eager[i])
                eager_out.append(o)
            torch.cuda.synchronize()
            for i in range(LAYERS):
                assert torch.equal(graph.out[i], eager_out[i]), (token, i)
                assert torch.equal(st_graph[i], st_eager[i]), (token, i)
            if token == 0:
                for i in (0, 17, 29):
                    h = {key: first[i][key].cpu() for key in keys}
                    o_ref, s_ref = oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"],
                                              first[i]["state_in"].cpu())
                    assert_parity(graph.out[i], st_graph[i], o_ref, s_ref, f"graph layer {i}")
    finally:
        graph.close()


def test_decode_graph_empty_and_reuse():
    """Zero layers records an empty graph; a handle replays after other graphs are made."""
    stream = torch.cuda.Stream()
    empty = gdn.DecodeGraph([], [], [], [], [], [], stream=stream)
    empty.launch()
    torch.cuda.synchronize()
    empty.close()
    c = token_inputs(3)[:2]
    st = [x["state_in"].clone() for x in c]
    ref = [x["state_in"].clone() for x in c]
    g1 = gdn.DecodeGraph([x["q"] for x in c], [x["k"] for x in c], [x["v"] for x in c],
                         [x["g"] for x in c], [x["beta"] for x in c], st, stream=stream)
    g2 = gdn.DecodeGraph([x["q"] for x in c], [x["k"] for x in c], [x["v"] for x in c],
                         [x["g"] for x in c], [x["beta"] for x in c],
                         [s.clone() for s in st], stream=stream)
    g1.launch()
    for i in range(2):
        gdn.gdn_decode_step(c[i]["q"], c[i]["k"], c[i]["v"], c[i]["g"], c[i]["beta"], ref[i],
                            state_out=ref[i])
    torch.cuda.synchronize()
    assert all(torch.equal(st[i], ref[i]) for i in range(2))
    g1.close()
    g2.close()
