"""GPU parity: gdn_prefill_chunked (and the scan/chunk sweep grid) against the fp64 oracle.

Large cases compare a sample of V heads: the oracle runs a problem built from the sampled
heads' slices with one QK head per V head, which is the same computation bitwise (pinned by
the oracle's head-mapping test).
"""
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity, out_error, state_error

pytestmark = pytest.mark.gpu
DEV = "cuda"
FULL = dict(h_qk=16, h_v=32, d=128)


def cpu(c):
    return {key: (None if val is None else val.cpu()) for key, val in c.items()}


def run_oracle(c, eps=1e-6):
    h = cpu(c)
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"], l2_eps=eps)


def head_slice(c, heads, grp):
    """Inputs of the given V heads alone, as a problem with one QK head per V head (V head
    i of the slice reads QK head i), on the CPU."""
    hs = list(heads)
    qk = [h // grp for h in hs]
    s = {"q": c["q"][:, :, qk], "k": c["k"][:, :, qk], "v": c["v"][:, :, hs],
         "g": c["g"][:, :, hs], "beta": c["beta"][:, :, hs],
         "state_in": None if c["state_in"] is None else c["state_in"][:, hs]}
    return {key: (None if val is None else val.contiguous().cpu()) for key, val in s.items()}


def oracle_heads(c, heads, grp):
    """{head: (out [n, t, 1, d], state [n, 1, d, d])} from one oracle run over the sample."""
    s = head_slice(c, heads, grp)
    o, st = oracle.run(s["q"], s["k"], s["v"], s["g"], s["beta"], s["state_in"])
    return {h: (o[:, :, i:i + 1], st[:, i:i + 1]) for i, h in enumerate(heads)}


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


# ------------------------------------------------------------------------ full sizes
def bench_chunk(shape):
    """The method gdn_prefill picks for a shape (what the benchmark times); chunked here."""
    chunk = gdn.gdn_prefill_choose(shape.t, shape.h_qk, shape.h_v, shape.d, shape.n, shape.dtype)
    assert chunk > 0, chunk
    return chunk


@pytest.mark.parametrize("which", ["dispatch", "C=64"])
def test_chunked_prefill_4k(which):
    """The 4096-token prefill workload (16 QK / 32 V heads, d=128, bf16, S0=0) in the launch
    configuration the benchmark times (the chunk gdn_prefill picks, 32 on MI355X) and at
    chunk 64: every output and the final state of a sample of V heads against the oracle;
    all heads against the direct scan."""
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=2, device=DEV)
    chunk = bench_chunk(gdn_inputs.PREFILL_4K) if which == "dispatch" else 64
    out, st = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    out_s, st_s = gdn.gdn_prefill_scan(**c)
    torch.cuda.synchronize()
    heads = [0, 5, 18, 31]
    ref = oracle_heads(c, heads, 2)
    for h in heads:
        assert_parity(out[:, :, h], st[:, h], ref[h][0][:, :, 0], ref[h][1][:, 0], f"4k head {h}")
    # every head: chunked and scan agree to the same bar
    assert_parity(out, st, out_s, st_s, "4k chunked vs scan, all heads")


def test_chunked_long_131072_segments():
    """The long-prefill workload: T = 131072 as 32 segments of 4096 with the state carried
    between calls, with the chunk gdn_prefill picks for a segment. Per-segment outputs and
    the final state of sampled V heads against one single-pass oracle run."""
    seg_t, nseg = gdn_inputs.LONG_SEGMENT.t, gdn_inputs.LONG_SEGMENTS
    heads = [3, 28]
    st = torch.zeros(1, 32, 128, 128, device=DEV)
    host = {key: [] for key in ("q", "k", "v", "g", "beta")}
    outs = []
    chunk = bench_chunk(gdn_inputs.LONG_SEGMENT)
    ws = torch.empty(gdn.gdn_workspace_bytes(1, seg_t, 16, 32, 128, chunk=chunk), device=DEV,
                     dtype=torch.uint8)
    out = torch.empty(1, seg_t, 32, 128, device=DEV)
    for s in range(nseg):
        c = gdn_inputs.make_case(gdn_inputs.LONG_SEGMENT, seed=4000 + s, device=DEV)
        gdn.gdn_prefill_chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], st, out=out,
                                state_out=st, workspace=ws, chunk=chunk)
        sl = head_slice(c, heads, 2)
        for key in host:
            host[key].append(sl[key])
        outs.append(out[:, :, heads].cpu())
    torch.cuda.synchronize()
    assert torch.isfinite(st).all()
    full = {key: torch.cat(val, dim=1) for key, val in host.items()}
    o_ref, s_ref = oracle.run(full["q"], full["k"], full["v"], full["g"], full["beta"])
    for i, h in enumerate(heads):
        worst = 0.0
        for s in range(nseg):
            sl = slice(s * seg_t, (s + 1) * seg_t)
            worst = max(worst, out_error(outs[s][:, :, i], o_ref[:, sl, i]))
        es = state_error(st[:, h], s_ref[:, i])
        print(f"long head {h}: worst segment out err {worst:.3e}, final state {es:.3e}")
        assert worst <= 2e-3 and es <= 1e-3, (h, worst, es)


@pytest.mark.parametrize("t", gdn_inputs.SWEEP_T)
def test_sweep_grid_parity(t):
    """The scan-versus-chunk sweep grid at one length: chunk 16, 32, 64 and 128, the direct
    scan and the dispatching gdn_prefill against one oracle run of sampled heads; then the
    retrieval inputs (g = 0, beta = 1) at the same length, where the same bar applies."""
    shape = Shape(n=1, t=t, **FULL)
    for retrieval in (False, True):
        c = gdn_inputs.make_case(shape, seed=5000 + t, device=DEV, retrieval=retrieval)
        heads = [7, 24]
        ref = oracle_heads(c, heads, 2)
        chunks = sorted({16, *gdn_inputs.SWEEP_CHUNKS})
        runs = {f"C={cs}": gdn.gdn_prefill_chunked(**c, chunk=cs) for cs in chunks}
        runs["scan"] = gdn.gdn_prefill_scan(**c)
        runs["dispatch"] = gdn.gdn_prefill(**c)
        torch.cuda.synchronize()
        for name, (out, st) in runs.items():
            assert torch.isfinite(out).all() and torch.isfinite(st).all(), name
            for h in heads:
                assert_parity(out[:, :, h], st[:, h], ref[h][0][:, :, 0], ref[h][1][:, 0],
                              f"sweep t={t} {name} head {h} retrieval={retrieval}")
            del out, st
        del runs, c
        torch.cuda.empty_cache()
