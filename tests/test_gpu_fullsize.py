"""GPU parity at the workloads' full sizes against the fp64 oracle, every V head (the long
prefill: the two V heads of every other QK head), with the worst errors recorded for the
error summary (tests/parity.py; GDN_PARITY_REPORT=<path> writes it).

Workloads (gdn_inputs):
  * the tiny case (T = 64, 1 QK + 2 V heads, d = 16, fp32 inputs): chunk 16, the direct scan
    and the dispatching entry point;
  * the 4096-token prefill (16 QK / 32 V heads, d = 128, bf16 q/k/v, S0 = 0) with every
    chunk size, the direct scan and the dispatching entry point;
  * the stacked decode: 30 layers x 32 V heads, S0 ~ N(0, 0.02^2), 4096 consecutive steps
    with the state carried, every output and the state every 512 steps of every
    (layer, head);
  * the 131072-token prefill as 32 segments of 4096 with the state carried between calls,
    chunks 32 and 64, against one single-pass oracle run;
  * the scan-versus-chunk sweep lengths with chunks 16, 32, 64 and 128, the direct scan and
    the dispatching entry point, on the standard inputs and the retrieval inputs
    (g = 0, beta = 1).

Errors are per V head, in fp64 on the GPU (the oracle's results are copied there): the
largest |out - out_oracle| over the head's outputs divided by their RMS, and the Frobenius
error of the head's state divided by the oracle state's norm. The bars are the tolerances
of parity.py, per head.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import OUT_TOL, STATE_TOL, record

pytestmark = pytest.mark.gpu
DEV = "cuda"
FULL = dict(h_qk=16, h_v=32, d=128)
METHODS = ("dispatch", "C=16", "C=32", "C=64", "C=128", "scan")


def to_dev64(a):
    if isinstance(a, torch.Tensor):
        return a.to(DEV, torch.float64)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def cpu(c):
    return {key: (None if val is None else val.cpu()) for key, val in c.items()}


def run_oracle(c, heads=None):
    h = cpu(c)
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"], heads=heads)


def out_errors(out, ref, reduce_dims):
    """max |out - ref| / RMS(ref) over `reduce_dims` (absolute where RMS is zero)."""
    assert torch.isfinite(out).all(), "non-finite output"
    diff = (out.double() - ref).abs().amax(dim=reduce_dims)
    rms = ref.square().mean(dim=reduce_dims).sqrt()
    return torch.where(rms > 0, diff / rms, diff)


def state_errors(st, ref):
    """Per-head Frobenius error over norm, st and ref [n, h, d, d] -> [h]."""
    assert torch.isfinite(st).all(), "non-finite state"
    ds = (st.double() - ref).square().sum(dim=(0, 2, 3)).sqrt()
    ns = ref.square().sum(dim=(0, 2, 3)).sqrt()
    return torch.where(ns > 0, ds / ns, ds)


def check(config, method, compared, eo, es):
    eo = np.asarray(eo.cpu() if isinstance(eo, torch.Tensor) else eo, dtype=np.float64)
    es = np.asarray(es.cpu() if isinstance(es, torch.Tensor) else es, dtype=np.float64)
    record(config, method, compared, eo.ravel(), es.ravel())
    bad_o = np.argwhere(eo > OUT_TOL).ravel().tolist()
    bad_s = np.argwhere(es > STATE_TOL).ravel().tolist()
    assert not bad_o and not bad_s, (
        f"{config} {method}: over the bar at out {bad_o[:8]} (worst {eo.max():.3e}, tol "
        f"{OUT_TOL}), state {bad_s[:8]} (worst {es.max():.3e}, tol {STATE_TOL})")


def run_method(c, method):
    if method == "dispatch":
        return gdn.gdn_prefill(**c)
    if method == "scan":
        return gdn.gdn_prefill_scan(**c)
    return gdn.gdn_prefill_chunked(**c, chunk=int(method[2:]))


def method_name(method, t, h_qk=16, h_v=32, d=128, dtype=torch.bfloat16):
    if method == "dispatch":
        chunk = gdn.gdn_prefill_choose(t, h_qk, h_v, d, 1, dtype)
        return f"gdn_prefill ({'scan' if chunk == 0 else f'C={chunk}'})"
    return method


# ------------------------------------------------------------------------- tiny
def test_tiny_scan_and_chunked():
    """T=64, 1 QK + 2 V heads, d=16, fp32 inputs, S0=0: chunk 16 and the direct scan."""
    c = gdn_inputs.make_case(gdn_inputs.TINY, seed=1, device=DEV)
    o_ref, s_ref = run_oracle(c)
    o_ref, s_ref = to_dev64(o_ref), to_dev64(s_ref)
    for method in ("C=16", "scan", "dispatch"):
        out, st = run_method(c, method)
        torch.cuda.synchronize()
        check("tiny T=64, 1 QK / 2 V heads, d=16, fp32",
              method_name(method, 64, 1, 2, 16, torch.float32),
              "2 V heads: every output, final state",
              out_errors(out, o_ref, (0, 1, 3)), state_errors(st, s_ref))


# ------------------------------------------------------------- 4096-token prefill
@pytest.fixture(scope="module")
def prefill_4k():
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=2, device=DEV)
    o_ref, s_ref = run_oracle(c)
    return c, to_dev64(o_ref), to_dev64(s_ref)


@pytest.mark.parametrize("method", METHODS)
def test_prefill_4k_every_head(prefill_4k, method):
    c, o_ref, s_ref = prefill_4k
    out, st = run_method(c, method)
    torch.cuda.synchronize()
    check("prefill T=4096, 16 QK / 32 V heads, d=128, bf16, S0=0", method_name(method, 4096),
          "32 V heads: every output, final state",
          out_errors(out, o_ref, (0, 1, 3)), state_errors(st, s_ref))


# ------------------------------------------------------------------ stacked decode
def test_decode_30_layers_4096_steps_every_head():
    """Every output of every step and the state every 512 steps of all 30 x 32 (layer, V
    head) pairs; the oracle follows the 30 layers as 30 sequences of 4096 tokens, in
    segments of 512 steps, each continuing from its own state."""
    L, steps, snap = 30, 4096, 512
    per_step = Shape(n=L * steps, t=1, **FULL)
    c = gdn_inputs.make_case(per_step, seed=3, device=DEV)
    x = {key: c[key].view(steps, L, *c[key].shape[1:]) for key in ("q", "k", "v", "g", "beta")}
    s0 = gdn_inputs.make_case(Shape(n=L, t=1, **FULL), seed=33, device=DEV,
                              s0_std=0.02)["state_in"]
    st = s0.clone()
    outs = torch.empty(steps, L, 1, 32, 128, device=DEV)
    snaps = []
    for s in range(steps):
        gdn.gdn_decode_step(x["q"][s], x["k"][s], x["v"][s], x["g"][s], x["beta"][s], st,
                            out=outs[s], state_out=st)
        if (s + 1) % snap == 0:
            snaps.append(st.clone())
    torch.cuda.synchronize()
    # [steps, L, 1, ...] -> [L, steps, ...]: the layers as sequences
    seq = {key: x[key][:, :, 0].transpose(0, 1).contiguous().cpu()
           for key in ("q", "k", "v", "g", "beta")}
    state = s0.cpu()
    worst_o = torch.zeros(L * 32, dtype=torch.float64, device=DEV)
    worst_s = torch.zeros(L * 32, dtype=torch.float64, device=DEV)
    for seg in range(steps // snap):
        sl = slice(seg * snap, (seg + 1) * snap)
        o_ref, s_ref = oracle.run(seq["q"][:, sl], seq["k"][:, sl], seq["v"][:, sl],
                                  seq["g"][:, sl], seq["beta"][:, sl], state)
        # (layer, head) pairs as 960 heads of one sequence
        got = outs[sl, :, 0].reshape(1, snap, L * 32, 128)
        ref = to_dev64(o_ref).transpose(0, 1).reshape(1, snap, L * 32, 128)
        worst_o = torch.maximum(worst_o, out_errors(got, ref, (0, 1, 3)))
        worst_s = torch.maximum(worst_s, state_errors(snaps[seg].reshape(1, L * 32, 128, 128),
                                                      to_dev64(s_ref).reshape(1, L * 32, 128, 128)))
        state = torch.from_numpy(s_ref)
    check("decode, 30 layers x 32 V heads, 4096 steps, S0~N(0,0.02^2)", "gdn_decode_step",
          "960 (layer, head) pairs: every step's output, state every 512 steps",
          worst_o, worst_s)


# ------------------------------------------------- 131072 tokens in 32 segments
def test_long_131072_as_32_segments():
    """Chunks 32 and 64 (the dispatch picks 64 for a 4096-token segment), the state carried
    between the 32 calls in place; per-segment outputs and the final state of the two V
    heads of every other QK head (16 heads) against one single-pass oracle run."""
    seg_t, nseg = gdn_inputs.LONG_SEGMENT.t, gdn_inputs.LONG_SEGMENTS
    heads = [h for qk in range(0, 16, 2) for h in (2 * qk, 2 * qk + 1)]
    chunks = (32, 64)
    states = {cs: torch.zeros(1, 32, 128, 128, device=DEV) for cs in chunks}
    ws = {cs: torch.empty(gdn.gdn_workspace_bytes(1, seg_t, 16, 32, 128, chunk=cs), device=DEV,
                          dtype=torch.uint8) for cs in chunks}
    out = torch.empty(1, seg_t, 32, 128, device=DEV)
    got = {cs: torch.empty(1, nseg * seg_t, len(heads), 128) for cs in chunks}
    host = {key: [] for key in ("q", "k", "v", "g", "beta")}
    idx = torch.tensor(heads, device=DEV)
    qk_idx = torch.tensor([h // 2 for h in heads], device=DEV)
    for s in range(nseg):
        c = gdn_inputs.make_case(gdn_inputs.LONG_SEGMENT, seed=4000 + s, device=DEV)
        for cs in chunks:
            gdn.gdn_prefill_chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], states[cs],
                                    out=out, state_out=states[cs], workspace=ws[cs], chunk=cs)
            got[cs][:, s * seg_t:(s + 1) * seg_t] = out.index_select(2, idx).cpu()
        # the sampled heads as a problem with one QK head per V head
        host["q"].append(c["q"].index_select(2, qk_idx).cpu())
        host["k"].append(c["k"].index_select(2, qk_idx).cpu())
        for key in ("v", "g", "beta"):
            host[key].append(c[key].index_select(2, idx).cpu())
    torch.cuda.synchronize()
    full = {key: torch.cat(val, dim=1) for key, val in host.items()}
    del host
    o_ref, s_ref = oracle.run(full["q"], full["k"], full["v"], full["g"], full["beta"])
    del full
    ref = to_dev64(o_ref).view(1, nseg, seg_t, len(heads), 128)
    s_ref = to_dev64(s_ref)
    for cs in chunks:
        o = got[cs].to(DEV).view(1, nseg, seg_t, len(heads), 128)
        eo = out_errors(o, ref, (0, 2, 4)).amax(dim=0)  # worst segment per head
        es = state_errors(states[cs].index_select(1, idx), s_ref)
        check("prefill T=131072 as 32 x 4096-token segments, state carried",
              f"C={cs}" + (" (dispatch)" if cs == gdn.gdn_prefill_choose(seg_t, **FULL) else ""),
              "16 V heads: every segment's outputs (RMS per segment), final state", eo, es)


# ------------------------------------------------------------------ sweep grid
@pytest.mark.parametrize("t", gdn_inputs.SWEEP_T)
def test_sweep_grid_every_head(t):
    shape = Shape(n=1, t=t, **FULL)
    for retrieval in (False, True):
        c = gdn_inputs.make_case(shape, seed=5000 + t, device=DEV, retrieval=retrieval)
        o_ref, s_ref = run_oracle(c)
        o_ref, s_ref = to_dev64(o_ref), to_dev64(s_ref)
        kind = "retrieval inputs (g=0, beta=1)" if retrieval else "standard inputs"
        for method in METHODS:
            out, st = run_method(c, method)
            torch.cuda.synchronize()
            eo, es = out_errors(out, o_ref, (0, 1, 3)), state_errors(st, s_ref)
            del out, st
            check(f"sweep T={t}, {kind}", method_name(method, t),
                  "32 V heads: every output, final state", eo, es)
        del c, o_ref, s_ref
        torch.cuda.empty_cache()
