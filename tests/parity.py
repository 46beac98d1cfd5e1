"""Comparison helpers for GPU-versus-oracle parity.

Tolerances (fixed for bf16 q/k/v inputs, and used as the bar for fp32 inputs too):
  out:    max |out - out_oracle| <= 2e-3 * RMS(out_oracle), RMS over the whole tensor
  state:  ||S - S_oracle||_F <= 1e-3 * ||S_oracle||_F (absolute when S_oracle is zero)
"""
import numpy as np
import torch

OUT_TOL = 2e-3
STATE_TOL = 1e-3


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def out_error(out, ref):
    """max|err| / RMS(ref) (absolute max error when ref is all zero)."""
    out, ref = to64(out), to64(ref)
    err = np.max(np.abs(out - ref)) if out.size else 0.0
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    return err / rms if rms > 0 else err


def state_error(st, ref):
    st, ref = to64(st), to64(ref)
    num = np.linalg.norm((st - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return num / den if den > 0 else num


def assert_parity(out, st, out_ref, st_ref, what="", out_tol=OUT_TOL, state_tol=STATE_TOL):
    eo = out_error(out, out_ref) if out is not None else 0.0
    es = state_error(st, st_ref)
    msg = f"{what}: out max|err|/RMS = {eo:.3e} (tol {out_tol}), state rel-F = {es:.3e} (tol {state_tol})"
    assert np.all(np.isfinite(to64(st))), "non-finite state: " + msg
    if out is not None:
        assert np.all(np.isfinite(to64(out))), "non-finite output: " + msg
    assert eo <= out_tol and es <= state_tol, msg
    return eo, es


# ---------------------------------------------------------------- error report
# Full-size cases record their worst errors here; with GDN_PARITY_REPORT=<path> set, the
# test session writes them as a markdown table at its end (tests/conftest.py).
REPORT = []


def record(config, method, compared, out_errs, state_errs, out_tol=OUT_TOL, state_tol=STATE_TOL):
    """Keep the worst output and state errors of one (workload, method) comparison.
    `compared` says what was compared (heads, steps, segments)."""
    eo = float(np.max(out_errs)) if len(out_errs) else 0.0
    es = float(np.max(state_errs)) if len(state_errs) else 0.0
    REPORT.append(dict(config=config, method=method, compared=compared, out=eo, state=es,
                       out_tol=out_tol, state_tol=state_tol))


def write_report(path, header=""):
    lines = ["# Parity at full size: GPU library against the fp64 oracle", "", header, "",
             "| workload | method | compared | worst out max\\|err\\|/RMS | worst state rel-F | "
             "tolerance (out / state) |", "|---|---|---|---|---|---|"]
    for r in REPORT:
        lines.append(f"| {r['config']} | {r['method']} | {r['compared']} | {r['out']:.3e} | "
                     f"{r['state']:.3e} | {r['out_tol']:g} / {r['state_tol']:g} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
