"""CPU tests: the oracle pins catch plausible mistakes.

Each case rebuilds the oracle's C source with one deliberate mistake (a flipped sign, a
dropped factor, a wrong index or a transposed layout) into a temporary library and checks
that at least one pin fails. The real oracle is never modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "delta_sign": ("Sj[i] - b * u * kh[i]", "Sj[i] + b * u * kh[i]"),
    "no_gate": ("alpha * (Sj[i] - b * u * kh[i])", "(Sj[i] - b * u * kh[i])"),
    "gate_not_on_delta": ("alpha * (Sj[i] - b * u * kh[i])", "alpha * Sj[i] - b * u * kh[i]"),
    "gate_is_g": ("exp(J->g[tok * J->h_v + hv])", "(J->g[tok * J->h_v + hv])"),
    "no_beta_on_v": ("+ b * vj * kh[i]", "+ vj * kh[i]"),
    "output_reads_k": ("o += Sj[i] * qh[i]", "o += Sj[i] * kh[i]"),
    "eps_outside_sqrt": ("sqrt(ss + eps)", "sqrt(ss) + eps"),
    "no_l2_norm": ("const double norm = sqrt(ss + eps);", "const double norm = 1.0 + 0.0 * (ss + eps);"),
    "interleaved_heads": ("hv / (J->h_v / J->h_qk)", "hv % J->h_qk"),
    "state_not_transposed": ("(int64_t)i * dv + row_lo + r", "(int64_t)(row_lo + r) * dk + i"),
}


def _build(name, src_text, tmp_path):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-I", os.path.dirname(SRC), str(c), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    f = lib.gdn_oracle_run
    f.restype = ctypes.c_int
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, ctypes.c_double,
                  P, P, P, ctypes.c_int64, ctypes.c_int32]

    def run(q, k, v, g, beta, s0, l2_eps, threads=None):
        arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.float64)
                for a in (q, k, v, g, beta, s0)]
        n, t, hq, dk = arrs[0].shape
        hv, dv = arrs[2].shape[2], arrs[2].shape[3]
        out = np.full((n, t, hv, dv), np.nan)
        st = np.full((n, hv, dk, dv), np.nan)
        p = [None if a is None else a.ctypes.data_as(P) for a in arrs]
        rc = f(n, t, hq, hv, dk, dv, *p, float(l2_eps), out.ctypes.data_as(P),
               st.ctypes.data_as(P), None, 0, 2)
        if rc != 0:
            raise ValueError(rc)
        return out, st
    return run


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    run = _build(name, src.replace(old, new), tmp_path)
    caught = []
    for pin in PINS:
        try:
            pin(run)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


def test_unmutated_build_passes_all_pins(tmp_path):
    run = _build("clean", open(SRC).read(), tmp_path)
    for pin in PINS:
        pin(run)
