"""fp64 CPU oracle for the Gated DeltaNet recurrence -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package. The GPU library never uses it and shares no code with it.

``run`` wraps ``gdn_oracle_run`` from ``libgdn_oracle.so`` (plain C, fp64, see
``gdn_oracle.h`` for the definition, its source passage and the layouts). Inputs of any
float dtype (numpy or CPU torch, including bfloat16) are upcast exactly to fp64 first.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        f = lib.gdn_oracle_run
        f.restype = ctypes.c_int
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, ctypes.c_double,
                      P, P, P, ctypes.c_int64, ctypes.c_int32]
        _lib = lib
    return _lib


def _f64(x):
    """Exact upcast to a contiguous fp64 numpy array (bf16 and fp32 embed in fp64)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    """Host threads to use: the CPUs this process may run on, capped by OMP_NUM_THREADS
    when set and at 16 (the CPU share of one GPU on a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def run(q, k, v, g, beta, state_in=None, l2_eps=1e-6, heads=None, threads=None):
    """Run the recurrence in fp64.

    q, k: [n, t, h_qk, d_k]; v: [n, t, h_v, d_v]; g, beta: [n, t, h_v];
    state_in: [n, h_v, d_k, d_v] (element [i][j] = S[j][i]) or None for zeros.
    heads: optional iterable of flattened head ids (seq * h_v + v_head) to compute; the
    other heads' outputs are left as NaN.
    Returns (out [n, t, h_v, d_v], state_out [n, h_v, d_k, d_v]) as fp64 numpy arrays.
    """
    q, k, v, g, beta, s0 = (_f64(a) for a in (q, k, v, g, beta, state_in))
    n, t, h_qk, d_k = q.shape
    h_v, d_v = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (n, t)
    assert g.shape == (n, t, h_v) and beta.shape == (n, t, h_v)
    if s0 is not None:
        assert s0.shape == (n, h_v, d_k, d_v)
    out = np.full((n, t, h_v, d_v), np.nan)
    s_out = np.full((n, h_v, d_k, d_v), np.nan)
    sel = None
    if heads is not None:
        sel = np.ascontiguousarray(np.asarray(list(heads), dtype=np.int64))
    rc = _load().gdn_oracle_run(
        n, t, h_qk, h_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
        float(l2_eps), _ptr(out), _ptr(s_out), _ptr(sel), 0 if sel is None else len(sel),
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"gdn_oracle_run failed with code {rc}")
    return out, s_out
