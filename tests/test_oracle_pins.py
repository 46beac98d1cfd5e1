"""CPU tests: the fp64 oracle against results the mathematics fixes (see oracle_pins.py)."""
import numpy as np
import pytest

import oracle
from oracle_pins import PINS, rand_case


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.run)


def test_thread_count_does_not_change_bits():
    q, k, v, g, beta, s0 = rand_case(20, n=2, t=33, h_qk=2, h_v=4, d_k=16, d_v=40)
    o1, s1 = oracle.run(q, k, v, g, beta, s0, threads=1)
    o7, s7 = oracle.run(q, k, v, g, beta, s0, threads=7)
    assert np.array_equal(o1, o7) and np.array_equal(s1, s7)


def test_head_selection_matches_full_run():
    q, k, v, g, beta, s0 = rand_case(21, n=2, t=9, h_qk=2, h_v=4, d_k=8, d_v=8)
    o, s = oracle.run(q, k, v, g, beta, s0)
    sel = [1, 6]
    o2, s2 = oracle.run(q, k, v, g, beta, s0, heads=sel)
    for hid in sel:
        b, h = divmod(hid, 4)
        assert np.array_equal(o2[b, :, h], o[b, :, h]) and np.array_equal(s2[b, h], s[b, h])
    assert np.isnan(o2[0, :, 0]).all()


def test_empty_sequence_passes_state_through():
    q, k, v, g, beta, s0 = rand_case(22, t=0, d_k=8, d_v=8)
    o, s = oracle.run(q, k, v, g, beta, s0)
    assert o.shape[1] == 0 and np.array_equal(s, s0)


def test_zero_key_with_eps_is_finite_and_without_is_nan():
    q, k, v, g, beta, s0 = rand_case(23, t=3, d_k=8, d_v=8)
    k[:, 1] = 0.0
    o, s = oracle.run(q, k, v, g, beta, s0, l2_eps=1e-6)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    o, s = oracle.run(q, k, v, g, beta, s0, l2_eps=0.0)
    assert np.isnan(s).all()


def test_bad_arguments_are_rejected():
    q, k, v, g, beta, s0 = rand_case(24, t=4, h_qk=3, h_v=4, d_k=8, d_v=8)
    with pytest.raises(ValueError):
        oracle.run(q, k, v, g, beta, s0)  # 4 V heads do not share 3 QK heads evenly


def test_golden_regression_fixture():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    doc = json.load(open(path))
    i = doc["inputs"]
    arr = {key: (np.array(val) if isinstance(val, list) else val) for key, val in i.items()}
    out, st = oracle.run(arr["q"], arr["k"], arr["v"], arr["g"], arr["beta"],
                         arr["state_in"], l2_eps=arr["l2_eps"], threads=1)
    np.testing.assert_allclose(out, np.array(doc["out"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(st, np.array(doc["state_out"]), rtol=1e-14, atol=1e-15)
