"""GPU parity over seeded random shapes: every prefill entry point and the decode step against
the fp64 oracle on shapes drawn from the supported space (one or two sequences, odd lengths,
1 to 4 V heads per QK head, every head dimension, both input dtypes, with and without an
initial state), so that combinations the targeted tests do not name are covered too.
"""
import random

import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
import oracle
from gdn_inputs import Shape
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"
NCASES = 24


def draw(i):
    """Shape, initial-state scale and segment length of case i (seeded, independent of order)."""
    r = random.Random(9000 + i)
    d = r.choice([16, 32, 64, 128])
    h_qk = r.choice([1, 2, 4])
    group = r.choice([1, 2, 4])
    n = r.choice([1, 2])
    t = r.choice([r.randint(1, 40), r.randint(41, 200), r.randint(201, 400)])
    dtype = r.choice([torch.bfloat16, torch.float32])
    s0 = r.choice([0.0, 0.1])
    seg_t = r.randint(1, t + 10)
    return Shape(n=n, t=t, h_qk=h_qk, h_v=h_qk * group, d=d, dtype=dtype), s0, seg_t


def run_oracle(c):
    h = {key: (None if val is None else val.cpu()) for key, val in c.items()}
    return oracle.run(h["q"], h["k"], h["v"], h["g"], h["beta"], h["state_in"])


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape_every_method(i):
    shape, s0, seg_t = draw(i)
    c = gdn_inputs.make_case(shape, seed=9100 + i, device=DEV, s0_std=s0)
    o_ref, s_ref = run_oracle(c)
    what = f"case {i}: {shape}, s0 {s0}"
    runs = {"scan": gdn.gdn_prefill_scan(**c), "dispatch": gdn.gdn_prefill(**c),
            f"segmented seg_t={seg_t}": gdn.gdn_prefill_segmented(**c, seg_t=seg_t)}
    for chunk in (16, 32, 64, 128):
        runs[f"C={chunk}"] = gdn.gdn_prefill_chunked(**c, chunk=chunk)
    torch.cuda.synchronize()
    for name, (out, st) in runs.items():
        assert_parity(out, st, o_ref, s_ref, f"{what}, {name}")


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape_decode(i):
    """The same shapes as one-token steps (t = 1): the stacked or split decode kernel,
    depending on the number of (sequence, V head) pairs."""
    shape, s0, _ = draw(i)
    shape = Shape(n=shape.n * 5, t=1, h_qk=shape.h_qk, h_v=shape.h_v, d=shape.d, dtype=shape.dtype)
    c = gdn_inputs.make_case(shape, seed=9200 + i, device=DEV, s0_std=s0)
    o_ref, s_ref = run_oracle(c)
    out, st = gdn.gdn_decode_step(**c)
    torch.cuda.synchronize()
    assert_parity(out, st, o_ref, s_ref, f"decode case {i}: {shape}, s0 {s0}")
