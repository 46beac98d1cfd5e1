"""Calls from several host threads at once (each on its own stream and buffers): chunked,
scan, decode and both segmented schedules (the overlapped one shares the library's side
stream and events, guarded on the host) give the bits of the same calls made one by one."""
import threading

import pytest
import torch

import gated_deltanet_linear_prefill_amd as gdn
import gdn_inputs
from gdn_inputs import Shape

pytestmark = pytest.mark.gpu
DEV = "cuda"


def job(kind, seed):
    shape = Shape(n=1, t=1 if kind == "decode" else 600, h_qk=4, h_v=8, d=128)
    c = gdn_inputs.make_case(shape, seed=seed, device=DEV, s0_std=0.05)

    def run():
        if kind == "chunked":
            return gdn.gdn_prefill_chunked(**c, chunk=32)
        if kind == "scan":
            return gdn.gdn_prefill_scan(**c)
        if kind == "decode":
            return gdn.gdn_decode_step(**c)
        return gdn.gdn_prefill_segmented(**c, seg_t=200, overlapped=(kind == "overlapped"))
    return run


def test_concurrent_host_threads():
    kinds = ["chunked", "scan", "decode", "in_order", "overlapped"] * 2
    runs = [job(k, 1600 + i) for i, k in enumerate(kinds)]
    ref = []
    for run in runs:
        ref.append(run())
        torch.cuda.synchronize()
    got = [None] * len(runs)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    got[i] = runs[i]()
            s.synchronize()
        except Exception as exc:  # reported below
            errors.append((i, exc))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(runs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (r, g) in enumerate(zip(ref, got)):
        assert torch.equal(r[0], g[0]) and torch.equal(r[1], g[1]), kinds[i]
