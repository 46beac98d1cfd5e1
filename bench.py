#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer recurrence on one MI355X.

One step is the whole hot path once:
  * prefill: a 4096-token prompt through 30 GDN layers, one library prefill call per layer
    (the method gdn_prefill_choose picks: the chunked kernels with 64-token chunks at this
    length), each layer on its own synthetic inputs (16 QK heads, 32 V heads,
    d_k = d_v = 128, bf16 q/k/v,
    fp32 gate and write strength, zero initial state), states written to a 30-layer stack;
  * decode: one token through the same 30 layers (one stacked gdn_decode_step, n = 30),
    continuing from the states the prefill produced, updated in place.
`value` is prefill tokens per second for the 30 layers (4096 / prefill seconds per step);
`decode_us_per_token` is the decode part. Inputs are resident in HBM before timing starts.
prefill_us_per_layer is the timed steps' prefill time over 30 (the mean duration of one of
the back-to-back calls); prefill_us_per_call_{median,min,p90} come from a separate pass with an
event around every call. prefill_c64_us_per_layer is the same 30 calls with 64-token chunks
(the chunk the 4096-token workload is specified with), timed the same way after the timed
region, with its fraction of the HBM roofline (prefill_c64_hbm_frac).

decode_us_per_token is the step's own decode token: its 60 MiB of state were last written by
the prefill calls, whose outputs have since pushed them out of the 256 MB MALL, so it reads
them from HBM. The JSON line also carries decode_steady_us_per_token (consecutive decode
steps on one state stack, as in the 4096-step decode workload: the state stays in the MALL
between steps), decode_cold_us_per_token (consecutive steps over six stacks used in turn,
360 MiB), stream_copy_{warm,cold}_GBps (the library's streaming-copy calibration kernel over
the same 60 MiB, one buffer pair or six in turn: the achievable read + write rate the decode
fractions are taken against), decode_per_layer_{eager,graph}_us_per_token (the same token as 30 dependent
per-layer steps of one sequence each, called one by one or replayed as one recorded HIP
graph), prefill_segmented_1024[_overlapped]_us_per_layer (one layer's prompt as four
1024-token segments with the smaller workspace they need, in order or with each segment's
per-chunk preparation on a side stream during the previous segment's sequential pass) and
hbm_copy_GBps (what a 1 GiB device copy reaches; the achievable HBM rate next to
the 8 TB/s peak), all measured after the timed region, and
  roofline:     the prefill call (its two kernels) against HBM: algorithmic bytes per call
                (q, k, v, g, beta read once, out and state_out written once) divided by the
                mean call duration (HIP events around the 30 back-to-back calls of every
                timed step, on the stream the kernels run on, divided by 30); traffic =
                HBM bytes per call from the committed rocprofv3 counter summary (null once
                the kernel source has changed);
  cpu_baseline: the fp64 oracle timed on this host's cores over the prefill step's layers
                (up to 30, or 20 s of oracle time), plus one layer on one thread.

Modes for counter collection (no JSON line): --mode pmc-prefill runs the prefill calls of
three layers; --mode pmc-copy runs a device copy of known size for counter calibration;
--mode segmented runs six segmented prefill calls (1024-token segments) in order, then six
overlapped, for a kernel trace; --mode ablation times the state-residency ablation at 2048
tokens (resident direct scan, the same scan with the state through device memory every 32
tokens, and the chunked call) and prints one JSON line of its own; --mode pmc-ablation makes
one call of each scan form for counter collection; --mode pmc-mfma runs one MFMA loop of
known flops (calibration of the MFMA counters); --mode pmc-decode runs three stacked decode
steps (30 layers); --mode decode-layers runs five decode tokens as 30 dependent per-layer
steps launched one by one, then five as replays of the recorded decode graph.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

T_PROMPT, LAYERS, H_QK, H_V, D = 4096, 30, 16, 32, 128
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published
COPY_BYTES = 256 << 20
METRIC = "GDN prefill tokens/s at T=4096 x30 layers; decode step us/token; % roofline"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--core-only", action="store_true",
                    help="skip the measurements after the timed region (their fields are null), "
                         "so that a kernel trace holds only the timed step's kernels")
    ap.add_argument("--mode", choices=["bench", "pmc-prefill", "pmc-copy", "segmented",
                                       "ablation", "pmc-ablation", "pmc-mfma", "pmc-decode",
                                       "decode-layers"],
                    default="bench")
    return ap.parse_args()


def prefill_bytes():
    """Algorithmic HBM bytes of one prefill call (S0 = 0, so no state read)."""
    qk = T_PROMPT * H_QK * D * 2
    v = T_PROMPT * H_V * D * 2
    gb = T_PROMPT * H_V * 4
    out = T_PROMPT * H_V * D * 4
    st = H_V * D * D * 4
    return 2 * qk + v + 2 * gb + out + st


def prefill_flops(chunk):
    """Algorithmic flops of one chunked prefill call: (6 d^2 + 4 C d) per token and V head
    (the state products, the Gram terms once per QK head, triangles counted as half)."""
    return (6 * D * D + 4 * chunk * D) * T_PROMPT * H_V


def decode_bytes():
    st = LAYERS * H_V * D * D * 4
    qk = LAYERS * H_QK * D * 2
    v = LAYERS * H_V * D * 2
    gb = LAYERS * H_V * 4
    out = LAYERS * H_V * D * 4
    return 2 * st + 2 * qk + v + 2 * gb + out


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "chunked_prefill_4k_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "gated_deltanet_linear_prefill_amd", "csrc", "gdn_chunked.hip")


def measured_traffic():
    """HBM bytes per prefill call from the committed rocprofv3 counter summary, or None when
    the kernel source has changed since the counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and line.split(":", 1)[0] in ("bytes_per_call", "source_sha256"):
            key, val = line.split(":", 1)
            fields[key] = val.strip()
    sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    if fields.get("source_sha256") != sha or "bytes_per_call" not in fields:
        return None
    return int(fields["bytes_per_call"])


def reference_rates(gdn, dec, dec_out, pre, dev):
    """Outside the timed region: the decode step with its state out of the 256 MB MALL
    (six independent 30-layer state stacks used in turn, 360 MiB), and the HBM rate a plain
    1 GiB device copy reaches (read + write bytes per second), the achievable counterpart
    of the 8 TB/s peak. Also one prefill layer run as 1024-token segments with the bounded
    workspace that needs (gdn_prefill_segmented, in order and overlapped)."""
    import torch
    stacks = [torch.zeros(LAYERS, H_V, D, D, device=dev) for _ in range(6)]
    calls = [gdn.bind_decode_step(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], st,
                                  dec_out, st) for st in stacks]

    def span_us(fns, reps=30):
        """Mean duration of fns[i % len(fns)] for i < reps, back to back between two events."""
        for i in range(3):
            fns[i % len(fns)]()
        torch.cuda.synchronize()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for i in range(reps):
            fns[i % len(fns)]()
        e0.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(e0) / reps * 1e3

    # consecutive decode steps on one 30-layer state stack (the 4096-step decode workload:
    # the 60 MiB of state stay in the 256 MB MALL from step to step), and the same steps
    # with six stacks used in turn (360 MiB, so every step reads its state from HBM)
    steady_us = span_us(calls[:1])
    cold_us = span_us(calls)
    del stacks, calls
    # the achievable read + write rate with the library's streaming copy over the decode
    # step's state bytes (60 MiB), warm (one buffer pair) and cold (six pairs in turn)
    nst = LAYERS * H_V * D * D
    pairs = [(torch.ones(nst, device=dev), torch.empty(nst, device=dev)) for _ in range(6)]
    cps = [(lambda a=a, b=b: gdn.calib_stream_copy(a, b, blocks=1024)) for a, b in pairs]
    copy_warm_us = span_us(cps[:1])
    copy_cold_us = span_us(cps)
    del pairs, cps

    # The same decode token as 30 dependent per-layer steps (one sequence each, the layer
    # order of a real model): called one by one, and recorded once as a HIP graph.
    st = torch.zeros(LAYERS, H_V, D, D, device=dev)
    per = {key: [dec[key][l:l + 1] for l in range(LAYERS)] for key in ("q", "k", "v", "g", "beta")}
    outs = [dec_out[l:l + 1] for l in range(LAYERS)]
    sts = [st[l:l + 1] for l in range(LAYERS)]
    eager = [gdn.bind_decode_step(per["q"][l], per["k"][l], per["v"][l], per["g"][l],
                                  per["beta"][l], sts[l], outs[l], sts[l]) for l in range(LAYERS)]
    graph = gdn.DecodeGraph(per["q"], per["k"], per["v"], per["g"], per["beta"], sts, outs,
                            stream=torch.cuda.Stream())

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            fn()
        e0.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(e0) / reps * 1e3

    layers_eager_us = timed(lambda: [c() for c in eager])
    layers_graph_us = timed(graph.launch)
    graph.close()
    del st, eager

    seg_t = 1024
    seg_out = torch.empty(1, T_PROMPT, H_V, D, device=dev)
    seg_st = torch.empty(1, H_V, D, D, device=dev)
    seg = {}
    for ov in (False, True):
        seg_ws = torch.empty(gdn.gdn_prefill_segmented_workspace_bytes(
            1, T_PROMPT, H_QK, H_V, D, seg_t, overlapped=ov), device=dev, dtype=torch.uint8)
        us = timed(lambda: gdn.gdn_prefill_segmented(
            pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], None, seg_t=seg_t,
            overlapped=ov, out=seg_out, state_out=seg_st, workspace=seg_ws))
        seg[ov] = (us, seg_ws.numel())
        del seg_ws
    del seg_out, seg_st
    # The achievable dense bf16 MFMA rate: a loop of independent MFMAs over the whole chip.
    sink = torch.empty(1024 * 256, device=dev)
    gdn.calib_mfma_bf16(100, 1024, sink)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        flops = gdn.calib_mfma_bf16(4000, 1024, sink)
        e0.record()
        torch.cuda.synchronize()
        best = min(best, s0.elapsed_time(e0) * 1e-3)
    mfma_tflops = flops / best / 1e12
    del sink
    a = torch.empty(1 << 28, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * a.numel() * 4 * 5 / (s.elapsed_time(e) * 1e-3) / 1e9
    return {"decode_cold_us": cold_us, "decode_steady_us": steady_us, "copy_GBps": copy_gbs,
            "stream_copy_warm_GBps": 2 * nst * 4 / (copy_warm_us * 1e-6) / 1e9,
            "stream_copy_cold_GBps": 2 * nst * 4 / (copy_cold_us * 1e-6) / 1e9,
            "layers_eager_us": layers_eager_us, "layers_graph_us": layers_graph_us,
            "seg": seg, "mfma_tflops": mfma_tflops}


def ablation(gdn, gdn_inputs, dev, counters):
    """The state-residency ablation at 2048 tokens (16 QK / 32 V heads, d = 128, bf16): the
    direct scan with the state resident for the whole prompt, against the same scan with
    the state sent through device memory every 32 tokens. counters: one call of each (for
    rocprofv3 --pmc) and no JSON line; else mean call times (HIP events, 10 calls after 2
    warm-up) as one JSON line."""
    import torch
    c = gdn_inputs.make_case(gdn_inputs.ABLATION_2K, seed=300, device=dev)
    shp = gdn_inputs.ABLATION_2K
    block_t = 32
    out = torch.empty(1, shp.t, shp.h_v, shp.d, device=dev)
    st = torch.empty(1, shp.h_v, shp.d, shp.d, device=dev)
    ws = torch.empty(gdn.gdn_workspace_bytes(1, shp.t, shp.h_qk, shp.h_v, shp.d, chunk=0),
                     device=dev, dtype=torch.uint8)
    chunk = gdn.gdn_prefill_choose(shp.t, shp.h_qk, shp.h_v, shp.d)
    ws_c = torch.empty(gdn.gdn_workspace_bytes(1, shp.t, shp.h_qk, shp.h_v, shp.d, chunk=chunk),
                       device=dev, dtype=torch.uint8)
    runs = {
        "resident": lambda: gdn.gdn_prefill_scan(**c, out=out, state_out=st, workspace=ws),
        "blockwise": lambda: gdn.gdn_prefill_scan_blockwise(**c, block_t=block_t, out=out,
                                                            state_out=st, workspace=ws),
        "chunked": lambda: gdn.gdn_prefill_chunked(**c, chunk=chunk, out=out, state_out=st,
                                                   workspace=ws_c),
    }
    if counters:
        for name in ("resident", "blockwise"):
            runs[name]()
            torch.cuda.synchronize()
            print(f"{name} call done", flush=True)
        return
    res = {}
    for name, fn in runs.items():
        for _ in range(2):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(10):
            fn()
        e.record()
        torch.cuda.synchronize()
        res[name + "_us"] = s.elapsed_time(e) / 10 * 1e3
    # fp32 state of one layer; with S0 = 0 the first block reads none, so the blockwise
    # form moves (2 blocks - 1) states and the resident one a single write
    state_bytes = shp.h_v * shp.d * shp.d * 4
    blocks = -(-shp.t // block_t)
    print(json.dumps({"workload": "GDN prefill, T=2048, 16 QK + 32 V heads, d=128, bf16, S0=0",
                      "block_t": block_t, "blocks": blocks,
                      "state_bytes_blockwise": state_bytes * (2 * blocks - 1),
                      "state_bytes_resident": state_bytes, "chunk": chunk, **res}), flush=True)


def matrix_fields(chunk, call_s, extra):
    """The chunked call's algorithmic MFMA rate against the published dense bf16 peak and
    against the MFMA loop's achievable rate (null when that was skipped)."""
    if not chunk:
        return None
    flops = prefill_flops(chunk)
    tf = flops / call_s / 1e12
    loop = (extra or {}).get("mfma_tflops")
    return {"algorithmic_flops_per_call": flops, "achieved_TFLOPs": tf,
            "peak_TFLOPs": BF16_PEAK_TFLOPS, "frac_peak": tf / BF16_PEAK_TFLOPS,
            "loop_TFLOPs": loop, "frac_loop": tf / loop if loop else None}


def extra_fields(extra):
    """The JSON fields of reference_rates (null when it was skipped)."""
    e = extra or {}
    seg = e.get("seg", {})
    cold = e.get("decode_cold_us")
    steady = e.get("decode_steady_us")
    rate = lambda us: decode_bytes() / (us * 1e-6) / 1e9 if us else None
    ratio = lambda a, b: a / b if a and b else None
    return {
        "decode_steady_us_per_token": steady,
        "decode_steady_GBps": rate(steady),
        "decode_cold_us_per_token": cold,
        "decode_cold_GBps": rate(cold),
        "stream_copy_warm_GBps": e.get("stream_copy_warm_GBps"),
        "stream_copy_cold_GBps": e.get("stream_copy_cold_GBps"),
        "decode_steady_frac_of_stream_copy": ratio(rate(steady), e.get("stream_copy_warm_GBps")),
        "decode_cold_frac_of_stream_copy": ratio(rate(cold), e.get("stream_copy_cold_GBps")),
        "decode_per_layer_eager_us_per_token": e.get("layers_eager_us"),
        "decode_per_layer_graph_us_per_token": e.get("layers_graph_us"),
        "prefill_segmented_1024_us_per_layer": seg.get(False, (None, None))[0],
        "prefill_segmented_1024_workspace_bytes": seg.get(False, (None, None))[1],
        "prefill_segmented_1024_overlapped_us_per_layer": seg.get(True, (None, None))[0],
        "prefill_segmented_1024_overlapped_workspace_bytes": seg.get(True, (None, None))[1],
        "hbm_copy_GBps": e.get("copy_GBps"),
        "mfma_bf16_loop_TFLOPs": e.get("mfma_tflops"),
    }


def _cpus_allowed():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return None


def _cpu_model():
    """The host CPU's model name (as lscpu prints it, read from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline():
    """The fp64 oracle on the prefill step's layers (each with its own inputs), all host
    threads it may use, until the 30 layers are done or 20 s of oracle time have passed."""
    import oracle
    import gdn_inputs
    threads = oracle.default_threads()
    spent, layers = 0.0, 0
    while layers < LAYERS and spent < 20.0:
        c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=100 + layers)
        t0 = time.perf_counter()
        oracle.run(c["q"], c["k"], c["v"], c["g"], c["beta"], None, threads=threads)
        spent += time.perf_counter() - t0
        layers += 1
    per_layer = spent / layers
    # the same oracle on one thread, one layer, for the scaling of the host figure
    c = gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=100)
    t0 = time.perf_counter()
    oracle.run(c["q"], c["k"], c["v"], c["g"], c["beta"], None, threads=1)
    one = time.perf_counter() - t0
    return {"value": T_PROMPT / (LAYERS * per_layer), "unit": "tokens/s", "cores": threads,
            "host_nproc": os.cpu_count(), "host_cpus_allowed": _cpus_allowed(),
            "host_cpu_model": _cpu_model(),
            "kind": "oracle",
            "sample": f"{layers} layer(s) of the prefill workload (T=4096, 32 V heads, d=128, "
                      f"each its own inputs), {spent:.1f} s of oracle time; value = 4096 / "
                      f"(30 x mean layer time)",
            "one_thread_layer_s": one,
            "one_thread_value": T_PROMPT / (LAYERS * one)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the recurrence shards by head with no communication, so the "
              "whole-job figure is N times the one-GPU figure and is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_linear_prefill_amd as gdn
    import gdn_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mode == "pmc-copy":
        a = torch.empty(COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"copied {COPY_BYTES} bytes x3", flush=True)
        return

    if args.mode == "pmc-mfma":
        sink = torch.empty(1024 * 256, device=dev)
        flops = gdn.calib_mfma_bf16(200, 1024, sink)
        torch.cuda.synchronize()
        print(f"MFMA loop done: {flops} flops", flush=True)
        return
    if args.mode in ("ablation", "pmc-ablation"):
        ablation(gdn, gdn_inputs, dev, counters=args.mode == "pmc-ablation")
        return

    # ---- inputs, all resident before timing
    layers = [gdn_inputs.make_case(gdn_inputs.PREFILL_4K, seed=100 + l, device=dev)
              for l in range(LAYERS)]
    dec = gdn_inputs.make_case(gdn_inputs.DECODE_30L, seed=200, device=dev)
    states = torch.zeros(LAYERS, H_V, D, D, device=dev)
    outs = torch.empty(LAYERS, 1, T_PROMPT, H_V, D, device=dev)
    dec_out = torch.empty(LAYERS, 1, H_V, D, device=dev)
    chunk = gdn.gdn_prefill_choose(T_PROMPT, H_QK, H_V, D)
    ws = torch.empty(max(1, gdn.gdn_workspace_bytes(1, T_PROMPT, H_QK, H_V, D, chunk=chunk)),
                     device=dev, dtype=torch.uint8)
    if chunk > 0:
        bind = lambda c, l: gdn.bind_prefill_chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], None,
                                                     outs[l], states[l:l + 1], ws, chunk=chunk)
    else:
        bind = lambda c, l: gdn.bind_prefill_scan(c["q"], c["k"], c["v"], c["g"], c["beta"], None,
                                                  outs[l], states[l:l + 1], ws)
    calls = [bind(c, l) for l, c in enumerate(layers)]
    decode = gdn.bind_decode_step(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], states,
                                  dec_out, states)

    if args.mode == "pmc-prefill":
        for l in range(3):
            calls[l]()
        torch.cuda.synchronize()
        print("prefill calls done", flush=True)
        return
    if args.mode == "pmc-decode":
        for _ in range(3):
            decode()
        torch.cuda.synchronize()
        print("decode steps done", flush=True)
        return
    if args.mode == "decode-layers":
        # one decode token as 30 dependent per-layer steps: 5 tokens launched one step at a
        # time, then 5 tokens as replays of the recorded graph (for a kernel trace)
        st = torch.zeros(LAYERS, H_V, D, D, device=dev)
        per = {key: [dec[key][l:l + 1] for l in range(LAYERS)]
               for key in ("q", "k", "v", "g", "beta")}
        outs1 = [dec_out[l:l + 1] for l in range(LAYERS)]
        sts = [st[l:l + 1] for l in range(LAYERS)]
        eager = [gdn.bind_decode_step(per["q"][l], per["k"][l], per["v"][l], per["g"][l],
                                      per["beta"][l], sts[l], outs1[l], sts[l])
                 for l in range(LAYERS)]
        graph = gdn.DecodeGraph(per["q"], per["k"], per["v"], per["g"], per["beta"], sts,
                                outs1, stream=torch.cuda.Stream())
        for _ in range(5):
            for c in eager:
                c()
        torch.cuda.synchronize()
        print("eager per-layer tokens done", flush=True)
        for _ in range(5):
            graph.launch()
        torch.cuda.synchronize()
        graph.close()
        print("graph per-layer tokens done", flush=True)
        return
    if args.mode == "segmented":
        c = layers[0]
        for ov in (False, True):
            seg_ws = torch.empty(gdn.gdn_prefill_segmented_workspace_bytes(
                1, T_PROMPT, H_QK, H_V, D, 1024, overlapped=ov), device=dev, dtype=torch.uint8)
            for _ in range(6):
                gdn.gdn_prefill_segmented(c["q"], c["k"], c["v"], c["g"], c["beta"], None,
                                          seg_t=1024, overlapped=ov, out=outs[0],
                                          state_out=states[0:1], workspace=seg_ws)
            torch.cuda.synchronize()
            print(f"segmented prefill calls done (overlapped={ov})", flush=True)
        return

    # A timed step records events only at its boundaries (an event between two calls
    # costs about 2 us on this stack); the per-call durations come from a separate pass
    # after the timed region.
    def step(evs=None):
        if evs is not None:
            evs[0].record()
        for c in calls:
            c()
        if evs is not None:
            evs[1].record()
        decode()
        if evs is not None:
            evs[2].record()

    for _ in range(args.warmup):
        step()
    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(all_evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    prefill_ms = [evs[0].elapsed_time(evs[1]) for evs in all_evs]
    decode_ms = [evs[1].elapsed_time(evs[2]) for evs in all_evs]
    prefill_s = sum(prefill_ms) / len(prefill_ms) / 1e3
    mean_call_s = prefill_s / LAYERS  # average duration of one of the back-to-back calls
    achieved = prefill_bytes() / mean_call_s / 1e9

    # per-call distribution (not part of the timed steps): an event around every call
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(LAYERS + 1)]
    call_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        for l, c in enumerate(calls):
            cev[l].record()
            c()
        cev[LAYERS].record()
        torch.cuda.synchronize()
        call_ms += [cev[l].elapsed_time(cev[l + 1]) for l in range(LAYERS)]

    # The 4096-token workload's configured chunk (64 tokens), timed as the timed steps time
    # the dispatched chunk: the 30 layers' calls back to back between two events, 3 rounds.
    c64_us = None
    if not args.core_only and chunk != 64:
        ws64 = torch.empty(gdn.gdn_workspace_bytes(1, T_PROMPT, H_QK, H_V, D, chunk=64),
                           device=dev, dtype=torch.uint8)
        calls64 = [gdn.bind_prefill_chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], None,
                                            outs[l], states[l:l + 1], ws64, chunk=64)
                   for l, c in enumerate(layers)]
        for f in calls64[:3]:
            f()
        torch.cuda.synchronize()
        e64 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e64[0].record()
        for _ in range(3):
            for f in calls64:
                f()
        e64[1].record()
        torch.cuda.synchronize()
        c64_us = e64[0].elapsed_time(e64[1]) / (3 * LAYERS) * 1e3
        del calls64, ws64
    elif chunk == 64:
        c64_us = mean_call_s * 1e6

    traffic = measured_traffic()
    extra = None if args.core_only else reference_rates(gdn, dec, dec_out, layers[0], dev)

    res = {
        "metric": METRIC,
        "value": T_PROMPT / prefill_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GDN prefill, T=4096 tokens through 30 layers (16 QK + 32 V "
                               "heads, d_k=d_v=128, bf16 q/k/v, fp32 g/beta/state, S0=0), "
                               "then one decode token through the 30 layers",
                   "method": f"chunked C={chunk}" if chunk else "direct scan",
                   "global_batch": 1, "seq_len": T_PROMPT, "layers": LAYERS},
        "decode_us_per_token": sum(decode_ms) / len(decode_ms) * 1e3,
        "decode_GBps": decode_bytes() / (sum(decode_ms) / len(decode_ms) / 1e3) / 1e9,
        "prefill_us_per_layer": mean_call_s * 1e6,
        "prefill_us_per_call_median": float(statistics.median(call_ms)) * 1e3,
        "prefill_us_per_call_min": min(call_ms) * 1e3,
        "prefill_us_per_call_p90": sorted(call_ms)[int(0.9 * (len(call_ms) - 1))] * 1e3,
        "prefill_c64_us_per_layer": c64_us,
        "prefill_c64_hbm_frac": (prefill_bytes() / (c64_us * 1e-6) / 1e9 / HBM_PEAK_GBS
                                 if c64_us else None),
        **extra_fields(extra),
        "prefill_workspace_bytes": ws.numel(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ("gdn_prefill_chunked call (chunk_prep_kernel + "
                                + ("chunk64_scan_kernel)" if chunk == 64 else "chunk_scan_kernel)")
                                if chunk else "gdn_prefill_scan call"),
                     "algorithmic_bytes_per_call": prefill_bytes()},
        "matrix": matrix_fields(chunk, mean_call_s, extra),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
