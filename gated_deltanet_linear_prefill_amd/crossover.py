"""Measure where the chunked prefill overtakes the direct scan on this GPU and write the
dispatch table gdn_prefill_choose reads (csrc/gdn_crossover.inc).

"Optimizing on-device inference for Apple Silicon", section "Qwen creates three distinct
workload shapes": whether the token-by-token scan or the re-blocked (chunked) evaluation is
faster depends on the dimensions, the workload and the hardware, so the choice is measured
rather than assumed. The sweep times one prefill call of the 16 QK / 32 V head, d = 128
layer (bf16 q/k/v, fp32 gate and write strength, zero initial state) at each length, for the
scan and every chunk size, in interleaved rounds, and keeps the median per method. As in a
layer stack, each call reads its own inputs and writes its own outputs: a round runs the
calls of several input sets back to back (enough sets that they do not all fit in the
GPU's caches, for lengths where that is possible) between two events, and a call's time is
the round's time over the call count. Inputs are synthetic (normal q/k/v, write strength
sigmoid(normal), gate log sigmoid(normal + 2)).

    python -m gated_deltanet_linear_prefill_amd.crossover            # print the sweep
    python -m gated_deltanet_linear_prefill_amd.crossover --write    # and rewrite the table

--write also writes a markdown summary (default profiles/crossover_sweep.md). Rebuild the
library afterwards (__graft_entry__.build()) so the new table is compiled in.
"""
import argparse
import os
import statistics
import sys

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TABLE = os.path.join(PKG, "csrc", "gdn_crossover.inc")
LENGTHS = (1, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)
CHUNKS = (16, 32, 64, 128)
H_QK, H_V, D = 16, 32, 128


def make_inputs(t, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    dev = "cuda"
    q = torch.randn(1, t, H_QK, D, device=dev, generator=gen).to(torch.bfloat16)
    k = torch.randn(1, t, H_QK, D, device=dev, generator=gen).to(torch.bfloat16)
    v = torch.randn(1, t, H_V, D, device=dev, generator=gen).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn(1, t, H_V, device=dev, generator=gen))
    g = torch.nn.functional.logsigmoid(torch.randn(1, t, H_V, device=dev, generator=gen) + 2.0)
    return q, k, v, g, beta


# Input sets per length: enough that their inputs and outputs together exceed this many
# bytes (more than the device's last-level cache), within [MIN_SETS, MAX_SETS].
ROTATE_BYTES = 1 << 30
MIN_SETS, MAX_SETS = 2, 32


def set_bytes(t):
    return t * (2 * H_QK * D * 2 + H_V * D * 2 + 2 * H_V * 4 + H_V * D * 4) + H_V * D * D * 4


def time_round(fns, repeat):
    """Time (us) per call of `repeat` passes over the calls `fns`, launched back to back
    between two events."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(repeat):
        for fn in fns:
            fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) * 1e3 / (repeat * len(fns))


def sweep(lengths, rounds):
    import gated_deltanet_linear_prefill_amd as gdn
    rows = []
    for t in lengths:
        nsets = max(MIN_SETS, min(MAX_SETS, -(-ROTATE_BYTES // set_bytes(t))))
        sets = []
        for i in range(nsets):
            q, k, v, g, beta = make_inputs(t, seed=5000 + 97 * i + t)
            out = torch.empty(1, t, H_V, D, device="cuda")
            st = torch.empty(1, H_V, D, D, device="cuda")
            sets.append((q, k, v, g, beta, out, st))
        methods = {}
        ws_scan = torch.empty(max(1, gdn.gdn_workspace_bytes(1, t, H_QK, H_V, D, chunk=0)),
                              device="cuda", dtype=torch.uint8)
        methods["scan"] = [gdn.bind_prefill_scan(q, k, v, g, beta, None, out, st, ws_scan)
                           for q, k, v, g, beta, out, st in sets]
        for c in CHUNKS:
            ws = torch.empty(max(1, gdn.gdn_workspace_bytes(1, t, H_QK, H_V, D, chunk=c)),
                             device="cuda", dtype=torch.uint8)
            methods[f"C{c}"] = [gdn.bind_prefill_chunked(q, k, v, g, beta, None, out, st, ws,
                                                         chunk=c)
                                for q, k, v, g, beta, out, st in sets]
        for fns in methods.values():  # warm-up
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        # about 2 ms of calls per round and method (at least one pass over the sets)
        probe = time_round(methods["C32"], 1)
        repeat = max(1, int(2000.0 / (probe * nsets)))
        times = {name: [] for name in methods}
        for _ in range(rounds):  # rounds alternate between the methods
            for name, fns in methods.items():
                times[name].append(time_round(fns, repeat))
        med = {name: statistics.median(v) for name, v in times.items()}
        best = min(med, key=med.get)
        rows.append((t, med, best, nsets))
        print(f"T={t:7d} sets={nsets:2d} " + " ".join(f"{n}={med[n]:9.1f}us" for n in methods) +
              f"  best {best}", flush=True)
        del sets, methods, ws_scan
        torch.cuda.empty_cache()
    return rows


def table_entries(rows):
    """Breakpoints {min_t, chunk}: each measured length's winner holds from that length up
    to the next measured length where the winner differs."""
    entries = []
    for t, _, best, _ in rows:
        chunk = 0 if best == "scan" else int(best[1:])
        if not entries or entries[-1][1] != chunk:
            entries.append((0 if not entries else t, chunk))
    return entries


def write_table(entries, device_name, path=TABLE):
    body = "\n".join(f"    {{{t}, {c}}}," for t, c in entries)
    text = f"""// gdn_crossover.inc -- prefill method by sequence length (written by crossover.py).
// Entries are sorted by min_t; the last entry whose min_t <= t wins. chunk 0 = direct scan.
// Measured on {device_name} with the 16 QK / 32 V head, d = 128, bf16 layout.
struct CrossoverEntry {{
    int64_t min_t;
    int32_t chunk;
}};
static const CrossoverEntry kCrossover[] = {{
{body}
}};
"""
    with open(path, "w") as f:
        f.write(text)


def write_summary(path, rows, entries, device_name, rounds):
    names = list(rows[0][1].keys())
    lines = [
        "# Scan vs chunked prefill crossover (16 QK / 32 V heads, d=128, bf16 q/k/v, S0=0)",
        "",
        "Command (repo root, MI355X):",
        "",
        "    python -m gated_deltanet_linear_prefill_amd.crossover " + " ".join(sys.argv[1:]),
        "",
        f"Device: {device_name}. Median of {rounds} interleaved rounds; a round times the calls "
        "of `sets` input sets (each with its own inputs and outputs, one shared workspace per "
        "method) back to back between two HIP events, and a call's time is the round's time "
        "over its call count.",
        "",
        "| T | sets | " + " | ".join(f"{n} us" for n in names) + " | best | best tokens/s |",
        "|---|---|" + "---|" * (len(names) + 2),
    ]
    for t, med, best, nsets in rows:
        lines.append(f"| {t} | {nsets} | " + " | ".join(f"{med[n]:.1f}" for n in names) +
                     f" | {best} | {t / (med[best] * 1e-6):.3e} |")
    lines += ["", "Dispatch table (csrc/gdn_crossover.inc; min_t -> chunk, 0 = scan): " +
              ", ".join(f"{t}->{c}" for t, c in entries), ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--write", action="store_true", help="rewrite csrc/gdn_crossover.inc")
    ap.add_argument("--rounds", type=int, default=7)
    ap.add_argument("--summary", default=os.path.join(ROOT, "profiles", "crossover_sweep.md"))
    ap.add_argument("--table", default=TABLE, help="where --write puts the table")
    ap.add_argument("--lengths", type=int, nargs="*", default=list(LENGTHS))
    args = ap.parse_args()
    if not torch.cuda.is_available():
        sys.exit("crossover.py measures on a GPU; none is visible")
    rows = sweep(sorted(args.lengths), args.rounds)
    entries = table_entries(rows)
    print("table:", entries, flush=True)
    if args.write:
        props = torch.cuda.get_device_properties(0)
        name = f"{props.name} ({getattr(props, 'gcnArchName', 'unknown arch')})"
        write_table(entries, name, args.table)
        write_summary(args.summary, rows, entries, name, args.rounds)
        print("wrote", args.table, "and", args.summary, flush=True)


if __name__ == "__main__":
    main()
