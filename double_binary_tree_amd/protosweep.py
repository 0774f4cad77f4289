"""Protocol sweep: the stepwise all-reduce with the slot protocol (SIMPLE:
a FIFO slot per step and a barrier after it) against LL (flag-in-line FIFO
words, no barriers), per algorithm and channel count.

8 virtual ranks on one node (ring, and the tree = intra-node chain) and 16
ranks on 16 nodes (the double binary tree, mirror), f32 sum, per-rank sizes
8 B .. 256 MiB in powers of two, values uniform in [-1, 1] drawn on the
device with a seeded generator.  Every point also checks that LL and SIMPLE
give bit-identical results and that no LL call was abandoned.

Reports per point the per-launch time of back-to-back launches replayed
from a HIP graph (so host call overhead is left out) and LL / SIMPLE, and per
(shape, algorithm, channel count) the size intervals where each protocol
wins, with the practical-tie rule of the course page ("NCCL 专家课程 13",
section "性能结果的判定规则": a loser within 5% of the winner is a tie).

    python -m double_binary_tree_amd.protosweep [--max-pow 26] [--out report.md]
"""

from __future__ import annotations

import argparse
import json
import sys

from double_binary_tree_amd.sweep import CHUNK, human, intervals

GRAPH_LAUNCHES = 20


def time_graph(E, sptr, rptr, count, torch, replays: int) -> float:
    """Per-launch time (us) of back-to-back launches replayed from a HIP
    graph: GRAPH_LAUNCHES all-reduces captured once (after warm calls, which
    build the shape's tables), the graph replayed `replays` times between
    two events.  Host-side call overhead is not in the figure."""
    stream = torch.cuda.current_stream()
    for _ in range(3):
        E.allreduce(sptr, rptr, count, "f32", "sum", stream.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(GRAPH_LAUNCHES):
            E.allreduce(sptr, rptr, count, "f32", "sum", cap.cuda_stream)
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        graph.replay()
    b.record(stream)
    b.synchronize()
    del graph
    return a.elapsed_time(b) * 1e3 / (replays * GRAPH_LAUNCHES)


SHAPES = ((8, 1), (16, 16))       # (ranks, nodes)
CHANNELS = (1, 12)
PROTOS = ("stepwise", "ll")


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--max-pow", type=int, default=26, help="largest count = 2**max_pow elements")
    ap.add_argument("--min-pow", type=int, default=1)
    ap.add_argument("--out", default=None, help="write a markdown report here")
    ap.add_argument("--jsonl", default=None, help="write one JSON line per point here")
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E

    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    maxc = 1 << args.max_pow
    nmax = max(n for n, _ in SHAPES)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261207)
    sends = [torch.rand(maxc, device="cuda", generator=g) * 2 - 1 for _ in range(nmax)]
    recvs = [torch.empty_like(s) for s in sends]
    rows = {}
    jl = open(args.jsonl, "w") if args.jsonl else None
    # one untimed point per shape and protocol first (the first launches of a
    # process pay one-time costs)
    for n, m in SHAPES:
        for proto in PROTOS:
            E.comm_init(n, m, "ring", 1, CHUNK, mode=proto)
            time_graph(E, [t.data_ptr() for t in sends[:n]], [t.data_ptr() for t in recvs[:n]], 2, torch, 1)
    for n, m in SHAPES:
        sptr = [t.data_ptr() for t in sends[:n]]
        rptr = [t.data_ptr() for t in recvs[:n]]
        for algo in ("ring", "tree"):
            for nch in CHANNELS:
                key = (n, m, algo, nch)
                rows[key] = []
                for p in range(args.min_pow, args.max_pow + 1):
                    count = 1 << p
                    row = {"nranks": n, "nnodes": m, "algo": algo, "nch": nch, "count": count, "bytes": 4 * count}
                    results = {}
                    for proto in PROTOS:
                        E.comm_init(n, m, algo, nch, CHUNK, mode=proto)
                        replays = 5 if count < (1 << 22) else 1
                        row[proto] = time_graph(E, sptr, rptr, count, torch, replays)
                        results[proto] = torch.cat([r[:count] for r in recvs[:n]]).view(torch.int32).clone()
                    if not torch.equal(results["ll"], results["stepwise"]):
                        print(f"MISMATCH LL vs SIMPLE: {key} count {count}", file=sys.stderr)
                        return 1
                    if E.protocol_status():
                        print(f"ABANDONED LL call: {key} count {count}", file=sys.stderr)
                        return 1
                    del results
                    rows[key].append(row)
                    if jl:
                        jl.write(json.dumps(row) + "\n")
                    print(f"n {n:2d} {algo:4s} nch {nch:2d} {human(4 * count):>8s}: simple {row['stepwise']:9.1f}us"
                          f"  ll {row['ll']:9.1f}us  ll/simple {row['ll'] / row['stepwise']:.3f}", flush=True)
    if jl:
        jl.close()
    if args.out:
        write_report(args.out, rows)
    return 0


def write_report(path, rows):
    lines = ["# Protocol sweep: stepwise all-reduce, SIMPLE vs LL (f32 sum, one MI355X)\n\n",
             "Command: `python -m double_binary_tree_amd.protosweep --out <this file>`. Per-launch time of "
             f"{GRAPH_LAUNCHES} back-to-back launches captured in a HIP graph and replayed (events on the stream "
             "around the replays; host call overhead excluded; buffers resident in HBM). "
             "SIMPLE = FIFO slot per step + workgroup barrier; LL = flag-in-line FIFO words polled by the "
             "reader, no barriers. Results bit-identical at every point.\n\n"]
    for (n, m, algo, nch), rs in rows.items():
        lines.append(f"## {n} ranks on {m} node(s), {algo}, {nch} channel(s)\n\n")
        lines.append("| S per rank | SIMPLE µs | LL µs | LL / SIMPLE | busbw SIMPLE GB/s | busbw LL GB/s |\n"
                     "|---|---|---|---|---|---|\n")
        for r in rs:
            f = r["bytes"] * 2 * (n - 1) / n / 1e3
            lines.append(f"| {human(r['bytes'])} | {r['stepwise']:.1f} | {r['ll']:.1f} | "
                         f"{r['ll'] / r['stepwise']:.3f} | {f / r['stepwise']:.2f} | {f / r['ll']:.2f} |\n")
        iv = intervals(rs, "ll", "stepwise")
        desc = "; ".join(f"{'LL' if v == 'll' else 'SIMPLE' if v == 'stepwise' else v} {human(a)}–{human(b)}"
                         for v, a, b in iv)
        lines.append(f"\nWinner (5% tie): {desc}\n\n")
    with open(path, "w", encoding="utf-8") as f:
        f.writelines(lines)


def main() -> int:
    from double_binary_tree_amd import emucomm as E
    try:
        return _main()
    finally:
        E.release()


if __name__ == "__main__":
    sys.exit(main())
