"""Message-size sweep: ring vs tree, fused vs stepwise, per channel count.

A workload's shape (ranks, nodes, element type, operator; by default the
8 ranks on one node of the size sweep, f32 sum, channels 1/4/12/32; other
workloads at their own channel count), per-rank sizes from 2 elements up in
powers of two, values from the workload's distribution drawn on the device
with a seeded generator.  The rank buffers are carved from one pool at
emu_buffer_layout's offsets, as the bench does.  Every point checks that the
fused and stepwise results of each algorithm are bit-identical.

Per point and leg: the per-launch time of back-to-back launches replayed from
a HIP graph (so host call overhead is left out), algbw = S/t, busbw = algbw *
2(N-1)/N and HBM GB/s = 2*N*S/t; per channel count the size intervals where
ring or tree wins, with the practical-tie rule of the course page ("NCCL 专家
课程 13", section "性能结果的判定规则": a loser within 5% of the winner is a
tie).

    python -m double_binary_tree_amd.sweep [--workload sweep8_f32] [--channels 1,4,12,32]
        [--max-pow 26] [--out report.md] [--jsonl points.jsonl]
"""

from __future__ import annotations

import argparse
import json
import sys

CHANNELS = (1, 4, 12, 32)
CHUNK = 512 * 1024
LEGS = (("ring", "fused"), ("tree", "fused"), ("ring", "stepwise"), ("tree", "stepwise"))
TIE = 0.05
GRAPH_LAUNCHES = 20
TORCH_DTYPES = {"i32": "int32", "i64": "int64", "f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def human(nbytes: int) -> str:
    for unit, div in (("GiB", 1 << 30), ("MiB", 1 << 20), ("KiB", 1 << 10)):
        if nbytes >= div:
            return f"{nbytes // div} {unit}"
    return f"{nbytes} B"


def time_graph(E, sptr, rptr, count, dtype, op, torch, replays: int) -> float:
    """Per-launch time (us) of back-to-back launches replayed from a HIP
    graph: GRAPH_LAUNCHES all-reduces captured once (after warm calls, which
    build the shape's tables), the graph replayed `replays` times between
    two events."""
    stream = torch.cuda.current_stream()
    for _ in range(3):
        E.allreduce(sptr, rptr, count, dtype, op, stream.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(GRAPH_LAUNCHES):
            E.allreduce(sptr, rptr, count, dtype, op, cap.cuda_stream)
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


def tree_depth(E, nch: int, n: int) -> int:
    """Deepest channel tree of the active communicator, from its records."""
    deepest = 0
    for c in range(nch):
        ups = [E.tree_topology(c, r)[0] for r in range(n)]
        for r in range(n):
            d, x = 0, r
            while ups[x] != -1:
                x, d = ups[x], d + 1
            deepest = max(deepest, d)
    return deepest


def intervals(rows, key_a, key_b):
    """Winner intervals between two legs over increasing sizes."""
    out = []
    for r in rows:
        ta, tb = r[key_a], r[key_b]
        winner = key_a if ta < tb else key_b
        loser_t, winner_t = max(ta, tb), min(ta, tb)
        verdict = "tie" if loser_t / winner_t - 1 < TIE else winner
        if out and out[-1][0] == verdict:
            out[-1][2] = r["bytes"]
        else:
            out.append([verdict, r["bytes"], r["bytes"]])
    return out


def fill(bufs, w, seed: int, torch) -> None:
    """Values of workload w's distribution, drawn on the device."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for b in bufs:
        if w.dist[0] == "int":
            b.copy_(torch.randint(w.dist[1], w.dist[2] + 1, b.shape, generator=g, device="cuda", dtype=torch.int64))
        elif w.dist[0] == "normal":
            b.copy_(torch.randn(b.shape, generator=g, device="cuda") * w.dist[1])
        else:
            b.copy_(torch.rand(b.shape, generator=g, device="cuda") * (w.dist[2] - w.dist[1]) + w.dist[1])


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="sweep8_f32")
    ap.add_argument("--channels", default=None, help="comma-separated channel counts (default: 1,4,12,32 for "
                                                     "sweep8_f32, else the workload's own)")
    ap.add_argument("--max-pow", type=int, default=26, help="largest count = 2**max_pow elements")
    ap.add_argument("--min-pow", type=int, default=1)
    ap.add_argument("--out", default=None, help="write a markdown report here")
    ap.add_argument("--jsonl", default=None, help="write one JSON line per point here")
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    w = I.WORKLOADS[args.workload]
    n = w.nranks
    if args.channels:
        channels = tuple(int(c) for c in args.channels.split(","))
    else:
        channels = CHANNELS if args.workload == "sweep8_f32" else (w.nchannels,)
    maxc = 1 << args.max_pow
    pool, sends, recvs = E.rank_buffers(n, maxc, getattr(torch, TORCH_DTYPES[w.dtype]))
    fill(sends, w, 20261206 + w.seed_index, torch)
    sptr = [t.data_ptr() for t in sends]
    rptr = [t.data_ptr() for t in recvs]
    rows = {c: [] for c in channels}
    jl = open(args.jsonl, "w") if args.jsonl else None
    for nch in channels:
        E.comm_init(n, w.nnodes, "tree", nch, CHUNK)
        depth = tree_depth(E, nch, n)
        for p in range(args.min_pow, args.max_pow + 1):
            count = 1 << p
            row = {"workload": w.name, "nranks": n, "nnodes": w.nnodes, "depth": depth, "dtype": w.dtype,
                   "op": w.op, "nch": nch, "count": count, "bytes": count * w.itemsize}
            results = {}
            for algo, mode in LEGS:
                E.comm_init(n, w.nnodes, algo, nch, CHUNK, mode=mode)
                replays = 3 if count * w.itemsize >= (1 << 24) else 10
                row[f"{algo}_{mode}"] = time_graph(E, sptr, rptr, count, w.dtype, w.op, torch, replays)
                results[(algo, mode)] = (recvs[0][:count].view(torch.uint8).clone(),
                                         recvs[-1][:count].view(torch.uint8).clone())
            for algo in ("ring", "tree"):
                f, s = results[(algo, "fused")], results[(algo, "stepwise")]
                if not (torch.equal(f[0], s[0]) and torch.equal(f[1], s[1])):
                    print(f"MISMATCH {algo} fused vs stepwise at count {count} nch {nch}", file=sys.stderr)
                    return 1
            del results
            rows[nch].append(row)
            line = {**row, **{f"{k}_busbw": row["bytes"] / (row[k] * 1e-6) / 1e9 * 2 * (n - 1) / n
                              for k in ("ring_fused", "tree_fused", "ring_stepwise", "tree_stepwise")}}
            if jl:
                jl.write(json.dumps(line) + "\n")
                jl.flush()
            print(f"{w.name} nch {nch:2d} {human(row['bytes']):>8s}: " +
                  "  ".join(f"{k} {row[k]:9.1f}us" for k in ("ring_fused", "tree_fused", "ring_stepwise",
                                                            "tree_stepwise")), flush=True)
    if jl:
        jl.close()
    if args.out:
        extra = "".join(f" --{k.replace('_', '-')} {v}" for k, v in
                        (("channels", args.channels), ("min_pow", args.min_pow), ("max_pow", args.max_pow))
                        if v is not None and v != ap.get_default(k))
        write_report(args.out, rows, w, extra)
    return 0


def write_report(path, rows, w, extra=""):
    n = w.nranks
    lines = [f"# Message-size sweep: ring vs tree, fused vs stepwise ({w.name}: {n} ranks on {w.nnodes} node(s), "
             f"{w.dtype} {w.op}, one MI355X)\n\n",
             f"Command: `python -m double_binary_tree_amd.sweep --workload {w.name}{extra} --out <this file>`. Per-launch "
             f"time of {GRAPH_LAUNCHES} back-to-back launches replayed from a HIP graph (events around the "
             "replays; buffers resident in HBM at the library's placement; no cache flush between launches, so "
             "sizes whose 2·N·S fits the 256 MB Infinity Cache run partly from cache). busbw = S/t · 2(N−1)/N; "
             "HBM = 2·N·S/t.\n\n"]
    for nch, rs in rows.items():
        lines.append(f"## {nch} channel(s)\n\n")
        lines.append("| S per rank | ring fused µs | tree fused µs | ring stepwise µs | tree stepwise µs | "
                     "best busbw GB/s | best HBM GB/s |\n|---|---|---|---|---|---|---|\n")
        for r in rs:
            best = min(r["ring_fused"], r["tree_fused"], r["ring_stepwise"], r["tree_stepwise"])
            busbw = r["bytes"] / (best * 1e-6) / 1e9 * 2 * (n - 1) / n
            hbm = 2 * n * r["bytes"] / (best * 1e-6) / 1e9
            lines.append(f"| {human(r['bytes'])} | {r['ring_fused']:.1f} | {r['tree_fused']:.1f} | "
                         f"{r['ring_stepwise']:.1f} | {r['tree_stepwise']:.1f} | {busbw:.1f} | {hbm:.0f} |\n")
        for mode in ("fused", "stepwise"):
            iv = intervals(rs, f"ring_{mode}", f"tree_{mode}")
            desc = "; ".join(f"{v.replace('_' + mode, '')} {human(a)}–{human(b)}" for v, a, b in iv)
            lines.append(f"\nRing vs tree ({mode}, 5% tie): {desc}\n")
        lines.append("\n")
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
