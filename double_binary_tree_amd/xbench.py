"""Transport comparison for the stepwise ring all-reduce: the step FIFOs in
LDS inside one workgroup (EMU_MODE_STEPWISE with EMU_PROTO_SIMPLE / LL)
against FIFOs in device memory between workgroups, one workgroup per
channel and ring position (EMU_TRANSPORT_DEVICE with SIMPLE / LL), and the
fused one-pass kernel for reference.

Workload: 8 virtual ranks on one node, f32 sum, 512 KiB chunks, values
uniform in [-1, 1] drawn on the device with a seeded generator; per-rank
sizes 64 MiB (the full-size ring workload) at 12, 32 and 64 channels, plus
a size sweep 1 KiB .. 64 MiB at 32 channels.  Per point: the per-launch
time of back-to-back launches replayed from a HIP graph (cooperative
launches capture like ordinary ones), and the HBM rate 2*N*S / t.  Every
point checks that all transports give the same bits and that no call was
abandoned.

    python -m double_binary_tree_amd.xbench [--out report.md]
"""

from __future__ import annotations

import argparse
import sys

from double_binary_tree_amd.sweep import human

GRAPH_LAUNCHES = 10
MODES = ("fused", "stepwise", "ll", "xwg", "xwg_ll")
NAMES = {"fused": "fused", "stepwise": "LDS SIMPLE", "ll": "LDS LL", "xwg": "device SIMPLE",
         "xwg_ll": "device LL"}
N = 8
CHUNK = 512 * 1024


def time_graph(E, sptr, rptr, count, torch, replays: int) -> float:
    stream = torch.cuda.current_stream()
    for _ in range(2):
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


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("--quick", action="store_true", help="full size at 32 channels only")
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E

    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    full = 16 << 20
    g = torch.Generator(device="cuda")
    g.manual_seed(20261209)
    sends = [torch.rand(full, device="cuda", generator=g) * 2 - 1 for _ in range(N)]
    recvs = [torch.empty_like(s) for s in sends]
    sptr = [t.data_ptr() for t in sends]
    rptr = [t.data_ptr() for t in recvs]
    points = [(nch, full) for nch in ((32,) if args.quick else (12, 32, 64))]
    if not args.quick:
        points += [(32, 1 << p) for p in range(8, 24, 2)]
    rows = []
    for nch, count in points:
        row = {"nch": nch, "count": count}
        ref = None
        for mode in MODES:
            E.comm_init(N, 1, "ring", nch, CHUNK, mode=mode)
            row[mode] = time_graph(E, sptr, rptr, count, torch, 3 if count >= (1 << 22) else 20)
            got = torch.cat([r[:count] for r in recvs]).view(torch.int32)
            if ref is None:
                ref = got.clone()
            elif not torch.equal(got, ref):
                print(f"MISMATCH {mode} nch {nch} count {count}", file=sys.stderr)
                return 1
        if E.protocol_status():
            print(f"ABANDONED call at nch {nch} count {count}", file=sys.stderr)
            return 1
        rows.append(row)
        hbm = 2 * N * count * 4 / 1e3
        print(f"nch {nch:2d} {human(4 * count):>8s}: " +
              "  ".join(f"{NAMES[m]} {row[m]:9.1f}us ({hbm / row[m]:5.0f} GB/s)" for m in MODES), flush=True)
    if args.out:
        lines = ["# Step FIFOs in LDS vs in device memory: stepwise ring all-reduce (8 ranks, f32 sum, one MI355X)\n\n",
                 "Command: `python -m double_binary_tree_amd.xbench --out <this file>`. Per-launch time of "
                 f"{GRAPH_LAUNCHES} back-to-back launches captured in a HIP graph and replayed (events around "
                 "the replays; buffers resident in HBM); GB/s = 2·N·S/t (HBM algorithmic rate, % of 8 TB/s in "
                 "brackets). 512 KiB chunks. LDS = one workgroup runs every rank of a ring task, step FIFOs in "
                 "LDS; device = one workgroup per (channel, ring position), step FIFOs in device memory "
                 "(SIMPLE: agent-scope release fence + tail counter, acquire fence on the reader; LL: 8-byte "
                 "flag-in-line words). fused = one pass, no steps. Same bits from every transport.\n\n",
                 "| channels | S per rank | " + " | ".join(f"{NAMES[m]} µs (GB/s, %)" for m in MODES) + " |\n",
                 "|---|---|" + "---|" * len(MODES) + "\n"]
        for r in rows:
            hbm = 2 * N * r["count"] * 4 / 1e3
            lines.append(f"| {r['nch']} | {human(4 * r['count'])} | " +
                         " | ".join(f"{r[m]:.1f} ({hbm / r[m]:.0f}, {hbm / r[m] / 80:.1f})" for m in MODES) + " |\n")
        with open(args.out, "w", encoding="utf-8") as f:
            f.writelines(lines)
    return 0


def main() -> int:
    from double_binary_tree_amd import emucomm as E
    try:
        return _main()
    finally:
        E.release()


if __name__ == "__main__":
    sys.exit(main())
