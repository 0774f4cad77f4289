"""Reduce-scatter and all-gather throughput on one GPU.

Shape: the all-reduce bench workload's ranks, channels and chunk (8 virtual
ranks, 12 channels, 512 KiB chunks, float32), with blocks of 2 Mi elements
(8 MiB): reduce-scatter reads 8 blocks from each of the 8 ranks (64 MiB per
rank in) and writes one block per rank; all-gather reads 8 MiB per rank and
writes 8 blocks per rank.  Algorithmic HBM bytes per call, either way:
(N^2 + N) * block bytes = 576 MiB.  Inputs N(0, 1), resident in HBM.

Prints one JSON line: per collective and mode the mean time per call
(events on the launch stream) and the HBM GB/s and fraction of 8 TB/s.

    python -m double_binary_tree_amd.collbench [--iters 20]
"""

from __future__ import annotations

import argparse
import json
import sys

HBM_PEAK_GBPS = 8000.0


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=20)
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    if not torch.cuda.is_available():
        print("collbench needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    w = I.WORKLOADS["chain8_f32"]
    n = w.nranks
    block = w.count // n
    esz = w.itemsize
    xs = I.rank_inputs(w)                                  # n blocks per rank
    rs_send = [torch.from_numpy(x).cuda() for x in xs]
    rs_recv = [torch.empty(block, dtype=torch.float32, device="cuda") for _ in range(n)]
    ag_send = [t[:block].clone() for t in rs_send]
    ag_recv = [torch.empty(n * block, dtype=torch.float32, device="cuda") for _ in range(n)]
    del xs
    stream = torch.cuda.current_stream()
    alg_bytes = (n * n + n) * block * esz
    out = {"shape": f"{n} virtual ranks x 1 node, {w.nchannels} channels, {w.chunk_bytes // 1024} KiB chunks, "
                    f"f32, block {block} elements ({block * esz // (1024 * 1024)} MiB)",
           "algorithmic_bytes_per_call": alg_bytes, "legs": {}}

    def call(coll):
        if coll == "reduce_scatter":
            E.reduce_scatter_tensors(rs_send, rs_recv, "sum", stream)
        else:
            E.all_gather_tensors(ag_send, ag_recv, stream)

    for mode in ("fused", "stepwise"):
        E.comm_init(n, w.nnodes, "ring", w.nchannels, w.chunk_bytes, mode=mode)
        for coll in ("reduce_scatter", "all_gather"):
            for _ in range(3):
                call(coll)
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for _ in range(args.iters):
                call(coll)
            end.record(stream)
            end.synchronize()
            t = start.elapsed_time(end) / 1e3 / args.iters
            gbps = alg_bytes / t / 1e9
            out["legs"][f"{coll}_{mode}"] = {"us": round(t * 1e6, 2), "hbm_GBps": round(gbps, 1),
                                             "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
            print(f"[collbench] {coll:14s} {mode:8s} {t * 1e6:8.1f} us  {gbps:7.1f} GB/s", file=sys.stderr,
                  flush=True)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    from double_binary_tree_amd import emucomm as E
    try:
        return _main()
    finally:
        E.release()


if __name__ == "__main__":
    sys.exit(main())
