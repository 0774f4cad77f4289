"""Helpers for the GPU tests: move seeded host inputs to the device, run the
C-ABI all-reduce, bring the results back as raw bits."""

from __future__ import annotations

import sys

import numpy as np

from double_binary_tree_amd import emucomm as E
from double_binary_tree_amd import inputs as I

TORCH_DTYPE = None


def _torch_dtype(dtype):
    import torch
    return {"i32": torch.int32, "i64": torch.int64, "f32": torch.float32,
            "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_device(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to("cuda")


def to_host_bits(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_allreduce(inputs, nnodes, algo, mode, nchannels, chunk_bytes, dtype, op, inplace=False,
                  sends=None, pattern="tree", intra=None):
    """Run one all-reduce through the C ABI; returns (outputs as numpy, send tensors)."""
    import torch
    n = len(inputs)
    E.comm_init(n, nnodes, algo, nchannels, chunk_bytes, mode=mode, pattern=pattern, intra=intra)
    if sends is None:
        sends = [to_device(x, dtype) for x in inputs]
    if inplace:
        recvs = [s.clone() for s in sends]
        bufs = recvs
        E.allreduce_tensors(bufs, bufs, op)
    else:
        recvs = [torch.empty_like(s) for s in sends]
        E.allreduce_tensors(sends, recvs, op)
    torch.cuda.synchronize()
    return [to_host_bits(r, dtype) for r in recvs], sends


# --- every-element parity at full size ---------------------------------------

_cache = {}


def clear_inputs() -> None:
    _cache.clear()


def full_inputs(w):
    """Host inputs and device send buffers of workload ``w``; one workload
    is kept at a time (the largest holds 2 GiB on each side)."""
    import torch
    key = (w.seed_index, w.nranks, w.count, w.dtype, w.dist)
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        xs = I.rank_inputs(w)
        _cache[key] = (xs, [to_device(x, w.dtype) for x in xs])
    return _cache[key]


def check_every_element(w, algo, modes=("fused", "stepwise"), inplace_modes=(False, True),
                        pattern="tree", intra=None, label=""):
    """Runs workload ``w`` with ``algo`` in every mode and placement and
    compares every element of every rank with the oracle."""
    import torch

    from oracle import allreduce as A
    xs, sends = full_inputs(w)
    announce(f"{label}oracle {w.name} {algo} ({w.nranks} ranks x {w.count} {w.dtype})")
    want = A.allreduce(xs, w.nnodes, algo, w.nchannels, w.chunk_bytes, w.dtype, w.op,
                       pattern=pattern, intra=intra)
    for r in range(1, w.nranks):
        assert np.array_equal(want[r].view(np.uint8), want[0].view(np.uint8)), "oracle ranks differ"
    want0 = want[0].view(np.uint8)
    del want
    for mode in modes:
        for inplace in inplace_modes:
            announce(f"  {label}{w.name} {algo} {mode} inplace={inplace}")
            E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode,
                        pattern=pattern, intra=intra)
            if inplace:
                recvs = [s.clone() for s in sends]
                E.allreduce_tensors(recvs, recvs, w.op)
            else:
                recvs = [torch.empty_like(s) for s in sends]
                E.allreduce_tensors(sends, recvs, w.op)
            torch.cuda.synchronize()
            if mode in ("ll", "xwg", "xwg_ll"):
                assert not E.protocol_status(), f"an {mode} call was abandoned"
            got0 = to_host_bits(recvs[0], w.dtype).view(np.uint8)
            bad = np.flatnonzero(got0 != want0)
            assert bad.size == 0, (f"{label}{w.name} {algo} {mode} inplace={inplace}: {bad.size} bytes differ "
                                   f"from the oracle, first at byte {bad[0]}")
            flat0 = recvs[0].view(torch.uint8)
            for r in range(1, w.nranks):
                assert torch.equal(recvs[r].view(torch.uint8), flat0), \
                    f"{label}{w.name} {algo} {mode} inplace={inplace}: rank {r} differs from rank 0"
            del recvs, got0, flat0
