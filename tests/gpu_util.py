"""Helpers for the GPU tests: move seeded host inputs to the device, run the
C-ABI all-reduce, bring the results back as raw bits."""

from __future__ import annotations

import sys

import numpy as np

from double_binary_tree_amd import emucomm as E

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
