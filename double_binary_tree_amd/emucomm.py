"""Thin ctypes binding of libemucomm (declared in include/emu_comm.h).

Argument marshalling only: every step of the all-reduce runs in the
library's HIP kernels.  The library is loaded on first use; a missing
library raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

# EMUCOMM_LIB may point at another build of the same library (e.g. a tuning
# variant); by default the in-tree build is used.
LIB_PATH = os.environ.get("EMUCOMM_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libemucomm.so")

ALGO = {"ring": 0, "tree": 1, "auto": 2}
# "ll": the stepwise mode with the LL protocol (EMU_PROTO_LL)
MODE = {"stepwise": 0x000, "fused": 0x100, "ll": 0x200, "xwg": 0x400, "xwg_ll": 0x600}
DTYPE = {"i32": 0, "i64": 1, "f32": 2, "f16": 3, "bf16": 4}
OP = {"sum": 0, "max": 1}
ITEMSIZE = {"i32": 4, "i64": 8, "f32": 4, "f16": 2, "bf16": 2}

SUCCESS = 0
ERR_INVALID_ARGUMENT = 1
ERR_NOT_INITIALIZED = 2
ERR_INTERNAL = 3
ERR_HIP = 4

_lib = None


class EmuError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (code {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.emu_comm_init.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t]
        L.emu_comm_init.restype = ctypes.c_int
        L.emu_comm_init_graph.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t,
                                          ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        L.emu_comm_init_graph.restype = ctypes.c_int
        L.emu_allreduce.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                    ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.emu_allreduce.restype = ctypes.c_int
        L.emu_allreduce_noalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.emu_allreduce_noalloc.restype = ctypes.c_int
        L.emu_reduce_scatter.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.emu_reduce_scatter.restype = ctypes.c_int
        L.emu_all_gather.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
        L.emu_all_gather.restype = ctypes.c_int
        L.emu_tree_topology.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_int)]
        L.emu_tree_topology.restype = ctypes.c_int
        L.emu_tree_depth.argtypes = [ctypes.POINTER(ctypes.c_int)]
        L.emu_tree_depth.restype = ctypes.c_int
        L.emu_comm_destroy.argtypes = []
        L.emu_comm_destroy.restype = ctypes.c_int
        L.emu_set_cost_model.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.emu_set_cost_model.restype = ctypes.c_int
        L.emu_set_cost_model_ranks.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.emu_set_cost_model_ranks.restype = ctypes.c_int
        L.emu_get_cost_model.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double)]
        L.emu_get_cost_model.restype = ctypes.c_int
        L.emu_predict_us.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
        L.emu_predict_us.restype = ctypes.c_int
        L.emu_select_algo.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        L.emu_select_algo.restype = ctypes.c_int
        L.emu_buffer_layout.argtypes = [ctypes.c_size_t, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.POINTER(ctypes.c_size_t)]
        L.emu_buffer_layout.restype = ctypes.c_int
        L.emu_protocol_status.argtypes = [ctypes.POINTER(ctypes.c_int)]
        L.emu_protocol_status.restype = ctypes.c_int
        L.emu_device_memory.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.emu_device_memory.restype = ctypes.c_int
        L.emu_stream_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        L.emu_stream_probe.restype = ctypes.c_int
        L.emu_strerror.argtypes = [ctypes.c_int]
        L.emu_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().emu_strerror(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != SUCCESS:
        raise EmuError(code, what)


def algo_code(algo: str, mode: str = "stepwise") -> int:
    return ALGO[algo] | MODE[mode]


def comm_init_raw(nranks: int, nnodes: int, algo: int, nchannels: int, chunk_bytes: int) -> int:
    return lib().emu_comm_init(nranks, nnodes, algo, nchannels, chunk_bytes)


PATTERNS = {"tree": 0, "split": 1, "balanced": 2}


def comm_init_graph_raw(nranks: int, nnodes: int, algo: int, nchannels: int, chunk_bytes: int,
                        pattern: int, intra=None) -> int:
    """emu_comm_init_graph; ``intra`` is None or nchannels rows of nranks ranks."""
    arr = None
    if intra is not None:
        flat = [int(r) for row in intra for r in row]
        arr = (ctypes.c_int * len(flat))(*flat)
    return lib().emu_comm_init_graph(nranks, nnodes, algo, nchannels, chunk_bytes, pattern, arr)


def comm_init(nranks: int, nnodes: int, algo: str, nchannels: int, chunk_bytes: int,
              mode: str = "stepwise", pattern: str = "tree", intra=None) -> None:
    """Build the communicator.  ``pattern`` ("tree", "split", "balanced") and
    ``intra`` (per-channel rank orders, node after node) select the graph;
    the defaults are the plain emu_comm_init."""
    if pattern == "tree" and intra is None:
        _check(comm_init_raw(nranks, nnodes, algo_code(algo, mode), nchannels, chunk_bytes), "emu_comm_init")
        return
    if pattern not in PATTERNS:
        raise ValueError(f"unknown pattern {pattern!r}")
    if intra is not None and (len(intra) != nchannels or any(len(row) != nranks for row in intra)):
        raise ValueError("intra needs nchannels rows of nranks ranks")
    _check(comm_init_graph_raw(nranks, nnodes, algo_code(algo, mode), nchannels, chunk_bytes,
                               PATTERNS[pattern], intra), "emu_comm_init_graph")


def allreduce_raw(sendptrs, recvptrs, count: int, dtype: int, op: int, stream: int = 0) -> int:
    n = len(sendptrs)
    send = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(int(p)) for p in sendptrs])
    recv = (ctypes.c_void_p * max(len(recvptrs), 1))(*[ctypes.c_void_p(int(p)) for p in recvptrs])
    return lib().emu_allreduce(send, recv, count, dtype, op, ctypes.c_void_p(int(stream)))


def allreduce(sendptrs, recvptrs, count: int, dtype: str, op: str, stream: int = 0) -> None:
    _check(allreduce_raw(sendptrs, recvptrs, count, DTYPE[dtype], OP[op], stream), "emu_allreduce")


def allreduce_noalloc_raw(sendptrs, recvptrs, count: int, dtype: int, op: int, stream: int = 0) -> int:
    return lib().emu_allreduce_noalloc(_ptrs(sendptrs), _ptrs(recvptrs), count, dtype, op,
                                       ctypes.c_void_p(int(stream)))


def allreduce_noalloc(sendptrs, recvptrs, count: int, dtype: str, op: str, stream: int = 0) -> None:
    _check(allreduce_noalloc_raw(sendptrs, recvptrs, count, DTYPE[dtype], OP[op], stream),
           "emu_allreduce_noalloc")


def _ptrs(ptrs):
    return (ctypes.c_void_p * max(len(ptrs), 1))(*[ctypes.c_void_p(int(p)) for p in ptrs])


def reduce_scatter_raw(sendptrs, recvptrs, recvcount: int, dtype: int, op: int, stream: int = 0) -> int:
    return lib().emu_reduce_scatter(_ptrs(sendptrs), _ptrs(recvptrs), recvcount, dtype, op,
                                    ctypes.c_void_p(int(stream)))


def reduce_scatter(sendptrs, recvptrs, recvcount: int, dtype: str, op: str, stream: int = 0) -> None:
    _check(reduce_scatter_raw(sendptrs, recvptrs, recvcount, DTYPE[dtype], OP[op], stream), "emu_reduce_scatter")


def all_gather_raw(sendptrs, recvptrs, sendcount: int, dtype: int, stream: int = 0) -> int:
    return lib().emu_all_gather(_ptrs(sendptrs), _ptrs(recvptrs), sendcount, dtype, ctypes.c_void_p(int(stream)))


def all_gather(sendptrs, recvptrs, sendcount: int, dtype: str, stream: int = 0) -> None:
    _check(all_gather_raw(sendptrs, recvptrs, sendcount, DTYPE[dtype], stream), "emu_all_gather")


def set_cost_model(algo: str, mode: str, alpha_us: float, bw_bytes_per_us: float) -> None:
    _check(lib().emu_set_cost_model(algo_code(algo, mode), alpha_us, bw_bytes_per_us), "emu_set_cost_model")


def set_cost_model_ranks(algo: str, mode: str, nranks: int, alpha_us: float, bw_bytes_per_us: float) -> None:
    """emu_set_cost_model_ranks: the parameters of the rank-count class of
    ``nranks`` (0: every class)."""
    _check(lib().emu_set_cost_model_ranks(algo_code(algo, mode), nranks, alpha_us, bw_bytes_per_us),
           "emu_set_cost_model_ranks")


def get_cost_model(algo: str, mode: str, nranks: int) -> tuple[float, float]:
    """(alpha us per stage, bandwidth bytes/us) of the class of ``nranks``."""
    a, b = ctypes.c_double(), ctypes.c_double()
    _check(lib().emu_get_cost_model(algo_code(algo, mode), nranks, ctypes.byref(a), ctypes.byref(b)),
           "emu_get_cost_model")
    return a.value, b.value


def predict_us(algo: str, mode: str, count: int, dtype: str) -> float:
    out = ctypes.c_double()
    _check(lib().emu_predict_us(algo_code(algo, mode), count, DTYPE[dtype], ctypes.byref(out)), "emu_predict_us")
    return out.value


def select_algo(count: int, dtype: str) -> str:
    out = ctypes.c_int()
    _check(lib().emu_select_algo(count, DTYPE[dtype], ctypes.byref(out)), "emu_select_algo")
    return {v: k for k, v in ALGO.items()}[out.value]


def tree_topology(channel: int, rank: int) -> tuple[int, list[int]]:
    up = ctypes.c_int(0)
    down = (ctypes.c_int * 3)()
    _check(lib().emu_tree_topology(channel, rank, ctypes.byref(up), down), "emu_tree_topology")
    return up.value, list(down)


def tree_depth() -> int:
    d = ctypes.c_int(0)
    _check(lib().emu_tree_depth(ctypes.byref(d)), "emu_tree_depth")
    return d.value


def buffer_layout(nbufs: int, nbytes: int) -> tuple[list[int], int]:
    """emu_buffer_layout: per-buffer byte offsets inside one pool, and the
    pool size (the pool base must be 64 KiB aligned)."""
    offs = (ctypes.c_size_t * max(nbufs, 1))()
    pool = ctypes.c_size_t(0)
    _check(lib().emu_buffer_layout(nbufs, nbytes, offs, ctypes.byref(pool)), "emu_buffer_layout")
    return [int(offs[i]) for i in range(nbufs)], int(pool.value)


def rank_buffers(nranks: int, count: int, dtype, device="cuda"):
    """Send and receive buffers of `count` elements for every rank, carved
    from one torch allocation at emu_buffer_layout's offsets (sends first,
    then receives).  Returns (pool, sends, recvs); the views keep the pool
    alive."""
    import torch
    itemsize = torch.empty((), dtype=dtype).element_size()
    offs, size = buffer_layout(2 * nranks, count * itemsize)
    align = 64 << 10
    pool = torch.empty(size + align, dtype=torch.uint8, device=device)
    base = (-pool.data_ptr()) % align
    bufs = [pool[base + o: base + o + count * itemsize].view(dtype) for o in offs]
    return pool, bufs[:nranks], bufs[nranks:]


def protocol_status() -> bool:
    """True if an LL all-reduce on the current device was abandoned since the
    last query (waits for the device; clears the flag)."""
    v = ctypes.c_int(0)
    _check(lib().emu_protocol_status(ctypes.byref(v)), "emu_protocol_status")
    return bool(v.value)


def comm_destroy() -> None:
    _check(lib().emu_comm_destroy(), "emu_comm_destroy")


STREAM = {"read": 0, "write": 1, "copy": 2}


def stream_probe(kind: str, src: int, dst: int, nbytes: int, stream: int = 0) -> None:
    """emu_stream_probe: one pass of the read-only, write-only or copy
    streaming kernel (pointers as integers)."""
    _check(lib().emu_stream_probe(STREAM[kind], ctypes.c_void_p(int(src)), ctypes.c_void_p(int(dst)), nbytes,
                                  ctypes.c_void_p(int(stream))), "emu_stream_probe")


def release() -> None:
    """emu_comm_destroy if the library was loaded: frees its device memory
    while the HIP runtime is still up.  Scripts call it before they return."""
    if _lib is not None:
        comm_destroy()


def device_memory() -> tuple[int, int]:
    """(allocations, bytes) of device memory the library holds now."""
    n = ctypes.c_size_t(0)
    b = ctypes.c_size_t(0)
    _check(lib().emu_device_memory(ctypes.byref(n), ctypes.byref(b)), "emu_device_memory")
    return int(n.value), int(b.value)


# --- torch convenience (device memory and streams only) ---------------------

def torch_dtype_name(t) -> str:
    import torch
    return {torch.int32: "i32", torch.int64: "i64", torch.float32: "f32",
            torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def allreduce_tensors(sends, recvs, op: str = "sum", stream=None) -> None:
    """All-reduce a list of per-rank CUDA tensors (same shape and dtype,
    contiguous) into ``recvs`` on ``stream`` (default: the current stream)."""
    import torch
    if len(sends) != len(recvs) or not sends:
        raise ValueError("need one send and one receive tensor per rank")
    dt = torch_dtype_name(sends[0])
    count = sends[0].numel()
    for t in list(sends) + list(recvs):
        if not t.is_cuda or not t.is_contiguous() or t.numel() != count or torch_dtype_name(t) != dt:
            raise ValueError("tensors must be contiguous CUDA tensors of one shape and dtype")
    s = torch.cuda.current_stream() if stream is None else stream
    allreduce([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count, dt, op, s.cuda_stream)


def _check_tensors(ts, numel, dt):
    import torch
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.numel() != numel or torch_dtype_name(t) != dt:
            raise ValueError("tensors must be contiguous CUDA tensors of the collective's size and one dtype")
    del torch


def reduce_scatter_tensors(sends, recvs, op: str = "sum", stream=None) -> None:
    """Reduce-scatter per-rank CUDA tensors: ``sends[r]`` holds nranks blocks
    of ``recvs[r].numel()`` elements; ``recvs[r]`` gets the reduced block r."""
    import torch
    if len(sends) != len(recvs) or not sends:
        raise ValueError("need one send and one receive tensor per rank")
    dt = torch_dtype_name(sends[0])
    rc = recvs[0].numel()
    _check_tensors(sends, rc * len(sends), dt)
    _check_tensors(recvs, rc, dt)
    s = torch.cuda.current_stream() if stream is None else stream
    reduce_scatter([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], rc, dt, op, s.cuda_stream)


def all_gather_tensors(sends, recvs, stream=None) -> None:
    """All-gather per-rank CUDA tensors: block k of every ``recvs[r]`` gets
    ``sends[k]``."""
    import torch
    if len(sends) != len(recvs) or not sends:
        raise ValueError("need one send and one receive tensor per rank")
    dt = torch_dtype_name(sends[0])
    sc = sends[0].numel()
    _check_tensors(sends, sc, dt)
    _check_tensors(recvs, sc * len(sends), dt)
    s = torch.cuda.current_stream() if stream is None else stream
    all_gather([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], sc, dt, s.cuda_stream)
