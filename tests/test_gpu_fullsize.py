"""Full-size parity: every workload at its real size, in the launch
configuration the bench uses, checked against the oracle position by
position on a sample (random positions plus the first and last element of
every channel, ring loop and rank-chunk), and by properties that hold at
any size (every rank holds the same bits; in-place equals out-of-place)."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from oracle import partition as P
from tests.gpu_util import announce, to_device, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    yield
    E.comm_destroy()
    torch.cuda.empty_cache()


def _sample(w, count, rng):
    unit = 16 // w.itemsize
    idx = set(rng.integers(0, count, size=4096).tolist())
    for off, ln in P.channel_ranges(count, unit, w.nchannels):
        if ln:
            idx.update((off, off + ln - 1))
            for blocks in P.ring_loops(off, ln, w.nranks, w.chunk_bytes // w.itemsize, unit):
                for o, n in blocks:
                    if n:
                        idx.update((o, o + n - 1))
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.parametrize("name", ["ring4_i32", "chain8_f32", "dtree16_bf16", "dtree15_bf16",
                                  "hier4x8_f16", "hier4x8_i64", "hier4x8_f32max"])
def test_full_size_sampled(name):
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.WORKLOADS[name]
    announce(f"full size {name}: {w.nranks} ranks x {w.count} {w.dtype}")
    xs = I.rank_inputs(w)
    idx = _sample(w, w.count, np.random.default_rng(5))
    sends = [to_device(x, w.dtype) for x in xs]
    for algo in w.algos:
        want = A.allreduce_at(xs, idx, w.nnodes, algo, w.nchannels, w.chunk_bytes, w.dtype, w.op)
        outs = {}
        for mode in ("fused", "stepwise"):
            for inplace in (False, True):
                announce(f"  {name} {algo} {mode} inplace={inplace}")
                E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
                recvs = [s.clone() for s in sends] if inplace else [torch.empty_like(s) for s in sends]
                E.allreduce_tensors(recvs if inplace else sends, recvs, w.op)
                torch.cuda.synchronize()
                flat = [r.view(torch.uint8) for r in recvs]
                for r in flat[1:]:
                    assert torch.equal(r, flat[0]), f"{name} {algo} {mode}: ranks differ"
                got = to_host_bits(recvs[0], w.dtype)
                g = got[idx]
                assert np.array_equal(g.view(np.uint8), want.view(np.uint8)), \
                    f"{name} {algo} {mode} inplace={inplace}: sampled outputs differ from the oracle"
                outs[(mode, inplace)] = flat[0]
                del recvs, flat
        ref = outs[("fused", False)]
        for key, o in outs.items():
            assert torch.equal(o, ref), f"{name} {algo} {key} differs from fused out-of-place"
        del outs
    del sends, xs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nch", [1, 32])
def test_sweep_largest_message_sampled(nch):
    """The largest point of the ring/tree size sweep (8 ranks, 256 MiB of f32
    per rank) at the smallest and largest channel count of the sweep, ring
    and tree, fused and stepwise: sampled positions (and every channel, loop
    and rank-chunk edge) equal the oracle's, all ranks hold the same bits,
    and the modes agree on every byte."""
    import torch
    from dataclasses import replace
    from double_binary_tree_amd import emucomm as E
    w = replace(I.WORKLOADS["sweep8_f32"], nchannels=nch, count=1 << 26)
    announce(f"sweep maximum: 8 ranks x 256 MiB f32, {nch} channels")
    xs = I.rank_inputs(w)
    idx = _sample(w, w.count, np.random.default_rng(6))
    sends = [to_device(x, w.dtype) for x in xs]
    for algo in ("ring", "tree"):
        outs = {}
        for mode in ("fused", "stepwise"):
            announce(f"  sweep maximum {nch} ch {algo} {mode}")
            E.comm_init(w.nranks, w.nnodes, algo, nch, w.chunk_bytes, mode=mode)
            recvs = [torch.empty_like(s) for s in sends]
            E.allreduce_tensors(sends, recvs, w.op)
            torch.cuda.synchronize()
            for r in recvs[1:]:
                assert torch.equal(r, recvs[0]), f"{algo} {mode}: ranks differ"
            outs[mode] = recvs[0]
            del recvs
        assert torch.equal(outs["fused"], outs["stepwise"]), f"{algo}: fused and stepwise differ"
        got = to_host_bits(outs["fused"], w.dtype)[idx]
        del outs
        want = A.allreduce_at(xs, idx, w.nnodes, algo, nch, w.chunk_bytes, w.dtype, w.op)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), f"{algo}: sampled outputs differ"
    del sends, xs
    torch.cuda.empty_cache()
