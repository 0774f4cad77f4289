"""Graph capture: once a shape has been run (its tables built), an
all-reduce, reduce-scatter or all-gather is one kernel launch on the
caller's stream, so it can be captured in a HIP graph and replayed.  Each
replay runs on new inputs written eagerly between replays, and every
replay is checked against the oracle."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from oracle import collectives as C
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


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint8)


# every mode where it applies: LL in LDS up to 16 ranks, the device-memory
# transport on the ring only
CAPTURE_CASES = [(name, algo, mode)
                 for name, algo in [("chain8_f32", "ring"), ("dtree16_bf16", "tree"), ("hier4x8_f16", "tree"),
                                    ("chain8_f32", "tree")]
                 for mode in ["fused", "stepwise", "ll", "xwg", "xwg_ll"]
                 if not (mode == "ll" and I.WORKLOADS[name].nranks > 16) and not (mode.startswith("xwg") and algo != "ring")]


@pytest.mark.parametrize("name,algo,mode", CAPTURE_CASES)
def test_captured_allreduce_replays(name, algo, mode):
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.WORKLOADS[name]
    count = 50_003
    E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, 8192, mode=mode)
    xs = I.rank_inputs(w, count=count)
    sends = [to_device(x, w.dtype) for x in xs]
    recvs = [torch.empty_like(s) for s in sends]
    E.allreduce_tensors(sends, recvs, w.op)          # builds the tables outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.allreduce_tensors(sends, recvs, w.op)
    torch.cuda.synchronize()
    for rep in range(3):
        announce(f"graph replay {rep}: {name} {algo} {mode}")
        ys = I.rank_inputs(w, count=count, salt=10 + rep)
        for s, y in zip(sends, ys):
            s.copy_(to_device(y, w.dtype))               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = A.allreduce(ys, w.nnodes, algo, w.nchannels, 8192, w.dtype, w.op)[0]
        for r in recvs:
            assert np.array_equal(_bits(to_host_bits(r, w.dtype)), _bits(want)), f"replay {rep}"
    if mode in ("ll", "xwg", "xwg_ll"):
        assert not E.protocol_status()


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_captured_reduce_scatter_and_all_gather_replay(mode):
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.WORKLOADS["chain8_f32"]
    n, rc = w.nranks, 4096 * 3
    E.comm_init(n, 1, "ring", w.nchannels, 8192, mode=mode)
    sends = [torch.empty(n * rc, device="cuda") for _ in range(n)]
    mid = [torch.empty(rc, device="cuda") for _ in range(n)]
    outs = [torch.empty(n * rc, device="cuda") for _ in range(n)]
    E.reduce_scatter_tensors(sends, mid)
    E.all_gather_tensors(mid, outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.reduce_scatter_tensors(sends, mid)
        E.all_gather_tensors(mid, outs)
    torch.cuda.synchronize()
    for rep in range(3):
        announce(f"graph replay {rep}: reduce-scatter + all-gather {mode}")
        ys = I.rank_inputs(w, count=n * rc, salt=20 + rep)
        for s, y in zip(sends, ys):
            s.copy_(torch.from_numpy(y).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rs = C.reduce_scatter(ys, 1, w.nchannels, 8192, "f32", "sum")
        ag = C.all_gather(rs, 1, w.nchannels, 8192, "f32")
        for r in range(n):
            assert np.array_equal(mid[r].cpu().numpy().view(np.uint32), rs[r].view(np.uint32)), f"replay {rep}"
            assert np.array_equal(outs[r].cpu().numpy().view(np.uint32), ag[r].view(np.uint32)), f"replay {rep}"
