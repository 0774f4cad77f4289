"""Full-size parity: every workload at its real size, in the launch
configuration the bench uses (the library's own plan for that shape: grid,
tiles, XCD-run mapping), compared with the oracle on every element of every
rank's output, for the ring and the tree, fused and stepwise, out of place
and in place.  The oracle runs once per (workload, algorithm) on the host;
rank 0's output is compared with it byte for byte on the host, and every
other rank's output with rank 0's on the device."""

import pytest

from double_binary_tree_amd import inputs as I
from tests.gpu_util import check_every_element, clear_inputs

pytestmark = pytest.mark.gpu

FULL = ["ring4_i32", "chain8_f32", "dtree16_bf16", "dtree15_bf16", "hier4x8_f16", "hier4x8_i64",
        "hier4x8_f32max"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    yield
    clear_inputs()
    E.comm_destroy()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("name", FULL)
def test_full_size_every_element(name, algo):
    """Every workload at full size, both algorithms (the ring runs on the
    tree workloads too), fused and stepwise, out of place and in place."""
    check_every_element(I.WORKLOADS[name], algo)


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("nch", [1, 32])
def test_sweep_largest_message_every_element(nch, algo):
    """The largest point of the ring/tree size sweep (8 ranks, 256 MiB of
    f32 per rank) at the smallest and largest channel count of the sweep,
    fused and stepwise, every element against the oracle."""
    from dataclasses import replace
    w = replace(I.WORKLOADS["sweep8_f32"], nchannels=nch, count=1 << 26)
    check_every_element(w, algo, inplace_modes=(False,))


@pytest.mark.parametrize("name,count", [("chain8_f32", (1 << 18) + 37), ("chain8_f32", (1 << 19) + 4099),
                                        ("dtree16_bf16", (1 << 19) + 11), ("dtree15_bf16", (3 << 18) + 5)])
def test_mid_size_tree_pieces_every_element(name, count):
    """Messages of 1-2 MiB per rank with a ragged tail, where the stepwise
    tree's pieces hold several slices each (at least min(H, slices per CU)
    rather than one piece per resident workgroup): ring and tree, fused and
    stepwise, every element against the oracle."""
    from dataclasses import replace
    w = replace(I.WORKLOADS[name], count=count)
    for algo in ("tree", "ring"):
        check_every_element(w, algo, inplace_modes=(False,))


@pytest.mark.parametrize("name,count,algo,over", [
    ("chain8_f32", (3 << 21) + 37, "tree", {}),
    ("dtree16_bf16", (5 << 21) + 11, "tree", {}),
    ("dtree15_bf16", (5 << 21) + 5, "tree", {}),
    ("chain8_f32", (9 << 18) + 3, "tree", {"nranks": 16}),
    ("chain8_f32", (28 << 20) + 4099, "ring", {"nchannels": 1}),
])
def test_balanced_plans_ragged_every_element(name, count, algo, over):
    """Sizes with a ragged tail large enough for the plans that let the
    hardware balance the CUs: the stepwise tree in short pieces, one
    workgroup each (at least one full round of resident workgroups; pieces
    of 8 slices, and of 16 on a 16-rank single-node chain, depth 15), and
    the stepwise ring with one workgroup per task (at least 12 tasks per
    resident workgroup: 8 ranks x 112 MiB on one channel).  Fused and
    stepwise, every element against the oracle."""
    from dataclasses import replace
    w = replace(I.WORKLOADS[name], count=count, **over)
    check_every_element(w, algo, inplace_modes=(False,))
