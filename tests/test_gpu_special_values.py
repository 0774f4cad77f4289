"""Parity on IEEE special values: subnormals and signed zeros (exact
subnormal sums, -0 only from all -0), sums that overflow to infinity,
infinities, and max with -0 below +0; every float type, both algorithms,
every mode and protocol, bit-exact to the oracle.  The oracle's behaviour on
these inputs is pinned from IEEE arithmetic in tests/test_oracle_special.py.
The inputs hold no NaN and never infinities of both signs at one position
(the header's contract), so no NaN can arise."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from tests.gpu_util import announce, run_allreduce

pytestmark = pytest.mark.gpu

SHAPES = [(2, 1, 2), (6, 3, 3), (8, 1, 4), (16, 16, 2), (15, 15, 3), (32, 4, 4)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    assert not E.protocol_status()
    yield
    E.comm_destroy()
    torch.cuda.empty_cache()


def _modes(n, algo):
    modes = ["fused", "stepwise"]
    if n <= 16:
        modes.append("ll")
    if algo == "ring":
        modes += ["xwg", "xwg_ll"]
    return modes


@pytest.mark.parametrize("n,m,nch", SHAPES)
@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("op", ["sum", "max"])
def test_special_values(n, m, nch, algo, dtype, op):
    from double_binary_tree_amd import emucomm as E
    count = 5 * 1024 + 11
    xs, _, _ = I.special_inputs(n, dtype, count, seed=1000 + n * 10 + nch)
    want = A.allreduce(xs, m, algo, nch, 1024, dtype, op)[0]
    wb = np.ascontiguousarray(want).view(np.uint8).reshape(count, -1)
    for mode in _modes(n, algo):
        announce(f"special n={n} m={m} nch={nch} {algo} {dtype} {op} {mode}")
        got, _ = run_allreduce(xs, m, algo, mode, nch, 1024, dtype, op, inplace=(mode == "stepwise"))
        assert not E.protocol_status(), f"{mode}: a call was abandoned"
        for r, g in enumerate(got):
            gb = np.ascontiguousarray(g).view(np.uint8).reshape(count, -1)
            if not np.array_equal(gb, wb):
                bad = np.nonzero((gb != wb).any(axis=1))[0]
                raise AssertionError(f"{mode} rank {r}: {len(bad)} elements differ, first at {bad[:8].tolist()}")
