"""The C ABI driven from plain C (tests/host/capi_check.c, built by
__graft_entry__.build() into tests/host/libcapi_check.so and called here
in-process): hipMalloc'd buffers, the default stream, no torch.  Exact
int32 sum and max against host-computed values for both algorithms in every
mode and protocol, in- and out-of-place, plus the error codes, count 0,
tree records, buffer layout, reduce-scatter and all-gather."""

import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "libcapi_check.so")


def test_c_program_uses_the_abi():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    from tests.gpu_util import announce
    E.lib()
    announce("capi_check: plain-C use of the ABI")
    lib = ctypes.CDLL(LIB)
    lib.capi_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    lib.capi_check.restype = ctypes.c_int
    buf = ctypes.create_string_buffer(512)
    rc = lib.capi_check(buf, len(buf))
    assert rc == 0, buf.value.decode()
    assert buf.value == b"ok"
