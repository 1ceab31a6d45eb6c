"""The WENO kernels' shortcut divisions on the GPU (the device functions the
kernels call, built into libvbm_divcheck.so) against the GPU's own IEEE
division, for every fp32 operand of the ranges the kernels use them on:

* recip(y) = 1 / y, and div_by_recip(n, y, recip(y)) = n / y for n = 6 and 3,
  for every y in [2^-40, 2^126) (the kernels' t^2 lies in [1e-12, 2^123));
* div_const(x, 6) = x / 6 and div_const(x, 12) = x / 12 for +0 and every
  finite x of magnitude at least 2^-124 (2^31 operands each); -0 gives +0
  where IEEE gives -0, which the kernels never pass on.

Below and above those ranges the shortcuts do miss (subnormal quotients, the
overflow edge), which each check must see, so a broken comparison cannot pass.
"""
import ctypes
import os
import struct

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from nanovdb_stencil_filtering_amd import build as B  # noqa: E402

BLOCKS, THREADS = 2048, 256


def bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.DIVCHECK_LIB):
        pytest.fail("libvbm_divcheck.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(B.DIVCHECK_LIB)
    for fn in (L.vbm_divcheck_recip, L.vbm_divcheck_const):
        fn.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32]
        fn.restype = ctypes.c_int
    return L


def run(fn, k, lo, hi):
    """Mismatch counts (k of them) over the bit patterns [lo, hi)."""
    counts = torch.full((BLOCKS * THREADS * k,), 0xFFFF, dtype=torch.int32, device="cuda")
    assert fn(lo, hi - lo, counts.data_ptr(), BLOCKS, THREADS) == 0
    torch.cuda.synchronize()
    return counts.view(-1, k).cpu().numpy().astype(np.int64).sum(axis=0)


def test_recip_and_weights(lib):
    assert list(run(lib.vbm_divcheck_recip, 3, bits(2.0 ** -40), bits(2.0 ** 126))) == [0, 0, 0]
    # past the range the quotients turn subnormal and the shortcut misses
    assert all(run(lib.vbm_divcheck_recip, 3, bits(2.0 ** 126), bits(2.0 ** 127)) > 0)


def test_constant_divisions(lib):
    # the zeros: +0 agrees, -0 gives +0 (one miss per divisor); then every finite
    # magnitude from 2^-124 on, both signs
    assert list(run(lib.vbm_divcheck_const, 2, 0, 1)) == [1, 1]
    assert list(run(lib.vbm_divcheck_const, 2, bits(2.0 ** -124), 0x7F800000)) == [0, 0]
    # subnormal dividends: the shortcut misses
    assert all(run(lib.vbm_divcheck_const, 2, 1, 0x00800000) > 0)
