"""A consumer written on the device header alone (tests/custom_consumer.hip,
built into libvbm_example.so): the decode, the staged neighbour-leaf table and
the streamed box taps of vbm_device.hpp, used from a kernel of the caller's
own, the way the pages' forEachBoxStencil callback is meant to be used.  Per
voxel, the number of active box neighbours and the largest channel-0 value
among them must equal what the oracle's taps give, with the Cached table and
with tree walks, at W128 and W512, including a grid whose blocks all span more
than 16 leaves (the table is then skipped)."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from nanovdb_stencil_filtering_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from nanovdb_stencil_filtering_amd import build as B  # noqa: E402
from nanovdb_stencil_filtering_amd import vbm  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.EXAMPLE_LIB):
        pytest.fail("libvbm_example.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(B.EXAMPLE_LIB)
    L.vbm_example_neighbour_stats.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    L.vbm_example_neighbour_stats.restype = ctypes.c_int
    return L


GRIDS = {
    "tiny_shell": lambda: I.shell_coords(**I.TINY_SHELL),
    "dense_cube": lambda: I.random_sparse_coords(4, (24, 24, 24), 1.0, (-8, -8, -8)),
    "straddle": lambda: I.random_sparse_coords(3, (18, 18, 18), 0.9, (4087, -9, -4100)),
    "one_per_leaf": lambda: I.one_per_cell_coords(5, 12),
}


@pytest.mark.parametrize("name", sorted(GRIDS))
def test_neighbour_stats(lib, name):
    coords = GRIDS[name]()
    ref = oracle.OracleGrid(coords)
    C = 3
    sc = I.sidecar(55, ref.n_active, C)
    taps = ref.taps(27).astype(np.int64)                     # rows for indices 1..N
    active = taps != 0
    want_count = active.sum(axis=1).astype(np.uint32)
    vals = np.where(active, sc[taps, 0], -np.inf).astype(np.float32)
    want_max = vals.max(axis=1)
    sct = torch.from_numpy(sc).cuda()
    for log2w in (7, 9):
        g = vbm.build(coords, log2w)
        for cached in (1, 0):
            largest = torch.full((g.n_slots,), float("nan"), dtype=torch.float32, device="cuda")
            count = torch.full((g.n_slots,), -1, dtype=torch.int32, device="cuda")
            rc = lib.vbm_example_neighbour_stats(ctypes.byref(g.hdr), ctypes.c_void_p(g.blob.data_ptr()),
                                                 ctypes.c_void_p(sct.data_ptr()), C, ctypes.c_void_p(largest.data_ptr()),
                                                 ctypes.c_void_p(count.data_ptr()), cached)
            assert rc == 0
            torch.cuda.synchronize()
            n = ref.n_active
            got_count = count.cpu().numpy().view(np.uint32)
            got_max = largest.cpu().numpy()
            assert np.array_equal(got_count[:n], want_count), (name, log2w, cached)
            assert np.array_equal(got_max[:n].view(np.uint32), want_max.view(np.uint32)), (name, log2w, cached)
            assert np.all(got_count[n:] == 0xFFFFFFFF)  # sentinel slots untouched
