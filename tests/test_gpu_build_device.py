"""Device-side grid build (vbm_build_device_plan / _fill) against the host
builder: the blob must be byte for byte the one vbm_build writes, on every test
grid and BlockWidth, for coordinates given in any order and with duplicates,
near the coordinate limit, and at the workloads' full sizes; bad input is
refused with the documented status.  The host builder is itself checked against
the oracle (tests/test_builder_cpu.py), and the grids below are also run through
the filters against the oracle."""
import ctypes
import sys

import numpy as np
import pytest

import oracle
from nanovdb_stencil_filtering_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from nanovdb_stencil_filtering_amd import vbm  # noqa: E402
from test_gpu_parity import GRIDS  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same_as_host(coords, log2w):
    hdr, host = vbm.build_host(coords, log2w)
    g = vbm.build_device(torch.from_numpy(np.ascontiguousarray(coords, np.int32)).cuda(), log2w)
    assert bytes(g.hdr) == bytes(hdr)
    assert np.array_equal(g.blob.cpu().numpy(), host)
    return g


@pytest.mark.parametrize("log2w", [6, 7, 8, 9])
@pytest.mark.parametrize("name", sorted(GRIDS))
def test_blob_equals_host(name, log2w):
    coords = GRIDS[name]()
    say("build_device %s W=%d n=%d" % (name, 1 << log2w, len(coords)))
    same_as_host(coords, log2w)
    # any order, duplicates collapsed
    rng = np.random.default_rng(log2w)
    dup = np.concatenate([coords, coords[rng.integers(0, len(coords), size=len(coords) // 3 + 1)]])
    same_as_host(I.shuffled(dup, 100 + log2w), log2w)


def test_empty_and_single():
    for c in (np.zeros((0, 3), np.int32), np.array([[-5, 1000, 3]], np.int32), np.array([[7, 7, 7]] * 5, np.int32)):
        for log2w in (6, 9):
            same_as_host(c, log2w)


def test_extreme_coordinates():
    coords = I.shell_coords(**I.TINY_SHELL)
    far = (1 << 30) - 2 * 4096
    for shift in ((far, -far, far), (-far, far, -far), (far - 4096 * 300, 17, -far)):
        moved = (coords.astype(np.int64) + np.array(shift)).astype(np.int32)
        same_as_host(moved, 7)


def test_device_built_grid_filters_match_the_oracle():
    coords = I.shuffled(I.random_sparse_coords(3, (18, 18, 18), 0.9, (4087, -9, -4100)), 9)
    ref = oracle.OracleGrid(coords)
    g = vbm.build_device(coords, 7)
    sc = I.sidecar(700, g.n_active, 16)
    out = vbm.box_filter(g, torch.from_numpy(sc).cuda(), vbm.CACHED | vbm.STREAMING)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.box(sc).view(np.uint32))


def test_cfg_shell_and_band_full_size():
    coords = I.shell_coords(**I.CFG_SHELL)
    for log2w in (7, 9):
        say("build_device cfg-shell W=%d" % (1 << log2w))
        same_as_host(I.shuffled(coords, 3), log2w)
    say("build_device band: generating coordinates")
    band = I.band_coords(5, **I.BAND)
    say("build_device band W=512 n=%d" % len(band))
    same_as_host(band, 9)


def run_plan(coords, log2w=7, ws_bytes=None):
    lib = vbm.load_library()
    c = torch.from_numpy(np.ascontiguousarray(coords, np.int32)).cuda()
    n = c.shape[0]
    need = ctypes.c_uint64()
    assert lib.vbm_build_device_workspace(n, ctypes.byref(need)) == 0
    ws = torch.empty(int(need.value), dtype=torch.uint8, device="cuda")
    hdr = vbm.GridHeader()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.vbm_build_device_plan(ctypes.c_void_p(c.data_ptr()), n, log2w, ctypes.c_void_p(ws.data_ptr()),
                                   need.value if ws_bytes is None else ws_bytes, ctypes.byref(hdr), st)
    return rc, hdr, ws, need.value, n


def test_errors():
    lib = vbm.load_library()
    assert run_plan(np.array([[0, 0, 1 << 30]], np.int64).astype(np.int32))[0] == -5      # c = 2^30
    assert run_plan(np.array([[-(1 << 30), 0, 0]], np.int32))[0] == -5                  # -2^30
    spread = np.array([[-(1 << 30) + 1] * 3, [(1 << 30) - 1] * 3], np.int32)
    assert run_plan(spread)[0] == -7                                                     # > 2^28 root tiles
    assert run_plan(I.shell_coords(**I.TINY_SHELL), ws_bytes=1024)[0] == -2              # workspace too small
    rc, hdr, ws, need, n = run_plan(I.shell_coords(**I.TINY_SHELL))
    assert rc == 0
    blob = torch.zeros(int(hdr.blob_bytes), dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bad = vbm.GridHeader.from_buffer_copy(hdr)
    bad.off_root += 256
    assert lib.vbm_build_device_fill(ctypes.byref(bad), n, ctypes.c_void_p(ws.data_ptr()), need,
                                     ctypes.c_void_p(blob.data_ptr()), st) == -1
    assert lib.vbm_build_device_fill(ctypes.byref(hdr), n, ctypes.c_void_p(ws.data_ptr()), 512,
                                     ctypes.c_void_p(blob.data_ptr()), st) == -2
    host_blob = np.zeros(int(hdr.blob_bytes), np.uint8)
    assert lib.vbm_build_device_fill(ctypes.byref(hdr), n, ctypes.c_void_p(ws.data_ptr()), need,
                                     ctypes.c_void_p(host_blob.ctypes.data), st) == -1
    torch.cuda.synchronize()
    assert int(blob.sum().item()) == 0
