"""Python binding of libvbm.so (the C ABI in include/vbm.h).

Argument marshalling only: every step of the stencil pipeline runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream.  The names mirror the C entry points:

    build(coords, log2_width)          vbm_build  (host) + copy of the blob to the GPU
    build_device(coords, log2_width)   vbm_build_device_workspace / _plan / _fill (on the GPU)
    build_metadata(grid)               vbm_build_metadata (device-side leaf/block metadata)
    decode(grid)                       vbm_decode
    decode_sweep(grid)                 vbm_decode_sweep
    stencil_indices(grid, shape, ...)  vbm_stencil_indices
    box_filter(grid, sidecar, ...)     vbm_box_filter
    cross_filter(grid, sidecar, ...)   vbm_cross_filter
    axis_filter(grid, sidecar, ...)    vbm_axis_filter
    weno_filter(grid, sidecar, ...)    vbm_weno_filter

There is no CPU fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libvbm.so")
# checking build used by the tests (brick cells poisoned before every brick pass)
POISON_LIB_PATH = os.path.join(_HERE, "_lib", "libvbm_poison.so")

CACHED = 0x1
STREAMING = 0x2
OP_SUM = 0x0
OP_LAPLACIAN = 0x4
WIDE_ROWS = 0x8  # filters: sidecar rows by 64-bit addresses (taken by itself from 0xFFFFFF00 bytes on)
MAX_CACHED_LEAVES = 16
GRID_MAGIC = 0x314D4256

STATUS = {0: "VBM_OK", -1: "VBM_ERR_ARG", -2: "VBM_ERR_SIZE", -3: "VBM_ERR_ALIGN", -4: "VBM_ERR_ALIAS",
          -5: "VBM_ERR_RANGE", -6: "VBM_ERR_HIP", -7: "VBM_ERR_UNSUPPORTED", -8: "VBM_ERR_NOMEM"}

EXPORTED = ("vbm_build", "vbm_free_blob", "vbm_build_metadata", "vbm_decode", "vbm_decode_sweep", "vbm_stencil_indices",
            "vbm_box_filter", "vbm_cross_filter", "vbm_axis_filter", "vbm_weno_filter",
            "vbm_build_device_workspace", "vbm_build_device_plan", "vbm_build_device_fill",
            "vbm_build_device_static", "vbm_strerror")


class VbmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, str(status)), _strerror(status)))


class GridHeader(ctypes.Structure):
    """Mirror of struct vbm_grid."""
    _fields_ = [
        ("magic", ctypes.c_uint32), ("log2_width", ctypes.c_int32), ("n_active", ctypes.c_uint64),
        ("n_leaves", ctypes.c_uint32), ("n_blocks", ctypes.c_uint32), ("n_root", ctypes.c_uint32),
        ("n_upper", ctypes.c_uint32), ("n_lower", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
        ("blob_bytes", ctypes.c_uint64), ("off_leaves", ctypes.c_uint64), ("off_root", ctypes.c_uint64),
        ("off_upper", ctypes.c_uint64), ("off_lower", ctypes.c_uint64),
        ("off_block_first_leaf", ctypes.c_uint64), ("off_block_jump", ctypes.c_uint64),
    ]


_libs = {}
_active_path = None  # set by using_library()


@contextlib.contextmanager
def using_library(path):
    """Route every call of this module to the library at `path` (the tests use it
    for the poisoned checking build) for the duration of the block."""
    global _active_path
    old = _active_path
    _active_path = path
    try:
        yield load_library()
    finally:
        _active_path = old


def load_library():
    """Load libvbm.so (raises if it has not been built)."""
    path = _active_path or LIB_PATH
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise ImportError("%s is not built; run __graft_entry__.build() or "
                          "python -m nanovdb_stencil_filtering_amd.build" % path)
    # torch brings its own HIP runtime; loading it first makes libvbm.so bind to
    # that same runtime, so torch's device pointers and streams are valid in the
    # library's launches (a second runtime would reject torch's stream handles).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    GP = ctypes.POINTER(GridHeader)
    lib.vbm_build.restype = I
    lib.vbm_build.argtypes = [P, I64, I, GP, ctypes.POINTER(ctypes.c_void_p)]
    lib.vbm_free_blob.restype = None
    lib.vbm_free_blob.argtypes = [P]
    lib.vbm_build_metadata.restype = I
    lib.vbm_build_metadata.argtypes = [GP, P, P, P]
    lib.vbm_decode.restype = I
    lib.vbm_decode.argtypes = [GP, P, P, P, P]
    lib.vbm_decode_sweep.restype = I
    lib.vbm_decode_sweep.argtypes = [GP, P, P, P, P]
    lib.vbm_stencil_indices.restype = I
    lib.vbm_stencil_indices.argtypes = [GP, P, I, I, P, P]
    lib.vbm_box_filter.restype = I
    lib.vbm_box_filter.argtypes = [GP, P, P, P, I, I, P]
    lib.vbm_cross_filter.restype = I
    lib.vbm_cross_filter.argtypes = [GP, P, P, P, I, I, P]
    lib.vbm_axis_filter.restype = I
    lib.vbm_axis_filter.argtypes = [GP, P, P, P, I, I, P]
    lib.vbm_build_device_workspace.restype = I
    lib.vbm_build_device_workspace.argtypes = [I64, ctypes.POINTER(ctypes.c_uint64)]
    lib.vbm_build_device_plan.restype = I
    lib.vbm_build_device_plan.argtypes = [P, I64, I, P, ctypes.c_uint64, GP, P]
    lib.vbm_build_device_fill.restype = I
    lib.vbm_build_device_fill.argtypes = [GP, I64, P, ctypes.c_uint64, P, P]
    lib.vbm_build_device_static.restype = I
    lib.vbm_build_device_static.argtypes = [P, I64, I, P, ctypes.c_uint64, GP, P]
    lib.vbm_weno_filter.restype = I
    lib.vbm_weno_filter.argtypes = [GP, P, P, P, I, I, P]
    lib.vbm_strerror.restype = ctypes.c_char_p
    lib.vbm_strerror.argtypes = [I]
    _libs[path] = lib
    return lib


def _strerror(status: int) -> str:
    try:
        return load_library().vbm_strerror(status).decode()
    except Exception:  # pragma: no cover - library missing while formatting an error
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise VbmError(status, what)


# ---------------------------------------------------------------------------
# host build
# ---------------------------------------------------------------------------

def build_host(coords: np.ndarray, log2_width: int):
    """vbm_build: returns (header, blob as a numpy uint8 array owned by Python)."""
    lib = load_library()
    c = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 3)
    hdr = GridHeader()
    blob = ctypes.c_void_p()
    ptr = c.ctypes.data_as(ctypes.c_void_p) if c.size else None
    _check(lib.vbm_build(ptr, c.shape[0], int(log2_width), ctypes.byref(hdr), ctypes.byref(blob)), "vbm_build")
    try:
        host = np.ctypeslib.as_array(ctypes.cast(blob, ctypes.POINTER(ctypes.c_uint8)),
                                     shape=(hdr.blob_bytes,)).copy()
    finally:
        lib.vbm_free_blob(blob)
    return hdr, host


def blob_sections(hdr: GridHeader, blob: np.ndarray) -> dict:
    """Numpy views of the blob's sections (layout of include/vbm.h)."""
    L, nb, W = hdr.n_leaves, hdr.n_blocks, 1 << hdr.log2_width
    leaf_dt = np.dtype([("mask", "<u8", (8,)), ("prefix", "<u8"), ("first", "<u8"), ("origin", "<i4", (3,)),
                        ("lower", "<u4"), ("upper", "<u4"), ("pad", "<u4", (7,))])
    root_dt = np.dtype([("key", "<i4", (3,)), ("upper", "<u4")])

    def sec(off, dt, count):
        return np.frombuffer(blob, dtype=dt, count=count, offset=off)

    return dict(
        leaves=sec(hdr.off_leaves, leaf_dt, L),
        root=sec(hdr.off_root, root_dt, hdr.n_root),
        upper=sec(hdr.off_upper, "<u4", hdr.n_upper * 32768).reshape(hdr.n_upper, 32768),
        lower=sec(hdr.off_lower, "<u4", hdr.n_lower * 4096).reshape(hdr.n_lower, 4096),
        block_first_leaf=sec(hdr.off_block_first_leaf, "<u4", nb),
        block_jump=sec(hdr.off_block_jump, "<u8", nb * (W // 64)).reshape(nb, W // 64),
    )


# ---------------------------------------------------------------------------
# device side
# ---------------------------------------------------------------------------

class Grid:
    """A built grid: its header and the blob resident in device memory."""

    def __init__(self, hdr: GridHeader, blob):
        self.hdr = hdr
        self.blob = blob  # torch.uint8 tensor on the device

    @property
    def n_active(self) -> int:
        return int(self.hdr.n_active)

    @property
    def n_leaves(self) -> int:
        return int(self.hdr.n_leaves)

    @property
    def n_blocks(self) -> int:
        return int(self.hdr.n_blocks)

    @property
    def log2_width(self) -> int:
        return int(self.hdr.log2_width)

    @property
    def width(self) -> int:
        return 1 << int(self.hdr.log2_width)

    @property
    def n_slots(self) -> int:
        return self.n_blocks * self.width


def build(coords: np.ndarray, log2_width: int, device="cuda") -> Grid:
    import torch
    hdr, host = build_host(coords, log2_width)
    blob = torch.from_numpy(host).to(device)
    return Grid(hdr, blob)


def build_device(coords, log2_width: int, device="cuda", stream=None) -> Grid:
    """vbm_build_device_*: build the grid on the GPU from coordinates (a torch int32
    [n, 3] tensor on the device, or anything numpy converts; copied to `device`).
    The workspace is a torch allocation released on return; the plan waits for the
    stream once (the blob's size depends on the data)."""
    import torch
    lib = load_library()
    c = coords if isinstance(coords, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(coords, np.int32))
    c = c.to(device=device, dtype=torch.int32).reshape(-1, 3).contiguous()
    dev = c.device
    if dev.type != "cuda":
        raise ValueError("build_device needs a GPU device, not %s" % dev)
    n = int(c.shape[0])
    need = ctypes.c_uint64()
    _check(lib.vbm_build_device_workspace(n, ctypes.byref(need)), "vbm_build_device_workspace")
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    hdr = GridHeader()
    sp = _stream_ptr(stream, dev)
    _check(lib.vbm_build_device_plan(_ptr(c), n, int(log2_width), _ptr(ws), need.value, ctypes.byref(hdr), sp),
           "vbm_build_device_plan")
    blob = torch.empty(int(hdr.blob_bytes), dtype=torch.uint8, device=dev)
    _check(lib.vbm_build_device_fill(ctypes.byref(hdr), n, _ptr(ws), need.value, _ptr(blob), sp),
           "vbm_build_device_fill")
    return Grid(hdr, blob)


def build_metadata(grid: Grid, stream=None):
    """vbm_build_metadata: recompute the leaf prefix directories and leafFirst and the
    block metadata of grid.blob on the device from its leaf masks; returns the total
    active count as a one-element int64 device tensor."""
    import torch
    dev = _device(grid)
    total = torch.zeros(1, dtype=torch.int64, device=dev)
    _check(load_library().vbm_build_metadata(ctypes.byref(grid.hdr), _blob_ptr(grid), _ptr(total),
                                             _stream_ptr(stream, dev)), "vbm_build_metadata")
    return total


def _device(grid: Grid):
    """The GPU holding the grid's blob.  Every pointer the C ABI receives must be
    device memory of that GPU: a host pointer handed to a kernel faults the GPU, so
    the binding refuses it here."""
    dev = grid.blob.device
    if dev.type != "cuda":
        raise ValueError("the grid's blob must be on a GPU (build(..., device='cuda')), not %s" % dev)
    return dev


def _on(t, dev, what: str):
    if t.device != dev:
        raise ValueError("%s must be on the grid's device %s, not %s" % (what, dev, t.device))


def _stream_ptr(stream, dev):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    if s.device != dev:
        raise ValueError("the stream must belong to the grid's device %s, not %s" % (dev, s.device))
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _blob_ptr(grid: Grid):
    return _ptr(grid.blob)


def decode(grid: Grid, stream=None, sweep: bool = False):
    """vbm_decode (or vbm_decode_sweep) -> (leafIndex as int32 tensor, voxelOffset as int16 tensor),
    n_blocks*W each (bit patterns of u32 / u16)."""
    import torch
    dev = _device(grid)
    leaf = torch.empty(grid.n_slots, dtype=torch.int32, device=dev)
    off = torch.empty(grid.n_slots, dtype=torch.int16, device=dev)
    lib = load_library()
    fn, name = (lib.vbm_decode_sweep, "vbm_decode_sweep") if sweep else (lib.vbm_decode, "vbm_decode")
    _check(fn(ctypes.byref(grid.hdr), _blob_ptr(grid), _ptr(leaf), _ptr(off), _stream_ptr(stream, dev)), name)
    return leaf, off


def decode_sweep(grid: Grid, stream=None):
    """vbm_decode_sweep: the same maps as decode(), by the sweep the select-based decode replaced."""
    return decode(grid, stream, sweep=True)


def stencil_indices(grid: Grid, shape: int, flags: int = 0, stream=None):
    """vbm_stencil_indices -> int64 tensor [n_blocks*W, shape] (u64 bit patterns)."""
    import torch
    dev = _device(grid)
    taps = torch.empty((grid.n_slots, shape), dtype=torch.int64, device=dev)
    _check(load_library().vbm_stencil_indices(ctypes.byref(grid.hdr), _blob_ptr(grid), int(shape), int(flags),
                                              _ptr(taps), _stream_ptr(stream, dev)), "vbm_stencil_indices")
    return taps


def _filter_out(grid: Grid, sidecar, out):
    """Validate the sidecar (and out) against the grid; returns (out, device)."""
    import torch
    dev = _device(grid)
    if sidecar.dtype != torch.float32 or sidecar.dim() != 2 or sidecar.shape[0] != grid.n_active + 1:
        raise ValueError("sidecar must be float32 [(N+1), C]")
    if not sidecar.is_contiguous():
        raise ValueError("sidecar must be contiguous")
    _on(sidecar, dev, "the sidecar")
    if out is None:
        out = torch.empty_like(sidecar)
    elif out.shape != sidecar.shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like the sidecar")
    _on(out, dev, "out")
    return out, dev


def box_filter(grid: Grid, sidecar, flags: int = CACHED | STREAMING, out=None, stream=None):
    """vbm_box_filter -> out float32 [(N+1), C]."""
    out, dev = _filter_out(grid, sidecar, out)
    _check(load_library().vbm_box_filter(ctypes.byref(grid.hdr), _blob_ptr(grid), _ptr(sidecar), _ptr(out),
                                         int(sidecar.shape[1]), int(flags), _stream_ptr(stream, dev)), "vbm_box_filter")
    return out


def cross_filter(grid: Grid, sidecar, flags: int = CACHED | OP_SUM, out=None, stream=None):
    """vbm_cross_filter -> out float32 [(N+1), C]."""
    out, dev = _filter_out(grid, sidecar, out)
    _check(load_library().vbm_cross_filter(ctypes.byref(grid.hdr), _blob_ptr(grid), _ptr(sidecar), _ptr(out),
                                           int(sidecar.shape[1]), int(flags), _stream_ptr(stream, dev)),
           "vbm_cross_filter")
    return out


def axis_filter(grid: Grid, sidecar, flags: int = CACHED | STREAMING, out=None, stream=None):
    """vbm_axis_filter (19-tap axis stencil sum) -> out float32 [(N+1), C]."""
    out, dev = _filter_out(grid, sidecar, out)
    _check(load_library().vbm_axis_filter(ctypes.byref(grid.hdr), _blob_ptr(grid), _ptr(sidecar), _ptr(out),
                                          int(sidecar.shape[1]), int(flags), _stream_ptr(stream, dev)), "vbm_axis_filter")
    return out


def weno_filter(grid: Grid, sidecar, flags: int = CACHED | STREAMING, out=None, stream=None):
    """vbm_weno_filter (fifth-order WENO |grad u|^2 on the 19 axis taps) -> out float32 [(N+1), C]."""
    out, dev = _filter_out(grid, sidecar, out)
    _check(load_library().vbm_weno_filter(ctypes.byref(grid.hdr), _blob_ptr(grid), _ptr(sidecar), _ptr(out),
                                          int(sidecar.shape[1]), int(flags), _stream_ptr(stream, dev)), "vbm_weno_filter")
    return out
