"""Seeded synthetic inputs for the VBM stencil pipeline.

This module only *generates inputs*: sets of integer voxel coordinates and
interleaved fp32 sidecar channels.  It contains none of the method's
arithmetic (no leaves, masks, indices, blocks or stencils), so both the HIP
path and the CPU oracle may consume what it produces.

The workloads stand in for the pages' scenes, which are not available:

* sphere shells -- openvdb PR #2263, "Measurements" (a sparse sphere shell of
  about 1.29M active voxels in 9140 leaves); a shell of radius R and half
  thickness h is every integer point p with | ||p|| - R | <= h;
* a decode-stress topology of random leaves with Bernoulli value masks of
  mixed density -- openvdb PR #2258 measures decode on real scenes whose leaf
  occupancy varies; this mixes the densities explicitly;
* a noisy narrow band around a sphere (a level-set band);
* sidecar channels uniform in [-1, 1) from a counter-based generator.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): the k-th output of a stream
with seed s is mix(s + (k + 1) * 0x9E3779B97F4A7C15) where mix is the
published 64-bit finaliser.
"""
from __future__ import annotations

import os

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """Outputs number ``counters`` (0-based) of the SplitMix64 stream ``seed``."""
    c = np.ascontiguousarray(counters, dtype=np.uint64).ravel()
    out = np.empty_like(c)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    step = 1 << 18
    with np.errstate(over="ignore"):
        for a in range(0, c.size, step):
            z = c[a:a + step] + np.uint64(1)
            z *= _GAMMA
            z += s
            t = z >> np.uint64(30)
            z ^= t
            z *= _M1
            np.right_shift(z, np.uint64(27), out=t)
            z ^= t
            z *= _M2
            np.right_shift(z, np.uint64(31), out=t)
            z ^= t
            out[a:a + step] = z
    return out.reshape(np.shape(counters))


def _uniform_pm1_f32(bits: np.ndarray) -> np.ndarray:
    """Top 24 bits of a 64-bit word -> exactly representable float32 in [-1, 1)."""
    top = (bits >> np.uint64(40)).astype(np.int64) - (1 << 23)
    return (top.astype(np.float64) / float(1 << 23)).astype(np.float32)


def sidecar(seed: int, n_active: int, channels: int) -> np.ndarray:
    """Interleaved sidecar, shape ((n_active + 1), channels), float32.

    Row 0 belongs to index 0 (inactive) and is zero; row i >= 1 holds the
    channels of active index i.  Element (i, ch) is counter i*channels + ch.
    """
    rows = n_active + 1
    k = np.arange(rows * channels, dtype=np.uint64)
    v = _uniform_pm1_f32(splitmix64(seed, k)).reshape(rows, channels)
    v[0, :] = 0.0
    return v


def sidecar_rows(seed: int, row0: int, row1: int, channels: int) -> np.ndarray:
    """Rows row0 .. row1-1 of ``sidecar(seed, n, channels)`` (same values), so a
    large sidecar can be produced a slice at a time."""
    k = np.arange(row0 * channels, row1 * channels, dtype=np.uint64)
    v = _uniform_pm1_f32(splitmix64(seed, k)).reshape(row1 - row0, channels)
    if row0 == 0:
        v[0, :] = 0.0
    return v


def sidecar_at(seed: int, rows: np.ndarray, channels: int) -> np.ndarray:
    """The given rows (any order) of ``sidecar(seed, n, channels)``, same values,
    so that a few rows of a sidecar too large to hold can be produced alone."""
    rows = np.asarray(rows, dtype=np.uint64).ravel()
    k = (rows[:, None] * np.uint64(channels) + np.arange(channels, dtype=np.uint64)[None, :]).ravel()
    v = _uniform_pm1_f32(splitmix64(seed, k)).reshape(rows.size, channels)
    v[rows == 0] = 0.0
    return v


def wide_range_sidecar(seed: int, n_active: int, channels: int, fraction: float = 0.01) -> np.ndarray:
    """A sidecar like ``sidecar`` in which a share ``fraction`` of the elements,
    picked one by one, are drawn from the rest of the finite fp32 range instead
    of [-1, 1), in six equally likely kinds: signed zeros, subnormals, normals
    from 1e-37 to 1e-12, the magnitudes 2^-41, 2^-40, 2^-39, 2^44, 2^45, 2^46 and
    the neighbours of 2^-40 and 2^45, large ones (4e13 .. 1e18), and huge ones
    (1e19 .. 1e38, whose squares overflow).  Row 0 (the background) keeps the
    ordinary value of each channel."""
    rows = n_active + 1
    n = rows * channels
    bits = splitmix64(seed, np.arange(4 * n, dtype=np.uint64)).reshape(4, n)
    ordinary = _uniform_pm1_f32(bits[0])
    u = (bits[1] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53       # kind
    w = (bits[2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53       # magnitude
    sign = np.where((bits[3] & np.uint64(1)) != 0, -1.0, 1.0)
    pick = ((bits[3] >> np.uint64(1)) % np.uint64(8)).astype(np.int64)
    edges = np.array([2.0 ** -40, float(np.nextafter(np.float32(2.0 ** -40), np.float32(0))), 2.0 ** 45,
                      float(np.nextafter(np.float32(2.0 ** 45), np.float32(np.inf))), 2.0 ** -41, 2.0 ** 46,
                      2.0 ** -39, 2.0 ** 44])
    kinds = [0.0 * sign,
             sign * w * 2.0 ** -126,                 # subnormal after rounding to fp32
             sign * 10.0 ** (-37 + 25 * w),          # 1e-37 .. 1e-12
             sign * edges[pick],
             sign * 10.0 ** (13.6 + 4.4 * w),        # 4e13 .. 1e18
             sign * 10.0 ** (19 + 19 * w)]           # 1e19 .. 1e38
    v = ordinary.astype(np.float64)
    for k, val in enumerate(kinds):
        sel = (u >= fraction * k / len(kinds)) & (u < fraction * (k + 1) / len(kinds))
        v = np.where(sel, val, v)
    out = v.astype(np.float32).reshape(rows, channels)
    out[0] = ordinary.reshape(rows, channels)[0]
    return out


def shell_coords(radius: float, half_thickness: float) -> np.ndarray:
    """All integer points p with | ||p|| - radius | <= half_thickness, centred on the origin.

    Evaluated exactly on squared norms: (R-h)^2 <= x^2+y^2+z^2 <= (R+h)^2
    (both bounds are exact in float64 for the radii used here).  Returns
    int32 [N, 3] in x-major, then y, then z ascending order.
    """
    r_in = radius - half_thickness
    r_out = radius + half_thickness
    assert r_in >= 0
    lo2 = r_in * r_in
    hi2 = r_out * r_out
    ext = int(np.floor(r_out))
    ax = np.arange(-ext, ext + 1, dtype=np.int64)
    out = []
    yy, zz = np.meshgrid(ax, ax, indexing="ij")
    yz2 = (yy * yy + zz * zz).ravel()
    y_flat = yy.ravel()
    z_flat = zz.ravel()
    for x in ax:
        r2 = yz2 + x * x
        sel = (r2 >= lo2) & (r2 <= hi2)
        n = int(sel.sum())
        if n:
            blk = np.empty((n, 3), dtype=np.int32)
            blk[:, 0] = x
            blk[:, 1] = y_flat[sel]
            blk[:, 2] = z_flat[sel]
            out.append(blk)
    return np.concatenate(out, axis=0) if out else np.zeros((0, 3), np.int32)


def random_sparse_coords(seed: int, extent: tuple[int, int, int], density: float,
                         offset: tuple[int, int, int] = (0, 0, 0)) -> np.ndarray:
    """Each point of the box offset + [0, extent) active with probability ``density``."""
    ex, ey, ez = extent
    k = np.arange(ex * ey * ez, dtype=np.uint64)
    u = (splitmix64(seed, k) >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    sel = np.nonzero(u < density)[0]
    x = sel // (ey * ez)
    y = (sel // ez) % ey
    z = sel % ez
    c = np.stack([x + offset[0], y + offset[1], z + offset[2]], axis=1)
    return c.astype(np.int32)


def leaf_bernoulli_coords(seed: int, n_leaves: int, domain_leaves: int,
                          probabilities: tuple[float, ...], leaf_edge: int = 8) -> np.ndarray:
    """Decode-stress topology: ``n_leaves`` distinct cells of edge ``leaf_edge`` at
    random positions of a ``domain_leaves``^3 lattice; in each cell every point is
    active independently with a probability drawn per cell from ``probabilities``.
    A cell whose draw comes out empty is drawn again (same probability, next
    counter block), so exactly ``n_leaves`` cells are non-empty.
    """
    d = domain_leaves
    total = d * d * d
    # distinct cells: order all lattice cells by a random key, keep the first n
    keys = splitmix64(seed, np.arange(total, dtype=np.uint64))
    cells = np.argsort(keys, kind="stable")[:n_leaves].astype(np.int64)
    cx, cy, cz = cells // (d * d), (cells // d) % d, cells % d
    pick = splitmix64(seed ^ 0x5EED, np.arange(n_leaves, dtype=np.uint64)) % np.uint64(len(probabilities))
    p = np.asarray(probabilities, dtype=np.float64)[pick.astype(np.int64)]
    per = leaf_edge ** 3
    out = []
    stream = seed ^ 0xB17
    attempt = np.zeros(n_leaves, dtype=np.int64)
    todo = np.arange(n_leaves)
    masks = np.zeros((n_leaves, per), dtype=bool)
    while todo.size:
        ctr = ((attempt[todo] * n_leaves + todo)[:, None] * per + np.arange(per)[None, :]).astype(np.uint64)
        u = (splitmix64(stream, ctr.ravel()) >> np.uint64(11)).astype(np.float64) / float(1 << 53)
        m = (u.reshape(todo.size, per) < p[todo, None])
        masks[todo] = m
        empty = ~m.any(axis=1)
        attempt[todo[empty]] += 1
        todo = todo[empty]
    li, lo = np.nonzero(masks)
    lx, ly, lz = lo // (leaf_edge * leaf_edge), (lo // leaf_edge) % leaf_edge, lo % leaf_edge
    out = np.stack([cx[li] * leaf_edge + lx, cy[li] * leaf_edge + ly, cz[li] * leaf_edge + lz], axis=1)
    return out.astype(np.int32)


def one_per_cell_coords(seed: int, n_cells_per_axis: int, cell_edge: int = 8) -> np.ndarray:
    """One active point at a random position inside each cell of an
    n^3 lattice of cells of edge ``cell_edge`` (a maximally sparse topology)."""
    n = n_cells_per_axis
    c = np.arange(n * n * n, dtype=np.int64)
    cx, cy, cz = c // (n * n), (c // n) % n, c % n
    r = (splitmix64(seed, c.astype(np.uint64)) % np.uint64(cell_edge ** 3)).astype(np.int64)
    out = np.stack([cx * cell_edge + r // (cell_edge * cell_edge),
                    cy * cell_edge + (r // cell_edge) % cell_edge,
                    cz * cell_edge + r % cell_edge], axis=1)
    return out.astype(np.int32)


# --------------------------------------------------------------------------
# noisy narrow band
# --------------------------------------------------------------------------

def _lattice_values(seed: int, octave: int, ix: np.ndarray, iy: np.ndarray, iz: np.ndarray) -> np.ndarray:
    """Lattice value in [-1, 1) for integer lattice points (seeded, per octave)."""
    m21 = np.int64((1 << 21) - 1)
    k = (((ix & m21) << 42) | ((iy & m21) << 21) | (iz & m21)).astype(np.uint64)
    bits = splitmix64((seed * 1000003 + octave * 7919) & 0xFFFFFFFFFFFFFFFF, k)
    return ((bits >> np.uint64(11)).astype(np.float64) / float(1 << 52)) - 1.0


def value_noise(seed: int, p: np.ndarray, wavelengths=(128.0, 64.0, 32.0),
                amplitudes=None, total_amplitude: float = 20.0) -> np.ndarray:
    """Multi-octave value noise at points p (float64 [M,3]): per octave, lattice
    values interpolated trilinearly with smoothstep weights, summed with
    amplitudes total_amplitude * (4, 2, 1) / 7 for three octaves."""
    if amplitudes is None:
        amplitudes = _octave_amplitudes(len(wavelengths), total_amplitude)
    n = np.zeros(p.shape[0], dtype=np.float64)
    for o, (lam, amp) in enumerate(zip(wavelengths, amplitudes)):
        u = p / lam
        i0 = np.floor(u).astype(np.int64)
        f = u - i0
        s = f * f * (3.0 - 2.0 * f)
        acc = np.zeros(p.shape[0], dtype=np.float64)
        for cx in (0, 1):
            wx = s[:, 0] if cx else 1.0 - s[:, 0]
            for cy in (0, 1):
                wy = s[:, 1] if cy else 1.0 - s[:, 1]
                for cz in (0, 1):
                    wz = s[:, 2] if cz else 1.0 - s[:, 2]
                    acc += wx * wy * wz * _lattice_values(seed, o, i0[:, 0] + cx, i0[:, 1] + cy, i0[:, 2] + cz)
        n += amp * acc
    return n


def _octave_amplitudes(n_octaves: int, total_amplitude: float):
    w = np.array([2.0 ** (n_octaves - 1 - i) for i in range(n_octaves)])
    return total_amplitude * w / w.sum()


class _LatticeNoise:
    """value_noise with each octave's lattice values tabulated once over a box.

    Same lattice values and the same float64 operations in the same order as
    ``value_noise``, so the results are identical (a CPU test checks this)."""

    def __init__(self, seed, lo, hi, wavelengths=(128.0, 64.0, 32.0), total_amplitude=20.0):
        self.wavelengths = wavelengths
        self.amplitudes = _octave_amplitudes(len(wavelengths), total_amplitude)
        self.tables = []
        for o, lam in enumerate(wavelengths):
            i_lo = int(np.floor(lo / lam)) - 1
            i_hi = int(np.floor(hi / lam)) + 2
            ax = np.arange(i_lo, i_hi + 1, dtype=np.int64)
            ix, iy, iz = np.meshgrid(ax, ax, ax, indexing="ij")
            vals = _lattice_values(seed, o, ix.ravel(), iy.ravel(), iz.ravel()).reshape(ix.shape)
            self.tables.append((i_lo, vals))

    def __call__(self, p):
        n = np.zeros(p.shape[0], dtype=np.float64)
        for (lam, amp, (i_lo, tab)) in zip(self.wavelengths, self.amplitudes, self.tables):
            u = p / lam
            i0 = np.floor(u).astype(np.int64)
            f = u - i0
            s = f * f * (3.0 - 2.0 * f)
            j = i0 - i_lo
            acc = np.zeros(p.shape[0], dtype=np.float64)
            for cx in (0, 1):
                wx = s[:, 0] if cx else 1.0 - s[:, 0]
                for cy in (0, 1):
                    wy = s[:, 1] if cy else 1.0 - s[:, 1]
                    for cz in (0, 1):
                        wz = s[:, 2] if cz else 1.0 - s[:, 2]
                        acc += wx * wy * wz * tab[j[:, 0] + cx, j[:, 1] + cy, j[:, 2] + cz]
            n += amp * acc
        return n


def _band_slab(args):
    seed, radius, half_width, amplitude, xs = args
    reach = amplitude + half_width
    r_in, r_out = radius - reach, radius + reach
    ext = int(np.ceil(r_out))
    noise = _LatticeNoise(seed, -ext, ext, total_amplitude=amplitude)
    ax = np.arange(-ext, ext + 1, dtype=np.int64)
    yy, zz = np.meshgrid(ax, ax, indexing="ij")
    y_flat, z_flat = yy.ravel(), zz.ravel()
    yz2 = y_flat * y_flat + z_flat * z_flat
    out = []
    for x in xs:
        r2 = yz2 + x * x
        cand = np.nonzero((r2 >= r_in * r_in) & (r2 <= r_out * r_out))[0]
        if cand.size == 0:
            continue
        p = np.empty((cand.size, 3), dtype=np.float64)
        p[:, 0] = x
        p[:, 1] = y_flat[cand]
        p[:, 2] = z_flat[cand]
        d = np.sqrt(r2[cand].astype(np.float64)) - (radius + noise(p))
        keep = np.abs(d) <= half_width
        if keep.any():
            out.append(p[keep].astype(np.int32))
    return np.concatenate(out, axis=0) if out else np.zeros((0, 3), np.int32)


def band_coords(seed: int, radius: float = 600.0, half_width: float = 3.0,
                amplitude: float = 20.0, workers: int | None = None) -> np.ndarray:
    """Narrow band |d(p)| <= half_width with d(p) = ||p|| - (radius + noise(p)),
    noise = 3-octave value noise of total amplitude ``amplitude`` (wavelengths
    128, 64, 32; amplitudes in ratio 4:2:1).  Slabs of constant x are
    evaluated in parallel processes; the result is in x-major order."""
    import multiprocessing as mp
    ext = int(np.ceil(radius + amplitude + half_width))
    xs = np.arange(-ext, ext + 1, dtype=np.int64)
    if workers is None:
        workers = max(1, min(16, (os.cpu_count() or 1)))
    n_chunks = max(1, workers * 4)
    bounds = np.linspace(0, xs.size, n_chunks + 1).astype(int)
    chunks = [xs[bounds[i]:bounds[i + 1]] for i in range(n_chunks) if bounds[i + 1] > bounds[i]]
    args = [(seed, radius, half_width, amplitude, c) for c in chunks]
    if workers == 1:
        parts = [_band_slab(a) for a in args]
    else:
        with mp.get_context("fork").Pool(workers) as pool:
            parts = pool.map(_band_slab, args)
    return np.concatenate(parts, axis=0)


def shuffled(coords: np.ndarray, seed: int) -> np.ndarray:
    """The same coordinate set in a seeded random order (inputs are sets)."""
    keys = splitmix64(seed, np.arange(coords.shape[0], dtype=np.uint64))
    return coords[np.argsort(keys, kind="stable")]


# Named workloads ----------------------------------------------------------

TINY_SHELL = dict(radius=16.0, half_thickness=1.0)          # ~6.5K voxels
CFG_SHELL = dict(radius=185.0, half_thickness=1.5)          # ~1.29M voxels
PAGES_SHELL = dict(radius=160.0, half_thickness=2.0)        # 1.29M voxels / 9140 leaves
STRESS = dict(n_leaves=20000, domain_leaves=64, probabilities=(0.02, 0.1, 0.5, 1.0))
BAND = dict(radius=600.0, half_width=3.0, amplitude=20.0)
