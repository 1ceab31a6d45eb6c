"""Pins of the oracle's WENO consumer (CPU only).

The pages name a 19-tap WENO consumer but not its arithmetic; the oracle
reads it as fifth-order WENO one-sided derivatives (Jiang and Shu, J. Comput.
Phys. 126, 1996) on the axis taps, combined by Godunov's upwind rule into the
squared gradient norm per channel, inactive taps reading sidecar row 0.  None
of these checks re-types that code path: they use what the mathematics fixes.

* closed forms of one WENO derivative: constant differences (a linear field)
  and differences of a quadratic give the exact derivative (every candidate
  is exact for quadratics); a jump on one side gives a derivative of order
  epsilon-squared from the smooth side (the ENO property), far from the
  ideal-weight value; an isolated spike has smoothness indicators 10/3, 10 and
  22 times c^2, whose weights give a value worked out by hand in fp64;
* a quadratic field with a different curvature per axis on a dense grid: the
  result is |grad u|^2 of the polynomial at every voxel at least 3 voxels
  inside the grid;
* mirror symmetry: reflecting the grid along any axis maps every output to the
  mirrored voxel's output bit for bit (the right-biased derivative is the
  left-biased one of the reflected field, negated);
* an isolated voxel on a nonzero background: every tap but the centre reads
  row 0, and the result follows from the spike closed form;
* brute force: a separate fp64 numpy evaluation on a dense array with the
  background outside the active set agrees to fp32 accuracy.
"""
import numpy as np
import pytest

import oracle
from nanovdb_stencil_filtering_amd import inputs as I

U = 2.0 ** -24  # unit roundoff of fp32


def test_linear_field_is_exact():
    for k in (1.0, -3.0, 0.5, 7.25, 1e-3):
        r = oracle.weno5(k, k, k, k, k)
        assert abs(r - k) <= 3 * U * abs(k), (k, r)


def test_quadratic_differences_give_the_exact_derivative():
    # u(x) = x^2 + s x: differences around x0 are u(x0+k) - u(x0+k-1) = 2(x0+k) - 1 + s
    for x0 in (-5, -1, 0, 2, 9):
        for s in (0.0, 3.0, -7.0):
            d = [2.0 * (x0 + k) - 1.0 + s for k in (-2, -1, 0, 1, 2)]
            exact = 2.0 * x0 + s
            left = oracle.weno5(*d)
            dr = [2.0 * (x0 + k) - 1.0 + s for k in (3, 2, 1, 0, -1)]
            right = oracle.weno5(*dr)
            for r in (left, right):
                assert abs(r - exact) <= 4 * U * abs(exact), (x0, s, r, exact)


def test_jump_is_ignored_by_the_smooth_side():
    # the jump sits in the last (first) difference only: the two other candidates see a
    # flat field, so the result is O(eps^2), while the ideal weights would give -0.05
    ideal = 0.3 * ((2 * 0 + 5 * 0) - 1) / 6
    assert abs(ideal + 0.05) < 1e-12
    assert abs(oracle.weno5(0, 0, 0, 0, 1)) < 1e-11
    assert abs(oracle.weno5(1, 0, 0, 0, 0)) < 1e-11
    assert abs(oracle.weno5(0, 0, 0, 0, -2)) < 1e-11


def spike_value(c):
    """weno5(0, 0, c, -c, 0) from its closed form: candidates 11c/6, c/2, -c/2;
    smoothness indicators 10/3 c^2, 10 c^2, 22 c^2; weights 1, 6, 3 over (s + eps)^2."""
    eps = 1e-6
    p = np.array([11 * c / 6, c / 2, -c / 2])
    s = np.array([10 / 3, 10, 22]) * c * c
    a = np.array([1, 6, 3]) / (s + eps) ** 2
    return float((a * p).sum() / a.sum())


def test_spike_closed_form():
    for c in (1.0, -0.5, 2.0, 0.125):
        r = oracle.weno5(0.0, 0.0, c, -c, 0.0)
        assert abs(r - spike_value(c)) <= 1e-6 * abs(spike_value(c)), (c, r, spike_value(c))


def dense_cube(n, lo=0):
    ax = np.arange(lo, lo + n)
    return np.stack(np.meshgrid(ax, ax, ax, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)


def test_quadratic_field_on_a_dense_grid():
    c = dense_cube(14, -4)
    ref = oracle.OracleGrid(c)
    vox = ref.voxels().astype(np.float64)
    x, y, z = vox[:, 0], vox[:, 1], vox[:, 2]
    # exact in fp32: integer values below 2^24
    u = x * x + 2 * y * y - 3 * z * z + 5 * x - y + 7 * z + 1
    sc = np.zeros((ref.n_active + 1, 1), np.float32)
    sc[1:, 0] = u
    out = ref.weno(sc)[1:, 0].astype(np.float64)
    grad2 = (2 * x + 5) ** 2 + (4 * y - 1) ** 2 + (-6 * z + 7) ** 2
    inner = ((vox >= -4 + 3) & (vox <= 9 - 3)).all(axis=1)
    assert inner.sum() == 8 ** 3
    err = np.abs(out[inner] - grad2[inner])
    assert np.all(err <= 16 * U * grad2[inner] + 1e-30), err.max()


def test_mirror_symmetry_bit_exact():
    c = I.random_sparse_coords(11, (12, 12, 12), 0.8, (-6, 3, -9)).astype(np.int64)
    ref = oracle.OracleGrid(c.astype(np.int32))
    C = 3
    rng = np.random.default_rng(5)
    vox = ref.voxels().astype(np.int64)
    vals = rng.uniform(-1, 1, size=(ref.n_active, C)).astype(np.float32)
    sc = np.zeros((ref.n_active + 1, C), np.float32)
    sc[0] = 0.375  # background
    sc[1:] = vals
    out = ref.weno(sc)
    by_coord = {tuple(p): out[i + 1] for i, p in enumerate(vox.tolist())}
    for axis in range(3):
        m = vox.copy()
        m[:, axis] = -m[:, axis]
        mref = oracle.OracleGrid(m.astype(np.int32))
        mvox = mref.voxels().astype(np.int64)
        # carry each voxel's values to its mirror image
        lookup = {tuple(p): vals[i] for i, p in enumerate(m.tolist())}
        msc = np.zeros_like(sc)
        msc[0] = sc[0]
        msc[1:] = np.array([lookup[tuple(p)] for p in mvox.tolist()], np.float32)
        mout = mref.weno(msc)
        for i, p in enumerate(mvox.tolist()):
            q = list(p)
            q[axis] = -q[axis]
            assert np.array_equal(mout[i + 1].view(np.uint32), by_coord[tuple(q)].view(np.uint32)), (axis, p)


def test_isolated_voxel_reads_the_background():
    c = np.array([[3, -2, 40]], np.int32)
    ref = oracle.OracleGrid(c)
    for bg, v in ((0.0, 1.0), (0.5, 1.5), (-1.0, 1.0), (2.0, -0.25)):
        sc = np.array([[bg], [v]], np.float32)
        out = float(ref.weno(sc)[1, 0])
        cdiff = v - bg                       # u[0] - u[-1]; u[1] - u[0] = -cdiff
        dm = spike_value(cdiff)              # weno5(0, 0, c, -c, 0)
        dp = spike_value(-cdiff)             # weno5(0, 0, -c, c, 0): the mirror image
        if v > 0:
            g = max(max(dm, 0) ** 2, min(dp, 0) ** 2)
        else:
            g = max(min(dm, 0) ** 2, max(dp, 0) ** 2)
        assert abs(out - 3 * g) <= 1e-5 * abs(3 * g) + 1e-30, (bg, v, out, 3 * g)


def weno5_f64(a, b, c, d, e):
    """Jiang-Shu fifth-order WENO in fp64 (vectorised)."""
    eps = 1e-6
    p1 = (2 * a - 7 * b + 11 * c) / 6
    p2 = (-b + 5 * c + 2 * d) / 6
    p3 = (2 * c + 5 * d - e) / 6
    s1 = 13 / 12 * (a - 2 * b + c) ** 2 + 0.25 * (a - 4 * b + 3 * c) ** 2
    s2 = 13 / 12 * (b - 2 * c + d) ** 2 + 0.25 * (b - d) ** 2
    s3 = 13 / 12 * (c - 2 * d + e) ** 2 + 0.25 * (3 * c - 4 * d + e) ** 2
    w1, w2, w3 = 0.1 / (s1 + eps) ** 2, 0.6 / (s2 + eps) ** 2, 0.3 / (s3 + eps) ** 2
    return (w1 * p1 + w2 * p2 + w3 * p3) / (w1 + w2 + w3)


def test_brute_force_fp64_on_a_dense_array():
    c = I.random_sparse_coords(12, (14, 13, 15), 0.7, (5, -7, 2))
    ref = oracle.OracleGrid(c)
    vox = ref.voxels()
    C = 2
    sc = I.sidecar(61, ref.n_active, C).astype(np.float32)
    sc[0] = (-0.75, 0.25)  # background row
    out = ref.weno(sc)[1:].astype(np.float64)
    lo = vox.min(0) - 3
    shape = vox.max(0) - lo + 4
    for ch in range(C):
        dense = np.full(shape, float(sc[0, ch]))
        dense[tuple((vox - lo).T)] = sc[1:, ch]
        p = vox - lo
        total = np.zeros(len(vox))
        centre = dense[tuple(p.T)]
        for axis in range(3):
            u = []
            for k in range(-3, 4):
                q = p.copy()
                q[:, axis] += k
                u.append(dense[tuple(q.T)])
            d = [u[j + 1] - u[j] for j in range(6)]
            dm = weno5_f64(d[0], d[1], d[2], d[3], d[4])
            dp = weno5_f64(d[5], d[4], d[3], d[2], d[1])
            g_out = np.maximum(np.maximum(dm, 0) ** 2, np.minimum(dp, 0) ** 2)
            g_in = np.maximum(np.minimum(dm, 0) ** 2, np.maximum(dp, 0) ** 2)
            total += np.where(centre > 0, g_out, g_in)
        err = np.abs(out[:, ch] - total)
        assert np.all(err <= 1e-4 * (1.0 + np.abs(total))), err.max()


@pytest.mark.parametrize("C", [1, 4])
def test_rows_match_the_whole_grid(C):
    ref = oracle.OracleGrid(I.shell_coords(**I.TINY_SHELL))
    sc = I.sidecar(62, ref.n_active, C)
    whole = ref.weno(sc)
    idx = np.array([1, 7, ref.n_active // 2, ref.n_active], np.uint64)
    assert np.array_equal(ref.weno(sc, idx).view(np.uint32), whole[idx.astype(np.int64)].view(np.uint32))
    assert np.all(whole[0] == 0)
