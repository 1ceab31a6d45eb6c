"""The oracle against brute force on small grids (no GPU).

Every quantity is recomputed by a second, independent route:
* indices: Python integer floor division/modulo and Python's tuple sort;
* taps: a dense 3-D array of indices, shifted per tap (no hash map);
* decode: rank by binary search on leafFirst and select by enumerating mask bits
  (the oracle sweeps instead);
* blocks: leaf starts found by searching leafFirst;
* filters: numpy float32 sequential sums over the dense-array taps.
Grids straddle leaf, lower-node (128) and root-tile (4096) boundaries and use
negative coordinates.
"""
import numpy as np
import pytest

import oracle
from nanovdb_stencil_filtering_amd import inputs as I

CASES = [
    # seed, extent, density, offset
    (1, (24, 24, 24), 0.05, (0, 0, 0)),
    (2, (20, 26, 22), 0.3, (-13, -5, 117)),        # y negative, z straddles 128
    (3, (18, 18, 18), 0.9, (4087, -9, -4100)),    # x straddles 4096, z straddles -4096
    (4, (16, 16, 16), 1.0, (-8, -8, -8)),
    (5, (30, 12, 30), 0.15, (120, 250, -140)),
]


def brute_index(coords):
    pts = sorted(set(map(tuple, coords.tolist())),
                 key=lambda p: (p[0] // 4096, p[1] // 4096, p[2] // 4096,
                                (p[0] % 4096) // 128, (p[1] % 4096) // 128, (p[2] % 4096) // 128,
                                (p[0] % 128) // 8, (p[1] % 128) // 8, (p[2] % 128) // 8,
                                p[0] % 8, p[1] % 8, p[2] % 8))
    return np.array(pts, dtype=np.int64).reshape(-1, 3)


def brute_leaves(vox):
    leaf_keys = [(x // 8, y // 8, z // 8) for x, y, z in vox.tolist()]
    origin, first, mask = [], [], []
    for i, k in enumerate(leaf_keys):
        if not origin or origin[-1] != k:
            origin.append(k)
            first.append(i + 1)
            mask.append([0] * 512)
        x, y, z = vox[i]
        mask[-1][(x % 8) * 64 + (y % 8) * 8 + (z % 8)] = 1
    return np.array(origin) * 8, np.array(first, np.int64), np.array(mask, np.uint8)


def dense_taps(vox, N):
    lo = vox.min(axis=0) - 1
    hi = vox.max(axis=0) + 1
    D = np.zeros(tuple(hi - lo + 1), np.uint64)
    rel = vox - lo
    D[rel[:, 0], rel[:, 1], rel[:, 2]] = np.arange(1, N + 1, dtype=np.uint64)
    taps = np.zeros((N, 27), np.uint64)
    t = 0
    for di in (-1, 0, 1):
        for dj in (-1, 0, 1):
            for dk in (-1, 0, 1):
                taps[:, t] = D[rel[:, 0] + di, rel[:, 1] + dj, rel[:, 2] + dk]
                t += 1
    return taps


@pytest.fixture(scope="module", params=CASES, ids=lambda c: "seed%d" % c[0])
def case(request):
    seed, extent, density, offset = request.param
    coords = I.random_sparse_coords(seed, extent, density, offset)
    g = oracle.OracleGrid(I.shuffled(coords, seed + 100))
    vox = brute_index(coords)
    return g, vox


def test_indices(case):
    g, vox = case
    assert g.n_active == vox.shape[0]
    assert np.array_equal(g.voxels().astype(np.int64), vox)


def test_leaves(case):
    g, vox = case
    origin, first, mask = brute_leaves(vox)
    lv = g.leaves()
    assert np.array_equal(lv["origin"], origin)
    assert np.array_equal(lv["first"].astype(np.int64), first)
    bits = np.unpackbits(lv["mask"].view(np.uint8).reshape(-1, 8, 8), axis=2, bitorder="little")
    assert np.array_equal(bits.reshape(-1, 512), mask)
    words = mask.reshape(-1, 8, 64).sum(axis=2).cumsum(axis=1)
    for k in range(7):
        assert np.array_equal((lv["prefix"] >> np.uint64(9 * k)) & np.uint64(511), words[:, k].astype(np.uint64))


@pytest.mark.parametrize("log2w", [6, 7, 8, 9])
def test_blocks_and_decode(case, log2w):
    g, vox = case
    N = g.n_active
    W = 1 << log2w
    origin, first, mask = brute_leaves(vox)
    nb = -(-N // W)
    b = g.blocks(log2w)
    assert b["first_leaf"].shape == (nb,)
    leaf_of = np.searchsorted(first, np.arange(1, N + 1), side="right") - 1
    assert np.array_equal(b["first_leaf"], leaf_of[np.arange(nb) * W])
    starts = set(first.tolist())
    for blk in range(nb):
        bits = [(s >= 1 and 1 + blk * W + s <= N and (1 + blk * W + s) in starts) for s in range(W)]
        words = [sum(1 << j for j in range(64) if bits[64 * k + j]) for k in range(W // 64)]
        assert [int(x) for x in b["jump"][blk]] == words
    leaf, off = g.decode(log2w)
    # select by definition: the r-th set bit of the owning leaf's mask
    for gidx in range(1, N + 1):
        l = leaf_of[gidx - 1]
        r = gidx - first[l]
        assert leaf[gidx - 1] == l
        assert off[gidx - 1] == np.nonzero(mask[l])[0][r]
    assert np.all(leaf[N:] == 0xFFFFFFFF) and np.all(off[N:] == 0xFFFF)
    assert leaf.size == nb * W


def test_taps(case):
    g, vox = case
    taps = dense_taps(vox, g.n_active)
    assert np.array_equal(g.taps(27), taps)
    assert np.array_equal(g.taps(7), taps[:, [4, 10, 12, 13, 14, 16, 22]])
    assert np.array_equal(taps[:, 13], np.arange(1, g.n_active + 1, dtype=np.uint64))


@pytest.mark.parametrize("C", [1, 3])
def test_filters(case, C):
    g, vox = case
    N = g.n_active
    taps = dense_taps(vox, N).astype(np.int64)
    sc = I.sidecar(40 + C, N, C)
    box = np.zeros((N, C), np.float32)
    for t in range(27):
        act = taps[:, t] != 0
        box[act] = box[act] + sc[taps[act, t]]
    assert np.array_equal(g.box(sc)[1:], box)
    assert np.all(g.box(sc)[0] == 0)
    cross_t = [4, 10, 12, 13, 14, 16, 22]
    cs = np.zeros((N, C), np.float32)
    lap = np.zeros((N, C), np.float32)
    for t in cross_t:
        act = taps[:, t] != 0
        cs[act] = cs[act] + sc[taps[act, t]]
        if t != 13:
            lap[act] = lap[act] + sc[taps[act, t]]
    lap = lap - np.float32(6.0) * sc[1:]
    assert np.array_equal(g.cross(sc, "sum")[1:], cs)
    assert np.array_equal(g.cross(sc, "laplacian")[1:], lap)
