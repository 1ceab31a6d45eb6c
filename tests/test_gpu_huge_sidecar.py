"""A sidecar past 4 GiB on the GPU: (N+1) * C * 4 bytes beyond the 32-bit
offsets of the buffer-resource path, which every filter then leaves for 64-bit
row addresses by itself.  The cfg-shell (1,290,538 voxels) with C = 836
channels (4.32 GB each way): sampled rows -- the first, random ones and the
last 800, whose rows and most of whose taps lie past the 4 GiB mark -- of every
filter against the oracle, bit for bit.  The oracle reads only the rows it
needs, from a zero-filled host array into which exactly those rows are
generated."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from nanovdb_stencil_filtering_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from nanovdb_stencil_filtering_amd import vbm  # noqa: E402

C = 836
SEED = 83


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def huge():
    coords = I.shell_coords(**I.CFG_SHELL)
    g = vbm.build(coords, 7)
    ref = oracle.OracleGrid(coords)
    N = g.n_active
    assert (N + 1) * C * 4 > 0xFFFFFF00
    say("huge sidecar: N=%d C=%d, %.2f GB each way" % (N, C, (N + 1) * C * 4 / 1e9))
    sc = torch.empty((N + 1, C), dtype=torch.float32, device="cuda")
    step = 1 << 15
    chunks = [(a, min(N + 1, a + step)) for a in range(0, N + 1, step)]
    with ThreadPoolExecutor(8) as pool:
        for (a, b), rows in zip(chunks, pool.map(lambda ab: I.sidecar_rows(SEED, ab[0], ab[1], C), chunks)):
            sc[a:b].copy_(torch.from_numpy(rows))
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([np.arange(1, 201), rng.integers(1, N + 1, 1500),
                                       np.arange(N - 799, N + 1)])).astype(np.uint64)
    need = np.unique(np.concatenate([ref.taps(27, sample).ravel(), ref.taps(19, sample).ravel(), sample, [0]]))
    full = np.zeros((N + 1, C), np.float32)  # pages never touched stay unallocated
    for a in range(0, need.size, 4096):
        part = need[a:a + 4096]
        full[part.astype(np.int64)] = I.sidecar_at(SEED, part, C)
    out = torch.empty_like(sc)
    yield g, ref, sc, out, full, sample
    del sc, out
    torch.cuda.empty_cache()


def check(out, want, sample, what):
    got = out[torch.from_numpy(sample.astype(np.int64)).cuda()].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), what


@pytest.mark.parametrize("flags", [vbm.CACHED | vbm.STREAMING, vbm.CACHED, vbm.STREAMING, 0])
def test_box_past_4_gib(huge, flags):
    g, ref, sc, out, full, sample = huge
    say("huge box flags=%d" % flags)
    vbm.box_filter(g, sc, flags, out=out)
    check(out, ref.box(full, sample), sample, "box")


@pytest.mark.parametrize("flags", [vbm.CACHED | vbm.STREAMING, 0])
def test_cross_and_axis_past_4_gib(huge, flags):
    g, ref, sc, out, full, sample = huge
    for what, run, want in (("sum", lambda: vbm.cross_filter(g, sc, flags, out=out), lambda: ref.cross(full, "sum", sample)),
                            ("lap", lambda: vbm.cross_filter(g, sc, flags | vbm.OP_LAPLACIAN, out=out),
                             lambda: ref.cross(full, "laplacian", sample)),
                            ("axis", lambda: vbm.axis_filter(g, sc, flags, out=out), lambda: ref.axis(full, sample))):
        say("huge %s flags=%d" % (what, flags))
        run()
        check(out, want(), sample, what)


@pytest.mark.parametrize("flags", [vbm.CACHED | vbm.STREAMING, 0])
def test_weno_past_4_gib(huge, flags):
    g, ref, sc, out, full, sample = huge
    say("huge weno flags=%d" % flags)
    vbm.weno_filter(g, sc, flags, out=out)
    check(out, ref.weno(full, sample), sample, "weno")
