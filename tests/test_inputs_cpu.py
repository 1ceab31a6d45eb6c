"""The seeded input generators (CPU only): the row-wise and row-subset forms of
the sidecar give the same values as the whole sidecar, and the wide-range
sidecar is deterministic and finite."""
import numpy as np

from nanovdb_stencil_filtering_amd import inputs as I


def test_sidecar_rows_and_subsets_match_the_whole():
    whole = I.sidecar(21, 5000, 7)
    assert np.array_equal(I.sidecar_rows(21, 0, 5001, 7), whole)
    assert np.array_equal(I.sidecar_rows(21, 1234, 4321, 7), whole[1234:4321])
    rows = np.array([0, 5000, 17, 17, 4999, 1], np.uint64)
    assert np.array_equal(I.sidecar_at(21, rows, 7), whole[rows.astype(np.int64)])
    assert np.all(I.sidecar_at(21, [0], 7) == 0)


def test_wide_range_sidecar_is_deterministic_and_finite():
    a = I.wide_range_sidecar(5, 20000, 3, 0.2)
    b = I.wide_range_sidecar(5, 20000, 3, 0.2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.isfinite(a).all()
    mag = np.abs(a[1:]).ravel()
    assert (mag == 0).any() and ((mag > 0) & (mag < 2.0 ** -126)).any() and (mag > 1e19).any()
    assert ((mag == 2.0 ** -40) | (mag == 2.0 ** 45)).any()
    # about 20 % of the elements leave [-1, 1)
    out = (mag >= 1) | (mag < 2.0 ** -40)
    assert 0.1 < out.mean() < 0.25
