"""The seeded generator: slices equal the same slice of the full tensor,
and the byte stream does not depend on the worker count."""
import numpy as np

import synth_inputs as si


def test_slices_match_full_tensor():
    k = si.kv_tensor(90, si.K, 2, 3, 40, 16, "f16", outliers=True)
    sub = si.kv_tensor(90, si.K, 2, 3, 40, 16, "f16", outliers=True,
                       heads=range(1, 3), tokens=range(7, 33))
    assert np.array_equal(k[:, 1:3, 7:33], sub)
    rows = si.flat_rows(91, 64 * 32, 32)
    assert np.array_equal(rows[5:9], si.flat_rows(91, 64 * 32, 32, rows=range(5, 9)))


def test_chunk_boundary_and_workers():
    n = si.CHUNK + 1000
    a = si.stream(92, 1, n, workers=1)
    b = si.stream(92, 1, n, workers=4)
    assert np.array_equal(a, b)
    c = si.stream(92, 1, 100, start=si.CHUNK - 50)
    assert np.array_equal(a[si.CHUNK - 50: si.CHUNK + 50], c)


def test_outliers_scale_by_twenty():
    base = si.kv_tensor(93, si.K, 1, 2, 8, 16, "f32")
    out = si.kv_tensor(93, si.K, 1, 2, 8, 16, "f32", outliers=True)
    ch = si.outlier_channels(93, 2, 16)
    for h in range(2):
        assert len(set(ch[h])) == 4
        mask = np.zeros(16, bool)
        mask[ch[h]] = True
        assert np.array_equal(out[0, h][:, mask], base[0, h][:, mask] * np.float32(20))
        assert np.array_equal(out[0, h][:, ~mask], base[0, h][:, ~mask])
