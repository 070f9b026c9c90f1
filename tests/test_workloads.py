"""Sanity of the seeded synthetic workloads (CPU only): shapes, dtypes,
determinism and the statistical shape of each routing law."""
import numpy as np
import pytest

from combine_get_dispatch_02_amd.workloads import CONFIGS, make_workload


@pytest.mark.parametrize("name", ["tiny", "dsv3", "skewed", "ll_fp8"])
def test_shapes_distinct_and_deterministic(name):
    wl = CONFIGS[name]
    x, idx, w = make_workload(wl, with_x=(wl.T * wl.H <= 2 ** 22))
    assert idx.shape == (wl.T, wl.k) and idx.dtype == np.int64
    assert idx.min() >= 0 and idx.max() < wl.E
    s = np.sort(idx, 1)
    assert np.all(s[:, 1:] != s[:, :-1])                      # distinct experts per token
    assert w.dtype == np.float32 and np.allclose(w.sum(1), 1.0, atol=1e-6) and np.all(w > 0)
    _, idx2, w2 = make_workload(wl, with_x=False)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    if x is not None:
        assert x.shape == (wl.T, wl.H) and x.dtype == np.uint16


def test_uniform_routing_is_flat():
    wl = CONFIGS["dsv3"]
    _, idx, _ = make_workload(wl, with_x=False)
    cnt = np.bincount(idx.ravel(), minlength=wl.E)
    mean = wl.T * wl.k / wl.E
    assert abs(cnt.mean() - mean) < 1e-9 and cnt.std() < 4 * np.sqrt(mean)


def test_zipf_is_skewed():
    wl = CONFIGS["skewed"]
    _, idx, _ = make_workload(wl, with_x=False)
    cnt = np.bincount(idx.ravel(), minlength=wl.E)
    assert cnt[0] == cnt.max() and cnt[0] > 0.8 * wl.T        # expert 0 in most tokens
    part0 = cnt[: wl.E // wl.R].sum() / cnt.sum()
    assert part0 > 0.5                                          # partition 0 is hot


def test_two_level_confinement():
    wl = CONFIGS["large"].scaled(T=4096)
    _, idx, _ = make_workload(wl, with_x=False)
    grp = idx // (wl.E // wl.G)
    confined = np.all(grp == grp[:, :1], axis=1)
    assert 0.45 < confined.mean() < 0.56                      # ~50% (+ chance confinement)


def test_x_distribution():
    wl = CONFIGS["ll_fp8"]
    x, _, _ = make_workload(wl)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.std() - 2.0) < 0.02 and abs(f.mean()) < 0.01
