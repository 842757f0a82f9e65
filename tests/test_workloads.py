"""The seeded input generator: deterministic, shaped and distributed as stated."""

import numpy as np
import pytest

import workloads as wl


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_deterministic_and_shaped(name):
    a = wl.make_workload(name)
    b = wl.make_workload(name)
    np.testing.assert_array_equal(a["x"], b["x"])
    np.testing.assert_array_equal(a["dy"], b["dy"])
    w = a["widths"]
    assert a["x"].shape == (a["N"], w[0]) and a["dy"].shape == (a["N"], w[-1])
    for l, (C, W) in enumerate(a["layers"]):
        assert C.shape == (w[l + 1], w[l], a["G"] + 3)
        assert (W is None) == (not a["base"])
    assert np.abs(a["x"]).max() <= 1.0


def test_prefix_rows_and_bf16_exact():
    full = wl.make_workload("c4", N=64)
    part = wl.make_workload("c4", N=16)
    np.testing.assert_array_equal(full["x"][:16], part["x"])
    for arr in [full["x"], full["layers"][0][0], full["layers"][1][1]]:
        bits = np.ascontiguousarray(arr, dtype=np.float32).view(np.uint32)
        assert np.all((bits & 0xFFFF) == 0)


def test_grid_variants_differ():
    a = wl.make_workload("c3", G=8, N=4)
    b = wl.make_workload("c3", G=20, N=4)
    assert a["layers"][0][0].shape[-1] == 11 and b["layers"][0][0].shape[-1] == 23


def test_random_layer_has_special_points():
    d = wl.random_layer(64, 9, 5, 8, seed=1)
    x = d["x"]
    assert (x == 1.0).any() and (x == -1.0).any() and (np.abs(x) > 3).any()


def test_samples():
    r = wl.sample_indices(1000, 10, 3)
    assert len(set(r.tolist())) == 10 and r.max() < 1000
    assert len(wl.sample_indices(5, 10, 3)) == 5
    p = wl.sample_pairs(7, 9, 20, 1)
    assert p.shape == (20, 2) and p[:, 0].max() < 7 and p[:, 1].max() < 9
