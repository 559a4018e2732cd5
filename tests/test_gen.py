"""The synthetic-input generator: determinism, distribution, and workload shapes."""
import numpy as np

import gen


def test_counter_based_slices_agree():
    wl = gen.Workload("s", 8, 256, 6, 3, "bf16", True)
    full = gen.Trajectory(wl, seed=3)
    part = gen.Trajectory(wl, seed=3, slot0=2, nslots=3, threads=1)
    for _ in range(3):
        a = full.next()
        b = part.next()
        assert np.array_equal(a[2:5], b)


def test_seed_changes_data():
    wl = gen.WORKLOADS["tiny"]
    a = gen.Trajectory(wl, 0).next()
    b = gen.Trajectory(wl, 1).next()
    assert not np.array_equal(a, b)


def test_normal_moments():
    z = gen.normals(0, 9, 0, 0, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.std() - 1) < 5e-3
    assert abs((z ** 4).mean() - 3) < 0.05


def test_outlier_channels():
    for n, want in ((3072, 31), (1920, 19)):
        c1 = np.empty(n, np.float32)
        c20 = np.empty(n, np.float32)
        gen.lib().cfgen_channel_scales(0, 5, n, 0.5, 0.01, 1.0, gen._ptr(c1))
        gen.lib().cfgen_channel_scales(0, 5, n, 0.5, 0.01, 20.0, gen._ptr(c20))
        ratio = c20 / c1
        assert np.sum(np.abs(ratio - 20) < 1e-5) == want
        assert np.sum(np.abs(ratio - 1) < 1e-6) == n - want
        lg = np.log(c1.astype(np.float64))
        assert abs(lg.std() - 0.5) < 0.05


def test_drift_and_bf16_rounding():
    wl = gen.Workload("s", 64, 512, 1, 2, "bf16", True)
    tr = gen.Trajectory(wl, 0)
    a0 = tr.next()
    s0 = tr.state.copy()
    a1 = tr.next()
    s1 = tr.state.copy()
    dz = (s1 - s0)[0] / tr.c[0][None, :]
    assert abs(dz.std() - 0.05) < 2e-3
    f = gen.as_f32(a1)
    assert np.all(np.abs(f - s1) <= np.spacing(np.abs(s1)) * 2 ** 15 + 1e-30)
    assert a0.dtype == np.uint16


def test_workload_table():
    assert gen.WORKLOADS["flux"].numel == 1024 * 3072
    assert gen.WORKLOADS["flux"].slots == 114 and gen.WORKLOADS["flux"].steps == 28
    assert gen.WORKLOADS["cogvideo"].numel == 2925 * 1920
    assert gen.WORKLOADS["cogvideo"].slots == 60 and gen.WORKLOADS["cogvideo"].steps == 50
    assert gen.WORKLOADS["tiny"].dtype == "f32"
