"""The seeded input generators: determinism, shapes and the stated value ranges (no GPU)."""

import numpy as np

from workloads import (CONFIGS, SMALL_CONFIGS, add_noise, config_phantom, config_trajectory,
                       sinogram_field)


def test_small_configs_mirror_full_ones():
    for name, full in CONFIGS.items():
        small = SMALL_CONFIGS[name]
        assert (small.beam, small.trajectory, small.layout, small.batch) == \
               (full.beam, full.trajectory, full.layout, full.batch)
        assert small.n_rays * 10 <= full.n_rays or name == "c1_parallel2d"


def test_phantoms_are_seeded_and_in_range():
    for cfg in SMALL_CONFIGS.values():
        a = config_phantom(cfg)
        b = config_phantom(cfg)
        assert a.dtype == np.float32 and np.array_equal(a, b)
        assert a.shape == ((cfg.batch,) if cfg.batch else ()) + cfg.shape
        assert a.min() >= 0.0 and a.max() > 0.1
        assert a.max() <= cfg.n_ellipsoids * cfg.intensity_range[1] + cfg.background + 1e-6


def test_trajectories_match_geometry():
    for cfg in list(SMALL_CONFIGS.values()) + list(CONFIGS.values()):
        t = config_trajectory(cfg)
        rank = 3 if cfg.beam == "cone" else 2
        for k in ("src", "det", "eu"):
            assert t[k].shape == (cfg.views, rank) and t[k].dtype == np.float64
        if cfg.beam == "parallel":
            np.testing.assert_allclose(np.linalg.norm(t["src"], axis=1), 1.0)
            continue
        d = np.linalg.norm(t["det"] - t["src"], axis=1)
        np.testing.assert_allclose(d, cfg.sdd, rtol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(t["src"][:, :2], axis=1), cfg.sid, rtol=1e-12)
        if cfg.beam == "cone":
            assert np.all(t["ev"][:, :2] == 0.0) and np.all(t["ev"][:, 2] == 1.0)
    h = config_trajectory(CONFIGS["c5_helical_b4"])
    z = h["src"][:, 2]
    assert abs(z[0] + 96.0) < 1e-12 and abs(z[480] - z[0] - 64.0) < 1e-9 and z.max() < 96.0


def test_noise_and_fields_are_seeded():
    s = np.zeros((4, 5, 6), np.float32)
    n1 = add_noise(s, 0.01, 3)
    assert np.array_equal(n1, add_noise(s, 0.01, 3)) and 0.005 < n1.std() < 0.02
    f = sinogram_field((2, 7, 5, 9), seed=4)
    assert f.shape == (2, 7, 5, 9) and f.dtype == np.float32
    assert np.array_equal(f, sinogram_field((2, 7, 5, 9), seed=4))
