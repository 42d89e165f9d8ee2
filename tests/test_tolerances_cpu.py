"""The tolerances the GPU parity tests derive, checked on the CPU against
brute force: they must hold for every perturbation they claim to cover."""

import numpy as np

from oracle import locks_oracle as lo

import reference as ref


def test_record_band_covers_every_perturbation_within_delta():
    """Two score sets within delta of each other select pages that differ only
    within record_band(delta) of the reference cut (random trials, G = 1..8,
    perturbations up to the bound)."""
    rng = np.random.default_rng(31)
    worst = 0.0
    for trial in range(400):
        G = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(6, 60))
        k = int(rng.integers(3, n))
        s = rng.normal(0.0, rng.uniform(0.05, 3.0), size=(G, n))
        delta = float(rng.choice([1e-6, 1e-4, 1e-3, 1e-2, 5e-2]))
        s2 = s + rng.uniform(-delta, delta, size=s.shape)
        n_mr = n  # pages 0..n-1 scored, n is the most recent page
        m1, m2 = lo.share_average(s), lo.share_average(s2)
        sel1, sel2 = lo.select_pages(m1, n_mr, k), lo.select_pages(m2, n_mr, k)
        band = ref.record_band(delta)
        assert ref.selection_mismatch(sel2, sel1, m1, n_mr, k, rel=band) is None
        diff = set(sel1.tolist()) ^ set(sel2.tolist())
        if diff:
            cand = list(range(1, n_mr))
            cut = m1[sorted(cand, key=lambda j: (-m1[j], j))[min(k - 2, len(cand)) - 1]]
            worst = max(worst, max(abs(m1[j] - cut) / cut for j in diff) / band)
    assert 0.0 < worst <= 1.0  # some trials swap pages, every swap inside the band


def test_bf16_ulps_counts_grid_steps():
    a = np.array([1.0, -1.0, 0.0, 1.0078125, 0.5, 2.0 ** -126])
    b = np.array([1.0078125, -1.0078125, -0.0, 1.0, 0.498046875, 0.0])
    np.testing.assert_array_equal(ref.bf16_ulps(a, b), [1, 1, 0, 1, 1, 128])
