"""Measurement helpers of bench.py against the oracle (CPU only)."""
import numpy as np

import bench
import oracle as O


def test_bench_representability_matches_the_oracle_fit():
    rng = np.random.default_rng(5)
    for n, d in [(300, 8), (2048, 16)]:
        X = rng.standard_normal((n, d))
        D = X + 0.3 * X @ rng.standard_normal((d, d)) + 0.1 * rng.standard_normal((n, d))
        energy, left = bench.affine_fit_energy(X, D)
        ref = O.affine_representability(X, D)
        np.testing.assert_allclose(energy, ref["energy"], rtol=1e-13)
        np.testing.assert_allclose(left, ref["remaining"], rtol=1e-10)
