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


def test_cpu_baseline_reports_the_later_call_and_the_oracle_error():
    """The CPU baseline times the oracle in the headline's regime (a later call from the oracle's own
    previous call) and reports the host it ran on and the oracle's error on its sample rows."""
    import free_block_sparse_sampled_amd as spr
    from workloads import config
    cfg = config("tiny")
    opc = spr.OperatorConfig(Ck=cfg.Ck, Cq=cfg.Cq, rK=cfg.rK, rQ=min(cfg.rQ, cfg.d), Ms=cfg.Ms,
                             max_iters=cfg.max_iters, tol=cfg.tol, M=cfg.M, rho=cfg.rho, lam=cfg.lam, seed=0)
    cb = bench.cpu_baseline(cfg, opc, True, 2, 1)
    rows = cb.pop("_rows")
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["nproc"] >= 1 and cb["cores"] >= 1
    assert "later call" in cb["regime"]
    att = cb["oracle_err_vs_dense"]
    assert att["rows"] == len(rows) > 0
    assert np.isfinite(att["corrected_mean"]) and np.isfinite(att["sparse_only_mean"])
    cold = bench.cpu_baseline(cfg, opc, False, 2, 0)
    assert "cold call" in cold["regime"]


def test_cpu_info():
    model, nproc = bench.cpu_info()
    assert nproc >= 1
    assert model is None or isinstance(model, str)
