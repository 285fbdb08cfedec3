"""GPU-vs-oracle parity of the HIP operator (run through the C ABI).

Discrete outputs (groups, permutations, routes, probes) must be identical to the oracle's
unless the oracle reports a decision whose relative margin is at most 1e-6 (a tie), in
which case the test says so and falls back to lockstep checks.  Continuous outputs must
match within 2e-3 relative L2 per row (attention outputs, bf16 inputs with fp32
accumulation) or tighter bounds derived from fp64 arithmetic."""
import numpy as np
import pytest
import torch

import free_block_sparse_sampled_amd as spr
import oracle as O
from tests.gpu_pipeline import device_inputs, op_config, pull, row_rel_err, run_operator
from workloads import batch_inputs, config, head_inputs

pytestmark = pytest.mark.gpu

TIE = 1e-6
ROW_TOL = 2e-3


def _oracle_params(opc, n_text=0):
    return O.Params(Ck=opc.Ck, Cq=opc.Cq, rK=opc.rK, rQ=opc.rQ, Ms=opc.Ms, max_iters=opc.max_iters, tol=opc.tol,
                    rms_eps=opc.rms_eps, eig_clamp=opc.eig_clamp, seed=opc.seed, M=opc.M, rho=opc.rho,
                    lam=opc.lam, std_eps=opc.std_eps, n_text=n_text)


# ------------------------------------------------------------------ dense kernel
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (64, torch.float32),
                                     (128, torch.float32)])
def test_dense_attention_matches_oracle(d, dtype):
    rng = np.random.default_rng([7, d])
    B, H, N = 1, 2, 333                       # several 64-row tiles and a ragged tail
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    x[1] *= 1.5
    t = torch.from_numpy(x).to(dtype)
    xq = t.float().numpy()
    q, k, v = (t[i].cuda() for i in range(3))
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    spr.sparsepr_attn_dense(spr.make_desc(q), q, k, v, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for h in range(H):
        ref = O.dense_attention_rows(xq[0, 0, h], xq[1, 0, h], xq[2, 0, h], np.arange(N))
        err = row_rel_err(got[0, h], ref)
        assert err.max() < ROW_TOL, (h, err.max())


# ------------------------------------------------------------------ k-means
def _clustered(n, r, C, seed):
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((C, r)) * 3
    return centres[rng.integers(0, C, n)] + rng.standard_normal((n, r))


@pytest.mark.parametrize("r,C,n", [(48, 20, 1000), (64, 37, 777), (16, 5, 300), (48, 700, 3001), (64, 1024, 2500),
                                   (128, 40, 1500), (128, 300, 3001)])
def test_kmeans_matches_oracle(r, C, n):
    BH = 2
    feats = np.stack([_clustered(n, r, C, [r, C, h]) for h in range(BH)])
    lab, cent, passes = spr.sparsepr_kmeans(torch.from_numpy(feats).cuda(), C, 11, 0, 25, 1e-4)
    torch.cuda.synchronize()
    lab, cent, passes = lab.cpu().numpy(), cent.cpu().numpy(), passes.cpu().numpy()
    for h in range(BH):
        ref = O.kmeans(feats[h], C, 11, h, 0, 25, 1e-4)
        assert ref["min_margin"] > TIE and ref["stop_margin"] > 1e-6
        assert passes[h] == ref["passes"]
        assert np.array_equal(lab[h], ref["labels"])
        np.testing.assert_allclose(cent[h], ref["centres"], rtol=0, atol=1e-12 * np.abs(ref["centres"]).max())


# ------------------------------------------------------------------ whole operator
def _compare_head(g, ref, hd, Nv, N, n_text, discrete_exact=True, kh=None):
    """Compare GPU outputs of query head hd (K/V head kh, default hd) against an oracle run."""
    kh = hd if kh is None else kh
    d = g["FK"].shape[1]
    # factors: F F^T is unique (eigenvector signs / rotations are not)
    for F, Fo in ((g["FK"][kh], ref["FK"]), (g["FQ"][kh], ref["FQ"])):
        if Fo is None:  # not formed by this partition mode
            continue
        A, Ao = F @ F.T, Fo @ Fo.T
        assert np.abs(A - Ao).max() <= 1e-9 * np.abs(Ao).max()
    nkv, nq = int(g["n_kv"][kh]), int(g["n_q"][hd])
    if discrete_exact:
        assert nkv == ref["n_kv"] and nq == ref["n_q"]
        assert np.array_equal(g["kv_label"][kh], ref["kv_label"])
        assert np.array_equal(g["q_label"][hd], ref["q_label"])
        perm_k, off_k = O.group_perm(ref["kv_label"], nkv)
        perm_q, off_q = O.group_perm(ref["q_label"], nq)
        assert np.array_equal(g["kv_perm"][kh], perm_k) and np.array_equal(g["kv_off"][kh][: nkv + 1], off_k)
        assert np.array_equal(g["q_perm"][hd], perm_q) and np.array_equal(g["q_off"][hd][: nq + 1], off_q)
        np.testing.assert_allclose(g["kbar"][kh][:nkv], ref["kbar"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["vbar"][kh][:nkv], ref["vbar"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["qbar"][hd][:nq], ref["qbar"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["qdist"][hd], ref["qdist"], rtol=1e-8, atol=1e-10)
        for a in range(nq):
            cnt = int(g["sel_cnt"][hd][a])
            sel = g["sel_kv"][hd][a][:cnt]
            want = list(ref["sel"][a]) + ([nkv] if n_text else [])
            assert list(sel) == want, (hd, a)
        assert int(g["pairs"][hd]) == ref["pairs"]
        assert abs(g["rho_exec"][hd] - ref["rho_exec"]) < 1e-15
        assert np.array_equal(g["probe_idx"][hd], ref["probes"])
        np.testing.assert_allclose(g["probe_w"][hd], ref["probe_w"], rtol=1e-15)
    # attention outputs: O^sp is stored in group-major order
    qperm = g["q_perm"][hd]
    osp = np.empty((N, d))
    osp[qperm] = g["o_sp"][hd][:Nv]
    osp[Nv:] = g["o_sp"][hd][Nv:]
    rows = ref["rows"]
    err = row_rel_err(osp[rows], ref["O_sp"])
    assert err.max() < ROW_TOL, ("o_sp", err.max())
    err = row_rel_err(g["o_probe"][hd], ref["probe_dense"])
    assert err.max() < ROW_TOL, ("o_probe", err.max())
    # fit in lockstep: the oracle's ridge on the GPU's probe features and residuals
    X = osp[ref["probes"]]
    fit = O.ridge_fit(X, g["o_probe"][hd] - X, g["probe_w"][hd], ref["lam"], 1e-6)
    fs = g["fit_state"][hd]
    Bg = fs[3 * d:].reshape(d, d)
    assert np.linalg.norm(Bg - fit["B"]) <= 1e-6 * max(np.linalg.norm(fit["B"]), 1e-12)
    np.testing.assert_allclose(fs[:d], fit["muX"], rtol=0, atol=1e-9)
    np.testing.assert_allclose(fs[2 * d:3 * d], fit["muR"], rtol=0, atol=1e-9)
    # final output: the oracle's correction of the GPU's sparse rows with that fit (probe rows
    # exact, text rows uncorrected) checks the fit and apply arithmetic on identical inputs
    want = osp[rows].copy()
    video = rows < Nv
    want[video] = O.correct(osp[rows][video], fit)
    pidx = {int(r): i for i, r in enumerate(g["probe_idx"][hd])}
    for ir, r in enumerate(rows):
        if int(r) in pidx:
            want[ir] = g["o_probe"][hd][pidx[int(r)]]
    err = row_rel_err(g["out"][hd][rows], want)
    assert err.max() < ROW_TOL, ("out (lockstep fit)", err.max())
    # end to end against the oracle's own output.  The difference splits into the lockstep
    # error above and the oracle's own response to the GPU's sub-2e-3 sparse and probe rows,
    # `own`, which an ill-conditioned ridge (probe count near d on diffuse attention) can
    # amplify; where the fit does not amplify (own < ROW_TOL / 2 everywhere) the bar is ROW_TOL
    e2e = row_rel_err(g["out"][hd][rows], ref["O_hat"])
    own = row_rel_err(want, ref["O_hat"])
    if own.max() < ROW_TOL / 2:
        assert e2e.max() < ROW_TOL, ("out", e2e.max())
    else:
        assert np.all(e2e <= own + ROW_TOL), ("out", e2e.max(), own.max())
        assert np.median(e2e) < ROW_TOL, ("out median", np.median(e2e))


def _oracle_is_tie_free(ref):
    return (ref["kmK"]["min_margin"] > TIE and ref["kmQ"]["min_margin"] > TIE
            and ref["kmK"]["stop_margin"] > 1e-6 and ref["kmQ"]["stop_margin"] > 1e-6
            and min(i["min_gap"] for i in ref["route_info"]) > TIE)


@pytest.mark.parametrize("name,heads", [("tiny", [(0, 0)]), ("small", [(0, 0), (0, 7)]),
                                        ("small_text", [(0, 0), (0, 1)])])
def test_operator_end_to_end(name, heads):
    cfg = config(name)
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    for (b, h) in heads:
        hd = b * cfg.H + h
        rows = None if cfg.N <= 2048 else np.unique(np.concatenate(
            [np.arange(0, cfg.N, 7), np.arange(cfg.N - 100, cfg.N)]))
        ref = O.sparsepr_head(q[b, h], k[b, h], v[b, h], p, head=hd, rows=rows)
        ref["lam"] = p.lam
        if _oracle_is_tie_free(ref):
            _compare_head(g, ref, hd, cfg.Nv, cfg.N, cfg.n_text)
        else:
            # a decision of the oracle's run lies within the 1e-6 tie margin: the two runs may
            # legitimately part there, so check every stage in lockstep instead
            _lockstep_head(g, q, k, v, cfg, opc, b, h, np.random.default_rng(1))
    assert np.all(g["head_status"] & 1 == 0)


@pytest.mark.parametrize("d,Ck,n_text", [
    (64, 128, 32),   # bf16 at d = 64 (every d = 64 instance of the bf16 path), with text tokens
    (64, 16, 0),     # K/V groups of about 500 keys: past what the fp64 rescoring stages in LDS at d = 64
    (128, 24, 0),    # the same at d = 128 (groups of about 340 keys against 180 staged)
])
def test_bf16_head_dims_and_large_groups(d, Ck, n_text):
    """The bf16 operator at d = 64, and with K/V groups larger than the fp64 rescoring keeps in LDS
    (it then reads the group's keys from memory), end to end against the oracle on two heads of a
    small video latent, with the usual lockstep fallback for decisions inside the tie margin."""
    cfg = config("small").with_(name=f"small_d{d}_ck{Ck}", H=2, d=d, Ck=Ck, n_text=n_text)
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    rows = np.unique(np.concatenate([np.arange(0, cfg.N, 7), np.arange(cfg.N - 100, cfg.N)]))
    for h in range(cfg.H):
        ref = O.sparsepr_head(q[0, h], k[0, h], v[0, h], p, head=h, rows=rows)
        ref["lam"] = p.lam
        if _oracle_is_tie_free(ref):
            _compare_head(g, ref, h, cfg.Nv, cfg.N, cfg.n_text)
        else:
            _lockstep_head(g, q, k, v, cfg, opc, 0, h, np.random.default_rng(h))
    assert np.all(g["head_status"] & 1 == 0)


@pytest.mark.parametrize("grid,Ck,Cq,M,rho,n_text", [
    ((4, 8, 8), 1, 1, 8, 0.5, 0),         # one group each: the route is every key
    ((4, 8, 8), 256, 256, 16, 0.3, 0),    # one group per key requested (duplicate draws leave empties)
    ((2, 8, 8), 7, 5, 4, 0.9, 16),        # an empty query group, text tokens, a budget near N
    ((1, 3, 43), 16, 16, 8, 0.22, 0),     # 129 video rows: ragged against every tile size
])
def test_degenerate_group_counts(grid, Ck, Cq, M, rho, n_text):
    """Edge cases of the partition and route on the tiny mixture workload (fp32, d = 64)."""
    cfg = config("tiny").with_(grid=grid, Ck=Ck, Cq=Cq, M=M, rho=rho, n_text=n_text, Ms=4096)
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    ref = O.sparsepr_head(q[0, 0], k[0, 0], v[0, 0], p, head=0)
    ref["lam"] = p.lam
    assert _oracle_is_tie_free(ref)
    _compare_head(g, ref, 0, cfg.Nv, cfg.N, cfg.n_text)
    empty_q = ref["n_q"] < Cq
    assert bool(g["head_status"][0] & 8) == empty_q  # SPR_HS_Q_GROUPS_EMPTY


@pytest.mark.parametrize("name,heads", [("tiny", [(0, 0)]), ("small", [(0, 0), (0, 7)]),
                                        ("small_text", [(0, 0), (0, 1)])])
def test_warm_start_end_to_end(name, heads):
    """A later call (App. C.1): call 1 cold on the step-0 inputs, call 2 on fresh-noise step-1
    inputs started from call 1's factors and centroids, with the warm iteration limit.  The
    oracle runs the same two calls from its own state (the factors agree up to a rotation,
    which neither the subspace iteration nor the distances see).  A head where either oracle
    call meets a tie is checked in lockstep on the GPU's own state instead."""
    cfg = config(name)
    opc = op_config(cfg)
    (q0, k0, v0), (tq0, tk0, tv0) = device_inputs(cfg, step=0)
    (q1, k1, v1), (tq1, tk1, tv1) = device_inputs(cfg, step=1)
    op = spr.SparsePR(tq0, opc, n_text=cfg.n_text, diagnostics=True, keep_scores=True)
    op.run(tq0, tk0, tv0)
    op.run(tq1, tk1, tv1, warm=True)
    torch.cuda.synchronize()
    g = pull(op)
    assert np.all(g["passes"] <= op.warm_iters)
    p = _oracle_params(opc, cfg.n_text)
    p2 = O.Params(**{**p.__dict__, "max_iters": op.warm_iters})
    for (b, h) in heads:
        hd = b * cfg.H + h
        first = O.sparsepr_head(q0[b, h], k0[b, h], v0[b, h], p, head=hd, full=False)
        rows = None if cfg.N <= 2048 else np.unique(np.concatenate(
            [np.arange(0, cfg.N, 7), np.arange(cfg.N - 100, cfg.N)]))
        ref = O.sparsepr_head(q1[b, h], k1[b, h], v1[b, h], p2, head=hd, rows=rows, warm=first["state"])
        ref["lam"] = p.lam
        if name == "tiny":
            assert ref["warm_ok"] == [True, False]  # M_Q has rank 15 < r_Q: cold factor
        else:
            assert ref["warm_ok"] == [True, True]
        if _oracle_is_tie_free(first) and _oracle_is_tie_free(ref):
            _compare_head(g, ref, hd, cfg.Nv, cfg.N, cfg.n_text)
        else:
            _lockstep_head(g, q1, k1, v1, cfg, opc, b, h, np.random.default_rng(3))


@pytest.mark.parametrize("name,rK,rQ", [("small", 8, 16), ("small", 32, 32), ("tiny", 16, 8)])
def test_warm_start_factor_ranks(name, rK, rQ):
    """Later calls at the other factor ranks (8 to 32) and at d = 64: the subspace update of both
    factors against the oracle's later-call path, then the whole head as in the test above."""
    cfg = config(name)
    opc = op_config(cfg, rK=rK, rQ=rQ)
    (q0, k0, v0), (tq0, tk0, tv0) = device_inputs(cfg, step=0)
    (q1, k1, v1), (tq1, tk1, tv1) = device_inputs(cfg, step=1)
    op = spr.SparsePR(tq0, opc, n_text=cfg.n_text, diagnostics=True, keep_scores=True)
    op.run(tq0, tk0, tv0)
    op.run(tq1, tk1, tv1, warm=True)
    torch.cuda.synchronize()
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    p2 = O.Params(**{**p.__dict__, "max_iters": op.warm_iters})
    first = O.sparsepr_head(q0[0, 0], k0[0, 0], v0[0, 0], p, head=0, full=False)
    rows = None if cfg.N <= 2048 else np.arange(0, cfg.N, 7)
    ref = O.sparsepr_head(q1[0, 0], k1[0, 0], v1[0, 0], p2, head=0, rows=rows, warm=first["state"])
    ref["lam"] = p.lam
    assert ref["warm_ok"] == [True, True]
    if _oracle_is_tie_free(first) and _oracle_is_tie_free(ref):
        _compare_head(g, ref, 0, cfg.Nv, cfg.N, cfg.n_text)
    else:
        for F, Fo in ((g["FK"][0], ref["FK"]), (g["FQ"][0], ref["FQ"])):
            A, Ao = F @ F.T, Fo @ Fo.T
            assert np.abs(A - Ao).max() <= 1e-9 * np.abs(Ao).max()


def _check_scores(gs, ge, sc):
    """GPU scores of one row against the oracle's: equal up to one positive row factor, within the
    bound the GPU reports for each score (0 where it was computed in fp64) plus fp64 rounding."""
    ge = np.abs(ge)
    assert np.all(np.isfinite(ge))
    exact = ge == 0
    r = int(np.argmax(np.where(exact, sc, -np.inf))) if exact.any() else int(np.argmax(sc))
    f = gs[r] / sc[r]                                            # one positive factor per row
    assert f > 0
    rel_f = ge[r] / gs[r]                                        # uncertainty of that factor
    assert rel_f < 1e-2
    tol = ge + rel_f / (1 - rel_f) * f * np.abs(sc) + 1e-9 * f * sc.max()
    assert np.all(np.abs(gs - f * sc) <= tol)


def test_lockstep_stages_small():
    """Each stage's oracle function applied to the GPU's own inputs of that stage."""
    cfg = config("small")
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    for hd in (0, 5, 11):
        qh, kh, vh = (x[0, hd].astype(np.float64) for x in (q, k, v))
        # key metric and factor
        FK = g["FK"][hd]
        _, wK = O.metric_factor(O.key_metric(qh, opc.Ms), opc.rK, opc.eig_clamp)
        np.testing.assert_allclose(g["phiK"][hd], O.project(kh, FK), rtol=0, atol=1e-12 * np.abs(g["phiK"][hd]).max())
        # last K/V assignment against the centres it used
        lab, _, margin = O.kmeans_assign(g["phiK"][hd], g["cK_last"][hd])
        lab_c, n = O.compact_labels(lab, opc.Ck)
        ok = margin > TIE
        assert np.array_equal(g["kv_label"][hd][ok], lab_c[ok])
        # query coordinates from the GPU's F_Q
        np.testing.assert_allclose(g["phiQ"][hd], O.query_coords(qh, g["FQ"][hd], opc.rms_eps), rtol=0, atol=1e-12)
        lab, _, margin = O.kmeans_assign(g["phiQ"][hd], g["cQ_last"][hd])
        lab_c, n = O.compact_labels(lab, opc.Cq)
        ok = margin > TIE
        assert np.array_equal(g["q_label"][hd][ok], lab_c[ok])
        # routing scores from the GPU's groups and centroids (order within a row must agree)
        nkv, nq = int(g["n_kv"][hd]), int(g["n_q"][hd])
        kvl = g["kv_label"][hd]
        sc, _ = O.route_scores(g["qbar"][hd][:nq], kh, vh, kvl, g["kbar"][hd][:nkv], g["vbar"][hd][:nkv],
                               groups=range(0, nq, 9))
        for ia, a in enumerate(range(0, nq, 9)):
            _check_scores(g["scores"][hd][a][:nkv], g["score_err"][hd][a][:nkv], sc[ia])
        # selections from the GPU's scores (groups flagged as outside the prefix rank last)
        size = np.diff(g["kv_off"][hd][: nkv + 1])
        T = O.key_budget(opc.rho, cfg.N, cfg.Nv, opc.M, 0)
        for a in range(nq):
            gs = np.where(g["score_err"][hd][a][:nkv] < 0, -1e300, g["scores"][hd][a][:nkv])
            sel, info = O.route_select(gs, size, T)
            cnt = int(g["sel_cnt"][hd][a])
            assert list(g["sel_kv"][hd][a][:cnt]) == list(sel)
        # probes from the GPU's groups and distances
        qs = np.diff(g["q_off"][hd][: nq + 1])
        rows_p, w, _ = O.select_probes(g["q_label"][hd], g["qdist"][hd], qs, opc.M)
        assert np.array_equal(g["probe_idx"][hd], rows_p)
        np.testing.assert_allclose(g["probe_w"][hd], w, rtol=1e-15)


def _lockstep_head(g, q, k, v, cfg, opc, b, h, rng, nrows=96, ngroups=6):
    """Every stage of head (b, h) checked on sampled outputs with the oracle's stage functions
    applied to the GPU's own inputs of that stage."""
    N, Nv, d = cfg.N, cfg.Nv, cfg.d
    T = O.key_budget(opc.rho, N, Nv, opc.M, cfg.n_text)
    G = cfg.H // cfg.Hkv if cfg.Hkv else 1             # query heads per K/V head
    hd, hk = b * cfg.H + h, b * (cfg.H // G) + h // G  # query head, its K/V head (flattened)
    qh = q[b, h].astype(np.float64)
    kh, vh = k[b, h // G].astype(np.float64), v[b, h // G].astype(np.float64)
    nkv, nq = int(g["n_kv"][hk]), int(g["n_q"][hd])
    # K/V and query partitions: final assignment pass and compaction
    for feat, cent, lab_g, C in ((g["phiK"][hk], g["cK_last"][hk], g["kv_label"][hk], opc.Ck),
                                 (g["phiQ"][hd], g["cQ_last"][hd], g["q_label"][hd], opc.Cq)):
        lab, _, margin = O.kmeans_assign(feat, cent)
        lab_c, n = O.compact_labels(lab, C)
        ok = margin > TIE
        assert ok.mean() > 0.99
        assert np.array_equal(lab_g[ok], lab_c[ok])
    perm, off = O.group_perm(g["kv_label"][hk], nkv)
    assert np.array_equal(g["kv_perm"][hk], perm) and np.array_equal(g["kv_off"][hk][: nkv + 1], off)
    perm, off = O.group_perm(g["q_label"][hd], nq)
    assert np.array_equal(g["q_perm"][hd], perm) and np.array_equal(g["q_off"][hd][: nq + 1], off)
    size, kbar, vbar = O.key_group_stats(kh[:Nv], vh[:Nv], g["kv_label"][hk], nkv)
    np.testing.assert_allclose(g["kbar"][hk][:nkv], kbar, rtol=0, atol=1e-12)
    # routing of sampled query groups from the GPU's centroids
    groups = rng.choice(nq, size=min(ngroups, nq), replace=False)
    sc, _ = O.route_scores(g["qbar"][hd][:nq], kh[:Nv], vh[:Nv], g["kv_label"][hk], g["kbar"][hk][:nkv],
                           g["vbar"][hk][:nkv], groups=groups)
    for ia, a in enumerate(groups):
        sel, info = O.route_select(sc[ia], size, T)
        cnt = int(g["sel_cnt"][hd][a])
        got = list(g["sel_kv"][hd][a][:cnt])
        if cfg.n_text:
            assert got[-1] == nkv
            got = got[:-1]
        if info["min_gap"] > TIE:
            assert got == list(sel), (hd, a)
    # probes
    qs = np.diff(g["q_off"][hd][: nq + 1])
    rows_p, w, _ = O.select_probes(g["q_label"][hd], g["qdist"][hd], qs, opc.M)
    assert np.array_equal(g["probe_idx"][hd], rows_p)
    # sparse and dense rows on the GPU's routes
    sel_all = [g["sel_kv"][hd][a][: int(g["sel_cnt"][hd][a]) - (1 if cfg.n_text else 0)] for a in range(nq)]
    qlab = np.concatenate([g["q_label"][hd], np.full(cfg.n_text, -1)])
    rows = np.unique(np.concatenate([rng.choice(N, nrows, replace=False), [0, Nv - 1, N - 1]]))
    qpos = g["q_pos"][hd]
    osp = O.sparse_attention_rows(qh, kh, vh, rows, qlab, g["kv_label"][hk], sel_all, cfg.n_text)
    pos = np.where(rows < Nv, qpos[np.minimum(rows, Nv - 1)], rows)
    err = row_rel_err(g["o_sp"][hd][pos], osp)
    assert err.max() < ROW_TOL, ("o_sp", err.max())
    od = O.dense_attention_rows(qh, kh, vh, g["probe_idx"][hd])
    err = row_rel_err(g["o_probe"][hd], od)
    assert err.max() < ROW_TOL, ("o_probe", err.max())
    # fit from the GPU's probe features and residuals, then the final rows
    X = g["o_sp"][hd][qpos[g["probe_idx"][hd]]].astype(np.float64)
    fit = O.ridge_fit(X, g["o_probe"][hd] - X, g["probe_w"][hd], opc.lam, opc.std_eps)
    Bg = g["fit_state"][hd][3 * d:].reshape(d, d)
    assert np.linalg.norm(Bg - fit["B"]) <= 1e-6 * max(np.linalg.norm(fit["B"]), 1e-12)
    want = O.correct(g["o_sp"][hd][pos].astype(np.float64), fit)
    want[rows >= Nv] = g["o_sp"][hd][pos][rows >= Nv]
    isprobe = np.isin(rows, g["probe_idx"][hd])
    err = row_rel_err(g["out"][hd][rows][~isprobe], want[~isprobe])
    assert err.max() < ROW_TOL, ("out", err.max())


def _full_size_lockstep(name, heads):
    """Full-size workload in the benchmark's launch configuration, checked in lockstep."""
    _full_size_lockstep_cfg(config(name), heads)


def _full_size_lockstep_cfg(cfg, heads):
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    del tq, tk, tv
    rng = np.random.default_rng(0)
    for (b, h) in heads:
        _lockstep_head(g, q, k, v, cfg, opc, b, h, rng)


def test_full_size_mid_sampled():
    _full_size_lockstep("mid", [(0, 0), (0, 39)])


def test_full_size_joint_text_sampled():
    _full_size_lockstep("joint", [(0, 0), (1, 23)])


def test_full_size_long_sampled():
    """The long workload (N = 118800, 1024 K/V and query groups, 512 probes) in the benchmark's
    launch configuration."""
    _full_size_lockstep("long", [(0, 0), (0, 23)])


@pytest.mark.parametrize("rho,M", [(0.10, 1024), (0.50, 64)])
def test_full_size_joint_density_and_probe_extremes(rho, M):
    """The ends of the density and probe-count sweep on the joint text + video workload."""
    _full_size_lockstep_cfg(config("joint").with_(rho=rho, M=M), [(0, 0), (1, 5)])


def test_full_size_mid_later_call_sampled():
    """A later call at full size (App. C.1), the regime the benchmark times: call 1 cold on the
    step-0 inputs, call 2 warm on fresh-noise step-1 inputs.  The factors of call 2 are checked
    against the oracle's subspace iteration started from call 1's factors, then every stage of two
    heads in lockstep."""
    cfg = config("mid")
    opc = op_config(cfg)
    _, (tq0, tk0, tv0) = device_inputs(cfg, step=0)
    op = run_operator(cfg, opc, tq0, tk0, tv0)
    FK0, FQ0 = op.part.FK.cpu().numpy(), op.part.FQ.cpu().numpy()
    del tq0, tk0, tv0
    (q, k, v), (tq, tk, tv) = device_inputs(cfg, step=1)
    op.run(tq, tk, tv, warm=True)
    torch.cuda.synchronize()
    g = pull(op)
    del tq, tk, tv
    assert np.all(g["passes"] <= op.warm_iters)
    rng = np.random.default_rng(2)
    for (b, h) in [(0, 0), (0, 31)]:
        hd = b * cfg.H + h
        qh = q[b, h].astype(np.float64)
        MK = O.key_metric(qh[: cfg.Nv], opc.Ms)
        FK, ok = O.metric_factor_warm(MK, FK0[hd], opc.rK, opc.eig_clamp)
        assert ok
        nkv = int(g["n_kv"][hd])
        MQ = O.query_metric(g["kbar"][hd][:nkv])
        FQ, okq = O.metric_factor_warm(MQ, FQ0[hd], opc.rQ, opc.eig_clamp)
        assert okq
        for F, Fo in ((g["FK"][hd], FK), (g["FQ"][hd], FQ)):
            A, Ao = F @ F.T, Fo @ Fo.T
            assert np.abs(A - Ao).max() <= 1e-9 * np.abs(Ao).max()
        _lockstep_head(g, q, k, v, cfg, opc, b, h, rng)


# ------------------------------------------------------------------ partition modes
@pytest.mark.parametrize("name,mode,heads", [("tiny", "semantic", [0]), ("tiny", "key_response", [0]),
                                             ("small", "semantic", [0, 3]), ("small", "key_response", [0, 3])])
def test_partition_modes_end_to_end(name, mode, heads):
    """The semantic reference partition of Sec. 3.1 (k-means on the raw keys and queries) and the
    key-response variant of Table 2 (response-coupled K/V groups, raw query groups), end to end
    against the oracle's run of the same mode; heads with an oracle decision inside the 1e-6
    tie margin are checked stage by stage instead."""
    cfg = config(name)
    opc = op_config(cfg, partition_mode=mode)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = O.Params(**{**_oracle_params(opc, cfg.n_text).__dict__, "partition_mode": mode})
    Nv = cfg.Nv
    for h in heads:
        # raw coordinates are the activations themselves, exactly
        if mode == "semantic":
            assert np.array_equal(g["phiK"][h], k[0, h][:Nv].astype(np.float64))
        assert np.array_equal(g["phiQ"][h], q[0, h][:Nv].astype(np.float64))
        ref = O.sparsepr_head(q[0, h], k[0, h], v[0, h], p, head=h)
        ref["lam"] = p.lam
        if _oracle_is_tie_free(ref):
            _compare_head(g, ref, h, Nv, cfg.N, cfg.n_text)
        else:
            _lockstep_head(g, q, k, v, cfg, opc, 0, h, np.random.default_rng(h))
    assert np.all(g["head_status"] & 1 == 0)


# ------------------------------------------------------------------ grouped-query attention
@pytest.mark.parametrize("name", ["tiny_gqa", "small_gqa"])
def test_gqa_end_to_end(name):
    """Grouped-query attention (Sec. 4.3, routing and GQA; App. C.2): one key metric and K/V
    partition per K/V head from the rows of its G query heads, the query side per query head.
    Every query head is compared with the oracle's group run of its K/V head."""
    cfg = config(name)
    G = cfg.H // cfg.Hkv
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    assert tk.shape[1] == cfg.Hkv
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    assert g["kv_label"].shape[0] == cfg.B * cfg.Hkv and g["q_label"].shape[0] == cfg.B * cfg.H
    p = _oracle_params(opc, cfg.n_text)
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            kh = b * cfg.Hkv + j
            heads = [b * cfg.H + j * G + i for i in range(G)]
            refs = O.sparsepr_group([q[b, j * G + i] for i in range(G)], k[b, j], v[b, j], p, kh, heads)
            # the shared key factor (no discrete decision before it): F F^T is unique
            A, Ao = g["FK"][kh] @ g["FK"][kh].T, refs[0]["FK"] @ refs[0]["FK"].T
            assert np.abs(A - Ao).max() <= 1e-9 * np.abs(Ao).max()
            for hd, ref in zip(heads, refs):
                ref["lam"] = p.lam
                if _oracle_is_tie_free(ref):
                    _compare_head(g, ref, hd, cfg.Nv, cfg.N, cfg.n_text, kh=kh)
                    assert g["passes"][kh][0] == ref["kmK"]["passes"] and g["passes"][hd][1] == ref["kmQ"]["passes"]
                else:
                    # a decision within the 1e-6 tie margin: every stage in lockstep instead
                    _lockstep_head(g, q, k, v, cfg, opc, b, hd - b * cfg.H, np.random.default_rng(hd))
    assert np.all(g["head_status"] & 1 == 0)


def test_gqa_warm_start():
    """A later call under grouped-query attention: the K/V-side state (factors, key centroids) is
    per K/V head, the query centroids per query head (App. C.1 with the sharing of Sec. 4.3)."""
    cfg = config("small_gqa")
    G = cfg.H // cfg.Hkv
    opc = op_config(cfg)
    (q0, k0, v0), (tq0, tk0, tv0) = device_inputs(cfg, step=0)
    (q1, k1, v1), (tq1, tk1, tv1) = device_inputs(cfg, step=1)
    op = spr.SparsePR(tq0, opc, n_text=cfg.n_text, diagnostics=True, keep_scores=True, k=tk0)
    op.run(tq0, tk0, tv0)
    op.run(tq1, tk1, tv1, warm=True)
    torch.cuda.synchronize()
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    p2 = O.Params(**{**p.__dict__, "max_iters": op.warm_iters})
    for j in range(cfg.Hkv):
        heads = [j * G + i for i in range(G)]
        first = O.sparsepr_group([q0[0, h] for h in heads], k0[0, j], v0[0, j], p, j, heads, full=False)
        refs = O.sparsepr_group([q1[0, h] for h in heads], k1[0, j], v1[0, j], p2, j, heads,
                                warm=[r["state"] for r in first])
        A, Ao = g["FK"][j] @ g["FK"][j].T, refs[0]["FK"] @ refs[0]["FK"].T
        assert np.abs(A - Ao).max() <= 1e-9 * np.abs(Ao).max()
        for hd, ref in zip(heads, refs):
            ref["lam"] = p.lam
            if all(_oracle_is_tie_free(r) for r in first) and _oracle_is_tie_free(ref):
                _compare_head(g, ref, hd, cfg.Nv, cfg.N, cfg.n_text, kh=j)
            else:
                _lockstep_head(g, q1, k1, v1, cfg, opc, 0, hd, np.random.default_rng(hd))
    # passes[j][0] holds the K/V passes of K/V head j (rows past B * Hkv are not written),
    # passes[hd][1] the query passes of query head hd
    BHkv = cfg.B * cfg.Hkv
    assert np.all(g["passes"][:BHkv, 0] <= op.warm_iters) and np.all(g["passes"][:, 1] <= op.warm_iters)


# ------------------------------------------------------------------ probe and estimator variants
@pytest.mark.parametrize("name,heads,probe_mode,family,out_rank", [
    ("tiny", [0], "random", "full", 0),
    ("tiny", [0], "uniform", "full", 0),
    ("tiny", [0], "stratified", "mean", 0),
    ("tiny", [0], "stratified", "scalar", 0),
    ("tiny", [0], "stratified", "diag", 0),
    ("tiny", [0], "stratified", "full", 8),
    ("small", [0, 5], "random", "diag", 16),
    ("small", [3], "uniform", "full", 32),
])
def test_probe_and_estimator_variants(name, heads, probe_mode, family, out_rank):
    """Table 4's probe choices and App. D.3-D.4's estimators through the C ABI: probe rows and
    weights bit-exact against the oracle's rule, then the fit in lockstep (the oracle's estimator
    on the GPU's own probe features and residuals) and the corrected rows."""
    cfg = config(name)
    opc = op_config(cfg, probe_mode=probe_mode, fit_family=family, out_rank=out_rank)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    N, Nv, d = cfg.N, cfg.Nv, cfg.d
    for hd in heads:
        if probe_mode == "random":
            rows, w = O.select_probes_random(Nv, opc.M, opc.seed, hd)
        elif probe_mode == "uniform":
            rows, w = O.select_probes_uniform(Nv, opc.M)
        else:
            rows, w = None, None
        if rows is not None:
            assert np.array_equal(g["probe_idx"][hd], rows)
            np.testing.assert_array_equal(g["probe_w"][hd], w)
        qpos = g["q_pos"][hd]
        P = g["probe_idx"][hd]
        X = g["o_sp"][hd][qpos[P]].astype(np.float64)
        fit = O.ridge_fit(X, g["o_probe"][hd] - X, g["probe_w"][hd], opc.lam, opc.std_eps, family, out_rank,
                          opc.eig_clamp)
        Bg = g["fit_state"][hd][3 * d:].reshape(d, d)
        assert np.linalg.norm(Bg - fit["B"]) <= 1e-6 * max(np.linalg.norm(fit["B"]), 1e-12), family
        if out_rank:
            pass  # the truncation mixes columns: B V_r V_r^T has no family structure left
        elif family == "mean":
            assert np.all(Bg == 0)
        elif family == "scalar":
            assert np.all(Bg[~np.eye(d, dtype=bool)] == 0) and np.ptp(np.diag(Bg)) == 0
        elif family == "diag":
            assert np.all(Bg[~np.eye(d, dtype=bool)] == 0)
        # corrected rows: every 5th video row that is not a probe
        rr = np.setdiff1d(np.arange(0, Nv, 5), P)
        want = O.correct(g["o_sp"][hd][qpos[rr]].astype(np.float64), fit)
        err = row_rel_err(g["out"][hd][rr], want)
        assert err.max() < ROW_TOL, ("out", err.max())
        # probe rows are the exact rows (up to the output's rounding)
        err = row_rel_err(g["out"][hd][P], g["o_probe"][hd])
        assert err.max() < ROW_TOL


@pytest.mark.gpu
def test_bf16_score_bounds_small():
    """bf16 keys: every routing score of two heads lies within its reported bound of the oracle's
    fp64 score (one positive factor per row), the bounds are tight enough to leave most scores
    unrecomputed, and each selection equals the oracle's selection on the oracle's scores unless
    the oracle's boundary gap is a tie."""
    cfg = config("small")
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    T = O.key_budget(opc.rho, cfg.N, cfg.Nv, opc.M, 0)
    n_exact = n_all = n_out = 0
    for hd in (3, 8):
        kh, vh = (x[0, hd].astype(np.float64) for x in (k, v))
        nkv, nq = int(g["n_kv"][hd]), int(g["n_q"][hd])
        sc, _ = O.route_scores(g["qbar"][hd][:nq], kh, vh, g["kv_label"][hd], g["kbar"][hd][:nkv],
                               g["vbar"][hd][:nkv])
        size = np.diff(g["kv_off"][hd][: nkv + 1])
        for a in range(nq):
            ge = g["score_err"][hd][a][:nkv]
            _check_scores(g["scores"][hd][a][:nkv], ge, sc[a])
            n_exact += int((ge == 0).sum())
            n_out += int((ge < 0).sum())
            n_all += nkv
            sel, info = O.route_select(sc[a], size, T)
            if info["min_gap"] > TIE:
                cnt = int(g["sel_cnt"][hd][a])
                assert list(g["sel_kv"][hd][a][:cnt]) == list(sel), (hd, a)
    assert n_exact < 0.2 * n_all and n_out > 0.3 * n_all, (n_exact, n_out, n_all)


@pytest.mark.gpu
@pytest.mark.parametrize("Ck", [48, 200, 640])
def test_bf16_route_widths(Ck):
    """The bounded bf16 routing path at other K/V group counts (one, four and sixteen entries per
    lane of its ranking network): two heads of small end to end against the oracle."""
    cfg = config("small").with_(H=2, Ck=Ck)
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    rows = np.unique(np.concatenate([np.arange(0, cfg.N, 7), np.arange(cfg.N - 100, cfg.N)]))
    for h in (0, 1):
        ref = O.sparsepr_head(q[0, h], k[0, h], v[0, h], p, head=h, rows=rows)
        ref["lam"] = p.lam
        if _oracle_is_tie_free(ref):
            _compare_head(g, ref, h, cfg.Nv, cfg.N, cfg.n_text)
        else:
            _lockstep_head(g, q, k, v, cfg, opc, 0, h, np.random.default_rng(1))
        nkv = int(g["n_kv"][h])
        e = g["score_err"][h][: int(g["n_q"][h]), :nkv]
        assert np.all(np.isfinite(e)) and (e < 0).any()
    assert np.all(g["head_status"] & 1 == 0)


@pytest.mark.gpu
@pytest.mark.parametrize("grid,Ck,Cq,M,rho", [
    ((2, 8, 8), 96, 8, 8, 0.6),      # mostly one-key groups (exact zero scores in the bf16 path)
    ((1, 5, 29), 40, 9, 8, 0.3),     # 145 rows, ragged against every tile
    # many K/V groups at high density: paired small query groups whose union runs to hundreds of
    # segments per category (the segment tables of the sparse tiles near their capacity)
    ((8, 16, 16), 800, 256, 64, 0.8),
    ((8, 16, 16), 1000, 256, 64, 0.5),
])
def test_bf16_degenerate_groups(grid, Ck, Cq, M, rho):
    """Edge cases of the bounded bf16 routing on the positional workload (bf16, d = 128)."""
    cfg = config("small").with_(grid=grid, H=1, Ck=Ck, Cq=Cq, M=M, rho=rho, Ms=64)
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    ref = O.sparsepr_head(q[0, 0], k[0, 0], v[0, 0], p, head=0)
    ref["lam"] = p.lam
    if _oracle_is_tie_free(ref):
        _compare_head(g, ref, 0, cfg.Nv, cfg.N, cfg.n_text)
    else:
        _lockstep_head(g, q, k, v, cfg, opc, 0, 0, np.random.default_rng(1), nrows=64, ngroups=min(6, Cq))


@pytest.mark.gpu
def test_large_and_small_magnitude_values():
    """V far outside the fp16 range (head 0 scaled by 2^20, |v| up to ~4e6) and far below it
    (head 1 scaled by 2^-30): the fp16 copy of V is scaled by a power of two per K/V head and the
    scale undone on the output, so every stage still matches the oracle in lockstep."""
    cfg = config("small").with_(H=2)
    opc = op_config(cfg)
    q, k, v = batch_inputs(cfg)
    v = v.astype(np.float64)
    v[0, 0] *= 2.0 ** 20
    v[0, 1] *= 2.0 ** -30
    v = v.astype(np.float32)  # exact: bf16 values times a power of two
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    assert torch.equal(tv.float().cpu(), torch.from_numpy(v))
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    assert np.all(np.isfinite(g["o_sp"])) and np.all(np.isfinite(g["out"]))
    rng = np.random.default_rng(4)
    for h in (0, 1):
        _lockstep_head(g, q, k, v, cfg, opc, 0, h, rng)


@pytest.mark.gpu
@pytest.mark.parametrize("Cq", [48, 24])
def test_sparse_tiles_of_large_query_groups(Cq):
    """Query groups of 170 and 340 rows on average: most groups span several sparse tiles, and the
    rows past a group's full tiles are offered for pairing with other groups.  Two heads of small
    end to end against the oracle."""
    cfg = config("small").with_(H=2, Cq=Cq)
    assert cfg.Nv >= 96 * Cq
    opc = op_config(cfg)
    (q, k, v), (tq, tk, tv) = device_inputs(cfg)
    op = run_operator(cfg, opc, tq, tk, tv)
    g = pull(op)
    p = _oracle_params(opc, cfg.n_text)
    rows = np.unique(np.concatenate([np.arange(0, cfg.N, 5), np.arange(cfg.N - 100, cfg.N)]))
    for h in (0, 1):
        ref = O.sparsepr_head(q[0, h], k[0, h], v[0, h], p, head=h, rows=rows)
        ref["lam"] = p.lam
        if _oracle_is_tie_free(ref):
            _compare_head(g, ref, h, cfg.Nv, cfg.N, cfg.n_text)
        else:
            _lockstep_head(g, q, k, v, cfg, opc, 0, h, np.random.default_rng(5), nrows=256)
