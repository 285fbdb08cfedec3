"""Plain fp64 NumPy oracle of SparsePR's per-call sparse attention operator.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; nothing in the HIP library uses
it and the two share no code.

Source: "Partition the Support, Reconstruct the Residual: Training-Free Sparse
Attention for Video Generation and World Models" (Taghavi, Langari, Pandey),
paper text as rendered on paperpeel.com.  Each function names the section or
equation it follows.  Every step is a separate function so that tests can run
it on intermediates produced by the GPU ("lockstep").

Everything is fp64.  Inputs (bf16 or fp32 values) convert to fp64 exactly.

Readings taken where the pages are silent or garbled (all "parity unpinned"
against the pages; the tests pin them against mathematics instead):

* F = U_r diag(sqrt(lambda_r)) from the eigendecomposition of the metric,
  eigenvalues below ``eig_clamp * lambda_1`` set to zero.
* mu_K is the unweighted mean of the nonempty key-group centroids; C_k in M_Q
  counts nonempty groups.
* k-means: initial centres are feature rows drawn uniformly with replacement
  by SplitMix64; ties go to the lowest centre index; an empty centre keeps its
  previous position; a run stops after an assignment pass whose labels did not
  change or whose assignment cost fell by at most ``tol`` relative to the
  previous pass, or after ``max_iters`` passes.  Nonempty clusters are then
  renumbered in ascending order.
* Routing score overflow is avoided by a per-query-group shift (the order of
  the scores within a query group does not depend on it).  Score ties go to the
  lower K/V group.  The prefix is the shortest one whose key count reaches the
  budget, at least one group, all groups if the budget cannot be reached.
* Probe allocation (the text of App. A.2 that defines m_a is missing):
  largest-remainder apportionment of M over query groups by size; remainder
  ties go to the larger group, then the lower group id; inside a group the
  rows with the smallest d_i (ties: lower row index).
* Text tokens (trailing ``n_text`` rows): not partitioned; their keys form one
  extra group that every query group selects; their query rows attend densely;
  they take no part in probes or the fit.
* Later calls (App. C.1): the previous centroids in the original space go through
  the current feature map, RMSNorm included for queries; centre slots beyond the
  previous number of nonempty groups take the cold draws of their index.  The two
  subspace iterations start from the previous factor's columns scaled to unit length,
  orthonormalise by Cholesky QR and give F = U L with L L^T = U^T M U; a pivot of
  Z^T Z at or below eig_clamp^2, or of U^T M U at or below eig_clamp, times the
  largest diagonal entry (or a zero previous column) sends the head back to the cold
  eigendecomposition.
* Probe and estimator variants (Table 4; App. D.3, D.4): random probes are the M rows
  with the smallest SplitMix64 draws of a separate probe stream (a sample without
  replacement, nested in M); uniform spatiotemporal probes are M evenly spaced rows of
  the row-major (t, h, w) sequence; both carry weights Nv / M.  The output truncation
  takes the leading eigenvectors of Rbar^T W Rbar, eigenvalues at or below eig_clamp
  times the largest counted as absent.
* Semantic partition (Sec. 3.1; Table 2): k-means on the raw video keys and queries (d
  coordinates, no RMSNorm), the same initialisation and stopping rules; values inherit their
  key's group.  The key-response variant keeps the response-coupled K/V groups and takes
  semantic query groups.  Probe distances d_i are taken in the coordinates the query groups
  were formed in; warm starts map the previous centroids through the mode's feature map.
* Affine representability (App. D.5): least squares on [1, O_sp] via an SVD of the centred,
  column-scaled sparse outputs (relative tolerance 1e-10); explained fraction relative to the
  uncentred residual energy.
* Grouped-query attention (Sec. 4.3; App. C.2): the concatenation of the G heads'
  video query rows is sampled like one head's rows with G * Ms in place of Ms, which
  takes the same evenly spaced rows from each head.  The K/V k-means draws from the
  stream of the K/V head's index b * Hkv + j; the query k-means and random probes from
  that of the query head b * H + h, which uses K/V head h // G.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Params", "splitmix64", "init_indices", "sample_rows", "key_metric", "metric_factor",
    "project", "kmeans_assign", "kmeans_update", "kmeans", "compact_labels", "group_perm",
    "key_group_stats", "query_metric", "query_coords", "query_group_stats", "key_budget",
    "route_scores", "route_select", "route", "sparse_attention_rows", "dense_attention_rows",
    "select_probes_random", "select_probes_uniform", "output_projector",
    "executed_density", "allocate_probes", "select_probes", "ridge_fit", "correct", "relative_error",
    "sparsepr_head", "cholesky_upper", "metric_factor_warm", "warm_centres",
    "key_metric_shared", "kv_side", "query_side", "sparsepr_group", "affine_representability",
]

U64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


@dataclasses.dataclass
class Params:
    """Operator hyperparameters (Table C.1 of the paper's App. C.2 gives the defaults)."""
    Ck: int = 1000
    Cq: int = 300
    rK: int = 48
    rQ: int = 64
    Ms: int = 2048
    max_iters: int = 25
    tol: float = 1e-4
    rms_eps: float = 1e-6
    eig_clamp: float = 1e-6
    seed: int = 0
    M: int = 64
    rho: float = 0.22
    lam: float = 1.0
    std_eps: float = 1e-6
    n_text: int = 0
    probe_mode: str = "stratified"   # "stratified" | "random" | "uniform" (Table 4)
    fit_family: str = "full"         # "full" | "mean" | "scalar" | "diag" (App. D.4)
    out_rank: int = 0                # rank of the output truncation (App. D.3); 0: none
    partition_mode: str = "response"  # "response" | "semantic" | "key_response" (Sec. 3.1, Table 2)


# --------------------------------------------------------------------------- RNG
def splitmix64(seed: int, counter: int) -> int:
    """Counter-based SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): the output
    that the generator seeded with ``seed`` returns on call ``counter`` (0-based)."""
    z = (seed + (counter + 1) * GOLDEN_GAMMA) & U64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & U64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & U64
    return z ^ (z >> 31)


def init_indices(seed: int, head: int, stage: int, C: int, N: int) -> np.ndarray:
    """Initial k-means centres: C feature rows drawn uniformly with replacement
    (App. C.1).  Counter = ((head*2 + stage) << 20) + m; stage 0 = K/V, 1 = query."""
    base = (head * 2 + stage) << 20
    return np.array([splitmix64(seed, base + m) % N for m in range(C)], dtype=np.int64)


# ------------------------------------------------------------- metric and factors
def sample_rows(Nv: int, Ms: int) -> np.ndarray:
    """Evenly spaced query rows for the key metric (App. C.2: up to Ms rows, all
    rows when fewer are available): s_i = floor(i * Nv / Ms)."""
    m = min(Ms, Nv)
    return (np.arange(m, dtype=np.int64) * Nv) // m


def key_metric(Q: np.ndarray, Ms: int) -> np.ndarray:
    """Key-response metric M_K = Q_s^T Q_s / M_s (Sec. 4.1, App. B.1)."""
    Qs = np.asarray(Q, dtype=np.float64)[sample_rows(Q.shape[0], Ms)]
    return Qs.T @ Qs / Qs.shape[0]


def key_metric_shared(Qs: Sequence[np.ndarray], Ms: int) -> np.ndarray:
    """Key-response metric shared by the G query heads of one K/V head under grouped-query
    attention (Sec. 4.3, routing and GQA; App. C.2): their query rows are concatenated and
    up to G * Ms evenly spaced rows of the concatenation give one metric."""
    Qc = np.concatenate([np.asarray(Q, dtype=np.float64) for Q in Qs], axis=0)
    return key_metric(Qc, Ms * len(Qs))


def metric_factor(Mmat: np.ndarray, r: int, clamp: float) -> Tuple[np.ndarray, np.ndarray]:
    """Rank-r factor F with F F^T = the rank-r truncation of the metric (Sec. 4.1:
    distances in phi = x F reproduce the truncated response metric).
    Returns (F [d, r], eigenvalues descending after clamping)."""
    w, U = np.linalg.eigh(np.asarray(Mmat, dtype=np.float64))
    w, U = w[::-1].copy(), U[:, ::-1]
    top = w[0] if w.size and w[0] > 0 else 0.0
    w[w < clamp * top] = 0.0
    w[w < 0] = 0.0
    return U[:, :r] * np.sqrt(w[:r])[None, :], w


def project(X: np.ndarray, F: np.ndarray) -> np.ndarray:
    """Response coordinates phi(x) = x F (Sec. 4.1)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(F, dtype=np.float64)


# ------------------------------------------------------------------------ k-means
def kmeans_assign(X: np.ndarray, cent: np.ndarray):
    """Nearest centre by squared Euclidean distance, ties to the lowest index.
    Returns (labels, distance to the chosen centre, relative margin
    (d_second - d_best) / d_second per point).

    Distances are evaluated once per distinct centre position, each standing for the
    lowest index that holds it: bitwise-equal centres (duplicates of the sampling with
    replacement) then tie exactly, which a library matmul does not guarantee for two
    equal columns.  Margins are taken over distinct positions."""
    X = np.asarray(X, dtype=np.float64)
    cent = np.asarray(cent, dtype=np.float64)
    uniq, first = np.unique(cent, axis=0, return_index=True)
    order = np.argsort(first)
    uniq, first = uniq[order], first[order]
    D = (X * X).sum(1)[:, None] + (uniq * uniq).sum(1)[None, :] - 2.0 * (X @ uniq.T)
    labels = first[np.argmin(D, axis=1)]
    diff = X - cent[labels]
    dbest = (diff * diff).sum(1)
    if uniq.shape[0] > 1:
        part = np.partition(D, 1, axis=1)
        d2 = np.maximum(part[:, 1], 0.0)
        d1 = np.maximum(part[:, 0], 0.0)
        margin = np.where(d2 > 0, (d2 - d1) / np.where(d2 > 0, d2, 1.0), 0.0)
    else:
        margin = np.full(X.shape[0], np.inf)
    return labels.astype(np.int64), dbest, margin


def kmeans_update(X: np.ndarray, labels: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Lloyd update: each centre moves to the mean of its members; a centre with no
    members keeps its position."""
    X = np.asarray(X, dtype=np.float64)
    C = cent.shape[0]
    sums = np.zeros((C, X.shape[1]))
    np.add.at(sums, labels, X)
    cnt = np.bincount(labels, minlength=C)
    new = np.array(cent, dtype=np.float64, copy=True)
    nz = cnt > 0
    new[nz] = sums[nz] / cnt[nz, None]
    return new


def kmeans(X: np.ndarray, C: int, seed: int, head: int, stage: int, max_iters: int, tol: float,
           init: Optional[np.ndarray] = None):
    """k-means with C requested clusters (Sec. 4.1; App. C.1 initialisation, Table C.1
    limits).  ``init`` (C x r) replaces the sampled initial centres (warm start).
    Returns dict(labels (uncompacted), centres used by the final assignment, passes,
    min_margin, stop_margin)."""
    X = np.asarray(X, dtype=np.float64)
    N = X.shape[0]
    if init is None:
        cent = X[init_indices(seed, head, stage, C, N)].copy()
    else:
        cent = np.array(init, dtype=np.float64, copy=True)
        assert cent.shape == (C, X.shape[1])
    prev = None
    J_prev = None
    min_margin = np.inf
    stop_margin = np.inf
    t = 0
    for t in range(1, max_iters + 1):
        labels, dbest, margin = kmeans_assign(X, cent)
        min_margin = min(min_margin, float(margin.min()) if margin.size else np.inf)
        J = float(dbest.sum())
        if t > 1:
            if np.array_equal(labels, prev):
                break
            # distance of the tolerance decision from its threshold, relative
            gap = (J_prev - J) - tol * J_prev
            stop_margin = min(stop_margin, abs(gap) / max(tol * J_prev, 1e-300))
            if J_prev - J <= tol * J_prev:
                break
        if t == max_iters:
            break
        cent = kmeans_update(X, labels, cent)
        prev, J_prev = labels, J
    return dict(labels=labels, centres=cent, passes=t, min_margin=min_margin,
                stop_margin=stop_margin)


def compact_labels(labels: np.ndarray, C: int) -> Tuple[np.ndarray, int]:
    """Drop empty clusters and renumber the rest in ascending order (Sec. 4.1:
    C_k counts nonempty K/V groups)."""
    nonempty = np.bincount(labels, minlength=C) > 0
    newid = np.cumsum(nonempty) - 1
    return newid[labels].astype(np.int64), int(nonempty.sum())


def group_perm(labels_c: np.ndarray, n_groups: int) -> Tuple[np.ndarray, np.ndarray]:
    """Contiguous group-major order (Sec. 4.3), rows of a group in ascending original
    index.  Returns (perm: position -> original row, offsets [n_groups + 1])."""
    perm = np.argsort(labels_c, kind="stable")
    off = np.zeros(n_groups + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.bincount(labels_c, minlength=n_groups))
    return perm.astype(np.int64), off


# ------------------------------------------------------------ query coordinates
def key_group_stats(K: np.ndarray, V: np.ndarray, labels_c: np.ndarray, n_groups: int):
    """Group sizes and key / value centroids (original space) of the K/V groups."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    size = np.bincount(labels_c, minlength=n_groups)
    kbar = np.zeros((n_groups, K.shape[1]))
    vbar = np.zeros((n_groups, V.shape[1]))
    np.add.at(kbar, labels_c, K)
    np.add.at(vbar, labels_c, V)
    return size, kbar / size[:, None], vbar / size[:, None]


def query_metric(kbar: np.ndarray) -> np.ndarray:
    """Query-response metric M_Q = K~^T K~ / (C_k d), K~ rows = kbar_b - mu_K
    (Sec. 4.1; the centring of App. B.2)."""
    Ck, d = kbar.shape
    Kt = kbar - kbar.mean(0)[None, :]
    return Kt.T @ Kt / (Ck * d)


def query_coords(Q: np.ndarray, FQ: np.ndarray, eps: float) -> np.ndarray:
    """phi_Q(q) = RMSNorm(q F_Q) = q F_Q / max(sqrt(|q F_Q|^2 / r_Q), eps) (App. B.2)."""
    Y = np.asarray(Q, dtype=np.float64) @ FQ
    rms = np.sqrt((Y * Y).sum(1) / FQ.shape[1])
    return Y / np.maximum(rms, eps)[:, None]


def query_group_stats(Q: np.ndarray, phi: np.ndarray, labels_c: np.ndarray, n_groups: int):
    """Query-group sizes, mean queries qbar_a (original space), mean coordinates c_a
    and the distances d_i = |phi_Q(q_i) - c_a| of App. A.2."""
    Q = np.asarray(Q, dtype=np.float64)
    size = np.bincount(labels_c, minlength=n_groups)
    qbar = np.zeros((n_groups, Q.shape[1]))
    cbar = np.zeros((n_groups, phi.shape[1]))
    np.add.at(qbar, labels_c, Q)
    np.add.at(cbar, labels_c, phi)
    qbar /= size[:, None]
    cbar /= size[:, None]
    dist = np.sqrt(((phi - cbar[labels_c]) ** 2).sum(1))
    return size, qbar, cbar, dist


# -------------------------------------------------------------------- warm start
def cholesky_upper(G: np.ndarray, clamp: float) -> Optional[np.ndarray]:
    """Textbook Cholesky G = R^T R with R upper triangular, column by column.  Returns
    None when a pivot is not above clamp times the largest diagonal entry of G (G not
    numerically positive definite at the metric's eigenvalue clamp)."""
    G = np.asarray(G, dtype=np.float64)
    n = G.shape[0]
    R = np.zeros_like(G)
    floor = clamp * float(np.max(np.diag(G))) if n else 0.0
    for j in range(n):
        piv = G[j, j] - R[:j, j] @ R[:j, j]
        if not piv > floor:
            return None
        R[j, j] = math.sqrt(piv)
        R[j, j + 1:] = (G[j, j + 1:] - R[:j, j] @ R[:j, j + 1:]) / R[j, j]
    return R


def metric_factor_warm(Mmat: np.ndarray, F_prev: np.ndarray, r: int, clamp: float,
                       iters: int = 2) -> Tuple[np.ndarray, bool]:
    """Factor update of later calls (App. C.1): subspace iterations started from the span
    of the previous factor (its columns scaled to unit length), U <- orth(M U), each
    orthonormalised by Cholesky QR (Z = M U, Z^T Z = R^T R, U = Z R^{-1}); then F = U L
    with L L^T = U^T M U (Cholesky), so that F F^T = U U^T M U U^T, the metric compressed
    to the iterated subspace.  Z^T Z has the squared singular values of Z as its scale, so
    its pivots are tested against clamp^2 (Z numerically rank deficient at the metric's
    eigenvalue clamp), those of U^T M U against clamp.  A zero column of the previous
    factor or a failed pivot returns the cold factor instead.  Returns (F [d, r], warm_ok)."""
    M = np.asarray(Mmat, dtype=np.float64)
    U = np.array(F_prev, dtype=np.float64, copy=True)
    norms = np.sqrt((U * U).sum(0))
    if not np.all(norms > 0):
        return metric_factor(M, r, clamp)[0], False
    U /= norms[None, :]
    for _ in range(iters):
        Z = M @ U
        R = cholesky_upper(Z.T @ Z, clamp * clamp)
        if R is None:
            return metric_factor(M, r, clamp)[0], False
        U = np.linalg.solve(R.T, Z.T).T
    H = U.T @ (M @ U)
    H = 0.5 * (H + H.T)
    R = cholesky_upper(H, clamp)
    if R is None:
        return metric_factor(M, r, clamp)[0], False
    return U @ R.T, True


def warm_centres(prev_orig: np.ndarray, feature_map, X: np.ndarray, C: int, seed: int, head: int,
                 stage: int) -> np.ndarray:
    """Initial centres of a later call (App. C.1): the previous call's centroids in the
    original space, mapped by the current feature map (k F_K for keys, RMSNorm(q F_Q)
    for queries) into the current coordinates.  Slots beyond the previous number of
    groups take the cold draws of their index."""
    init = np.asarray(X, dtype=np.float64)[init_indices(seed, head, stage, C, X.shape[0])].copy()
    n = min(C, prev_orig.shape[0])
    if n:
        init[:n] = feature_map(prev_orig[:n])
    return init


# ---------------------------------------------------------------------- routing
def key_budget(rho: float, N: int, Nv: int, M: int, n_text: int) -> int:
    """Common per-query key budget after reserving probe cost (Sec. 4.3).  The
    executed-pair target rho * N^2 minus the fixed costs (probe rows against all
    keys, text query rows, text keys of every video row) is spread over the Nv
    video query rows; a prefix count is an integer, so reaching the real budget T
    means reaching ceil(T)."""
    total = rho * N * N
    fixed = float(n_text) * N + float(M) * N + float(Nv) * n_text
    T = (total - fixed) / Nv
    return int(math.ceil(T))


def executed_density(route_pairs: int, N: int, M: int, n_text: int) -> float:
    """rho_exec = rho_route + M / N_q (Sec. 4.3): routed pairs plus every exact pair of
    the M probe rows (counted although they are recomputed) and, with text tokens,
    the dense text query rows, over the N x N grid."""
    return (route_pairs + n_text * N + M * N) / float(N) ** 2


def route_scores(qbar: np.ndarray, K: np.ndarray, V: np.ndarray, kv_labels_c: np.ndarray,
                 kbar: np.ndarray, vbar: np.ndarray, groups: Optional[Sequence[int]] = None):
    """Value-error routing score of App. B.3:
    s_ab = 1/|G_b| sum_{j in G_b} | e^{qbar_a kbar_b / sqrt d} vbar_b - e^{qbar_a k_j / sqrt d} v_j |^2,
    evaluated with every exponent shifted by m_a = max over all logits of row a
    (one positive factor per query group, so the order within a row is unchanged).
    Returns scores [len(groups), C_k] and the shifts."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = K.shape[1]
    Ck = kbar.shape[0]
    size = np.bincount(kv_labels_c, minlength=Ck)
    rows = range(qbar.shape[0]) if groups is None else groups
    out = np.zeros((len(rows), Ck))
    shifts = np.zeros(len(rows))
    order = np.argsort(kv_labels_c, kind="stable")
    starts = np.concatenate([[0], np.cumsum(size)[:-1]])
    for ia, a in enumerate(rows):
        lbar = kbar @ qbar[a] / math.sqrt(d)
        lkey = K @ qbar[a] / math.sqrt(d)
        m = max(lbar.max(), lkey.max())
        A = np.exp(lbar - m)
        Bj = np.exp(lkey - m)
        diff = A[kv_labels_c][:, None] * vbar[kv_labels_c] - Bj[:, None] * V
        err = (diff * diff).sum(1)
        out[ia] = np.add.reduceat(err[order], starts) / size
        shifts[ia] = m
    return out, shifts


def route_select(scores_a: np.ndarray, kv_size: np.ndarray, T: int) -> Tuple[np.ndarray, Dict]:
    """Budgeted prefix (Sec. 4.3): rank K/V groups by descending score (ties to the
    lower group), keep the shortest prefix whose cumulative key count reaches T
    (at least one group; all groups if T is out of reach).  Returns the ranked
    selected groups and the relative score gaps next to the prefix boundary."""
    Ck = scores_a.shape[0]
    order = np.lexsort((np.arange(Ck), -scores_a))
    cum = np.cumsum(kv_size[order])
    hit = np.nonzero(cum >= T)[0]
    L = int(hit[0]) + 1 if hit.size else Ck
    L = max(L, 1)
    s = scores_a[order]
    gaps = []
    for t in range(max(L - 2, 0), min(L + 1, Ck - 1)):
        hi, lo = s[t], s[t + 1]
        gaps.append((hi - lo) / max(abs(hi), 1e-300))
    return order[:L].astype(np.int64), dict(L=L, min_gap=min(gaps) if gaps else np.inf)


def route(qbar, K, V, kv_labels_c, kbar, vbar, kv_size, T):
    """Scores and prefix for every query group.  Returns (list of ranked selections,
    scores, info list)."""
    scores, _ = route_scores(qbar, K, V, kv_labels_c, kbar, vbar)
    sel, info = [], []
    for a in range(qbar.shape[0]):
        s, inf = route_select(scores[a], kv_size, T)
        sel.append(s)
        info.append(inf)
    return sel, scores, info


# -------------------------------------------------------------------- attention
def _softmax_rows(Z: np.ndarray) -> np.ndarray:
    Z = Z - Z.max(1, keepdims=True)
    E = np.exp(Z)
    return E / E.sum(1, keepdims=True)


def dense_attention_rows(Q, K, V, rows) -> np.ndarray:
    """Dense attention O = softmax(Q K^T / sqrt d) V (Sec. 3) for the given rows."""
    Q = np.asarray(Q, dtype=np.float64)[np.asarray(rows)]
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    return _softmax_rows(Q @ K.T / math.sqrt(K.shape[1])) @ V


def sparse_attention_rows(Q, K, V, rows, q_labels_c, kv_labels_c, selections, n_text: int = 0):
    """Renormalised block-sparse output (Eq. (2) of Sec. 3): row i of video query
    group a attends to the keys of the selected K/V groups of a, plus the text keys;
    text query rows attend to every key."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = K.shape
    Nv = N - n_text
    kv_labels_c = np.asarray(kv_labels_c)
    out = np.zeros((len(rows), V.shape[1]))
    text = np.arange(Nv, N)
    for r, i in enumerate(rows):
        if i >= Nv:
            keys = np.arange(N)
        else:
            sel = selections[int(q_labels_c[i])]
            keys = np.nonzero(np.isin(kv_labels_c, sel))[0]
            keys = np.concatenate([keys, text])
        z = K[keys] @ Q[i] / math.sqrt(d)
        p = np.exp(z - z.max())
        out[r] = (p / p.sum()) @ V[keys]
    return out


# ------------------------------------------------------------------------ probes
def allocate_probes(q_size: np.ndarray, M: int) -> np.ndarray:
    """m_a: largest-remainder apportionment of M probes by group size, capped at the
    group size; remainder ties to the larger group, then the lower group id."""
    q_size = np.asarray(q_size, dtype=np.int64)
    Nv = int(q_size.sum())
    prod = M * q_size
    m = np.minimum(prod // Nv, q_size)
    rem = prod % Nv
    left = M - int(m.sum())
    order = sorted(range(q_size.size), key=lambda a: (-int(rem[a]), -int(q_size[a]), a))
    while left > 0:
        progressed = False
        for a in order:
            if left == 0:
                break
            if m[a] < q_size[a]:
                m[a] += 1
                left -= 1
                progressed = True
        if not progressed:
            break
    return m


def select_probes(q_labels_c: np.ndarray, dist: np.ndarray, q_size: np.ndarray, M: int):
    """Query-group-stratified probes (App. A.2): in each group the m_a rows closest to
    the group's mean coordinate (smallest d_i, ties to the lower row); weights
    w_p = |G_a| / m_a.  Returns (rows in group-major order, w, m_a)."""
    m = allocate_probes(q_size, M)
    rows, w = [], []
    for a in range(q_size.size):
        if m[a] == 0:
            continue
        members = np.nonzero(q_labels_c == a)[0]
        order = np.lexsort((members, dist[members]))
        take = members[order[: m[a]]]
        rows.extend(take.tolist())
        w.extend([q_size[a] / m[a]] * int(m[a]))
    return np.array(rows, dtype=np.int64), np.array(w, dtype=np.float64), m


PROBE_STREAM = 0x70726F6265  # "probe": the seed offset of the probe draws


def select_probes_random(Nv: int, M: int, seed: int, head: int):
    """Random probes (Table 4): the M video rows whose SplitMix64 draws
    splitmix64(seed xor "probe", head Nv + i) are smallest (ties to the lower row), i.e. a
    uniform sample without replacement whose draws for M probes contain those for fewer
    (nested probes, App. D.3).  Listed in ascending row; weights Nv / M."""
    keys = np.array([splitmix64(seed ^ PROBE_STREAM, head * Nv + i) for i in range(Nv)], dtype=np.uint64)
    order = np.lexsort((np.arange(Nv), keys))
    rows = np.sort(order[:M]).astype(np.int64)
    return rows, np.full(M, Nv / M)


def select_probes_uniform(Nv: int, M: int):
    """Uniform spatiotemporal probes (Table 4): with tokens in row-major (t, h, w) order, rows
    evenly spaced over the sequence, row_i = floor((2 i + 1) Nv / (2 M)) (the centre of each
    of M equal stretches); weights Nv / M."""
    i = np.arange(M, dtype=np.int64)
    return (2 * i + 1) * Nv // (2 * M), np.full(M, Nv / M)


# -------------------------------------------------------------------------- fit
def output_projector(Rb: np.ndarray, wt: np.ndarray, r: int, clamp: float) -> np.ndarray:
    """V_r V_r^T for the leading r right singular vectors of W^{1/2} Rbar (App. D.3), from
    the eigendecomposition of Rbar^T W Rbar; directions whose eigenvalue is at or below
    clamp times the largest count as absent (as in the metric factors)."""
    C = Rb.T @ (wt[:, None] * Rb)
    lam, U = np.linalg.eigh(C)
    idx = np.argsort(-lam, kind="stable")[:r]
    keep = [i for i in idx if lam[i] > 0 and lam[i] >= clamp * lam.max()]
    V = U[:, keep]
    return V @ V.T


def ridge_fit(X: np.ndarray, R: np.ndarray, w: np.ndarray, lam: float, std_eps: float, family: str = "full",
              out_rank: int = 0, clamp: float = 1e-6):
    """Weighted affine fit of Sec. 4.2 / App. A.3:
    alpha = w / sum w, W = diag(M w / sum w); features standardised with the
    alpha-weighted mean and sqrt(weighted variance + std_eps) (App. D.3); residuals
    centred by their alpha-weighted mean mu_R; B minimises
    |W^{1/2}(Rbar - Xbar B)|_F^2 + lam |B|_F^2, solved through the normal equations
    by Cholesky.  ``family`` restricts B as in App. D.4 (same weighted error and penalty):
    "mean" B = 0; "scalar" B = a I (penalty lam d a^2, a = tr H / tr G); "diag"
    B = diag(b) (b_c = H_cc / G_cc); "full" unrestricted.  ``out_rank`` r in [1, d)
    projects the centred prediction onto the leading r right singular vectors of
    W^{1/2} Rbar (App. D.3): B <- B V_r V_r^T; mu_R is not truncated.
    Returns dict(muX, sd, muR, B)."""
    X = np.asarray(X, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    M, d = X.shape
    alpha = w / w.sum()
    wt = M * w / w.sum()
    muX = alpha @ X
    var = alpha @ ((X - muX) ** 2)
    sd = np.sqrt(var + std_eps)
    Xb = (X - muX) / sd
    muR = alpha @ R
    Rb = R - muR
    G = Xb.T @ (wt[:, None] * Xb) + lam * np.eye(d)
    H = Xb.T @ (wt[:, None] * Rb)
    if family == "full":
        L = np.linalg.cholesky(G)
        B = np.linalg.solve(L.T, np.linalg.solve(L, H))
    elif family == "mean":
        B = np.zeros((d, d))
    elif family == "scalar":
        B = (np.trace(H) / np.trace(G)) * np.eye(d)
    elif family == "diag":
        B = np.diag(np.diag(H) / np.diag(G))
    else:
        raise ValueError(family)
    if 0 < out_rank < d:
        B = B @ output_projector(Rb, wt, out_rank, clamp)
    return dict(muX=muX, sd=sd, muR=muR, B=B)


def correct(O_sp: np.ndarray, fit: Dict) -> np.ndarray:
    """Residual prediction and corrected output for unprobed rows (Sec. 4.2):
    O_i + mu_R + ((O_i - mu_X) / sd) B."""
    O_sp = np.asarray(O_sp, dtype=np.float64)
    return O_sp + fit["muR"] + ((O_sp - fit["muX"]) / fit["sd"]) @ fit["B"]


def affine_representability(O_sp: np.ndarray, O_dense: np.ndarray, tol: float = 1e-10) -> Dict:
    """Oracle affine fit of App. D.5: the residual R = O_dense - O_sp of the given rows regressed
    on the features [1, O_sp] with all rows fitted.  Least squares through an SVD of the centred
    sparse outputs with columns scaled to unit norm, singular values at or below tol times the
    largest dropped; the residual mean is the intercept.  Returns the residual energy |R|^2, the
    remaining energy |R - R_hat|^2 and the explained fraction 1 - remaining / energy."""
    X = np.asarray(O_sp, dtype=np.float64)
    R = np.asarray(O_dense, dtype=np.float64) - X
    Xc = X - X.mean(axis=0)
    Rc = R - R.mean(axis=0)
    scale = np.linalg.norm(Xc, axis=0)
    scale[scale == 0.0] = 1.0
    U, S, _ = np.linalg.svd(Xc / scale, full_matrices=False)
    keep = S > tol * S[0] if S.size and S[0] > 0 else np.zeros(S.shape, dtype=bool)
    Uk = U[:, keep]
    remaining = float(((Rc - Uk @ (Uk.T @ Rc)) ** 2).sum())
    energy = float((R ** 2).sum())
    return dict(energy=energy, remaining=remaining, explained=1.0 - remaining / energy if energy > 0 else 1.0)


def relative_error(O: np.ndarray, O_dense: np.ndarray) -> np.ndarray:
    """Per-row |O_i - O_i^dense|_2 / (|O_i^dense|_2 + 1e-8) (caption of Table D.1)."""
    O = np.asarray(O, dtype=np.float64)
    O_dense = np.asarray(O_dense, dtype=np.float64)
    return np.linalg.norm(O - O_dense, axis=1) / (np.linalg.norm(O_dense, axis=1) + 1e-8)


# ------------------------------------------------------------------ whole head
def kv_side(qs: Sequence, k, v, p: Params, kv_head: int = 0, warm: Optional[Dict] = None) -> Dict:
    """The K/V side of one K/V head (Sec. 4.1, 4.2): key metric from the query rows of the heads
    in ``qs`` (one head, or the G heads that share this K/V head), key factor, K/V k-means, group
    statistics, query metric and query factor.  The k-means stream is that of ``kv_head``.
    ``p.partition_mode`` "semantic" clusters the raw keys instead (no metric or factor, Sec. 3.1);
    the query metric and factor are formed in "response" mode only, the one whose query
    coordinates use them."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = k.shape
    Nv = N - p.n_text
    kv, vv = k[:Nv], v[:Nv]
    qvs = [np.asarray(q, dtype=np.float64)[:Nv] for q in qs]
    warm_ok = []
    MK = FK = wK = None
    if p.partition_mode == "semantic":
        phiK = kv.copy()
        feature_map = lambda x: np.asarray(x, dtype=np.float64)  # noqa: E731
    else:
        MK = key_metric(qvs[0], p.Ms) if len(qvs) == 1 else key_metric_shared(qvs, p.Ms)
        if warm is None:
            FK, wK = metric_factor(MK, p.rK, p.eig_clamp)
        else:
            FK, ok = metric_factor_warm(MK, warm["FK"], p.rK, p.eig_clamp)
            warm_ok.append(ok)
        phiK = project(kv, FK)
        feature_map = lambda x: project(x, FK)  # noqa: E731
    initK = None if warm is None else warm_centres(warm["kbar"], feature_map, phiK, p.Ck, p.seed, kv_head, 0)
    km = kmeans(phiK, p.Ck, p.seed, kv_head, 0, p.max_iters, p.tol, init=initK)
    kv_lab, nkv = compact_labels(km["labels"], p.Ck)
    kv_size, kbar, vbar = key_group_stats(kv, vv, kv_lab, nkv)
    MQ = FQ = wQ = None
    if p.partition_mode == "response":
        MQ = query_metric(kbar)
        if warm is None:
            FQ, wQ = metric_factor(MQ, p.rQ, p.eig_clamp)
        else:
            FQ, ok = metric_factor_warm(MQ, warm["FQ"], p.rQ, p.eig_clamp)
            warm_ok.append(ok)
    return dict(MK=MK, FK=FK, wK=wK, phiK=phiK, kmK=km, kv_label=kv_lab, n_kv=nkv, kv_size=kv_size,
                kbar=kbar, vbar=vbar, MQ=MQ, FQ=FQ, wQ=wQ, warm_ok=warm_ok)


def query_side(q, k, v, kvs: Dict, p: Params, head: int = 0, rows: Optional[Sequence[int]] = None,
               full: bool = True, warm: Optional[Dict] = None) -> Dict:
    """The query side of one query head given its K/V head's ``kv_side`` result: query
    partition (Sec. 4.2), routing (Sec. 4.3), probes (App. A.2), and with ``full`` the sparse
    and probe attention, the ridge fit and the correction (Sec. 4.4).  Streams are those of
    ``head``; ``warm`` supplies the previous query centroids ``qbar``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    Nv = N - p.n_text
    qv, kv, vv = q[:Nv], k[:Nv], v[:Nv]
    FQ, kv_lab, kv_size = kvs["FQ"], kvs["kv_label"], kvs["kv_size"]
    out: Dict = dict(kvs)
    if p.partition_mode == "response":
        phiQ = query_coords(qv, FQ, p.rms_eps)
        feature_map = lambda x: query_coords(x, FQ, p.rms_eps)  # noqa: E731
    else:  # semantic query groups: k-means on the raw queries (Sec. 3.1)
        phiQ = qv.copy()
        feature_map = lambda x: np.asarray(x, dtype=np.float64)  # noqa: E731
    initQ = None if warm is None else warm_centres(warm["qbar"], feature_map, phiQ, p.Cq, p.seed, head, 1)
    qm = kmeans(phiQ, p.Cq, p.seed, head, 1, p.max_iters, p.tol, init=initQ)
    q_lab, nq = compact_labels(qm["labels"], p.Cq)
    q_size, qbar, cbar, dist = query_group_stats(qv, phiQ, q_lab, nq)
    T = key_budget(p.rho, N, Nv, p.M, p.n_text)
    sel, scores, rinfo = route(qbar, kv, vv, kv_lab, kvs["kbar"], kvs["vbar"], kv_size, T)
    pairs = int(sum(int(q_size[a]) * (int(kv_size[sel[a]].sum()) + p.n_text) for a in range(nq)))
    rho_exec = executed_density(pairs, N, p.M, p.n_text)
    if p.probe_mode == "stratified":
        probes, w, m_a = select_probes(q_lab, dist, q_size, p.M)
    elif p.probe_mode == "random":
        (probes, w), m_a = select_probes_random(Nv, p.M, p.seed, head), None
    elif p.probe_mode == "uniform":
        (probes, w), m_a = select_probes_uniform(Nv, p.M), None
    else:
        raise ValueError(p.probe_mode)
    out.update(phiQ=phiQ, kmQ=qm, q_label=q_lab, n_q=nq,
               q_size=q_size, qbar=qbar, cbar=cbar, qdist=dist, T=T, sel=sel, scores=scores,
               route_info=rinfo, pairs=pairs, rho_exec=rho_exec, probes=probes, probe_w=w, m_a=m_a,
               state=dict(FK=kvs["FK"], FQ=FQ, kbar=kvs["kbar"], qbar=qbar))
    if not full:
        return out
    q_lab_full = np.concatenate([q_lab, np.full(p.n_text, -1)])
    X = sparse_attention_rows(q, k, v, probes, q_lab_full, kv_lab, sel, p.n_text)
    Od = dense_attention_rows(q, k, v, probes)
    fit = ridge_fit(X, Od - X, w, p.lam, p.std_eps, p.fit_family, p.out_rank, p.eig_clamp)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    Osp = sparse_attention_rows(q, k, v, rows, q_lab_full, kv_lab, sel, p.n_text)
    Ohat = Osp.copy()
    video = rows < Nv
    Ohat[video] = correct(Osp[video], fit)
    pos = {int(r): i for i, r in enumerate(probes)}
    for ir, r in enumerate(rows):
        if int(r) in pos:
            Ohat[ir] = Od[pos[int(r)]]
    out.update(rows=rows, O_sp=Osp, O_hat=Ohat, probe_dense=Od, probe_sparse=X, fit=fit)
    return out


def sparsepr_head(q, k, v, p: Params, head: int = 0, rows: Optional[Sequence[int]] = None,
                  full: bool = True, warm: Optional[Dict] = None) -> Dict:
    """One head of the operator, every stage in the order of Sec. 4 and App. C.3.
    ``rows`` limits the attention outputs to a subset (default: all rows).  ``warm``
    (the ``state`` of the previous call of this head: FK, FQ, kbar, qbar) selects the
    later-call path of App. C.1: factors by subspace iteration from the previous ones
    and k-means started from the previous centroids."""
    kvs = kv_side([q], k, v, p, head, warm)
    return query_side(q, k, v, kvs, p, head, rows, full, warm)


def sparsepr_group(qs: Sequence, k, v, p: Params, kv_head: int, heads: Sequence[int],
                   rows: Optional[Sequence[int]] = None, full: bool = True,
                   warm: Optional[Sequence[Dict]] = None) -> List[Dict]:
    """Grouped-query attention (Sec. 4.3, routing and GQA; App. C.2): the G query heads ``qs``
    (stream indices ``heads``) share K/V head ``kv_head`` (k, v): one shared key metric and K/V
    partition, then a query partition, routing, probes and fit per query head.  ``warm`` is the
    list of the heads' previous ``state``s (their K/V-side entries are the shared ones)."""
    kvs = kv_side(qs, k, v, p, kv_head, None if warm is None else warm[0])
    return [query_side(q, k, v, kvs, p, h, rows, full, None if warm is None else warm[g])
            for g, (q, h) in enumerate(zip(qs, heads))]
