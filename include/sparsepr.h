/*
 * sparsepr.h - C ABI of an MI355X (gfx950) implementation of SparsePR's
 * per-call sparse attention operator.
 *
 * Source of the method: "Partition the Support, Reconstruct the Residual:
 * Training-Free Sparse Attention for Video Generation and World Models"
 * (Taghavi, Langari, Pandey).  Section references below are to that paper.
 *
 * One operator call, for every (batch, head), maps Q, K, V [N, d] to the
 * corrected output O^hat [N, d] in five stream-ordered calls:
 *
 *   sparsepr_partition    response-coupled partitioning (Sec. 4.1, App. B.1-B.2)
 *   sparsepr_route        routing scores, budgeted prefixes, probe choice
 *                         (Sec. 4.3, App. B.3, App. A.2)
 *   sparsepr_attn_sparse  renormalised block-sparse attention (Eq. (2), Sec. 3)
 *   sparsepr_probe_exact  exact dense attention of the probe rows (Sec. 4.2)
 *   sparsepr_fit_correct  weighted ridge fit + correction + order restore
 *                         (Sec. 4.2, App. A.3)
 *
 * Conventions shared by every call
 * ---------------------------------
 *  - All data pointers are DEVICE pointers unless a parameter says "host".
 *    The caller allocates every buffer (the library never allocates device
 *    memory) and keeps it alive until the stream has passed the call.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Nothing synchronises with the host; counts that depend on the data stay
 *    on the device.
 *  - Heads are flattened: head index hd = b * H + h, BH = B * H.  Per-head
 *    arrays below are laid out [BH][...] with the stated inner size even where
 *    the used part is smaller (for example only n_kv[hd] of Ck groups).
 *  - The last n_text of the N tokens of a head are text tokens: they are not
 *    partitioned, their keys form one extra K/V group (index n_kv[hd]) that
 *    every query group selects, and their query rows attend to all keys.
 *    Nv = N - n_text video tokens are partitioned.
 *  - Every call first validates its arguments on the host and returns a
 *    status without launching anything when they are invalid:
 *      SPR_EINVAL        null pointer, bad size or parameter (see each call)
 *      SPR_EUNSUPPORTED  head dimension or dtype not built, or one head's rows
 *                        span 2 GiB or more (the kernels use 32-bit offsets
 *                        within a head)
 *      SPR_EWORKSPACE    workspace smaller than sparsepr_workspace_size()
 *      SPR_EHIP          a HIP launch failed (the stream state is undefined)
 *      SPR_ETOOLARGE     the problem needs more scratch than the fixed array of
 *                        the allocation-free call holds
 *    Anomalies that depend on the data are reported per head in the device
 *    array `head_status` of sparsepr_fit_correct (SPR_HS_* bits).
 *  - The workspace `ws` is scratch owned by the caller; the same workspace
 *    must be passed to all five calls of one operator invocation (later calls
 *    read state that earlier ones left there) and must not be shared by two
 *    invocations in flight.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPR_OK = 0,
  SPR_EINVAL = 1,
  SPR_EUNSUPPORTED = 2,
  SPR_EWORKSPACE = 3,
  SPR_EHIP = 4,
  SPR_ETOOLARGE = 5
} spr_status;

typedef enum { SPR_BF16 = 0, SPR_F32 = 1 } spr_dtype;

/* per-head status bits written by sparsepr_fit_correct */
enum {
  SPR_HS_CHOLESKY_FALLBACK = 1, /* normal matrix not positive definite: mean-only correction */
  SPR_HS_BUDGET_UNREACHED = 2,  /* some query group selected every K/V group below budget */
  SPR_HS_KV_GROUPS_EMPTY = 4,   /* fewer nonempty K/V groups than requested */
  SPR_HS_Q_GROUPS_EMPTY = 8,    /* fewer nonempty query groups than requested */
  SPR_HS_RMS_FLOOR = 16,        /* some query coordinate norm fell below rms_eps */
  SPR_HS_EIGEN_NOCONV = 32      /* a metric eigendecomposition did not converge in 60 QL iterations */
};

/* Shape of q, k, v: element (b, h, n, c) of q lives at b*sb + h*sh + n*sn + c.
   Grouped-query attention: with 0 < Hkv < H (H % Hkv == 0, G = H / Hkv) k and v hold Hkv heads,
   element (b, j, n, c) at b*ksb + j*ksh + n*ksn + c, and query head h attends with K/V head
   h / G; the key metric and the K/V partition are shared by the G query heads of a K/V head,
   the query partition and the routing are per query head (Sec. 4.3, routing and GQA; App. C.2,
   which samples up to G * Ms rows of the G heads for the shared metric).  Hkv = 0 or
   Hkv = H: one K/V head per query head, k and v with the strides of q (ksb .. ksn unused). */
typedef struct {
  int32_t B, H, N, d; /* d in {64, 128}; N includes the n_text trailing text tokens */
  int32_t n_text;     /* 0 <= n_text < N */
  int32_t dtype;      /* spr_dtype of q, k, v */
  int64_t sb, sh, sn; /* element strides; the innermost stride is 1 */
  int32_t Hkv;        /* K/V heads (see above) */
  int32_t reserved;   /* 0 */
  int64_t ksb, ksh, ksn; /* element strides of k and v when 0 < Hkv < H */
} spr_desc;

/* Partition construction (spr_part_params.mode).  RESPONSE is the operator's response-coupled
   partition (Sec. 4.1).  SEMANTIC is the reference partition of Sec. 3.1 and Table 2: k-means
   on the raw key and query activations (d coordinates, no factor, no normalisation), each value
   inheriting its key's group.  KEY_RESPONSE is the Table 2 variant that changes only the K/V
   grouping: response-coupled K/V groups, semantic (raw) query groups.  Routing, probes and the
   fit are the same in every mode, and the query distances d_i of App. A.2 are taken in the
   coordinates the query groups were formed in. */
typedef enum { SPR_PART_RESPONSE = 0, SPR_PART_SEMANTIC = 1, SPR_PART_KEY_RESPONSE = 2 } spr_part_mode;

/* Partition hyperparameters (defaults of Table C.1, App. C.2, in brackets). */
typedef struct {
  int32_t Ck, Cq;    /* requested K/V and query groups [1000, 300]; 1 <= C <= min(Nv, 1024) */
  int32_t rK, rQ;    /* response ranks [48, 64]; in {8, 16, 32, 48, 64}, <= d */
  int32_t Ms;        /* metric query-sampling budget [2048]; min(Ms, Nv) evenly spaced rows */
  int32_t max_iters; /* k-means assignment passes [25]; >= 1 */
  double tol;        /* k-means relative cost-decrease tolerance [1e-4]; >= 0 */
  double rms_eps;    /* RMSNorm floor of the query coordinates [1e-6]; > 0 */
  double eig_clamp;  /* eigenvalues below eig_clamp * lambda_max count as zero [1e-6] */
  uint64_t seed;     /* k-means initialisation seed (SplitMix64) */
  int32_t mode;      /* spr_part_mode [SPR_PART_RESPONSE]; raw coordinates have rank d (k-means
                        coordinates, phiK / phiQ and the k-means centres are then d wide) */
  int32_t reserved;  /* 0 */
} spr_part_params;

/* Outputs of sparsepr_partition (caller-owned device buffers).  Arrays of the K/V side are per
   K/V head, BHkv = B * Hkv (BHkv = BH without grouped-query attention); K/V head j serves the
   query heads j G .. j G + G - 1 of the flattened index. */
typedef struct {
  int32_t* kv_label; /* [BHkv][Nv] K/V group of each video key, original order, groups renumbered
                                  0..n_kv-1 in ascending cluster id (empty clusters dropped) */
  int32_t* q_label;  /* [BH][Nv]  query group of each video query row, likewise */
  int32_t* kv_perm;  /* [BHkv][Nv] group-major position -> original key row (stable) */
  int32_t* q_perm;   /* [BH][Nv]  group-major position -> original query row (stable) */
  int32_t* q_pos;    /* [BH][Nv]  original query row -> group-major position */
  int32_t* kv_off;   /* [BHkv][Ck+1] start of each K/V group in kv_perm order; kv_off[n_kv] = Nv */
  int32_t* q_off;    /* [BH][Cq+1] start of each query group; q_off[n_q] = Nv */
  int32_t* n_kv;     /* [BHkv] nonempty K/V groups */
  int32_t* n_q;      /* [BH] nonempty query groups */
  double* kbar;      /* [BHkv][Ck][d] key centroids of the K/V groups (original space) */
  double* vbar;      /* [BHkv][Ck][d] value centroids */
  double* qbar;      /* [BH][Cq][d] mean query of each query group */
  double* qdist;     /* [BH][Nv]  |phi_Q(q_i) - c_a| (App. A.2), original order */
  double* FK;        /* [BHkv][d][rK] key response factor, F F^T = rank-rK truncation of M_K
                        (not written in SEMANTIC mode) */
  double* FQ;        /* [BHkv][d][rQ] query response factor (M_Q depends on the K/V side only;
                        written in RESPONSE mode only) */
  void* Qp;          /* [BH][N][d] q rows in group-major order, then the text rows; input dtype */
  void* Kp;          /* [BHkv][N][d] k rows likewise (kv_perm order) */
  void* Vp;          /* [BHkv][N][d] v rows likewise (kv_perm order) */
  /* optional diagnostics, each may be NULL */
  double* phiK;      /* [BHkv][Nv][rK] key coordinates k F_K (raw k, rank d, in SEMANTIC mode) */
  double* phiQ;      /* [BH][Nv][rQ] query coordinates RMSNorm(q F_Q) (raw q, rank d, unless
                        RESPONSE mode) */
  double* cK_last;   /* [BHkv][Ck][rK] k-means centres used by the final K/V assignment pass */
  double* cQ_last;   /* [BH][Cq][rQ] k-means centres used by the final query assignment pass
                        (rK, rQ: the coordinate ranks of the mode) */
  int32_t* passes;   /* [BH][2] assignment passes: [j][0] of the K/V k-means of K/V head j < BHkv,
                                  [hd][1] of the query k-means of query head hd */
} spr_partition;

/* State of the previous call of the same heads, for the later-call path of App. C.1
   (device buffers laid out as the corresponding spr_partition outputs; they may be the
   very buffers this call writes: every one is read before it is overwritten). */
typedef struct {
  const double* FK;    /* [BHkv][d][rK] previous key response factor */
  const double* FQ;    /* [BHkv][d][rQ] previous query response factor */
  const double* kbar;  /* [BHkv][Ck][d] previous key centroids (original space) */
  const double* qbar;  /* [BH][Cq][d] previous mean queries (original space) */
  const int32_t* n_kv; /* [BHkv] previous nonempty K/V groups */
  const int32_t* n_q;  /* [BH] previous nonempty query groups */
} spr_warm;

/* Outputs of sparsepr_route (caller-owned device buffers). */
typedef struct {
  int32_t* sel_cnt;   /* [BH][Cq+1] number of selected K/V groups of each query group; entry n_q
                                    is the text query group (when n_text > 0) */
  int32_t* sel_kv;    /* [BH][Cq+1][Ck+1] selected video K/V groups in descending score order,
                                    followed by the text group n_kv when n_text > 0 */
  int32_t* probe_idx; /* [BH][M] original row of each probe: stratified probes group-major, nearest
                                 first; the other modes in ascending row */
  double* probe_w;    /* [BH][M] coverage weight w_p (|G_a| / m_a, or Nv / M) */
  int64_t* pairs;     /* [BH] routed query-key pairs, text keys of video rows included */
  double* rho_exec;   /* [BH] executed-pair density incl. probes and text rows */
  double* scores;     /* optional [BH][Cq][Ck] routing scores times a positive per-row factor */
  double* score_err;  /* optional [BH][Cq][Ck] bound on |scores - exact score| (same factor): 0 where
                                 the score was computed in fp64 (every score of fp32 inputs),
                                 negated where the group cannot enter the budgeted prefix */
} spr_route;

/* Probe choice of sparsepr_route (Table 4; App. D.3).  Weights w_p: |G_a| / m_a for stratified
   probes, Nv / M for the others. */
typedef enum {
  SPR_PROBES_STRATIFIED = 0, /* query-group stratified (App. A.2), the operator's choice */
  SPR_PROBES_RANDOM = 1,     /* the M video rows i with the smallest SplitMix64 draws
                                splitmix64(seed ^ 0x70726F6265, hd * Nv + i) (ties to the lower row):
                                a uniform sample without replacement, nested in M */
  SPR_PROBES_UNIFORM = 2     /* evenly spaced rows floor((2 i + 1) Nv / (2 M)), i < M (row-major
                                (t, h, w) tokens: uniform over the spatiotemporal grid) */
} spr_probe_mode;

typedef struct {
  int32_t mode;  /* spr_probe_mode */
  uint64_t seed; /* SPR_PROBES_RANDOM only */
} spr_probe_options;

/* Estimator of sparsepr_fit_correct (App. D.3, D.4).  Every family minimises the same weighted
   squared error with penalty lam |B|_F^2. */
typedef enum {
  SPR_FIT_FULL = 0,   /* unrestricted B (the operator's choice) */
  SPR_FIT_MEAN = 1,   /* B = 0: the weighted mean residual only */
  SPR_FIT_SCALAR = 2, /* B = a I, a = tr H / tr G (penalty lam d a^2) */
  SPR_FIT_DIAG = 3    /* B = diag(b), b_c = H_cc / G_cc */
} spr_fit_family;

typedef struct {
  int32_t family;   /* spr_fit_family */
  int32_t out_rank; /* r in [1, d): the centred prediction is projected onto the r leading right
                       singular vectors of W^{1/2} Rb (B <- B V_r V_r^T; eigenvalues of Rb^T W Rb
                       at or below eig_clamp times the largest count as absent); 0 or >= d: none */
} spr_fit_options;

/* Bytes of workspace the five calls need for this shape (host function, no device work).
   Returns 0 when the arguments are invalid. */
size_t sparsepr_workspace_size(const spr_desc* desc, const spr_part_params* params, int32_t M);

/* Response-coupled partitioning (Sec. 4.1, App. B.1-B.2, App. C.1):
   M_K from min(Ms, Nv) evenly spaced video query rows; F_K from its eigendecomposition;
   k-means of phi_K = k F_K into Ck K/V groups (values follow their keys); key/value
   centroids; M_Q = K~^T K~ / (n_kv d) with K~ the centred key centroids; F_Q;
   phi_Q = RMSNorm(q F_Q); k-means into Cq query groups; group-major copies of Q, K, V.
   `warm` (nullable) selects the later-call path of App. C.1: each factor comes from two
   subspace iterations started at the previous factor (Cholesky QR, then F = U L with
   L L^T = U^T M U), a head whose Cholesky meets a pivot at or below eig_clamp times the
   largest diagonal entry takes the eigendecomposition instead; each k-means starts from
   the previous centroids mapped into the current coordinates (k F_K, RMSNorm(q F_Q)), slots
   beyond the previous group count from the cold draws.  The caller sets max_iters (2 in
   Table C.1) for such calls.
   EINVAL: null required pointer, B, H < 1, N < 2, n_text out of range, strides,
   C, r, Ms, max_iters, tol, rms_eps, eig_clamp out of range, a null member of *warm. */
spr_status sparsepr_partition(const spr_desc* desc, const void* q, const void* k, const void* v,
                              const spr_part_params* params, const spr_warm* warm, spr_partition* out,
                              void* ws, size_t ws_bytes, void* stream);

/* Routing and probe selection (Sec. 4.3, App. B.3, App. A.2):
   value-error scores s_ab for every (query group, K/V group); per query group the
   shortest descending-score prefix whose key count reaches the common budget
   ceil((rho*N^2 - n_text*N - M*N - Nv*n_text) / Nv); M probe rows stratified by query
   group (or the choice in `probes`, host, nullable: NULL is SPR_PROBES_STRATIFIED).
   `rho_exec_target` is the total executed-pair target including probes.
   The prefixes and their order are those of the fp64 scores: for bf16 keys the scores run on
   the bf16 matrix cores with a rigorous bound each, and the scores the prefix depends on are
   recomputed in fp64 (ties of exactly equal scores go to the lower group).
   EINVAL: 1 <= M < Nv violated, the budget is below one key, an unknown probe mode. */
spr_status sparsepr_route(const spr_desc* desc, const spr_part_params* params, const spr_partition* part,
                          double rho_exec_target, int32_t M, const spr_probe_options* probes, spr_route* out,
                          void* ws, size_t ws_bytes, void* stream);

/* Renormalised block-sparse attention (Eq. (2)): each row of query group a attends to the
   keys of its selected K/V groups (and the text keys); text rows attend to all keys.
   o_sp: [BH][N][d] fp32, rows in Qp order.
   Numeric domain of bf16 inputs: scores are exact products summed in fp32; P and V enter the
   P V products in fp16, V scaled per K/V head by the power of two 2^e that puts its largest
   magnitude in [2^14, 2^15) (|e| <= 100, undone on the output), so the whole bf16 range is
   accepted; entries below 2^-24 of their head's largest magnitude are rounded to fp16 steps
   of that size.  Non-finite values propagate. */
spr_status sparsepr_attn_sparse(const spr_desc* desc, const spr_part_params* params,
                                const spr_partition* part, const spr_route* route, float* o_sp,
                                void* ws, size_t ws_bytes, void* stream);

/* Exact dense attention (Eq. (1)) of the probe rows probe_idx [BH][M] against all N keys of the
   original q, k, v.  o_probe: [BH][M][d] fp32.  The workspace of this call is its own (split-K
   partials and, for bf16, a scaled fp16 copy of v; numeric domain as sparsepr_attn_sparse), of
   sparsepr_probe_workspace_size() bytes; it may be any buffer not in use by the other calls.
   EWORKSPACE: ws_bytes below that size. */
spr_status sparsepr_probe_exact(const spr_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* probe_idx, int32_t M, float* o_probe, void* ws,
                                size_t ws_bytes, void* stream);

/* Workspace bytes of sparsepr_probe_exact (host; 0 for invalid arguments). */
size_t sparsepr_probe_workspace_size(const spr_desc* desc, int32_t M);

/* Weighted ridge fit of the probe residuals against the sparse outputs and correction of the
   unprobed rows (Sec. 4.2, App. A.3, App. D.3): alpha = w / sum w; W = diag(M w / sum w);
   features standardised by the alpha-weighted mean and sqrt(weighted variance + std_eps);
   residuals centred by their weighted mean mu_R; B = (Xb^T W Xb + lam I)^-1 Xb^T W Rb (fp64
   Cholesky); O^hat_i = O^sp_i + mu_R + Xb_i B for unprobed video rows, the exact row for probes,
   O^sp for text rows.  `out` is [B][H][N][d] contiguous in original row order, fp32 or bf16
   (out_dtype).  `opts` (host, nullable: NULL is the full ridge without truncation) selects the
   estimator family and output truncation of App. D.3-D.4.  `fit_state` (nullable) receives
   [BH][3d + d*d] fp64: mu_X, sd, mu_R, B.  `head_status` [BH] receives SPR_HS_* bits.
   EINVAL: lam < 0, std_eps <= 0, M out of range, an unknown family, out_rank < 0. */
spr_status sparsepr_fit_correct(const spr_desc* desc, const spr_part_params* params,
                                const spr_partition* part, const spr_route* route, const float* o_sp,
                                const float* o_probe, int32_t M, double lam, double std_eps,
                                const spr_fit_options* opts, void* out, int32_t out_dtype, double* fit_state,
                                int32_t* head_status, void* ws, size_t ws_bytes, void* stream);

/* Baseline: dense flash attention softmax(q k^T / sqrt d) v for every row, same kernel as
   sparsepr_attn_sparse.  out: [B][H][N][d] contiguous, fp32 or bf16 (out_dtype).  ws: scratch of
   sparsepr_dense_workspace_size() bytes (the scaled fp16 copy of v for bf16 inputs).
   EWORKSPACE: ws_bytes below that size. */
spr_status sparsepr_attn_dense(const spr_desc* desc, const void* q, const void* k, const void* v,
                               void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of sparsepr_attn_dense (host; 0 for an invalid descriptor). */
size_t sparsepr_dense_workspace_size(const spr_desc* desc);

/* sparsepr_attn_dense for callers that cannot allocate device memory (work under HIP graph
   capture, tight serving loops, harnesses that forbid allocation): same arguments, kernels and
   result, without a workspace argument.  The scratch (the scaled fp16 copy of v for bf16 inputs)
   is a fixed array of SPR_NOALLOC_SCRATCH_BYTES in device memory that the library holds on every
   device it runs on until the process ends; its address is looked up once per device on the first
   call there.  The call allocates nothing.  Every call on one device shares that array, which keeps
   the last call's contents: calls that overlap on one device (two streams, two host threads) race
   and must be serialised by the caller.  ETOOLARGE: sparsepr_dense_workspace_size(desc) exceeds
   SPR_NOALLOC_SCRATCH_BYTES (for bf16, B * kv heads * N * d above about 32 Mi elements).
   EHIP: the scratch's device address could not be obtained. */
#define SPR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
spr_status sparsepr_attn_dense_noalloc(const spr_desc* desc, const void* q, const void* k, const void* v,
                                       void* out, int32_t out_dtype, void* stream);

/* Test helper: k-means of `feat` [BH][n][r] fp64 (r in {8, 16, 32, 48, 64, 128},
   C <= min(n, 1024)) with the operator's initialisation (stage 0 or 1), assignment, update and
   stopping rules.  labels [BH][n] receive
   the uncompacted cluster ids; centres [BH][C][r] the centres used by the final assignment pass;
   passes [BH] the number of assignment passes. */
spr_status sparsepr_kmeans(int32_t BH, int32_t n, int32_t r, int32_t C, const double* feat, uint64_t seed,
                           int32_t stage, int32_t max_iters, double tol, int32_t* labels, double* centres,
                           int32_t* passes, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of sparsepr_kmeans. */
size_t sparsepr_kmeans_workspace_size(int32_t BH, int32_t n, int32_t r, int32_t C);

/* Static description of a status code (host). */
const char* sparsepr_status_string(spr_status s);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEPR_H */
