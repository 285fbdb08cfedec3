// extern "C" entry points of libsparsepr: argument validation, workspace layout and the
// stream-ordered stage launches.  Validation runs on the host before any HIP call, so a
// rejected call has no effect on the device.
#include <cmath>

#include "common.hpp"
#include "stages.hpp"

namespace spr {

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

Workspace layout(const spr_desc& desc, const spr_part_params& p, int M) {
  Workspace L = {};
  const size_t BH = size_t(desc.B) * desc.H, d = desc.d, Nv = size_t(desc.N - desc.n_text);
  const int rK = kv_coord_rank(p, int(d)), rQ = q_coord_rank(p, int(d));
  L.Cmax = p.Ck > p.Cq ? p.Ck : p.Cq;
  L.rmax = rK > rQ ? rK : rQ;
  L.nblk = int((Nv + kAssignThreads - 1) / kAssignThreads);
  L.splits = kProbeSplits;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.metric = take(BH * d * d * 8);
  L.ktilde = take(BH * p.Ck * d * 8);
  L.phiK = take(BH * Nv * rK * 8);
  L.phiQ = take(BH * Nv * rQ * 8);
  L.km_cent = take(BH * L.Cmax * L.rmax * 8);
  L.km_lab = take(BH * Nv * 4);
  L.km_region = take(kmeans_ws_bytes(int(BH), int(Nv), L.Cmax, L.rmax));
  L.cbar = take(BH * p.Cq * rQ * 8);
  L.vstat = take(BH * Nv * 4 * 8);
  L.gstat = take(2 * BH * 8 * 4);  // per query head, then per K/V head
  L.pstat = take(BH * p.Cq * 2 * 4);
  L.shift = take(BH * p.Cq * 8);
  L.lbar = take(BH * p.Cq * p.Ck * 8);
  L.scores = take(BH * p.Cq * p.Ck * 8);
  const size_t nsc = desc.dtype == SPR_BF16 ? BH * p.Cq * p.Ck : 0;
  L.serr = take(nsc * 8);
  L.qsplit = take(desc.dtype == SPR_BF16 ? BH * p.Cq * 3 * d * 2 : 0);
  {  // the bf16 routing resolve: request bits, and each query group's ranking (64 E >= Ck entries)
    const size_t bf = desc.dtype == SPR_BF16 ? 1 : 0;
    const size_t e64 = p.Ck <= 64 ? 64 : p.Ck <= 128 ? 128 : p.Ck <= 256 ? 256 : p.Ck <= 512 ? 512 : 1024;
    L.rr_bits = take(bf * BH * p.Ck * ((p.Cq + 63) / 64) * 8);
    L.rr_order = take(bf * BH * p.Cq * e64 * 4);
    L.rr_nin = take(bf * BH * p.Cq * 4);
  }
  L.qnorm = take(BH * p.Cq * 8);
  const size_t BHkv = size_t(desc.B) * kv_heads(desc);
  L.vh = take(desc.dtype == SPR_BF16 ? BHkv * size_t(desc.N) * d * 2 : 0);
  L.vamax = take(BHkv * 4);
  L.vscale = take(2 * BHkv * 4);
  const size_t Mm = M > 0 ? size_t(M) : 1;
  L.fitX = take(BH * Mm * d * 8);
  L.fitR = take(BH * Mm * d * 8);
  L.fitG = take(BH * d * d * 8);
  L.fitH = take(BH * d * d * 8);
  L.fitS = take(BH * 4 * d * 8);
  L.fitW = take(BH * Mm * 8);
  L.applyB = take(BH * d * d * 4);
  L.applyC = take(BH * d * 4);
  L.fitF = take(BH * d * d * 8);
  L.tmax = sparse_tile_capacity(p.Cq, int(Nv), desc.n_text);
  L.tiles = take(BH * size_t(L.tmax) * 8 * 4);
  L.ntiles = take(BH * 4);
  L.tile_prefix = take((BH + 1) * 4);
  L.pair_ov = take(BH * p.Cq * p.Cq * 2);
  L.sel_bits = take(BH * p.Cq * 16 * 8);
  L.total = o;
  return L;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static spr_status check_desc(const spr_desc* d) {
  if (!d) return SPR_EINVAL;
  if (d->B < 1 || d->H < 1 || d->N < 2) return SPR_EINVAL;
  if (d->dtype != SPR_BF16 && d->dtype != SPR_F32) return SPR_EUNSUPPORTED;
  if (d->d != 64 && d->d != 128) return SPR_EUNSUPPORTED;
  if (d->n_text < 0 || d->N - d->n_text < 2) return SPR_EINVAL;
  const int64_t es = d->dtype == SPR_BF16 ? 2 : 4;
  if (d->sn < d->d || d->sh < 1 || d->sb < 1) return SPR_EINVAL;
  if ((d->sn * es) % 16 || (d->sh * es) % 16 || (d->sb * es) % 16) return SPR_EINVAL;
  if (d->Hkv < 0 || d->Hkv > d->H || d->reserved != 0) return SPR_EINVAL;
  if (is_gqa(*d)) {
    if (d->H % d->Hkv) return SPR_EINVAL;
    if (d->ksn < d->d || d->ksh < 1 || d->ksb < 1) return SPR_EINVAL;
    if ((d->ksn * es) % 16 || (d->ksh * es) % 16 || (d->ksb * es) % 16) return SPR_EINVAL;
  }
  return SPR_OK;
}

// The attention kernels address one head's rows with 32-bit byte offsets.
static bool head_fits_32bit(const spr_desc* d) {
  const int64_t es = d->dtype == SPR_BF16 ? 2 : 4;
  const int64_t sn = is_gqa(*d) && d->ksn > d->sn ? d->ksn : d->sn;
  return (int64_t(d->N) - 1) * sn * es + int64_t(d->d) * es < (int64_t(1) << 31);
}

static spr_status check_params(const spr_desc* d, const spr_part_params* p) {
  if (!p) return SPR_EINVAL;
  const int Nv = d->N - d->n_text;
  if (p->Ck < 1 || p->Cq < 1 || p->Ck > 1024 || p->Cq > 1024 || p->Ck > Nv || p->Cq > Nv) return SPR_EINVAL;
  if (p->rK < 1 || p->rQ < 1 || p->rK > d->d || p->rQ > d->d) return SPR_EINVAL;
  // response ranks up to 64 (the projection's tiles); rank 128 only for raw coordinates
  if (p->rK > 64 || p->rQ > 64 || !kmeans_rank_supported(p->rK) || !kmeans_rank_supported(p->rQ))
    return SPR_EUNSUPPORTED;
  if (p->Ms < 1 || p->max_iters < 1) return SPR_EINVAL;
  if (!(p->tol >= 0.0) || !(p->rms_eps > 0.0) || !(p->eig_clamp >= 0.0)) return SPR_EINVAL;
  if (p->mode < SPR_PART_RESPONSE || p->mode > SPR_PART_KEY_RESPONSE || p->reserved != 0) return SPR_EINVAL;
  return SPR_OK;
}

// ceil of the per-query key budget of Sec. 4.3 (same expression order as the documented one)
static int64_t key_budget(double rho, int N, int Nv, int M, int n_text) {
  const double total = rho * double(N) * double(N);
  const double fixed = double(n_text) * double(N) + double(M) * double(N) + double(Nv) * double(n_text);
  const double T = (total - fixed) / double(Nv);
  return int64_t(std::ceil(T));
}

static spr_status check_ws(const spr_desc* d, const spr_part_params* p, int M, void* ws, size_t ws_bytes,
                           Workspace* L) {
  *L = layout(*d, *p, M);
  if (!ws || !aligned16(ws)) return SPR_EINVAL;
  if (ws_bytes < L->total) return SPR_EWORKSPACE;
  return SPR_OK;
}

}  // namespace spr

using namespace spr;

extern "C" {

const char* sparsepr_status_string(spr_status s) {
  switch (s) {
    case SPR_OK: return "ok";
    case SPR_EINVAL: return "invalid argument";
    case SPR_EUNSUPPORTED: return "unsupported head dimension, rank or dtype";
    case SPR_EWORKSPACE: return "workspace too small";
    case SPR_EHIP: return "HIP launch failed";
    case SPR_ETOOLARGE: return "problem exceeds the fixed scratch of the allocation-free call";
  }
  return "unknown status";
}

size_t sparsepr_workspace_size(const spr_desc* desc, const spr_part_params* params, int32_t M) {
  if (check_desc(desc) != SPR_OK || check_params(desc, params) != SPR_OK) return 0;
  return layout(*desc, *params, M).total;
}

spr_status sparsepr_partition(const spr_desc* desc, const void* q, const void* k, const void* v,
                              const spr_part_params* params, const spr_warm* warm, spr_partition* out, void* ws,
                              size_t ws_bytes, void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if ((s = check_params(desc, params)) != SPR_OK) return s;
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v)) return SPR_EINVAL;
  const void* req[] = {out->kv_label, out->q_label, out->kv_perm, out->q_perm, out->q_pos, out->kv_off,
                       out->q_off, out->n_kv, out->n_q, out->kbar, out->vbar, out->qbar, out->qdist,
                       out->FK, out->FQ, out->Qp, out->Kp, out->Vp};
  for (const void* p : req)
    if (!p) return SPR_EINVAL;
  if (!aligned16(out->Qp) || !aligned16(out->Kp) || !aligned16(out->Vp)) return SPR_EINVAL;
  if (int64_t(desc->N) * desc->d * 4 >= (int64_t(1) << 31)) return SPR_EUNSUPPORTED;
  if (warm && (!warm->FK || !warm->FQ || !warm->kbar || !warm->qbar || !warm->n_kv || !warm->n_q))
    return SPR_EINVAL;
  Workspace L;
  if ((s = check_ws(desc, params, 1, ws, ws_bytes, &L)) != SPR_OK) return s;
  return run_partition(*desc, q, k, v, *params, warm, *out, ws, L, static_cast<hipStream_t>(stream));
}

spr_status sparsepr_route(const spr_desc* desc, const spr_part_params* params, const spr_partition* part,
                          double rho_exec_target, int32_t M, const spr_probe_options* probes, spr_route* out,
                          void* ws, size_t ws_bytes, void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if ((s = check_params(desc, params)) != SPR_OK) return s;
  if (!part || !out) return SPR_EINVAL;
  const int Nv = desc->N - desc->n_text;
  if (M < 1 || M >= Nv) return SPR_EINVAL;
  if (!(rho_exec_target > 0.0) || rho_exec_target > 1.0) return SPR_EINVAL;
  const int64_t Tk = key_budget(rho_exec_target, desc->N, Nv, M, desc->n_text);
  if (Tk < 1) return SPR_EINVAL;
  if (!out->sel_cnt || !out->sel_kv || !out->probe_idx || !out->probe_w || !out->pairs ||
      !out->rho_exec)
    return SPR_EINVAL;
  spr_probe_options po = {SPR_PROBES_STRATIFIED, 0};
  if (probes) po = *probes;
  if (po.mode != SPR_PROBES_STRATIFIED && po.mode != SPR_PROBES_RANDOM && po.mode != SPR_PROBES_UNIFORM)
    return SPR_EINVAL;
  Workspace L;
  if ((s = check_ws(desc, params, M, ws, ws_bytes, &L)) != SPR_OK) return s;
  return run_route(*desc, *params, *part, rho_exec_target, M, Tk, po, *out, ws, L, static_cast<hipStream_t>(stream));
}

spr_status sparsepr_attn_sparse(const spr_desc* desc, const spr_part_params* params, const spr_partition* part,
                                const spr_route* route, float* o_sp, void* ws, size_t ws_bytes, void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if ((s = check_params(desc, params)) != SPR_OK) return s;
  if (!part || !route || !o_sp || !aligned16(o_sp)) return SPR_EINVAL;
  Workspace L;
  if ((s = check_ws(desc, params, 1, ws, ws_bytes, &L)) != SPR_OK) return s;
  return run_attn_sparse(*desc, *params, *part, *route, o_sp, ws, L, static_cast<hipStream_t>(stream));
}

// Workspace of the probe call: split-K partials, then (bf16) the scaled fp16 copy of v.
static Workspace probe_layout(const spr_desc& desc, int M) {
  Workspace L = {};
  L.splits = kProbeSplits;
  L.pr_part = 0;
  L.pr_vcopy = align_up(size_t(desc.B) * desc.H * M * kProbeSplits * (desc.d + 2) * 4);
  L.total = L.pr_vcopy + v_copy_bytes(desc);
  return L;
}

spr_status sparsepr_probe_exact(const spr_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* probe_idx, int32_t M, float* o_probe, void* ws, size_t ws_bytes,
                                void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if (!q || !k || !v || !probe_idx || !o_probe || !aligned16(q) || !aligned16(k) || !aligned16(v)) return SPR_EINVAL;
  if (!head_fits_32bit(desc)) return SPR_EUNSUPPORTED;
  const int Nv = desc->N - desc->n_text;
  if (M < 1 || M >= Nv) return SPR_EINVAL;
  const Workspace L = probe_layout(*desc, M);
  if (!ws || !aligned16(ws)) return SPR_EINVAL;
  if (ws_bytes < L.total) return SPR_EWORKSPACE;
  return run_probe_exact(*desc, q, k, v, probe_idx, M, o_probe, ws, L, static_cast<hipStream_t>(stream));
}

size_t sparsepr_probe_workspace_size(const spr_desc* desc, int32_t M) {
  if (check_desc(desc) != SPR_OK || M < 1) return 0;
  return probe_layout(*desc, M).total;
}

spr_status sparsepr_fit_correct(const spr_desc* desc, const spr_part_params* params, const spr_partition* part,
                                const spr_route* route, const float* o_sp, const float* o_probe, int32_t M,
                                double lam, double std_eps, const spr_fit_options* opts, void* out,
                                int32_t out_dtype, double* fit_state, int32_t* head_status, void* ws,
                                size_t ws_bytes, void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if ((s = check_params(desc, params)) != SPR_OK) return s;
  const int Nv = desc->N - desc->n_text;
  if (M < 1 || M >= Nv) return SPR_EINVAL;
  if (!(lam >= 0.0) || !(std_eps > 0.0)) return SPR_EINVAL;
  if (out_dtype != SPR_BF16 && out_dtype != SPR_F32) return SPR_EUNSUPPORTED;
  if (!part || !route || !o_sp || !o_probe || !out || !head_status) return SPR_EINVAL;
  spr_fit_options fo = {SPR_FIT_FULL, 0};
  if (opts) fo = *opts;
  if (fo.family < SPR_FIT_FULL || fo.family > SPR_FIT_DIAG || fo.out_rank < 0) return SPR_EINVAL;
  Workspace L;
  if ((s = check_ws(desc, params, M, ws, ws_bytes, &L)) != SPR_OK) return s;
  return run_fit_correct(*desc, *params, *part, *route, o_sp, o_probe, M, lam, std_eps, fo.family, fo.out_rank, out,
                         out_dtype, fit_state, head_status, ws, L, static_cast<hipStream_t>(stream));
}

size_t sparsepr_dense_workspace_size(const spr_desc* desc) {
  if (check_desc(desc) != SPR_OK) return 0;
  const size_t n = v_copy_bytes(*desc);
  return n ? n : 256;
}

spr_status sparsepr_attn_dense(const spr_desc* desc, const void* q, const void* k, const void* v, void* out,
                               int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v)) return SPR_EINVAL;
  if (out_dtype != SPR_BF16 && out_dtype != SPR_F32) return SPR_EUNSUPPORTED;
  if (!head_fits_32bit(desc)) return SPR_EUNSUPPORTED;
  if (!ws || !aligned16(ws)) return SPR_EINVAL;
  if (ws_bytes < v_copy_bytes(*desc)) return SPR_EWORKSPACE;
  return run_attn_dense(*desc, q, k, v, out, out_dtype, ws, static_cast<hipStream_t>(stream));
}

spr_status sparsepr_attn_dense_noalloc(const spr_desc* desc, const void* q, const void* k, const void* v, void* out,
                                       int32_t out_dtype, void* stream) {
  spr_status s = check_desc(desc);
  if (s != SPR_OK) return s;
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v)) return SPR_EINVAL;
  if (out_dtype != SPR_BF16 && out_dtype != SPR_F32) return SPR_EUNSUPPORTED;
  if (!head_fits_32bit(desc)) return SPR_EUNSUPPORTED;
  if (v_copy_bytes(*desc) > kNoallocScratchBytes) return SPR_ETOOLARGE;
  void* scratch = nullptr;
  if ((s = noalloc_scratch(&scratch)) != SPR_OK) return s;
  return run_attn_dense(*desc, q, k, v, out, out_dtype, scratch, static_cast<hipStream_t>(stream));
}

size_t sparsepr_kmeans_workspace_size(int32_t BH, int32_t n, int32_t r, int32_t C) {
  if (BH < 1 || n < 1 || C < 1 || C > n || C > 1024 || !kmeans_rank_supported(r)) return 0;
  return kmeans_ws_bytes(BH, n, C, r);
}

spr_status sparsepr_kmeans(int32_t BH, int32_t n, int32_t r, int32_t C, const double* feat, uint64_t seed,
                           int32_t stage, int32_t max_iters, double tol, int32_t* labels, double* centres,
                           int32_t* passes, void* ws, size_t ws_bytes, void* stream) {
  if (BH < 1 || n < 1 || C < 1 || C > n || C > 1024 || max_iters < 1 || !(tol >= 0.0)) return SPR_EINVAL;
  if (stage != 0 && stage != 1) return SPR_EINVAL;
  if (!kmeans_rank_supported(r)) return SPR_EUNSUPPORTED;
  if (!feat || !labels || !centres || !passes || !ws || !aligned16(ws) || !aligned16(feat)) return SPR_EINVAL;
  if (ws_bytes < kmeans_ws_bytes(BH, n, C, r)) return SPR_EWORKSPACE;
  KmArgs a = kmeans_carve(ws, BH, n, C, r);
  a.BH = BH; a.n = n; a.r = r; a.C = C; a.stage = stage; a.max_iters = max_iters; a.tol = tol;
  a.seed = seed; a.feat = feat; a.cent = centres; a.labels = labels;
  hipStream_t st = static_cast<hipStream_t>(stream);
  spr_status s = run_kmeans(a, st);
  if (s != SPR_OK) return s;
  launch_copy_passes(a.ctrl, BH, passes, 1, 0, st);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

}  // extern "C"
