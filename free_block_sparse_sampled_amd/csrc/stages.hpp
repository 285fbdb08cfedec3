// Stage drivers of libsparsepr (host side), implemented in the per-stage .hip files.
#pragma once
#include "common.hpp"

namespace spr {

struct KmArgs {
  int BH, n, r, C, stage, max_iters, nsl;  // nsl: slices of the label sort
  double tol;
  uint64_t seed;
  const double* feat;  // [BH][n][r] coordinates
  double* cent;        // [BH][C][r] centres
  bool cent_given;     // cent already holds the initial centres (later calls)
  bool stats_given;    // the producer of feat accumulated the point statistics (see km_stats_target)
  int* labels;         // [BH][n] labels after the last pass
  // scratch carved by kmeans_carve()
  double* sums;
  int* cnt;
  int* lab_new;
  double* jpart;
  int* cpart;
  int* hist;
  int* cstart;
  int* order;
  double* ctrl;
  double* mu;
  void* xh;
  void* xl;
  float* xnrm;
  void* ch;
  void* cl;
  float* cn2;
  int* rq_count;
  int* rq_list;
};

size_t kmeans_ws_bytes(int BH, int n, int C, int rmax);
KmArgs kmeans_carve(void* ws, int BH, int n, int C, int rmax);
void launch_copy_passes(const double* ctrl, int BH, int* passes, int stride, int slot, hipStream_t st);

spr_status run_kmeans(const KmArgs& a, hipStream_t st);
// Where a producer of the k-means coordinates accumulates the point statistics itself: fp64
// column sums into mu[head * mu_stride + column] (atomics) and the largest |x| into
// ctrl[head * ctrl_stride + amax_slot] (atomicMax on the non-negative bit pattern), after
// kmeans_stats_zero has cleared them; run_kmeans then skips its own statistics pass.
struct KmStatsTarget {
  double* mu;
  double* ctrl;
  int mu_stride, ctrl_stride, amax_slot;
};
KmStatsTarget km_stats_target(const KmArgs& a);
void kmeans_stats_zero(const KmArgs& a, hipStream_t st);
bool kmeans_rank_supported(int r);
size_t jacobi_smem(int d);
// Groups from the final labels of a run_kmeans call (its scratch reused): empty clusters dropped,
// the others renumbered in ascending id (lab_c), offsets, group count, status bit, and a stable
// counting sort (perm: members of each group in ascending point index; pos_of: its inverse).
spr_status launch_compact(const KmArgs& a, int* lab_c, int* perm, int* pos_of, int* off, int* ngroups, int* gstat,
                          int empty_bit, hipStream_t st);

spr_status run_partition(const spr_desc& desc, const void* q, const void* k, const void* v, const spr_part_params& p,
                         const spr_warm* warm, spr_partition& out, void* ws, const Workspace& L, hipStream_t st);
spr_status run_route(const spr_desc& desc, const spr_part_params& p, const spr_partition& part, double rho, int M,
                     int64_t Tk, const spr_probe_options& probes, spr_route& out, void* ws, const Workspace& L,
                     hipStream_t st);
spr_status run_attn_sparse(const spr_desc& desc, const spr_part_params& p, const spr_partition& part,
                           const spr_route& route, float* o_sp, void* ws, const Workspace& L, hipStream_t st);
spr_status run_probe_exact(const spr_desc& desc, const void* q, const void* k, const void* v, const int* probe_idx,
                           int M, float* o_probe, void* ws, const Workspace& L, hipStream_t st);
spr_status run_fit_correct(const spr_desc& desc, const spr_part_params& p, const spr_partition& part,
                           const spr_route& route, const float* o_sp, const float* o_probe, int M, double lam,
                           double std_eps, int family, int out_rank, void* out, int out_dtype, double* fit_state,
                           int* head_status, void* ws, const Workspace& L, hipStream_t st);
// Factor F = U_r Lambda_r^{1/2} [BH][d][r] of the symmetric d x d matrices Mall (eigendecomposition
// of the partitioning stage; eigenvalues at or below clamp times the largest give zero columns).
spr_status launch_eigen_factor(const double* Mall, int BH, int d, int r, double clamp, double* Fall, int* gstat,
                               hipStream_t st);
spr_status run_attn_dense(const spr_desc& desc, const void* q, const void* k, const void* v, void* out,
                          int out_dtype, void* ws, hipStream_t st);
// device address of the fixed scratch of the allocation-free dense call on the current device
constexpr size_t kNoallocScratchBytes = SPR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
spr_status noalloc_scratch(void** ptr);
// Power-of-two scaling of bf16 values into fp16 (attention.hip): the largest |v| of every K/V head
// of v (geometry gk) into amax, then scale[hk] = 2^e and scale[heads + hk] = 2^-e.
void launch_v_scale(const void* v, const HeadGeom& gk, int heads, unsigned* amax, float* scale, hipStream_t st);
// Bytes of a scaled fp16 copy of v with its scales (0 for fp32 inputs).
size_t v_copy_bytes(const spr_desc& desc);

// Raise the dynamic-LDS limit of a kernel above the 64 KB default once per process.
template <typename K>
inline void allow_lds(K kernel, size_t bytes) {
  if (bytes > 65536) hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

template <typename T>
inline T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace spr
