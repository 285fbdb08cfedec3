// Response-coupled partitioning ("Partition the Support, Reconstruct the Residual",
// Sec. 4.1, App. B.1-B.2, App. C.1) on gfx950.
//
// Stages per head: key metric M_K from evenly spaced sampled queries -> rank-rK factor
// F_K (one-sided Jacobi, fp64, in LDS) -> phi_K = K F_K -> k-means on phi_K -> K/V groups,
// stable group-major permutation, key/value centroids -> M_Q from the centred key
// centroids -> F_Q -> phi_Q = RMSNorm(Q F_Q) -> k-means -> query groups and their means.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

// ------------------------------------------------------------------ key metric
// M_K = Q_s^T Q_s / M_s over rows s_i = floor(i * Nv / M_s) (Sec. 4.1 / App. B.1 for the
// metric, App. C.2 for the evenly spaced sampling).  16x16 output tile per block, fp64 sums.
template <int DT>
__global__ __launch_bounds__(256) void key_metric_kernel(const void* __restrict__ q, HeadGeom g, int Ms,
                                                         double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int tiles = g.d / 16;
  const int i0 = (blockIdx.x / tiles) * 16, j0 = (blockIdx.x % tiles) * 16;
  const int ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
  __shared__ float As[32][17], Bs[32][17];
  const int m = min(Ms, g.Nv);
  const int64_t base = g.base(hd);
  double acc = 0.0;
  for (int s0 = 0; s0 < m; s0 += 32) {
    for (int e = threadIdx.x; e < 32 * 16; e += 256) {
      const int rr = e >> 4, cc = e & 15, s = s0 + rr;
      float a = 0.f, b = 0.f;
      if (s < m) {
        const int64_t row = (int64_t(s) * g.Nv) / m;
        a = load_elem<DT>(q, base + row * g.sn + i0 + cc);
        b = load_elem<DT>(q, base + row * g.sn + j0 + cc);
      }
      As[rr][cc] = a;
      Bs[rr][cc] = b;
    }
    __syncthreads();
#pragma unroll 8
    for (int rr = 0; rr < 32; ++rr) acc = fma(double(As[rr][ti]), double(Bs[rr][tj]), acc);
    __syncthreads();
  }
  out[size_t(hd) * g.d * g.d + size_t(i0 + ti) * g.d + j0 + tj] = acc / double(m);
}

// Centred key centroids K~ = kbar_b - mu_K over the n_kv nonempty groups (App. B.2).
__global__ void ktilde_kernel(const double* __restrict__ kbar, const int* __restrict__ n_kv, int Ck, int d,
                              double* __restrict__ kt) {
  const int hd = blockIdx.x, c = threadIdx.x;
  if (c >= d) return;
  const int n = n_kv[hd];
  const double* kb = kbar + size_t(hd) * Ck * d;
  double mu = 0.0;
  for (int b = 0; b < n; ++b) mu += kb[size_t(b) * d + c];
  mu /= double(n);
  double* o = kt + size_t(hd) * Ck * d;
  for (int b = 0; b < n; ++b) o[size_t(b) * d + c] = kb[size_t(b) * d + c] - mu;
}

// M_Q = K~^T K~ / (n_kv d) (Sec. 4.1).
__global__ __launch_bounds__(256) void query_metric_kernel(const double* __restrict__ kt,
                                                           const int* __restrict__ n_kv, int Ck, int d,
                                                           double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int tiles = d / 16;
  const int i0 = (blockIdx.x / tiles) * 16, j0 = (blockIdx.x % tiles) * 16;
  const int ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
  __shared__ double As[32][17], Bs[32][17];
  const int n = n_kv[hd];
  const double* src = kt + size_t(hd) * Ck * d;
  double acc = 0.0;
  for (int s0 = 0; s0 < n; s0 += 32) {
    for (int e = threadIdx.x; e < 32 * 16; e += 256) {
      const int rr = e >> 4, cc = e & 15, s = s0 + rr;
      As[rr][cc] = s < n ? src[size_t(s) * d + i0 + cc] : 0.0;
      Bs[rr][cc] = s < n ? src[size_t(s) * d + j0 + cc] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int rr = 0; rr < 32; ++rr) acc = fma(As[rr][ti], Bs[rr][tj], acc);
    __syncthreads();
  }
  out[size_t(hd) * d * d + size_t(i0 + ti) * d + j0 + tj] = acc / (double(n) * double(d));
}

// ------------------------------------------------------------------ factor
// Rank-r factor F with F F^T = the eigenvalue-clamped rank-r truncation of a symmetric PSD
// d x d matrix.  One-sided (Hestenes) Jacobi applied to X = M itself: rotating column pairs
// until all columns are orthogonal leaves X = M V = V diag(lambda), so column i is
// lambda_i v_i and F's columns are x_i / sqrt(|x_i|) in descending |x_i| order.  Parallel
// round-robin ordering: d/2 disjoint pairs per round, d-1 rounds per sweep; blockDim/(d/2)
// consecutive lanes share one pair.  X lives in LDS in fp64 (128 KB at d = 128).
__global__ __launch_bounds__(256) void jacobi_factor_kernel(const double* __restrict__ Mall, int d, int r,
                                                            double clamp, double* __restrict__ Fall) {
  extern __shared__ double X[];  // column-major d x d, column stride ld (padded against bank conflicts)
  __shared__ int rotated;
  const int ld = d + 1;
  __shared__ double lam[128];
  __shared__ double red[32];
  const int hd = blockIdx.x;
  const double* Mm = Mall + size_t(hd) * d * d;
  for (int e = threadIdx.x; e < d * d; e += blockDim.x) X[(e / d) * ld + e % d] = Mm[e];  // symmetric
  __syncthreads();
  // largest squared column norm sets the scale below which columns count as null
  double nmax2 = 0.0;
  if (threadIdx.x < d) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += X[threadIdx.x * ld + i] * X[threadIdx.x * ld + i];
    nmax2 = s;
  }
  for (int o = 32; o > 0; o >>= 1) nmax2 = fmax(nmax2, __shfl_xor(nmax2, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = nmax2;
  __syncthreads();
  nmax2 = 0.0;
  for (int w = 0; w < int(blockDim.x >> 6); ++w) nmax2 = fmax(nmax2, red[w]);
  const double tiny = fmax(nmax2 * 1e-30, 1e-300);
  const double tol = 1e-14;

  const int npairs = d / 2;
  const int G = blockDim.x / npairs;  // lanes per pair: 4 at d = 128, 8 at d = 64
  const int p = threadIdx.x / G, sub = threadIdx.x % G;
  for (int sweep = 0; sweep < 60; ++sweep) {
    if (threadIdx.x == 0) rotated = 0;
    __syncthreads();
    for (int rd = 0; rd < d - 1; ++rd) {
      const int i = (p == 0) ? 0 : 1 + ((p - 1 + rd) % (d - 1));
      const int kk = d - 1 - p;
      const int j = 1 + ((kk - 1 + rd) % (d - 1));
      double* xi = X + size_t(i) * ld;
      double* xj = X + size_t(j) * ld;
      double a = 0.0, b = 0.0, c = 0.0;
      for (int rr = sub; rr < d; rr += G) {
        const double u = xi[rr], v = xj[rr];
        a = fma(u, u, a);
        b = fma(v, v, b);
        c = fma(u, v, c);
      }
      for (int o = G >> 1; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
        c += __shfl_xor(c, o);
      }
      if (a > tiny && b > tiny && fabs(c) > tol * sqrt(a * b)) {
        const double z = (b - a) / (2.0 * c);
        const double t = (z >= 0.0 ? 1.0 : -1.0) / (fabs(z) + sqrt(1.0 + z * z));
        const double cs = 1.0 / sqrt(1.0 + t * t), sn = cs * t;
        for (int rr = sub; rr < d; rr += G) {
          const double u = xi[rr], v = xj[rr];
          xi[rr] = cs * u - sn * v;
          xj[rr] = sn * u + cs * v;
        }
        if (sub == 0) rotated = 1;
      }
      __syncthreads();
    }
    const int again = rotated;
    __syncthreads();
    if (!again) break;
  }
  // eigenvalues = column norms; rank by descending value (ties: lower column first)
  if (threadIdx.x < d) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s = fma(X[threadIdx.x * ld + i], X[threadIdx.x * ld + i], s);
    lam[threadIdx.x] = sqrt(s);
  }
  __syncthreads();
  double lmax = 0.0;
  for (int i = 0; i < d; ++i) lmax = fmax(lmax, lam[i]);
  double* F = Fall + size_t(hd) * d * r;
  for (int e = threadIdx.x; e < d * r; e += blockDim.x) F[e] = 0.0;
  __syncthreads();
  if (threadIdx.x < d) {
    const int i = threadIdx.x;
    const double li = lam[i];
    int rank = 0;
    for (int j = 0; j < d; ++j) rank += (lam[j] > li) || (lam[j] == li && j < i);
    if (rank < r && li > 0.0 && li >= clamp * lmax) {
      const double s = 1.0 / sqrt(li);
      for (int row = 0; row < d; ++row) F[size_t(row) * r + rank] = X[size_t(i) * ld + row] * s;
    }
  }
}

// ------------------------------------------------------------------ projection
typedef double f64x4_t __attribute__((ext_vector_type(4)));

// phi = X F (Sec. 4.1) on v_mfma_f64_16x16x4f64, 128 rows per block (8 waves x 16 rows); with
// RMS the rows are RMS-normalised as in App. B.2: phi / max(sqrt(|phi|^2 / r), eps).  The
// fp64 MFMA takes A[i][k] from lane i + 16k and B[k][j] from lane j + 16k, and returns
// D[(lane / 16) + 4 v][lane % 16] in slot v.
template <int DT, bool RMS>
__global__ __launch_bounds__(512) void project_kernel(const void* __restrict__ x, HeadGeom g, int rows,
                                                      const double* __restrict__ Fall, int r, double eps,
                                                      double* __restrict__ out, int* __restrict__ gstat) {
  extern __shared__ double smem[];
  const int d = g.d;
  const int NT = (r + 15) >> 4;
  const int FS = NT * 16 + 8;  // F row stride (doubles)
  const int XS = d + 4;        // X tile row stride (floats)
  double* Fs = smem;                                      // [d][FS]
  float* Xs = reinterpret_cast<float*>(smem + d * FS);  // [128][XS]
  const int hd = blockIdx.y, row0 = blockIdx.x * 128;
  const double* F = Fall + size_t(hd) * d * r;
  for (int e = threadIdx.x; e < d * FS; e += 512) {
    const int kk = e / FS, c = e % FS;
    Fs[e] = c < r ? F[size_t(kk) * r + c] : 0.0;
  }
  const int64_t base = g.base(hd);
  for (int e = threadIdx.x; e < 128 * d; e += 512) {
    const int rr = e / d, cc = e % d, row = row0 + rr;
    Xs[rr * XS + cc] = row < rows ? load_elem<DT>(x, base + int64_t(row) * g.sn + cc) : 0.f;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r16 = lane & 15;
  f64x4_t acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  for (int ks = 0; ks < d / 4; ++ks) {
    const double av = Xs[(w * 16 + r16) * XS + ks * 4 + gq];
    const double* fr = Fs + (ks * 4 + gq) * FS + r16;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (nt < NT) acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, fr[nt * 16], acc[nt], 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    double scale = 1.0;
    const int row = row0 + w * 16 + gq + 4 * v;
    if constexpr (RMS) {
      double s2 = 0.0;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (nt < NT) s2 = fma(acc[nt][v], acc[nt][v], s2);
      s2 += __shfl_xor(s2, 1);
      s2 += __shfl_xor(s2, 2);
      s2 += __shfl_xor(s2, 4);
      s2 += __shfl_xor(s2, 8);
      const double rms = sqrt(s2 / double(r));
      scale = 1.0 / fmax(rms, eps);
      if (rms < eps && row < rows && r16 == 0) atomicOr(gstat + hd * 8 + 0, SPR_HS_RMS_FLOOR);
    }
    if (row < rows) {
      double* o = out + (size_t(hd) * rows + row) * r;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int c = nt * 16 + r16;
        if (nt < NT && c < r) o[c] = acc[nt][v] * scale;
      }
    }
  }
}

size_t project_smem(int d, int r) {
  const int NT = (r + 15) >> 4;
  return size_t(d) * (NT * 16 + 8) * sizeof(double) + size_t(128) * (d + 4) * sizeof(float);
}

// ------------------------------------------------------------------ compaction
// One block of 1024 threads per head: drop empty clusters (renumber the rest in ascending
// id), group offsets, and a stable counting-sort scatter that lists each group's members in
// ascending original index.  Ranks inside a wave come from ballots, ranks across the 16
// waves of a 1024-point chunk from per-wave counts in LDS.
__global__ __launch_bounds__(1024) void km_compact_kernel(const int* __restrict__ lab_raw, int n, int C,
                                                          int* __restrict__ lab_c, int* __restrict__ perm,
                                                          int* __restrict__ pos_of, int* __restrict__ off,
                                                          int* __restrict__ ngroups, int* __restrict__ gstat,
                                                          int empty_bit) {
  extern __shared__ int sm[];
  int* cntr = sm;              // [C]
  int* cursor = sm + C;        // [C]
  int* remap = sm + 2 * C;     // [C]
  int* scan = sm + 3 * C;      // [1024]
  int* wcnt = sm + 3 * C + 1024;  // [16][C]
  const int hd = blockIdx.x, t = threadIdx.x;
  const int* lr = lab_raw + size_t(hd) * n;
  for (int m = t; m < C; m += 1024) cntr[m] = 0;
  for (int e = t; e < 16 * C; e += 1024) wcnt[e] = 0;
  __syncthreads();
  for (int j = t; j < n; j += 1024) atomicAdd(&cntr[lr[j]], 1);
  __syncthreads();
  // C <= 1024: one cluster per thread
  const int cm = t < C ? cntr[t] : 0;
  int ng;
  const int newid = block_exscan_i(cm > 0 ? 1 : 0, scan, &ng);
  int tot;
  const int start = block_exscan_i(cm, scan, &tot);
  if (t < C) {
    remap[t] = newid;
    cursor[t] = start;
    if (cm > 0) off[size_t(hd) * (C + 1) + newid] = start;
  }
  if (t == 0) {
    off[size_t(hd) * (C + 1) + ng] = n;
    ngroups[hd] = ng;
    if (ng < C) atomicOr(gstat + hd * 8 + 0, empty_bit);
  }
  __syncthreads();
  const int lane = t & 63, w = t >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < n; c0 += 1024) {
    const int j = c0 + t;
    const bool valid = j < n;
    const int L = valid ? lr[j] : -1;
    unsigned long long todo = __ballot(valid);
    int myrank = 0, mycnt = 0;
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int Ll = __shfl(L, leader);
      const unsigned long long msk = __ballot(L == Ll);
      if (L == Ll) {
        myrank = __popcll(msk & lt);
        mycnt = __popcll(msk);
      }
      todo &= ~msk;
    }
    if (valid && myrank == 0) wcnt[w * C + L] = mycnt;
    __syncthreads();
    int before = 0, after = 0, pos = 0;
    if (valid) {
      for (int w2 = 0; w2 < w; ++w2) before += wcnt[w2 * C + L];
      for (int w2 = w + 1; w2 < 16; ++w2) after += wcnt[w2 * C + L];
      pos = cursor[L] + before + myrank;
    }
    __syncthreads();
    if (valid) {
      if (myrank == mycnt - 1 && after == 0) cursor[L] = pos + 1;
      if (myrank == 0) wcnt[w * C + L] = 0;
      perm[size_t(hd) * n + pos] = j;
      if (pos_of) pos_of[size_t(hd) * n + j] = pos;
      lab_c[size_t(hd) * n + j] = remap[L];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ gathers and means
// Group-major copy of the rows of one tensor: dst[hd][pos] = src[hd][perm[pos]] for video
// positions and dst[hd][pos] = src[hd][pos] for the trailing text rows.  16-byte pieces.
template <int DT>
__global__ __launch_bounds__(256) void gather_rows_kernel(const void* __restrict__ src, HeadGeom g,
                                                          const int* __restrict__ perm, void* __restrict__ dst) {
  constexpr int ES = ElemSize<DT>::value;
  const int hd = blockIdx.y;
  const int pieces = g.d * ES / 16;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(g.N) * pieces) return;
  const int pos = int(idx / pieces), pc = int(idx % pieces);
  const int row = pos < g.Nv ? perm[size_t(hd) * g.Nv + pos] : pos;
  const char* s = static_cast<const char*>(src) + (g.base(hd) + int64_t(row) * g.sn) * ES + pc * 16;
  char* dd = static_cast<char*>(dst) + ((size_t(hd) * g.N + pos) * g.d) * ES + pc * 16;
  *reinterpret_cast<uint4*>(dd) = *reinterpret_cast<const uint4*>(s);
}

// fp16 copy of the group-major bf16 values (the operand type of the P V products).
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ src, _Float16* __restrict__ dst,
                                                          size_t n) {
  const size_t i = (size_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const uint4 u = *reinterpret_cast<const uint4*>(src + i);
  const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 o;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o[2 * c] = _Float16(__uint_as_float(wv[c] << 16));
    o[2 * c + 1] = _Float16(__uint_as_float(wv[c] & 0xFFFF0000u));
  }
  *reinterpret_cast<h8*>(dst + i) = o;
}

// Means of rows [off[b], off[b+1]) of a group-major [BH][N][d] tensor, one wave per group.
template <int DT>
__global__ __launch_bounds__(256) void group_mean_kernel(const void* __restrict__ src, int N, int d,
                                                         const int* __restrict__ off, const int* __restrict__ ngroups,
                                                         int C, double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= C) return;
  double* o = out + (size_t(hd) * C + b) * d;
  if (b >= ngroups[hd]) {
    for (int c = lane; c < d; c += 64) o[c] = 0.0;
    return;
  }
  const int r0 = off[size_t(hd) * (C + 1) + b], r1 = off[size_t(hd) * (C + 1) + b + 1];
  double a0 = 0.0, a1 = 0.0;
  for (int rr = r0; rr < r1; ++rr) {
    const size_t base = (size_t(hd) * N + rr) * d;
    a0 += load_elem<DT>(src, base + lane);
    if (lane + 64 < d) a1 += load_elem<DT>(src, base + lane + 64);
  }
  const double inv = 1.0 / double(r1 - r0);
  o[lane] = a0 * inv;
  if (lane + 64 < d) o[lane + 64] = a1 * inv;
}

// c_a = mean of phi_Q over group a (App. A.2), members listed by perm.
__global__ __launch_bounds__(256) void group_mean_perm_kernel(const double* __restrict__ feat, int n, int r,
                                                              const int* __restrict__ perm,
                                                              const int* __restrict__ off,
                                                              const int* __restrict__ ngroups, int C,
                                                              double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= C || b >= ngroups[hd] || lane >= r) return;
  const int r0 = off[size_t(hd) * (C + 1) + b], r1 = off[size_t(hd) * (C + 1) + b + 1];
  double a = 0.0;
  for (int p = r0; p < r1; ++p) a += feat[(size_t(hd) * n + perm[size_t(hd) * n + p]) * r + lane];
  out[(size_t(hd) * C + b) * r + lane] = a / double(r1 - r0);
}

// d_i = |phi_Q(q_i) - c_a| for every video query row (App. A.2), original order.
__global__ __launch_bounds__(256) void qdist_kernel(const double* __restrict__ feat, int n, int r,
                                                    const int* __restrict__ lab, const double* __restrict__ cbar,
                                                    int C, double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int a = lab[size_t(hd) * n + i];
  const double* f = feat + (size_t(hd) * n + i) * r;
  const double* c = cbar + (size_t(hd) * C + a) * r;
  double s = 0.0;
  for (int e = 0; e < r; ++e) {
    const double t = f[e] - c[e];
    s = fma(t, t, s);
  }
  out[size_t(hd) * n + i] = sqrt(s);
}

// ------------------------------------------------------------------ host drivers
size_t compact_smem(int C) { return size_t(3 * C + 1024 + 16 * C) * sizeof(int); }

spr_status launch_compact(const int* lab_raw, int BH, int n, int C, int* lab_c, int* perm, int* pos_of, int* off,
                          int* ngroups, int* gstat, int empty_bit, hipStream_t st) {
  allow_lds(km_compact_kernel, compact_smem(C));
  hipLaunchKernelGGL(km_compact_kernel, dim3(BH), dim3(1024), compact_smem(C), st, lab_raw, n, C, lab_c, perm,
                     pos_of, off, ngroups, gstat, empty_bit);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

__global__ void copy_doubles_kernel(const double* src, double* dst, size_t n) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ void zero_ints_kernel(int* p, size_t n) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <typename T>
static T* wsp(void* ws, size_t off) {
  return ws_ptr<T>(ws, off);
}

template <int DT>
static spr_status partition_impl(const spr_desc& desc, const void* q, const void* k, const void* v,
                                 const spr_part_params& p, spr_partition& out, void* ws, const Workspace& L,
                                 hipStream_t st) {
  const HeadGeom g = make_geom(desc);
  const int BH = desc.B * desc.H, d = desc.d, Nv = g.Nv;
  double* metric = wsp<double>(ws, L.metric);
  double* phiK = out.phiK ? out.phiK : wsp<double>(ws, L.phiK);
  double* phiQ = out.phiQ ? out.phiQ : wsp<double>(ws, L.phiQ);
  int* gstat = wsp<int>(ws, L.gstat);
  hipLaunchKernelGGL(zero_ints_kernel, dim3(ceil_div(BH * 8, 256)), dim3(256), 0, st, gstat, size_t(BH) * 8);

  // M_K and F_K
  hipLaunchKernelGGL(key_metric_kernel<DT>, dim3((d / 16) * (d / 16), BH), dim3(256), 0, st, q, g, p.Ms, metric);
  SPR_CHECK_LAUNCH();
  const size_t jac_smem = jacobi_smem(d);
  allow_lds(jacobi_factor_kernel, jac_smem);
  hipLaunchKernelGGL(jacobi_factor_kernel, dim3(BH), dim3(256), jac_smem, st, metric, d, p.rK, p.eig_clamp, out.FK);
  SPR_CHECK_LAUNCH();
  // phi_K = K F_K
  const size_t prj_smem = project_smem(d, p.rK > p.rQ ? p.rK : p.rQ);
  allow_lds(project_kernel<DT, false>, prj_smem);
  allow_lds(project_kernel<DT, true>, prj_smem);
  hipLaunchKernelGGL((project_kernel<DT, false>), dim3(ceil_div(Nv, 128), BH), dim3(512), prj_smem, st, k, g, Nv,
                     out.FK, p.rK, p.rms_eps, phiK, gstat);
  SPR_CHECK_LAUNCH();
  // K/V k-means
  KmArgs ka = kmeans_carve(wsp<char>(ws, L.km_region), BH, Nv, L.Cmax, L.rmax);
  ka.BH = BH; ka.n = Nv; ka.r = p.rK; ka.C = p.Ck; ka.feat = phiK; ka.seed = p.seed; ka.stage = 0;
  ka.max_iters = p.max_iters; ka.tol = p.tol;
  ka.cent = wsp<double>(ws, L.km_cent); ka.labels = wsp<int>(ws, L.km_lab);
  spr_status s = run_kmeans(ka, st);
  if (s != SPR_OK) return s;
  if (out.passes) launch_copy_passes(ka.ctrl, BH, out.passes, 2, 0, st);
  if (out.cK_last) {
    // centres are stored with stride rK, exactly the caller's layout
    const size_t nel = size_t(BH) * p.Ck * p.rK;
    hipLaunchKernelGGL(copy_doubles_kernel, dim3(unsigned(ceil_div64(nel, 256))), dim3(256), 0, st, ka.cent,
                       out.cK_last, nel);
  }
  s = launch_compact(ka.labels, BH, Nv, p.Ck, out.kv_label, out.kv_perm, nullptr, out.kv_off, out.n_kv, gstat,
                     SPR_HS_KV_GROUPS_EMPTY, st);
  if (s != SPR_OK) return s;
  // group-major K and V, key / value centroids
  const int pieces = d * ElemSize<DT>::value / 16;
  const dim3 ggrid(unsigned(ceil_div64(int64_t(desc.N) * pieces, 256)), BH);
  hipLaunchKernelGGL(gather_rows_kernel<DT>, ggrid, dim3(256), 0, st, k, g, out.kv_perm, out.Kp);
  hipLaunchKernelGGL(gather_rows_kernel<DT>, ggrid, dim3(256), 0, st, v, g, out.kv_perm, out.Vp);
  SPR_CHECK_LAUNCH();
  if constexpr (DT == SPR_BF16) {
    const size_t nel = size_t(BH) * desc.N * d;
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(unsigned(ceil_div64(int64_t(nel / 8), 256))), dim3(256), 0, st,
                       static_cast<const uint16_t*>(out.Vp), wsp<_Float16>(ws, L.vh), nel);
    SPR_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(group_mean_kernel<DT>, dim3(ceil_div(p.Ck, 4), BH), dim3(256), 0, st, out.Kp, desc.N, d,
                     out.kv_off, out.n_kv, p.Ck, out.kbar);
  hipLaunchKernelGGL(group_mean_kernel<DT>, dim3(ceil_div(p.Ck, 4), BH), dim3(256), 0, st, out.Vp, desc.N, d,
                     out.kv_off, out.n_kv, p.Ck, out.vbar);
  SPR_CHECK_LAUNCH();
  // M_Q and F_Q
  double* kt = wsp<double>(ws, L.ktilde);
  hipLaunchKernelGGL(ktilde_kernel, dim3(BH), dim3(d), 0, st, out.kbar, out.n_kv, p.Ck, d, kt);
  hipLaunchKernelGGL(query_metric_kernel, dim3((d / 16) * (d / 16), BH), dim3(256), 0, st, kt, out.n_kv, p.Ck, d,
                     metric);
  hipLaunchKernelGGL(jacobi_factor_kernel, dim3(BH), dim3(256), jac_smem, st, metric, d, p.rQ, p.eig_clamp, out.FQ);
  SPR_CHECK_LAUNCH();
  // phi_Q = RMSNorm(Q F_Q)
  hipLaunchKernelGGL((project_kernel<DT, true>), dim3(ceil_div(Nv, 128), BH), dim3(512), prj_smem, st, q, g, Nv,
                     out.FQ, p.rQ, p.rms_eps, phiQ, gstat);
  SPR_CHECK_LAUNCH();
  // query k-means
  KmArgs qa = ka;
  qa.r = p.rQ; qa.C = p.Cq; qa.feat = phiQ; qa.stage = 1;
  s = run_kmeans(qa, st);
  if (s != SPR_OK) return s;
  if (out.passes) launch_copy_passes(qa.ctrl, BH, out.passes, 2, 1, st);
  if (out.cQ_last) {
    const size_t nel = size_t(BH) * p.Cq * p.rQ;
    hipLaunchKernelGGL(copy_doubles_kernel, dim3(unsigned(ceil_div64(nel, 256))), dim3(256), 0, st, qa.cent,
                       out.cQ_last, nel);
  }
  s = launch_compact(qa.labels, BH, Nv, p.Cq, out.q_label, out.q_perm, out.q_pos, out.q_off, out.n_q, gstat,
                     SPR_HS_Q_GROUPS_EMPTY, st);
  if (s != SPR_OK) return s;
  hipLaunchKernelGGL(gather_rows_kernel<DT>, ggrid, dim3(256), 0, st, q, g, out.q_perm, out.Qp);
  hipLaunchKernelGGL(group_mean_kernel<DT>, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, out.Qp, desc.N, d,
                     out.q_off, out.n_q, p.Cq, out.qbar);
  double* cbar = wsp<double>(ws, L.cbar);
  hipLaunchKernelGGL(group_mean_perm_kernel, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, phiQ, Nv, p.rQ,
                     out.q_perm, out.q_off, out.n_q, p.Cq, cbar);
  hipLaunchKernelGGL(qdist_kernel, dim3(ceil_div(Nv, 256), BH), dim3(256), 0, st, phiQ, Nv, p.rQ, out.q_label, cbar,
                     p.Cq, out.qdist);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_partition(const spr_desc& desc, const void* q, const void* k, const void* v, const spr_part_params& p,
                         spr_partition& out, void* ws, const Workspace& L, hipStream_t st) {
  if (desc.dtype == SPR_BF16) return partition_impl<SPR_BF16>(desc, q, k, v, p, out, ws, L, st);
  return partition_impl<SPR_F32>(desc, q, k, v, p, out, ws, L, st);
}

size_t jacobi_smem(int d) { return size_t(d) * (d + 1) * sizeof(double); }

}  // namespace spr
