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
typedef double f64x4_t __attribute__((ext_vector_type(4)));

// M_K = Q_s^T Q_s / M_s over rows s_i = floor(i * Nv / M_s) (Sec. 4.1 / App. B.1 for the
// metric, App. C.2 for the evenly spaced sampling); with grouped-query attention Q_s stacks the
// sampled rows of the G query heads of K/V head j (heads j G .. j G + G - 1), M_K = Q_s^T Q_s /
// (G M_s).  On the fp64 matrix cores: one block per 16 rows of M_K (i0 .. i0 + 15) and head; the
// sampled rows stream through LDS in chunks of 64 (widened to fp64, the next chunk loaded into
// registers meanwhile), and wave w accumulates columns 16 TW w .. 16 TW (w + 1) - 1.
template <int DT, int D>
__global__ __launch_bounds__(256) void key_metric_kernel(const void* __restrict__ q, HeadGeom g, int Ms, int G,
                                                         double* __restrict__ out) {
  constexpr int KC = 64, XS = D + 2, TW = D / 64, PER = KC * D / 8 / 256;
  extern __shared__ double km_xs[];  // [KC][XS]
  const int hj = blockIdx.y, i0 = blockIdx.x * 16;
  const int m = min(Ms, g.Nv), total = m * G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, kq = lane >> 4;
  Raw8<DT> xr8[PER];  // the next chunk's rows as stored (zero past the last sampled row)
  auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u, kk = e / (D / 8), c8 = (e % (D / 8)) * 8, k = k0 + kk;
      if (k < total) {
        const int gi = k / m, sidx = k % m;
        const int64_t row = (int64_t(sidx) * g.Nv) / m;
        xr8[u] = load8_raw<DT>(q, g.base(hj * G + gi) + row * g.sn + c8);
      } else {
        xr8[u] = Raw8<DT>{};
      }
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u, kk = e / (D / 8), c8 = (e % (D / 8)) * 8;
      float xv[8];
      widen8<DT>(xr8[u], xv);
#pragma unroll
      for (int t = 0; t < 8; t += 2)
        *reinterpret_cast<double2*>(km_xs + kk * XS + c8 + t) = make_double2(xv[t], xv[t + 1]);
    }
  };
  f64x4_t acc[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  fetch(0);
  for (int k0 = 0; k0 < total; k0 += KC) {
    __syncthreads();
    stage();
    __syncthreads();
    if (k0 + KC < total) fetch(k0 + KC);
#pragma unroll 4
    for (int kk = 0; kk < KC; kk += 4) {
      const double* xr = km_xs + (kk + kq) * XS;
      const double a = xr[i0 + r16];
#pragma unroll
      for (int t = 0; t < TW; ++t)
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, xr[(w * TW + t) * 16 + r16], acc[t], 0, 0, 0);
    }
  }
  const double den = double(m) * G;
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      out[size_t(hj) * D * D + size_t(i0 + kq + 4 * v) * D + (w * TW + t) * 16 + r16] = acc[t][v] / den;
}

// Centred key centroids K~ = kbar_b - mu_K over the n_kv nonempty groups (App. B.2).  One block
// of 1024 threads per head: 1024 / d row stripes accumulate column sums, combined in LDS.
__global__ __launch_bounds__(1024) void ktilde_kernel(const double* __restrict__ kbar, const int* __restrict__ n_kv,
                                                      int Ck, int d, double* __restrict__ kt) {
  __shared__ double part[1024];
  const int hd = blockIdx.x, c = threadIdx.x % d, stripe = threadIdx.x / d, ns = blockDim.x / d;
  const int n = n_kv[hd];
  const double* kb = kbar + size_t(hd) * Ck * d;
  double s0 = 0.0, s1 = 0.0;
  int b = stripe;
  for (; b + ns < n; b += 2 * ns) {
    s0 += kb[size_t(b) * d + c];
    s1 += kb[size_t(b + ns) * d + c];
  }
  if (b < n) s0 += kb[size_t(b) * d + c];
  part[threadIdx.x] = s0 + s1;
  __syncthreads();
  double mu = 0.0;
  for (int t = 0; t < ns; ++t) mu += part[t * d + c];
  mu /= double(n);
  double* o = kt + size_t(hd) * Ck * d;
  for (b = stripe; b < n; b += ns) o[size_t(b) * d + c] = kb[size_t(b) * d + c] - mu;
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
// d x d matrix (d <= 128), one workgroup per head, everything in fp64 in LDS:
//  1. Householder reduction to tridiagonal form.  Step i (i = d-1 .. 1) takes the reflector u
//     of row i restricted to columns 0..i-1 (u^T u = 2h), forms p = A u / h, q = p - (u^T p /
//     2h) u and updates the leading block A -= u q^T + q u^T (kept fully symmetric).  Row i
//     keeps u and column i keeps u / h.
//  2. Explicit accumulation of Q = H_{d-1} ... H_1 in place of A.
//  3. Implicit QL iterations with Wilkinson-type shifts on the tridiagonal matrix.  In each
//     sweep one lane runs the Givens recurrence and records the rotations; then every lane
//     applies the sweep's rotations, in order, to its own row of Q, so eigenvectors need two
//     barriers per sweep rather than per rotation.
// Columns of F are sqrt(lambda_i) times the eigenvectors, in descending lambda order (ties: lower
// index first); eigenvalues below clamp * lambda_max (or not positive) give zero columns.
constexpr int kEigMax = 128;

__global__ __launch_bounds__(256) void eigen_factor_kernel(const double* __restrict__ Mall, int d, int r,
                                                           double clamp, double* __restrict__ Fall,
                                                           int* __restrict__ gstat, int skip_slot) {
  extern __shared__ double A[];  // d x ld, row-major
  // heads whose factor the later-call update produced are left alone
  if (skip_slot >= 0 && gstat[blockIdx.x * 8 + skip_slot]) return;
  __shared__ double dg[kEigMax], ev[kEigMax], pv[kEigMax], rc[kEigMax], rs[kEigMax];
  __shared__ double red[8];
  __shared__ double sh_h, sh_scale;
  __shared__ int sh_nrot, sh_m, sh_fail;
  const int ld = d + 1;
  const int hd = blockIdx.x, tid = threadIdx.x, nth = blockDim.x;
  const int lane = tid & 63, wv = tid >> 6, nw = nth >> 6;
  const double* Mm = Mall + size_t(hd) * d * d;
  for (int e = tid; e < d * d; e += nth) A[(e / d) * ld + e % d] = Mm[e];
  if (tid == 0) sh_fail = 0;
  __syncthreads();

  auto block_sum = [&](double x) -> double {
    x = wave_sum_d(x);
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    double t = 0.0;
    for (int k = 0; k < nw; ++k) t += red[k];
    return t;
  };

  // 1. tridiagonal reduction
  for (int i = d - 1; i >= 1; --i) {
    const int l = i - 1;
    double* Ai = A + size_t(i) * ld;
    double part = 0.0;
    for (int k = tid; k <= l; k += nth) part += fabs(Ai[k]);
    const double scale = block_sum(part);
    if (l == 0 || scale == 0.0) {
      if (tid == 0) {
        ev[i] = Ai[l];
        dg[i] = 0.0;
      }
      __syncthreads();
      continue;
    }
    part = 0.0;
    for (int k = tid; k <= l; k += nth) {
      const double u = Ai[k] / scale;
      Ai[k] = u;
      part += u * u;
    }
    double h = block_sum(part);
    const double f = Ai[l];
    const double g = f >= 0.0 ? -sqrt(h) : sqrt(h);
    h -= f * g;
    __syncthreads();
    if (tid == 0) {
      ev[i] = scale * g;
      Ai[l] = f - g;
      dg[i] = h;
    }
    __syncthreads();
    // u/h into column i; p = A u / h
    for (int j = tid; j <= l; j += nth) A[size_t(j) * ld + i] = Ai[j] / h;
    part = 0.0;
    for (int j = tid; j <= l; j += nth) {
      const double* Aj = A + size_t(j) * ld;
      double s = 0.0;
#pragma unroll 8
      for (int k = 0; k <= l; ++k) s = fma(Aj[k], Ai[k], s);
      pv[j] = s / h;
      part += pv[j] * Ai[j];
    }
    const double K = block_sum(part) / (h + h);
    for (int j = tid; j <= l; j += nth) pv[j] -= K * Ai[j];
    __syncthreads();
#pragma unroll 4
    for (int e = tid; e < (l + 1) * (l + 1); e += nth) {
      const int j = e / (l + 1), k = e % (l + 1);
      A[size_t(j) * ld + k] -= Ai[j] * pv[k] + pv[j] * Ai[k];
    }
    __syncthreads();
  }
  if (tid == 0) {
    dg[0] = 0.0;
    ev[0] = 0.0;
  }
  __syncthreads();
  // 2. accumulate Q in place
  for (int i = 0; i < d; ++i) {
    const int l = i - 1;
    if (dg[i] != 0.0) {  // a reflector was applied at step i
      for (int j = tid; j <= l; j += nth) {
        double s = 0.0;
#pragma unroll 8
        for (int k = 0; k <= l; ++k) s = fma(A[size_t(i) * ld + k], A[size_t(k) * ld + j], s);
        pv[j] = s;
      }
      __syncthreads();
#pragma unroll 4
      for (int e = tid; e < (l + 1) * (l + 1); e += nth) {
        const int k = e / (l + 1), j = e % (l + 1);
        A[size_t(k) * ld + j] -= pv[j] * A[size_t(k) * ld + i];
      }
      __syncthreads();
    }
    if (tid == 0) dg[i] = A[size_t(i) * ld + i];
    __syncthreads();
    if (tid == 0) A[size_t(i) * ld + i] = 1.0;
    for (int j = tid; j <= l; j += nth) {
      A[size_t(j) * ld + i] = 0.0;
      A[size_t(i) * ld + j] = 0.0;
    }
    __syncthreads();
  }
  // 3. implicit QL on (dg, ev); e[i] couples i and i + 1 after the shift below
  if (tid == 0) {
    for (int i = 1; i < d; ++i) ev[i - 1] = ev[i];
    ev[d - 1] = 0.0;
  }
  __syncthreads();
  for (int l = 0; l < d; ++l) {
    for (int iter = 0;; ++iter) {
      if (wv == 0) {
        // first m >= l whose off-diagonal is negligible (m = d - 1 if none), by ballots
        int m = d - 1;
        for (int m0 = l; m0 < d - 1; m0 += 64) {
          const int mm = m0 + lane;
          bool small = false;
          if (mm < d - 1) {
            const double dd = fabs(dg[mm]) + fabs(dg[mm + 1]);
            small = fabs(ev[mm]) <= 1e-17 * dd || fabs(ev[mm]) + dd == dd;
          }
          const unsigned long long bal = __ballot(small);
          if (bal) {
            m = m0 + __builtin_ctzll(bal);
            break;
          }
        }
        if (lane == 0) {
          sh_m = m;
          int nrot = 0;
          if (m != l) {
            if (iter >= 60) sh_fail = 1;  // no convergence: keep the current values, flag the head
            double g = (dg[l + 1] - dg[l]) / (2.0 * ev[l]);
            double rr = sqrt(g * g + 1.0);
            g = dg[m] - dg[l] + ev[l] / (g + (g >= 0.0 ? rr : -rr));
            double s = 1.0, c = 1.0, p = 0.0;
            int i = m - 1;
            bool early = false;
            // dg[i + 1] and (dg[i], ev[i]) of the next rotation are carried in registers
            double d_hi = dg[m], d_i = dg[i], e_i = ev[i];
            for (; i >= l; --i) {
              const double d_lo = i > l ? dg[i - 1] : 0.0, e_lo = i > l ? ev[i - 1] : 0.0;
              const double f = s * e_i;
              const double b = c * e_i;
              const double x = fma(f, f, g * g);
              if (x == 0.0) {
                ev[i + 1] = 0.0;
                dg[i + 1] = d_hi - p;
                ev[m] = 0.0;
                early = true;
                break;
              }
              // 1 / sqrt(x): hardware estimate and two Newton steps
              double y = __builtin_amdgcn_rsq(x);
              y = y * fma(-0.5 * x * y, y, 1.5);
              y = y * fma(-0.5 * x * y, y, 1.5);
              ev[i + 1] = x * y;
              s = f * y;
              c = g * y;
              g = d_hi - p;
              rr = (d_i - g) * s + 2.0 * c * b;
              p = s * rr;
              dg[i + 1] = g + p;
              g = c * rr - b;
              rc[nrot] = c;
              rs[nrot] = s;
              ++nrot;
              d_hi = d_i;
              d_i = d_lo;
              e_i = e_lo;
            }
            if (!early) {
              dg[l] -= p;
              ev[l] = g;
              ev[m] = 0.0;
            }
          }
          sh_nrot = nrot;
        }
      }
      __syncthreads();
      const int m = sh_m, nrot = sh_nrot;
      if (m == l || sh_fail) break;
      // rotation t acts on columns (m - 1 - t, m - t)
      if (tid < d) {
        double* Zk = A + size_t(tid) * ld;
        double zhi = Zk[m];
#pragma unroll 4
        for (int t = 0; t < nrot; ++t) {
          const int i = m - 1 - t;
          const double zi = Zk[i];
          const double c = rc[t], s = rs[t];
          Zk[i + 1] = s * zi + c * zhi;
          zhi = c * zi - s * zhi;
        }
        Zk[m - nrot] = zhi;
      }
      __syncthreads();
    }
    if (sh_fail) break;
  }
  if (tid == 0 && sh_fail) atomicOr(gstat + hd * 8 + 0, SPR_HS_EIGEN_NOCONV);
  // ranks and output
  __syncthreads();
  double lmax = 0.0;
  for (int i = 0; i < d; ++i) lmax = fmax(lmax, dg[i]);
  double* F = Fall + size_t(hd) * d * r;
  for (int e = tid; e < d * r; e += nth) F[e] = 0.0;
  __syncthreads();
  if (tid < d) {
    const int i = tid;
    const double li = dg[i];
    int rank = 0;
    for (int j = 0; j < d; ++j) rank += (dg[j] > li) || (dg[j] == li && j < i);
    if (rank < r && li > 0.0 && li >= clamp * lmax) {
      const double s = sqrt(li);
      for (int row = 0; row < d; ++row) F[size_t(row) * r + rank] = A[size_t(row) * ld + i] * s;
    }
  }
}

// ------------------------------------------------------------------ later-call factor

// C (m x n, row stride ldc) = op(A) op(B) on the fp64 matrix cores (16x16x4 tiles).  Each wave
// takes 16-row blocks of C with all TN = ceil(n / 16) column tiles at once, so one A fragment
// feeds TN independent accumulation chains.  op(A)(i, k) = A[i * lda + k], or A[k * lda + i]
// when AT; op(B)(k, j) = B[k * ldb + j], or B[j * ldb + k] when BT.  K % 4 == 0; rows at or
// past m and columns at or past n read as zero and are not stored.  Fragments: lane l supplies A(i0 + l % 16,
// k + l / 16) and B(k + l / 16, 16 t + l % 16); it receives C(i0 + l / 16 + 4 v, 16 t + l % 16).
template <int TN, bool AT, bool BT>
__device__ inline void gemm_f64(const double* A, int lda, const double* B, int ldb, double* C, int ldc, int m, int n,
                                int K) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, kq = lane >> 4;
  for (int i0 = w * 16; i0 < m; i0 += nw * 16) {
    f64x4_t acc[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
    for (int k = 0; k < K; k += 4) {
      const double a = i0 + i >= m ? 0.0 : AT ? A[size_t(k + kq) * lda + i0 + i] : A[size_t(i0 + i) * lda + k + kq];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int col = t * 16 + i;
        const double b = col < n ? (BT ? B[size_t(col) * ldb + k + kq] : B[size_t(k + kq) * ldb + col]) : 0.0;
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int col = t * 16 + i;
      if (col < n)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (i0 + kq + 4 * v < m) C[size_t(i0 + kq + 4 * v) * ldc + col] = acc[t][v];
    }
  }
}

__device__ __forceinline__ double readlane_d(double x, int l) {
  const unsigned long long u = __double_as_longlong(x);
  const unsigned lo = __builtin_amdgcn_readlane(unsigned(u), l);
  const unsigned hi = __builtin_amdgcn_readlane(unsigned(u >> 32), l);
  return __longlong_as_double((long long)((unsigned long long)hi << 32 | lo));
}

// Upper Cholesky G = R^T R of the R x R matrix in LDS (row stride R) by one wave, with the
// trailing matrix in registers: lane c holds column c, g[a] being row j + a at step j, so that
// every register index is a constant and the rows shift down by one per step as they are
// updated.  Step j: pivot from lane j, row j of R (R[j][c] = G[j][c] / R[j][j]) written to G and
// to `rowbuf` (2R doubles of LDS scratch; entries past R stay zero), then g[a - 1] = g[a] -
// R[j][j + a] R[j][c] with the multipliers read back from rowbuf as broadcasts.  LDS accesses of
// one wave complete in program order, so wave barriers (which stop the compiler from moving
// memory operations across them) are the only synchronisation.  A pivot not above scale times
// the largest diagonal entry fails; the remaining steps then run on a unit pivot.  On success G
// holds R (upper triangular, row-major); on failure G[0] is -1, a value R[0][0] = sqrt(pivot) > 0
// never takes, so that every wave can read the outcome after a block barrier.
template <int R>
__device__ inline void chol_wave(double* G, double* rowbuf, double scale) {
  const int c = threadIdx.x & 63;
  const int cc = c < R ? c : R - 1;  // lanes past R shadow the last column and store nothing
  double g[R];
#pragma unroll
  for (int a = 0; a < R; ++a) g[a] = G[a * R + cc];
  double dmax = G[cc * R + cc];
  for (int o = 32; o > 0; o >>= 1) dmax = fmax(dmax, __shfl_xor(dmax, o));
  const double floor = scale * dmax;
  if (c < R) rowbuf[R + c] = 0.0;
  bool ok = true;
#pragma unroll 1
  for (int j = 0; j < R; ++j) {
    const double piv = readlane_d(g[0], j);
    ok = ok && piv > floor;
    const double rjj = ok ? sqrt(piv) : 1.0;
    const double rjc = c == j ? rjj : (c > j ? g[0] / rjj : 0.0);
    __builtin_amdgcn_wave_barrier();
    if (c < R) {
      rowbuf[c] = rjc;
      G[j * R + c] = rjc;
    }
    __builtin_amdgcn_wave_barrier();
    // in chunks of 16, so that the loaded values fit in registers beside g
#pragma unroll
    for (int a = 1; a < R; ++a) {
      g[a - 1] = fma(-rowbuf[j + a], rjc, g[a]);
      if (a % 16 == 0) __builtin_amdgcn_sched_barrier(0);
    }
    g[R - 1] = 0.0;
    __builtin_amdgcn_wave_barrier();
  }
  if (!ok && c == 0) G[0] = -1.0;
}

// Ut = (Z R^{-1})^T from Zt = Z^T (R x D) and the upper R (row-major, R x R): row i of U solves
// u R = z_i, one thread per row.  Column by column, u_c = z_c / R_cc and then z_k -= u_c R_ck
// for k > c, with the remaining z in registers shifted down by one per column (every register
// index a constant) and row c of R read as broadcasts.  Reads past row c of R run into the rows
// after it (or the buffer that follows R in LDS); they only touch the shifted-out tail, which
// never feeds a column below R.  Thread i touches column i of Zt and Ut, so a wave's accesses
// are contiguous.
template <int R, int D>
__device__ inline void right_solve_upper(const double* Zt, const double* Rm, double* Ut) {
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    double z[R];
#pragma unroll
    for (int a = 0; a < R; ++a) z[a] = Zt[a * D + i];
#pragma unroll 1
    for (int c = 0; c < R; ++c) {
      const double* row = Rm + c * (R + 1);  // R[c][c + a] = row[a]
      const double uc = z[0] / row[0];
      Ut[c * D + i] = uc;
      // in chunks of 16, so that the loaded values fit in registers beside z
#pragma unroll
      for (int a = 1; a < R; ++a) {
        z[a - 1] = fma(-uc, row[a], z[a]);
        if (a % 16 == 0) __builtin_amdgcn_sched_barrier(0);
      }
      z[R - 1] = 0.0;
    }
  }
}

// Factor update of later calls (App. C.1): two subspace iterations from the span of the previous
// factor (columns scaled to unit length), U <- orth(M U) by Cholesky QR (Z = M U, Z^T Z = R^T R,
// U = Z R^{-1}), then F = U L with L L^T = U^T M U, so F F^T = U U^T M U U^T.  One workgroup per
// head: the products on the fp64 matrix cores, each Cholesky factorisation by one wave, the
// triangular solve one row per thread.  U and Z are kept transposed in LDS (Ut, Zt: R x D) so
// that the solve reads them contiguously; M is symmetric, so Zt = Ut M.  M is read from global
// memory; one R x R matrix, Ut and Zt live in LDS, in that order.  A pivot of Z^T Z at or below clamp^2, or of
// U^T M U at or below clamp, times the largest diagonal entry of its matrix (or a zero previous
// column) stops the head: ok = 0 in gstat[hd][slot] and the eigendecomposition takes over;
// otherwise ok = 1 and F is written.
// The previous factor may be the very buffer the new one is written to (a later call that passes
// the operator's own outputs as its state): each block reads its head's previous factor before a
// barrier and writes the new one last, and neither pointer is restrict-qualified.
template <int D, int R>
__global__ __launch_bounds__(256) void subspace_factor_kernel(const double* __restrict__ Mall,
                                                              const double* Fprev, double clamp,
                                                              double* Fall, int* __restrict__ gstat,
                                                              int ok_slot) {
  constexpr int TD = D / 16, TR = (R + 15) / 16;
  extern __shared__ double sub_sm[];
  const int hd = blockIdx.x, tid = threadIdx.x, nth = blockDim.x;
  const double* M = Mall + size_t(hd) * D * D;
  double* G = sub_sm;                   // [R][R]
  double* Ut = sub_sm + R * R;          // [R][D]
  double* Zt = sub_sm + R * R + D * R;  // [R][D]
  // U^T: consecutive threads take consecutive rows of U, so the LDS writes are contiguous
  for (int e = tid; e < D * R; e += nth) {
    const int j = e / D, i = e % D;
    Ut[e] = Fprev[size_t(hd) * D * R + size_t(i) * R + j];
  }
  __syncthreads();
  // the previous factor's span, columns scaled to unit length; a zero column means a rank
  // below R, which the update cannot recover.  Wave w forms the norms of columns w, w + 4, ..
  // (rows of U^T) and leaves 1 / norm, or 0 for a zero column, in G, unused until the first
  // product.
  const int lane = tid & 63, w = tid >> 6, nw = nth >> 6;
  for (int j = w; j < R; j += nw) {
    double cs = 0.0;
    for (int i = lane; i < D; i += 64) cs = fma(Ut[j * D + i], Ut[j * D + i], cs);
    for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o);
    if (lane == 0) G[j] = cs > 0.0 ? 1.0 / sqrt(cs) : 0.0;
  }
  __syncthreads();
  bool ok = true;
  for (int j = 0; j < R; ++j) ok = ok && G[j] > 0.0;
  if (ok) {
    for (int e = tid; e < D * R; e += nth) Ut[e] *= G[e / D];
  }
  __syncthreads();
  for (int it = 0; it < 2 && ok; ++it) {
    gemm_f64<TD, false, false>(Ut, D, M, D, Zt, D, R, D, D);  // Zt = Ut M = (M U)^T
    __syncthreads();
    gemm_f64<TR, false, true>(Zt, D, Zt, D, G, R, R, R, D);   // G = Z^T Z
    __syncthreads();
    // Z^T Z scales with the squared singular values of Z: tested against clamp^2
    if (tid < 64) chol_wave<R>(G, Ut, clamp * clamp);  // U is dead until the solve rewrites it
    __syncthreads();
    ok = G[0] > 0.0;
    if (!ok) break;
    right_solve_upper<R, D>(Zt, G, Ut);  // U = Z R^{-1}
    __syncthreads();
  }
  if (ok) {
    gemm_f64<TD, false, false>(Ut, D, M, D, Zt, D, R, D, D);  // Wt = (M U)^T
    __syncthreads();
    gemm_f64<TR, false, true>(Ut, D, Zt, D, G, R, R, R, D);   // U^T W
    __syncthreads();
    for (int e = tid; e < R * R; e += nth) {
      const int a = e / R, b = e % R;
      if (b > a) {
        const double h = 0.5 * (G[a * R + b] + G[b * R + a]);
        G[a * R + b] = h;
        G[b * R + a] = h;
      }
    }
    __syncthreads();
    if (tid < 64) chol_wave<R>(G, Zt, clamp);  // W is dead after U^T W
    __syncthreads();
    ok = G[0] > 0.0;
    // F = U R^T
    if (ok) gemm_f64<TR, true, true>(Ut, D, G, R, Fall + size_t(hd) * D * R, R, D, R, R);
  }
  if (tid == 0) gstat[hd * 8 + ok_slot] = ok ? 1 : 0;
}

// The instantiation for (d, r); d in {64, 128}, r in {8, 16, 32, 48, 64}.
template <int D>
static void launch_subspace_d(int BH, int r, size_t smem, hipStream_t st, const double* M, const double* Fprev,
                              double clamp, double* F, int* gstat, int slot) {
  auto go = [&](auto kern) {
    allow_lds(kern, smem);
    hipLaunchKernelGGL(kern, dim3(BH), dim3(256), smem, st, M, Fprev, clamp, F, gstat, slot);
  };
  switch (r) {
    case 8: go(subspace_factor_kernel<D, 8>); break;
    case 16: go(subspace_factor_kernel<D, 16>); break;
    case 32: go(subspace_factor_kernel<D, 32>); break;
    case 48: go(subspace_factor_kernel<D, 48>); break;
    default: go(subspace_factor_kernel<D, 64>); break;
  }
}

static void launch_subspace(int BH, int d, int r, hipStream_t st, const double* M, const double* Fprev, double clamp,
                            double* F, int* gstat, int slot) {
  const size_t smem = (2 * size_t(d) * r + size_t(r) * r) * sizeof(double);
  if (d == 128) launch_subspace_d<128>(BH, r, smem, st, M, Fprev, clamp, F, gstat, slot);
  else launch_subspace_d<64>(BH, r, smem, st, M, Fprev, clamp, F, gstat, slot);
}

// Initial centres of a later call (App. C.1): previous centroid m (original space) mapped to the
// current coordinates, x F on the fp64 matrix cores (RMS-normalised as in App. B.2 for queries);
// slots m >= n_prev take the cold draw of index m.  One block per 64 centres of a head.
template <bool RMS, int TN>
__global__ __launch_bounds__(256) void warm_centres_kernel(const double* __restrict__ prev,
                                                           const int* __restrict__ n_prev, int C, int d,
                                                           const double* __restrict__ Fall, int r, double eps,
                                                           const double* __restrict__ feat, int n, uint64_t seed,
                                                           int stage, int fdiv, double* __restrict__ cent) {
  __shared__ double ys[64][65];
  const int hd = blockIdx.y, m0 = blockIdx.x * 64;
  const int np = min(n_prev[hd], C);
  const double* F = Fall + size_t(hd / fdiv) * d * r;  // factor of the head's K/V head
  // rows of slots at or past n_prev are stale previous centroids; they are replaced below
  gemm_f64<TN, false, false>(prev + (size_t(hd) * C + m0) * d, d, F, r, &ys[0][0], 65, min(64, C - m0), r, d);
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * r; e += blockDim.x) {
    const int ml = e / r, j = e % r, m = m0 + ml;
    if (m >= C || m < np) continue;
    const uint64_t ctr = ((uint64_t(hd) * 2ull + uint64_t(stage)) << 20) + uint64_t(m);
    const int row = int(splitmix64(seed, ctr) % uint64_t(n));
    ys[ml][j] = feat[(size_t(hd) * n + row) * r + j];
  }
  __syncthreads();
  if (RMS && threadIdx.x < 64) {
    const int ml = threadIdx.x, m = m0 + ml;
    if (m < np) {
      double s = 0.0;
      for (int j = 0; j < r; ++j) s = fma(ys[ml][j], ys[ml][j], s);
      const double den = fmax(sqrt(s / double(r)), eps);
      for (int j = 0; j < r; ++j) ys[ml][j] /= den;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * r; e += blockDim.x) {
    const int ml = e / r, j = e % r, m = m0 + ml;
    if (m < C) cent[(size_t(hd) * C + m) * r + j] = ys[ml][j];
  }
}

template <bool RMS>
static void launch_warm_centres(dim3 grid, hipStream_t st, const double* prev, const int* n_prev, int C, int d,
                                const double* F, int r, double eps, const double* feat, int n, uint64_t seed,
                                int stage, int fdiv, double* cent) {
  switch ((r + 15) / 16) {
    case 1:
      hipLaunchKernelGGL((warm_centres_kernel<RMS, 1>), grid, dim3(256), 0, st, prev, n_prev, C, d, F, r, eps, feat,
                         n, seed, stage, fdiv, cent);
      break;
    case 2:
      hipLaunchKernelGGL((warm_centres_kernel<RMS, 2>), grid, dim3(256), 0, st, prev, n_prev, C, d, F, r, eps, feat,
                         n, seed, stage, fdiv, cent);
      break;
    case 3:
      hipLaunchKernelGGL((warm_centres_kernel<RMS, 3>), grid, dim3(256), 0, st, prev, n_prev, C, d, F, r, eps, feat,
                         n, seed, stage, fdiv, cent);
      break;
    default:
      hipLaunchKernelGGL((warm_centres_kernel<RMS, 4>), grid, dim3(256), 0, st, prev, n_prev, C, d, F, r, eps, feat,
                         n, seed, stage, fdiv, cent);
      break;
  }
}

// ------------------------------------------------------------------ projection

// phi = X F (Sec. 4.1) on v_mfma_f64_16x16x4f64; with RMS the rows are RMS-normalised as in
// App. B.2: phi / max(sqrt(|phi|^2 / r), eps).  With a statistics target the kernel also
// accumulates the k-means point statistics of phi (column sums and the largest |phi|): per wave
// over its chunks in registers, then one atomic per column and block.  The fp64 MFMA takes A[i][k] from lane i + 16k
// and B[k][j] from lane j + 16k, and returns D[(lane / 16) + 4 v][lane % 16] in slot v.  F is
// staged in LDS once per block; the block then walks `chunks` chunks of 128 rows (8 waves x 16
// rows), the next chunk's rows loaded into registers (16-byte loads) while the current one is
// multiplied, then widened to fp32 in LDS.  The row width D and the NT = ceil(r / 16) column
// tiles are compile-time, so the product loop is straight-line code whose LDS reads run ahead of
// the matrix-core chain.
template <int DT, bool RMS, int D, int NT>
__global__ __launch_bounds__(512) void project_kernel(const void* __restrict__ x, HeadGeom g, int rows,
                                                      const double* __restrict__ Fall, int r, double eps,
                                                      double* __restrict__ out, int* __restrict__ gstat, int chunks,
                                                      int fdiv, KmStatsTarget kst) {
  extern __shared__ double smem[];
  constexpr int FS = NT * 16 + 8;  // F row stride (doubles)
  constexpr int XS = D + 4;        // X tile row stride (floats)
  double* Fs = smem;                                      // [D][FS]
  float* Xs = reinterpret_cast<float*>(smem + D * FS);  // [128][XS]
  const int hd = blockIdx.y;
  const double* F = Fall + size_t(hd / fdiv) * D * r;  // factor of the head's K/V head
  for (int e = threadIdx.x; e < D * FS; e += 512) {
    const int kk = e / FS, c = e % FS;
    Fs[e] = c < r ? F[size_t(kk) * r + c] : 0.0;
  }
  const int64_t base = g.base(hd);
  // this thread's share of a chunk: groups of 8 elements e8 = threadIdx.x + 512 u, u < D / 32
  constexpr int PER = D >> 5;  // 4 for d = 128, 2 for d = 64
  Raw8<DT> xr8[PER];  // the next chunk's rows as stored
  auto fetch = [&](int row0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = (threadIdx.x + 512 * u) * 8, rr = e / D, cc = e % D;
      const int row = row0 + rr < rows ? row0 + rr : rows - 1;
      xr8[u] = load8_raw<DT>(x, base + int64_t(row) * g.sn + cc);
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = (threadIdx.x + 512 * u) * 8, rr = e / D, cc = e % D;
      float xv[8];
      widen8<DT>(xr8[u], xv);
      float* dst = Xs + rr * XS + cc;
      *reinterpret_cast<float4*>(dst) = make_float4(xv[0], xv[1], xv[2], xv[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(xv[4], xv[5], xv[6], xv[7]);
    }
  };
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r16 = lane & 15;
  const int first = blockIdx.x * chunks * 128;
  double csum[NT], cmax = 0.0;  // this lane's rows of columns nt * 16 + r16
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) csum[nt] = 0.0;
  fetch(first);
  for (int ch = 0; ch < chunks; ++ch) {
    const int row0 = first + ch * 128;
    if (row0 >= rows) break;
    __syncthreads();
    stage();
    __syncthreads();
    if (ch + 1 < chunks && row0 + 128 < rows) fetch(row0 + 128);
    f64x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    const float* xr = Xs + (w * 16 + r16) * XS + gq;
    const double* fr = Fs + gq * FS + r16;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) {
      const double av = xr[ks * 4];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, fr[ks * 4 * FS + nt * 16], acc[nt], 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double scale = 1.0;
      const int row = row0 + w * 16 + gq + 4 * v;
      if constexpr (RMS) {
        double s2 = 0.0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s2 = fma(acc[nt][v], acc[nt][v], s2);
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
        for (int nt = 0; nt < NT; ++nt) {
          const int c = nt * 16 + r16;
          if (c < r) {
            const double y = acc[nt][v] * scale;
            o[c] = y;
            csum[nt] += y;
            cmax = fmax(cmax, fabs(y));
          }
        }
      }
    }
  }
  if (kst.mu) {
    // the four row groups of a column, then the waves of the block through LDS (Xs is free)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      csum[nt] += __shfl_xor(csum[nt], 16);
      csum[nt] += __shfl_xor(csum[nt], 32);
    }
    for (int o = 32; o > 0; o >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, o));
    __syncthreads();
    double* red = reinterpret_cast<double*>(Xs);  // [8 waves][64 columns + 1]
    if (gq == 0)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) red[w * 65 + nt * 16 + r16] = nt < NT ? csum[nt] : 0.0;
    if (lane == 0) red[w * 65 + 64] = cmax;
    __syncthreads();
    if (threadIdx.x < r) {
      double t = 0.0;
      for (int q = 0; q < 8; ++q) t += red[q * 65 + threadIdx.x];
      atomicAdd(kst.mu + size_t(hd) * kst.mu_stride + threadIdx.x, t);
    }
    if (threadIdx.x == 64) {
      double m = 0.0;
      for (int q = 0; q < 8; ++q) m = fmax(m, red[q * 65 + 64]);
      atomicMax(reinterpret_cast<unsigned long long*>(kst.ctrl + size_t(hd) * kst.ctrl_stride + kst.amax_slot),
                (unsigned long long)__double_as_longlong(m));
    }
  }
}

size_t project_smem(int d, int r) {
  const int NT = (r + 15) >> 4;
  return size_t(d) * (NT * 16 + 8) * sizeof(double) + size_t(128) * (d + 4) * sizeof(float);
}

// Chunks of 128 rows per projection block (one block per CU fits in LDS): the count in [4, 16]
// with the shortest schedule, rounds of 256 blocks times chunks per block, the larger on ties.
static int project_chunks(int rows, int BH) {
  const int total = ceil_div(rows, 128);
  int best = 4, best_cost = 1 << 30;
  for (int c = 4; c <= 16; ++c) {
    const int64_t blocks = int64_t(BH) * ceil_div(total, c);
    const int64_t cost = (blocks + 255) / 256 * c;
    if (cost <= best_cost) {
      best = c;
      best_cost = int(cost);
    }
  }
  return best;
}

// Projection launch for row width d (64 or 128) and rank r <= 64 (NT = ceil(r / 16) tiles).
template <int DT, bool RMS>
static void launch_project(int d, int r, dim3 grid, size_t smem, hipStream_t st, const void* x, const HeadGeom& g,
                           int rows, const double* F, double eps, double* out, int* gstat, int chunks, int fdiv,
                           const KmStatsTarget& kst) {
  auto go = [&](auto kernel) {
    allow_lds(kernel, smem);
    hipLaunchKernelGGL(kernel, grid, dim3(512), smem, st, x, g, rows, F, r, eps, out, gstat, chunks, fdiv, kst);
  };
  const int nt = (r + 15) >> 4;
  if (d == 128) {
    if (nt == 1) go(project_kernel<DT, RMS, 128, 1>);
    else if (nt == 2) go(project_kernel<DT, RMS, 128, 2>);
    else if (nt == 3) go(project_kernel<DT, RMS, 128, 3>);
    else go(project_kernel<DT, RMS, 128, 4>);
  } else {
    if (nt == 1) go(project_kernel<DT, RMS, 64, 1>);
    else if (nt == 2) go(project_kernel<DT, RMS, 64, 2>);
    else if (nt == 3) go(project_kernel<DT, RMS, 64, 3>);
    else go(project_kernel<DT, RMS, 64, 4>);
  }
}

// ------------------------------------------------------------------ gathers and means
// Group-major copy of the rows of one tensor: dst[hd][pos] = src[hd][perm[pos]] for video
// positions and dst[hd][pos] = src[hd][pos] for the trailing text rows.  16-byte pieces.
template <int DT>
__global__ __launch_bounds__(256) void gather_rows_kernel(const void* __restrict__ src, HeadGeom g,
                                                          const int* __restrict__ perm, void* __restrict__ dst,
                                                          _Float16* __restrict__ dst16 = nullptr,
                                                          const float* __restrict__ scale16 = nullptr) {
  constexpr int ES = ElemSize<DT>::value;
  const int hd = blockIdx.y;
  const int pieces = g.d * ES / 16;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(g.N) * pieces) return;
  const int pos = int(idx / pieces), pc = int(idx % pieces);
  const int row = pos < g.Nv ? perm[size_t(hd) * g.Nv + pos] : pos;
  const char* s = static_cast<const char*>(src) + (g.base(hd) + int64_t(row) * g.sn) * ES + pc * 16;
  char* dd = static_cast<char*>(dst) + ((size_t(hd) * g.N + pos) * g.d) * ES + pc * 16;
  const uint4 u = *reinterpret_cast<const uint4*>(s);
  *reinterpret_cast<uint4*>(dd) = u;
  if (dst16) {  // bf16 rows: also the fp16 copy scaled by 2^e (the operand of the P V products)
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
    const float f = scale16[hd];
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      o[2 * c] = _Float16(__uint_as_float(wv[c] << 16) * f);
      o[2 * c + 1] = _Float16(__uint_as_float(wv[c] & 0xFFFF0000u) * f);
    }
    *reinterpret_cast<h8*>(dst16 + (size_t(hd) * g.N + pos) * g.d + pc * 8) = o;
  }
}

// Means of rows [off[b], off[b+1]) of a group-major [BH][N][d] tensor, one wave per group: d / 8
// lanes cover a row with 16-byte loads, so one load instruction reads 64 / (d / 8) rows; the row
// slots are summed across lanes at the end.
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
  const int L = d >> 3, step = 64 / L, slot = lane / L, sub = lane % L;
  const int r0 = off[size_t(hd) * (C + 1) + b], r1 = off[size_t(hd) * (C + 1) + b + 1];
  double acc[8] = {};
  int rr = r0 + slot;
  for (; rr + step < r1; rr += 2 * step) {
    float x[8], y[8];
    load8<DT>(src, (int64_t(hd) * N + rr) * d + sub * 8, x);
    load8<DT>(src, (int64_t(hd) * N + rr + step) * d + sub * 8, y);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += double(x[c]) + double(y[c]);
  }
  if (rr < r1) {
    float x[8];
    load8<DT>(src, (int64_t(hd) * N + rr) * d + sub * 8, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += double(x[c]);
  }
  for (int o2 = L; o2 < 64; o2 <<= 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], o2);
  if (slot == 0) {
    const double inv = 1.0 / double(r1 - r0);
#pragma unroll
    for (int c = 0; c < 8; ++c) o[sub * 8 + c] = acc[c] * inv;
  }
}

// c_a = mean of phi_Q over group a (App. A.2), members listed by perm.  One wave per group and
// block of 64 columns: each half-wave reads a member row as 16-byte pairs, two rows per step,
// four steps in flight.
__global__ __launch_bounds__(256) void group_mean_perm_kernel(const double* __restrict__ feat, int n, int r,
                                                              const int* __restrict__ perm,
                                                              const int* __restrict__ off,
                                                              const int* __restrict__ ngroups, int C,
                                                              double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= C || b >= ngroups[hd]) return;
  const int half = lane >> 5, col = blockIdx.z * 64 + (lane & 31) * 2;
  const bool act = col < r;
  const int r0 = off[size_t(hd) * (C + 1) + b], r1 = off[size_t(hd) * (C + 1) + b + 1];
  const int* pm = perm + size_t(hd) * n;
  const double* fh = feat + size_t(hd) * n * r + (act ? col : 0);
  double a0 = 0.0, a1 = 0.0;
  int p = r0 + half;
  for (; p + 6 < r1; p += 8) {
    double2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const double2*>(fh + size_t(pm[p + 2 * u]) * r);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a0 += v[u].x;
      a1 += v[u].y;
    }
  }
  for (; p < r1; p += 2) {
    const double2 v = *reinterpret_cast<const double2*>(fh + size_t(pm[p]) * r);
    a0 += v.x;
    a1 += v.y;
  }
  a0 += __shfl_xor(a0, 32);
  a1 += __shfl_xor(a1, 32);
  if (half == 0 && act) {
    const double inv = 1.0 / double(r1 - r0);
    out[(size_t(hd) * C + b) * r + col] = a0 * inv;
    out[(size_t(hd) * C + b) * r + col + 1] = a1 * inv;
  }
}

// d_i = |phi_Q(q_i) - c_a| for every video query row (App. A.2), original order.  16 lanes per row,
// strided over the r coordinates, reduced across those lanes.
__global__ __launch_bounds__(256) void qdist_kernel(const double* __restrict__ feat, int n, int r,
                                                    const int* __restrict__ lab, const double* __restrict__ cbar,
                                                    int C, double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int i = blockIdx.x * 16 + (threadIdx.x >> 4), sub = threadIdx.x & 15;
  double s = 0.0;
  if (i < n) {
    const int a = lab[size_t(hd) * n + i];
    const double* f = feat + (size_t(hd) * n + i) * r;
    const double* c = cbar + (size_t(hd) * C + a) * r;
    for (int e = sub; e < r; e += 16) {
      const double t = f[e] - c[e];
      s = fma(t, t, s);
    }
  }
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (i < n && sub == 0) out[size_t(hd) * n + i] = sqrt(s);
}

// Raw activations as k-means coordinates (the semantic partition of Sec. 3.1): the video rows of
// x widened to fp64, [BH][rows][d].  Eight consecutive elements per thread.
template <int DT>
__global__ __launch_bounds__(256) void raw_rows_kernel(const void* __restrict__ x, HeadGeom g, int rows,
                                                       double* __restrict__ out) {
  const int hd = blockIdx.y;
  const int64_t e8 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (e8 >= int64_t(rows) * g.d) return;
  const int row = int(e8 / g.d), c = int(e8 % g.d);
  float v[8];
  load8<DT>(x, g.base(hd) + int64_t(row) * g.sn + c, v);
  double* o = out + (size_t(hd) * rows + row) * g.d + c;
#pragma unroll
  for (int t = 0; t < 8; t += 2) *reinterpret_cast<double2*>(o + t) = make_double2(v[t], v[t + 1]);
}

// Initial centres of a later call on raw coordinates: previous centroid m as it stands; slots
// m >= n_prev take the cold draw of index m.
__global__ __launch_bounds__(256) void warm_centres_raw_kernel(const double* __restrict__ prev,
                                                               const int* __restrict__ n_prev, int C, int d,
                                                               const double* __restrict__ feat, int n, uint64_t seed,
                                                               int stage, double* __restrict__ cent) {
  const int hd = blockIdx.y, m = blockIdx.x;
  const int np = min(n_prev[hd], C);
  const double* src;
  if (m < np) {
    src = prev + (size_t(hd) * C + m) * d;
  } else {
    const uint64_t ctr = ((uint64_t(hd) * 2ull + uint64_t(stage)) << 20) + uint64_t(m);
    src = feat + (size_t(hd) * n + int(splitmix64(seed, ctr) % uint64_t(n))) * d;
  }
  for (int e = threadIdx.x; e < d; e += blockDim.x) cent[(size_t(hd) * C + m) * d + e] = src[e];
}

// Status bits of the K/V side (kvstat, per K/V head) into every query head of the group.
__global__ void merge_kv_status_kernel(int* __restrict__ gstat, const int* __restrict__ kvstat, int BH, int G) {
  const int hd = blockIdx.x * 256 + threadIdx.x;
  if (hd < BH) gstat[hd * 8 + 0] |= kvstat[(hd / G) * 8 + 0];
}

// ------------------------------------------------------------------ host drivers
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

spr_status launch_eigen_factor(const double* Mall, int BH, int d, int r, double clamp, double* Fall, int* gstat,
                               hipStream_t st) {
  const size_t sm = jacobi_smem(d);
  allow_lds(eigen_factor_kernel, sm);
  hipLaunchKernelGGL(eigen_factor_kernel, dim3(BH), dim3(256), sm, st, Mall, d, r, clamp, Fall, gstat, -1);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

template <int DT>
static spr_status partition_impl(const spr_desc& desc, const void* q, const void* k, const void* v,
                                 const spr_part_params& p, const spr_warm* warm, spr_partition& out, void* ws,
                                 const Workspace& L, hipStream_t st) {
  // The K/V side (M_K, F_K, the K/V partition, the centroids, M_Q and F_Q) runs once per K/V
  // head (BHkv heads, geometry gk); the query side per query head, which takes the factor F_Q
  // of its K/V head hd / G.  Status bits of the K/V side go to kvstat and are merged at the end.
  const HeadGeom g = make_geom(desc), gk = make_kv_geom(desc);
  const int BH = desc.B * desc.H, d = desc.d, Nv = g.Nv;
  const int G = kv_group_size(desc), BHkv = BH / G;
  double* metric = wsp<double>(ws, L.metric);
  double* phiK = out.phiK ? out.phiK : wsp<double>(ws, L.phiK);
  double* phiQ = out.phiQ ? out.phiQ : wsp<double>(ws, L.phiQ);
  int* gstat = wsp<int>(ws, L.gstat);
  int* kvstat = gstat + size_t(BH) * 8;
  hipLaunchKernelGGL(zero_ints_kernel, dim3(ceil_div((BH + BHkv) * 8, 256)), dim3(256), 0, st, gstat,
                     size_t(BH + BHkv) * 8);

  // Coordinates of the two k-means: response-coupled (factor products) or raw activations
  // (semantic partition), per mode; raw coordinates have rank d.
  const bool kv_raw = p.mode == SPR_PART_SEMANTIC, q_raw = p.mode != SPR_PART_RESPONSE;
  const int rK = kv_coord_rank(p, d), rQ = q_coord_rank(p, d);
  const size_t jac_smem = jacobi_smem(d);
  allow_lds(eigen_factor_kernel, jac_smem);
  // M_K and F_K
  if (!kv_raw) {
    const size_t kms = size_t(64) * (d + 2) * sizeof(double);
    if (d == 128) {
      allow_lds(key_metric_kernel<DT, 128>, kms);
      hipLaunchKernelGGL((key_metric_kernel<DT, 128>), dim3(d / 16, BHkv), dim3(256), kms, st, q, g, p.Ms, G, metric);
    } else {
      allow_lds(key_metric_kernel<DT, 64>, kms);
      hipLaunchKernelGGL((key_metric_kernel<DT, 64>), dim3(d / 16, BHkv), dim3(256), kms, st, q, g, p.Ms, G, metric);
    }
  }
  SPR_CHECK_LAUNCH();
  if (!kv_raw) {
    if (warm)  // later call: subspace update, the eigendecomposition only for heads it rejects
      launch_subspace(BHkv, d, p.rK, st, metric, warm->FK, p.eig_clamp, out.FK, kvstat, 2);
    hipLaunchKernelGGL(eigen_factor_kernel, dim3(BHkv), dim3(256), jac_smem, st, metric, d, p.rK, p.eig_clamp,
                       out.FK, kvstat, warm ? 2 : -1);
    SPR_CHECK_LAUNCH();
  }
  // phi_K = K F_K, or the raw keys
  const size_t prj_smem = project_smem(d, p.rK > p.rQ ? p.rK : p.rQ);
  const int pchunks = project_chunks(Nv, BH), kchunks = project_chunks(Nv, BHkv);
  const dim3 rgrid(unsigned(ceil_div64(int64_t(Nv) * d / 8, 256)), BHkv), rqgrid(rgrid.x, BH);
  KmArgs ka = kmeans_carve(wsp<char>(ws, L.km_region), BH, Nv, L.Cmax, L.rmax);
  ka.BH = BHkv;
  const KmStatsTarget kst = km_stats_target(ka);
  if (kv_raw) {
    hipLaunchKernelGGL(raw_rows_kernel<DT>, rgrid, dim3(256), 0, st, k, gk, Nv, phiK);
  } else {
    kmeans_stats_zero(ka, st);  // the projection accumulates the k-means point statistics
    launch_project<DT, false>(d, p.rK, dim3(ceil_div(ceil_div(Nv, 128), kchunks), BHkv), prj_smem, st, k, gk, Nv,
                              out.FK, p.rms_eps, phiK, kvstat, kchunks, 1, kst);
    ka.stats_given = true;
  }
  SPR_CHECK_LAUNCH();
  // K/V k-means
  ka.n = Nv; ka.r = rK; ka.C = p.Ck; ka.feat = phiK; ka.seed = p.seed; ka.stage = 0;
  ka.max_iters = p.max_iters; ka.tol = p.tol;
  ka.cent = wsp<double>(ws, L.km_cent); ka.labels = wsp<int>(ws, L.km_lab);
  if (warm) {
    if (kv_raw)
      hipLaunchKernelGGL(warm_centres_raw_kernel, dim3(p.Ck, BHkv), dim3(128), 0, st, warm->kbar, warm->n_kv, p.Ck, d,
                         phiK, Nv, p.seed, 0, ka.cent);
    else
      launch_warm_centres<false>(dim3(ceil_div(p.Ck, 64), BHkv), st, warm->kbar, warm->n_kv, p.Ck, d, out.FK, p.rK,
                                 p.rms_eps, phiK, Nv, p.seed, 0, 1, ka.cent);
    SPR_CHECK_LAUNCH();
    ka.cent_given = true;
  }
  spr_status s = run_kmeans(ka, st);
  if (s != SPR_OK) return s;
  if (out.passes) launch_copy_passes(ka.ctrl, BHkv, out.passes, 2, 0, st);
  if (out.cK_last) {
    // centres are stored with stride rK, exactly the caller's layout
    const size_t nel = size_t(BHkv) * p.Ck * rK;
    hipLaunchKernelGGL(copy_doubles_kernel, dim3(unsigned(ceil_div64(nel, 256))), dim3(256), 0, st, ka.cent,
                       out.cK_last, nel);
  }
  s = launch_compact(ka, out.kv_label, out.kv_perm, nullptr, out.kv_off, out.n_kv, kvstat, SPR_HS_KV_GROUPS_EMPTY, st);
  if (s != SPR_OK) return s;
  // group-major K and V, key / value centroids
  const int pieces = d * ElemSize<DT>::value / 16;
  const dim3 ggrid(unsigned(ceil_div64(int64_t(desc.N) * pieces, 256)), BH);
  const dim3 kgrid(unsigned(ceil_div64(int64_t(desc.N) * pieces, 256)), BHkv);
  hipLaunchKernelGGL(gather_rows_kernel<DT>, kgrid, dim3(256), 0, st, k, gk, out.kv_perm, out.Kp);
  if (DT == SPR_BF16) {
    // power-of-two scale of each K/V head's values for their fp16 copy
    launch_v_scale(v, gk, BHkv, wsp<unsigned>(ws, L.vamax), wsp<float>(ws, L.vscale), st);
    hipLaunchKernelGGL(gather_rows_kernel<DT>, kgrid, dim3(256), 0, st, v, gk, out.kv_perm, out.Vp,
                       wsp<_Float16>(ws, L.vh), static_cast<const float*>(wsp<float>(ws, L.vscale)));
  } else {
    hipLaunchKernelGGL(gather_rows_kernel<DT>, kgrid, dim3(256), 0, st, v, gk, out.kv_perm, out.Vp, nullptr,
                       nullptr);
  }
  SPR_CHECK_LAUNCH();
  hipLaunchKernelGGL(group_mean_kernel<DT>, dim3(ceil_div(p.Ck, 4), BHkv), dim3(256), 0, st, out.Kp, desc.N, d,
                     out.kv_off, out.n_kv, p.Ck, out.kbar);
  hipLaunchKernelGGL(group_mean_kernel<DT>, dim3(ceil_div(p.Ck, 4), BHkv), dim3(256), 0, st, out.Vp, desc.N, d,
                     out.kv_off, out.n_kv, p.Ck, out.vbar);
  SPR_CHECK_LAUNCH();
  if (!q_raw) {
    // M_Q and F_Q
    double* kt = wsp<double>(ws, L.ktilde);
    hipLaunchKernelGGL(ktilde_kernel, dim3(BHkv), dim3(1024), 0, st, out.kbar, out.n_kv, p.Ck, d, kt);
    hipLaunchKernelGGL(query_metric_kernel, dim3((d / 16) * (d / 16), BHkv), dim3(256), 0, st, kt, out.n_kv, p.Ck,
                       d, metric);
    if (warm)
      launch_subspace(BHkv, d, p.rQ, st, metric, warm->FQ, p.eig_clamp, out.FQ, kvstat, 3);
    hipLaunchKernelGGL(eigen_factor_kernel, dim3(BHkv), dim3(256), jac_smem, st, metric, d, p.rQ, p.eig_clamp,
                       out.FQ, kvstat, warm ? 3 : -1);
    SPR_CHECK_LAUNCH();
    // phi_Q = RMSNorm(Q F_Q), with the query k-means statistics (after the K/V k-means is done
    // with the shared buffers)
    KmArgs qz = ka;
    qz.BH = BH;
    kmeans_stats_zero(qz, st);
    launch_project<DT, true>(d, p.rQ, dim3(ceil_div(ceil_div(Nv, 128), pchunks), BH), prj_smem, st, q, g, Nv,
                             out.FQ, p.rms_eps, phiQ, gstat, pchunks, G, kst);
  } else {
    hipLaunchKernelGGL(raw_rows_kernel<DT>, rqgrid, dim3(256), 0, st, q, g, Nv, phiQ);
  }
  SPR_CHECK_LAUNCH();
  // query k-means
  KmArgs qa = ka;
  qa.BH = BH; qa.r = rQ; qa.C = p.Cq; qa.feat = phiQ; qa.stage = 1; qa.cent_given = warm != nullptr;
  qa.stats_given = !q_raw;
  if (warm) {
    if (q_raw)
      hipLaunchKernelGGL(warm_centres_raw_kernel, dim3(p.Cq, BH), dim3(128), 0, st, warm->qbar, warm->n_q, p.Cq, d,
                         phiQ, Nv, p.seed, 1, qa.cent);
    else
      launch_warm_centres<true>(dim3(ceil_div(p.Cq, 64), BH), st, warm->qbar, warm->n_q, p.Cq, d, out.FQ, p.rQ,
                                p.rms_eps, phiQ, Nv, p.seed, 1, G, qa.cent);
    SPR_CHECK_LAUNCH();
  }
  s = run_kmeans(qa, st);
  if (s != SPR_OK) return s;
  if (out.passes) launch_copy_passes(qa.ctrl, BH, out.passes, 2, 1, st);
  if (out.cQ_last) {
    const size_t nel = size_t(BH) * p.Cq * rQ;
    hipLaunchKernelGGL(copy_doubles_kernel, dim3(unsigned(ceil_div64(nel, 256))), dim3(256), 0, st, qa.cent,
                       out.cQ_last, nel);
  }
  s = launch_compact(qa, out.q_label, out.q_perm, out.q_pos, out.q_off, out.n_q, gstat, SPR_HS_Q_GROUPS_EMPTY, st);
  if (s != SPR_OK) return s;
  hipLaunchKernelGGL(gather_rows_kernel<DT>, ggrid, dim3(256), 0, st, q, g, out.q_perm, out.Qp);
  hipLaunchKernelGGL(group_mean_kernel<DT>, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, out.Qp, desc.N, d,
                     out.q_off, out.n_q, p.Cq, out.qbar);
  double* cbar = wsp<double>(ws, L.cbar);
  hipLaunchKernelGGL(group_mean_perm_kernel, dim3(ceil_div(p.Cq, 4), BH, ceil_div(rQ, 64)), dim3(256), 0, st, phiQ,
                     Nv, rQ, out.q_perm, out.q_off, out.n_q, p.Cq, cbar);
  hipLaunchKernelGGL(qdist_kernel, dim3(ceil_div(Nv, 16), BH), dim3(256), 0, st, phiQ, Nv, rQ, out.q_label, cbar,
                     p.Cq, out.qdist);
  hipLaunchKernelGGL(merge_kv_status_kernel, dim3(ceil_div(BH, 256)), dim3(256), 0, st, gstat, kvstat, BH, G);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_partition(const spr_desc& desc, const void* q, const void* k, const void* v, const spr_part_params& p,
                         const spr_warm* warm, spr_partition& out, void* ws, const Workspace& L, hipStream_t st) {
  if (desc.dtype == SPR_BF16) return partition_impl<SPR_BF16>(desc, q, k, v, p, warm, out, ws, L, st);
  return partition_impl<SPR_F32>(desc, q, k, v, p, warm, out, ws, L, st);
}

size_t jacobi_smem(int d) { return size_t(d) * (d + 1) * sizeof(double); }

}  // namespace spr
