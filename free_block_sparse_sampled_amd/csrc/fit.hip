// Probe-fitted residual reconstruction ("Partition the Support, Reconstruct the Residual",
// Sec. 4.2, App. A.3, App. D.3) on gfx950.
//
// Per head: coverage weights alpha = w / sum w and W = diag(M w / sum w); probe features
// X = O^sp rows standardised by their alpha-weighted mean and sqrt(weighted variance + eps);
// residuals R = O^dense - O^sp centred by their alpha-weighted mean mu_R; the normal
// equations (Xb^T W Xb + lam I) B = Xb^T W Rb are built in fp64 and solved by an fp64
// Cholesky factorisation in one workgroup.  The correction is then folded into one affine
// map, O^hat = O^sp (I + diag(1/sd) B) + (mu_R - (mu_X / sd) B), applied to every row while
// it is scattered back to the original row order.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

// Probe features and residuals of one head and 32 columns per block: thread (column c,
// stripe s) takes probes p = s, s + 8, ...; the weighted means and variance are combined over
// the 8 stripes in LDS.
__global__ __launch_bounds__(256) void fit_prep_kernel(const float* __restrict__ o_sp, const float* __restrict__ o_probe,
                                                       const int* __restrict__ probe_idx, const double* __restrict__ probe_w,
                                                       const int* __restrict__ q_pos, int N, int Nv, int d, int M,
                                                       double std_eps, double* __restrict__ Xb, double* __restrict__ Rb,
                                                       double* __restrict__ S, double* __restrict__ Wt) {
  __shared__ double red[32];
  __shared__ double part[2][8][32];
  const int hd = blockIdx.y, c = blockIdx.x * 32 + (threadIdx.x & 31), st = threadIdx.x >> 5;
  const int* pidx = probe_idx + size_t(hd) * M;
  const double* pw = probe_w + size_t(hd) * M;
  double ws = 0.0;
  for (int p = threadIdx.x; p < M; p += blockDim.x) ws += pw[p];
  const double wsum = block_sum_d(ws, red);
  if (blockIdx.x == 0)
    for (int p = threadIdx.x; p < M; p += blockDim.x) Wt[size_t(hd) * M + p] = double(M) * pw[p] / wsum;
  double* xb = Xb + size_t(hd) * M * d + c;
  double* rb = Rb + size_t(hd) * M * d + c;
  double mx = 0.0, mr = 0.0;
#pragma unroll 4
  for (int p = st; p < M; p += 8) {
    const int pos = q_pos[size_t(hd) * Nv + pidx[p]];
    const double x = o_sp[(size_t(hd) * N + pos) * d + c];
    const double r = double(o_probe[(size_t(hd) * M + p) * d + c]) - x;
    const double al = pw[p] / wsum;
    mx = fma(al, x, mx);
    mr = fma(al, r, mr);
    xb[size_t(p) * d] = x;
    rb[size_t(p) * d] = r;
  }
  part[0][st][threadIdx.x & 31] = mx;
  part[1][st][threadIdx.x & 31] = mr;
  __syncthreads();
  mx = 0.0;
  mr = 0.0;
  for (int t = 0; t < 8; ++t) {
    mx += part[0][t][threadIdx.x & 31];
    mr += part[1][t][threadIdx.x & 31];
  }
  double var = 0.0;
  for (int p = st; p < M; p += 8) {
    const double t = xb[size_t(p) * d] - mx;
    var = fma(pw[p] / wsum, t * t, var);
  }
  __syncthreads();
  part[0][st][threadIdx.x & 31] = var;
  __syncthreads();
  var = 0.0;
  for (int t = 0; t < 8; ++t) var += part[0][t][threadIdx.x & 31];
  const double sd = sqrt(var + std_eps);
  for (int p = st; p < M; p += 8) {
    xb[size_t(p) * d] = (xb[size_t(p) * d] - mx) / sd;
    rb[size_t(p) * d] -= mr;
  }
  if (st == 0) {
    S[(size_t(hd) * 4 + 0) * d + c] = mx;
    S[(size_t(hd) * 4 + 1) * d + c] = sd;
    S[(size_t(hd) * 4 + 2) * d + c] = mr;
  }
}

// G = Xb^T W Xb + lam I and H = Xb^T W Rb on v_mfma_f64_16x16x4f64; with WITH_C also
// Cr = Rb^T W Rb (the residual second moment of the output truncation, App. D.3).  Block
// (i0 / 16, head) forms rows i0 .. i0 + 15 of each product, wave w its column tiles w, w + 4, ..;
// the probes stream through LDS in chunks of 16.  Products with A = rows of w Xb (or w Rb) and
// B = rows of Xb or Rb: lane l feeds probe k0 + l / 16 of column i0 + l % 16 (A) and of column
// j0 + l % 16 (B); accumulator v of lane l is entry (i0 + l / 16 + 4 v, j0 + l % 16).
typedef double fit_f64x4 __attribute__((ext_vector_type(4)));
constexpr int kNePc = 16;
template <bool WITH_C, int D>
__global__ __launch_bounds__(256) void normal_eq_kernel(const double* __restrict__ Xb, const double* __restrict__ Rb,
                                                        const double* __restrict__ Wt, int M, double lam,
                                                        double* __restrict__ G, double* __restrict__ Hm,
                                                        double* __restrict__ Cr) {
  constexpr int XS = D + 1, TW = D / 64;  // LDS row stride; column tiles per wave
  __shared__ double Xs[kNePc][XS], Rs[kNePc][XS], Ws[kNePc];
  const int hd = blockIdx.y, i0 = blockIdx.x * 16;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, kq = lane >> 4;
  fit_f64x4 ag[TW], ah[TW], ac[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) ag[u] = ah[u] = ac[u] = fit_f64x4{0.0, 0.0, 0.0, 0.0};
  for (int p0 = 0; p0 < M; p0 += kNePc) {
    __syncthreads();
    for (int e = threadIdx.x; e < kNePc * D; e += 256) {
      const int pp = e / D, c = e % D, p = p0 + pp;
      const bool ok = p < M;
      Xs[pp][c] = ok ? Xb[(size_t(hd) * M + p) * D + c] : 0.0;
      Rs[pp][c] = ok ? Rb[(size_t(hd) * M + p) * D + c] : 0.0;
    }
    if (threadIdx.x < kNePc) Ws[threadIdx.x] = p0 + threadIdx.x < M ? Wt[size_t(hd) * M + p0 + threadIdx.x] : 0.0;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kNePc; kk += 4) {
      const int p = kk + kq;
      const double a = Ws[p] * Xs[p][i0 + r16];
      const double ar = WITH_C ? Ws[p] * Rs[p][i0 + r16] : 0.0;
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        const int j = (w + 4 * u) * 16 + r16;
        ag[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Xs[p][j], ag[u], 0, 0, 0);
        ah[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Rs[p][j], ah[u], 0, 0, 0);
        if constexpr (WITH_C) ac[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(ar, Rs[p][j], ac[u], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TW; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + kq + 4 * v, j = (w + 4 * u) * 16 + r16;
      const size_t at = size_t(hd) * D * D + size_t(i) * D + j;
      G[at] = ag[u][v] + (i == j ? lam : 0.0);
      Hm[at] = ah[u][v];
      if constexpr (WITH_C) Cr[at] = ac[u][v];
    }
}

// C (m x n, row stride ldc) = op(A) op(B) with 4 x 4 register tiles per thread; op(A)(i, k) is
// A[i * lda + k], or A[k * lda + i] when AT; op(B)(k, j) is B[k * ldb + j], or B[j * ldb + k]
// when BT; m, n multiples of 4.
template <bool AT, bool BT = false>
__device__ inline void fit_gemm(const double* A, int lda, const double* B, int ldb, double* C, int ldc, int m, int n,
                                int K) {
  const int tr = m / 4, tc = n / 4;
  for (int t = threadIdx.x; t < tr * tc; t += blockDim.x) {
    const int i0 = (t / tc) * 4, j0 = (t % tc) * 4;
    double acc[4][4] = {};
#pragma unroll 2
    for (int k = 0; k < K; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) a[x] = AT ? A[size_t(k) * lda + i0 + x] : A[size_t(i0 + x) * lda + k];
#pragma unroll
      for (int y = 0; y < 4; ++y) b[y] = BT ? B[size_t(j0 + y) * ldb + k] : B[size_t(k) * ldb + j0 + y];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(a[x], b[y], acc[x][y]);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) C[size_t(i0 + x) * ldc + j0 + y] = acc[x][y];
  }
}

// Round to the nearest bf16 (ties to even) as a bit pattern.
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The affine map of the apply step from B (in the H buffer): E = diag(1 / sd) B, stored
// transposed (E^T[n][k]) as bf16 high and low parts so that hi + lo carries E to about 2^-16,
// and c = mu_R - (mu_X / sd) B in fp32; the fit state and the head status.  8 D threads:
// column b = t / 8 of B, rows s + 8 i.
template <int D>
__device__ inline void fit_epilogue(const double* __restrict__ Hall, const double* __restrict__ S,
                                    uint16_t* __restrict__ applyE, float* __restrict__ applyC,
                                    double* __restrict__ fit_state, const int* __restrict__ gstat,
                                    int* __restrict__ head_status, double* isd, double* wmx) {
  constexpr int NI = D / 8;
  const int hd = blockIdx.x, tid = threadIdx.x, nth = 8 * D;
  const int b = tid >> 3, s = tid & 7;
  const double* Hm = Hall + size_t(hd) * D * D;
  const double* mx = S + (size_t(hd) * 4 + 0) * D;
  const double* sd = S + (size_t(hd) * 4 + 1) * D;
  const double* mr = S + (size_t(hd) * 4 + 2) * D;
  for (int c = tid; c < D; c += nth) {
    isd[c] = 1.0 / sd[c];
    wmx[c] = mx[c] / sd[c];
  }
  __syncthreads();
  uint16_t* Eh = applyE + size_t(hd) * 2 * D * D;
  uint16_t* El = Eh + size_t(D) * D;
  for (int e = tid; e < D * D; e += nth) {
    const int k = e / D, n = e % D;
    const float x = float(Hm[e] * isd[k]);
    const uint16_t h = bf16_rne(x);
    Eh[size_t(n) * D + k] = h;
    El[size_t(n) * D + k] = bf16_rne(x - __uint_as_float(uint32_t(h) << 16));
  }
  {
    // c_j = mu_R_j - sum_i (mu_X_i / sd_i) B_ij: column j = b, rows i = s + 8 t, lanes combined
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < NI; ++i) part = fma(wmx[s + 8 * i], Hm[size_t(s + 8 * i) * D + b], part);
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    part += __shfl_xor(part, 4);
    if (s == 0) applyC[size_t(hd) * D + b] = float(mr[b] - part);
  }
  if (fit_state) {
    double* fs = fit_state + size_t(hd) * (3 * D + D * D);
    for (int c = tid; c < D; c += nth) {
      fs[c] = mx[c];
      fs[D + c] = sd[c];
      fs[2 * D + c] = mr[c];
    }
    for (int e = tid; e < D * D; e += nth) fs[3 * D + e] = Hm[e];
  }
  if (tid == 0) head_status[hd] = gstat[hd * 8 + 0];
}

template <int D>
__global__ __launch_bounds__(8 * D) void fit_epilogue_kernel(const double* __restrict__ Hall,
                                                             const double* __restrict__ S,
                                                             uint16_t* __restrict__ applyE,
                                                             float* __restrict__ applyC,
                                                             double* __restrict__ fit_state,
                                                             const int* __restrict__ gstat,
                                                             int* __restrict__ head_status) {
  __shared__ double isd[D], wmx[D];
  fit_epilogue<D>(Hall, S, applyE, applyC, fit_state, gstat, head_status, isd, wmx);
}

template <int D>
__device__ inline void solve_full(double* Gm, double* Hm, double* Rm, double (*rowbuf)[D], int* gstat);

// Per head, one workgroup of 8 D threads: thread t owns column b = t / 8 of the d x d matrix,
// rows a = (t % 8) + 8 i (i < D / 8) in registers, so the 8 owners of a column sit in adjacent
// lanes.
//  - Upper Cholesky G = R^T R, right-looking: step k publishes row k of the reduced matrix in
//    LDS (double-buffered, one barrier per step), every thread scales it by 1 / sqrt(pivot)
//    and updates its own entries a_ab -= r_ka r_kb (k < a <= b).
//  - R^{-1} row by row from the bottom (R T = I): T_ij = -(sum_{i<k<=j} R_ik T_kj) / R_ii,
//    T_ii = 1 / R_ii; row i of R is published in LDS, each thread sums over its own rows k
//    and the 8 owners of column j combine their sums by lane shuffles.
//  - B = R^{-1} (R^{-T} H) by two register-tiled products (R^{-1} in LDS; R^{-T} H goes to the
//    G buffer, B to the H buffer).
// A pivot <= 0 (possible only with lam = 0) gives B = 0: the mean-only correction, flagged in
// head_status.  The restricted families of App. D.4 minimise the same penalised error over
// smaller sets and need no factorisation: B = 0 (mean-only), B = a I with a = tr H / tr G
// (scalar, penalty lam d a^2), B = diag(H_cc / G_cc) (diagonal).  B goes to the H buffer.
template <int D>
__global__ __launch_bounds__(8 * D) void cholesky_solve_kernel(double* __restrict__ Gall, double* __restrict__ Hall,
                                                               int family, int* __restrict__ gstat, bool epilogue,
                                                               const double* __restrict__ S,
                                                               uint16_t* __restrict__ applyE,
                                                               float* __restrict__ applyC,
                                                               double* __restrict__ fit_state,
                                                               int* __restrict__ head_status) {
  extern __shared__ double Rm[];  // D x D row-major (R^{-1})
  __shared__ double rowbuf[2][D];
  const int hd = blockIdx.x, tid = threadIdx.x, nth = 8 * D;
  double* Gm = Gall + size_t(hd) * D * D;
  double* Hm = Hall + size_t(hd) * D * D;
  if (family != SPR_FIT_FULL) {
    double* gd = rowbuf[0];
    double* hdg = rowbuf[1];
    for (int c = tid; c < D; c += nth) {
      gd[c] = Gm[size_t(c) * D + c];
      hdg[c] = Hm[size_t(c) * D + c];
    }
    __syncthreads();
    double a = 0.0;
    if (family == SPR_FIT_SCALAR) {
      double tg = 0.0, th = 0.0;
      for (int c = 0; c < D; ++c) {
        tg += gd[c];
        th += hdg[c];
      }
      a = tg > 0.0 ? th / tg : 0.0;
    }
    for (int e = tid; e < D * D; e += nth) {
      const int i = e / D, j = e % D;
      double v = 0.0;
      if (i == j) {
        if (family == SPR_FIT_SCALAR) v = a;
        else if (family == SPR_FIT_DIAG) v = gd[i] > 0.0 ? hdg[i] / gd[i] : 0.0;
      }
      Hm[e] = v;
    }
  } else {
    solve_full<D>(Gm, Hm, Rm, rowbuf, gstat);
  }
  if (epilogue) {
    __syncthreads();
    fit_epilogue<D>(Hall, S, applyE, applyC, fit_state, gstat, head_status, rowbuf[0], rowbuf[1]);
  }
}

// Full ridge: Cholesky, triangular inverse and the two products (see above).
template <int D>
__device__ inline void solve_full(double* Gm, double* Hm, double* Rm, double (*rowbuf)[D], int* gstat) {
  constexpr int NI = D / 8;
  const int hd = blockIdx.x, tid = threadIdx.x, nth = 8 * D;
  const int b = tid >> 3, s = tid & 7;
  double A[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) A[i] = Gm[size_t(s + 8 * i) * D + b];
  // Row k = 8 ib + s0 lives in register slot ib of the threads with s == s0.  The slot loop is
  // unrolled so that every register index is a constant (a runtime index would send the array
  // to scratch memory).
  bool failed = false;
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
#pragma unroll 1
    for (int s0 = 0; s0 < 8; ++s0) {
      const int k = 8 * ib + s0;
      double* rb = rowbuf[k & 1];
      if (s == s0) rb[b] = A[ib];
      __syncthreads();
      const double piv = rb[k];
      if (!(piv > 0.0)) {  // uniform: every thread read the same pivot
        failed = true;
        break;
      }
      const double inv = 1.0 / sqrt(piv);
      const double rkb = b > k ? rb[b] * inv : (b == k ? sqrt(piv) : 0.0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i < ib) continue;  // rows above the pivot row are final
        const int a = s + 8 * i;
        const double upd = fma(-rb[a] * inv, rkb, A[i]);
        A[i] = a == k ? rkb : (a > k && a <= b ? upd : A[i]);
      }
    }
    if (failed) break;
  }
  __syncthreads();  // the last step's row buffer is the first one the inverse writes
  if (!failed) {
    // the strict lower triangle holds leftovers of G: clear it
#pragma unroll
    for (int i = 0; i < NI; ++i) A[i] = s + 8 * i > b ? 0.0 : A[i];
#pragma unroll
    for (int ib = NI - 1; ib >= 0; --ib) {
#pragma unroll 1
      for (int s0 = 7; s0 >= 0; --s0) {
        const int i0 = 8 * ib + s0;
        double* rb = rowbuf[i0 & 1];
        if (s == s0) rb[b] = A[ib];
        __syncthreads();
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i < ib) continue;  // rows k <= i0 do not enter row i0 of the inverse
          const int kk = s + 8 * i;
          part = kk > i0 && kk <= b ? fma(rb[kk], A[i], part) : part;
        }
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        const double rii = rb[i0];
        const double t = b > i0 ? -part / rii : (b == i0 ? 1.0 / rii : 0.0);
        A[ib] = s == s0 ? t : A[ib];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) Rm[(s + 8 * i) * D + b] = A[i];
    __syncthreads();
    fit_gemm<true>(Rm, D, Hm, D, Gm, D, D, D, D);  // Y = R^{-T} H
    __syncthreads();
    fit_gemm<false>(Rm, D, Gm, D, Hm, D, D, D, D);  // B = R^{-1} Y
  } else {
    for (int e = tid; e < D * D; e += nth) Hm[e] = 0.0;
    if (tid == 0) gstat[hd * 8 + 0] |= SPR_HS_CHOLESKY_FALLBACK;
  }
}

// Output truncation (App. D.3): B <- B V_r V_r^T with V_r the leading eigenvectors of
// Rb^T W Rb, given as the columns f_k of its factor F = U_r Lambda_r^{1/2} ([D][r], zero columns
// for clamped eigenvalues): V_r V_r^T = sum_k f_k f_k^T / |f_k|^2.  F is staged in LDS with the
// rank padded to a multiple of 4 by zero columns; T = B F goes to the G buffer.
template <int D>
__global__ __launch_bounds__(256) void truncate_kernel(double* __restrict__ Hall, double* __restrict__ Gall,
                                                       const double* __restrict__ Fall, int r) {
  extern __shared__ double Fs[];  // [D][r4], then norms [r4]
  const int hd = blockIdx.x, tid = threadIdx.x;
  const int r4 = (r + 3) & ~3;
  double* nrm = Fs + D * r4;
  const double* F = Fall + size_t(hd) * D * r;
  double* Hm = Hall + size_t(hd) * D * D;
  double* Tm = Gall + size_t(hd) * D * D;
  for (int e = tid; e < D * r4; e += 256) {
    const int i = e / r4, k = e % r4;
    Fs[e] = k < r ? F[size_t(i) * r + k] : 0.0;
  }
  __syncthreads();
  for (int k = tid; k < r4; k += 256) {
    double x = 0.0;
    for (int i = 0; i < D; ++i) x = fma(Fs[i * r4 + k], Fs[i * r4 + k], x);
    nrm[k] = x > 0.0 ? 1.0 / x : 0.0;
  }
  fit_gemm<false>(Hm, D, Fs, r4, Tm, r4, D, r4, D);  // T = B F
  __syncthreads();
  for (int e = tid; e < D * r4; e += 256) Fs[e] *= nrm[e % r4];
  __syncthreads();
  fit_gemm<false, true>(Tm, r4, Fs, r4, Hm, D, D, D, r4);  // B = T (F diag(1/|f|^2))^T
}

typedef __bf16 fit_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float fit_f32x4_t __attribute__((ext_vector_type(4)));

// O^hat = X + X E + c for 16-row tiles of group-major positions (X = O^sp rows, fp32), each
// video row scattered to its original row, text rows copied.  X E runs on the bf16 matrix cores
// as X_hi E_hi + X_hi E_lo + X_lo E_hi with fp32 accumulation (X = X_hi + X_lo, likewise E), the
// identity term X stays exact fp32.  E^T (hi and lo) sits in LDS; each wave takes 16-row tiles,
// loads them straight into A fragments (lane l: row l % 16, columns 32 ks + 8 (l / 16) .. + 7),
// and turns the C fragments back into that row layout through a per-wave LDS tile.
template <int D, int OUT_DT>
__global__ __launch_bounds__(512) void apply_kernel(const float* __restrict__ o_sp, const int* __restrict__ q_perm,
                                                    const uint16_t* __restrict__ applyE,
                                                    const float* __restrict__ applyC, int N, int Nv,
                                                    int tiles_per_block, void* __restrict__ out) {
  constexpr int KS = D / 32, CT = D / 16, LDE = D + 8, LDO = D + 4;
  extern __shared__ uint16_t esm[];  // [2][D][LDE] E^T hi, lo; then 8 x [16][LDO] fp32 tiles
  float* otile = reinterpret_cast<float*>(esm + 2 * D * LDE) + (threadIdx.x >> 6) * 16 * LDO;
  const int hd = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
  const uint16_t* Eg = applyE + size_t(hd) * 2 * D * D;
  for (int e = threadIdx.x * 8; e < 2 * D * D; e += 512 * 8) {
    const int part = e / (D * D), n = (e % (D * D)) / D, k = e % D;
    *reinterpret_cast<uint4*>(esm + (part * D + n) * LDE + k) = *reinterpret_cast<const uint4*>(Eg + e);
  }
  float cb[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) cb[ct] = applyC[size_t(hd) * D + ct * 16 + r16];
  __syncthreads();
  const int ntiles = (N + 15) / 16;
  const int t0 = blockIdx.x * tiles_per_block, t1 = min(t0 + tiles_per_block, ntiles);
  for (int t = t0 + w; t < t1; t += 8) {
    const int pos = t * 16 + r16;
    const float* xr = o_sp + (size_t(hd) * N + (pos < N ? pos : 0)) * D + 8 * kg;
    float x[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 u = *reinterpret_cast<const float4*>(xr + 32 * ks);
      const float4 v = *reinterpret_cast<const float4*>(xr + 32 * ks + 4);
      x[ks][0] = u.x; x[ks][1] = u.y; x[ks][2] = u.z; x[ks][3] = u.w;
      x[ks][4] = v.x; x[ks][5] = v.y; x[ks][6] = v.z; x[ks][7] = v.w;
    }
    fit_f32x4_t acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = fit_f32x4_t{cb[ct], cb[ct], cb[ct], cb[ct]};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fit_bf16x8_t ah, al;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint16_t h = bf16_rne(x[ks][c]);
        const float hf = __uint_as_float(uint32_t(h) << 16);
        ah[c] = __builtin_bit_cast(__bf16, h);
        al[c] = __builtin_bit_cast(__bf16, bf16_rne(x[ks][c] - hf));
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int off = (ct * 16 + r16) * LDE + 32 * ks + 8 * kg;
        const fit_bf16x8_t bh = *reinterpret_cast<const fit_bf16x8_t*>(esm + off);
        const fit_bf16x8_t bl = *reinterpret_cast<const fit_bf16x8_t*>(esm + D * LDE + off);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[ct], 0, 0, 0);
      }
    }
    // C fragment: lane l holds rows 4 (l / 16) + v, column 16 ct + l % 16
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) otile[(4 * kg + v) * LDO + ct * 16 + r16] = acc[ct][v];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (pos < N) {
      const bool video = pos < Nv;
      const size_t row = video ? size_t(q_perm[size_t(hd) * Nv + pos]) : size_t(pos);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int col = 32 * ks + 8 * kg;
        const float4 u = *reinterpret_cast<const float4*>(otile + r16 * LDO + col);
        const float4 v = *reinterpret_cast<const float4*>(otile + r16 * LDO + col + 4);
        const float cx[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
        float y[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] = video ? x[ks][c] + cx[c] : x[ks][c];
        const size_t dst = (size_t(hd) * N + row) * D + col;
        if constexpr (OUT_DT == SPR_BF16) {
          uint4 o;
          o.x = uint32_t(bf16_rne(y[0])) | (uint32_t(bf16_rne(y[1])) << 16);
          o.y = uint32_t(bf16_rne(y[2])) | (uint32_t(bf16_rne(y[3])) << 16);
          o.z = uint32_t(bf16_rne(y[4])) | (uint32_t(bf16_rne(y[5])) << 16);
          o.w = uint32_t(bf16_rne(y[6])) | (uint32_t(bf16_rne(y[7])) << 16);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + dst) = o;
        } else {
          float* o = static_cast<float*>(out) + dst;
          *reinterpret_cast<float4*>(o) = make_float4(y[0], y[1], y[2], y[3]);
          *reinterpret_cast<float4*>(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int OUT_DT>
__global__ void probe_write_kernel(const float* __restrict__ o_probe, const int* __restrict__ probe_idx, int N, int d,
                                   int M, void* __restrict__ out) {
  const int hd = blockIdx.y, p = blockIdx.x;
  const int row = probe_idx[size_t(hd) * M + p];
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    store_out<OUT_DT>(out, (size_t(hd) * N + row) * d + c, o_probe[(size_t(hd) * M + p) * d + c]);
}

template <int D, int OUT_DT>
static void launch_apply(const spr_desc& desc, const float* o_sp, const int* q_perm, const uint16_t* E, const float* C,
                         void* out, hipStream_t st) {
  const size_t sm = size_t(2) * D * (D + 8) * sizeof(uint16_t) + size_t(8) * 16 * (D + 4) * sizeof(float);
  constexpr int kTilesPerBlock = 64;
  allow_lds(apply_kernel<D, OUT_DT>, sm);
  hipLaunchKernelGGL((apply_kernel<D, OUT_DT>), dim3(ceil_div(ceil_div(desc.N, 16), kTilesPerBlock), desc.B * desc.H),
                     dim3(512), sm, st, o_sp, q_perm, E, C, desc.N, desc.N - desc.n_text, kTilesPerBlock, out);
}

spr_status run_fit_correct(const spr_desc& desc, const spr_part_params& p, const spr_partition& part,
                           const spr_route& route, const float* o_sp, const float* o_probe, int M, double lam,
                           double std_eps, int family, int out_rank, void* out, int out_dtype, double* fit_state,
                           int* head_status, void* ws, const Workspace& L, hipStream_t st) {
  const int BH = desc.B * desc.H, d = desc.d, N = desc.N, Nv = N - desc.n_text;
  double* Xb = ws_ptr<double>(ws, L.fitX);
  double* Rb = ws_ptr<double>(ws, L.fitR);
  double* G = ws_ptr<double>(ws, L.fitG);
  double* Hm = ws_ptr<double>(ws, L.fitH);
  double* S = ws_ptr<double>(ws, L.fitS);
  double* Wt = ws_ptr<double>(ws, L.fitW);
  uint16_t* AB = ws_ptr<uint16_t>(ws, L.applyB);
  float* AC = ws_ptr<float>(ws, L.applyC);
  int* gstat = ws_ptr<int>(ws, L.gstat);
  const bool trunc = out_rank > 0 && out_rank < d;
  double* Cr = trunc ? ws_ptr<double>(ws, L.metric) : nullptr;  // the metric buffer is free after partitioning
  double* Fr = ws_ptr<double>(ws, L.fitF);
  hipLaunchKernelGGL(fit_prep_kernel, dim3(d / 32, BH), dim3(256), 0, st, o_sp, o_probe, route.probe_idx, route.probe_w,
                     part.q_pos, N, Nv, d, M, std_eps, Xb, Rb, S, Wt);
  const dim3 neg(d / 16, BH);
  if (d == 128) {
    if (trunc)
      hipLaunchKernelGGL((normal_eq_kernel<true, 128>), neg, dim3(256), 0, st, Xb, Rb, Wt, M, lam, G, Hm, Cr);
    else
      hipLaunchKernelGGL((normal_eq_kernel<false, 128>), neg, dim3(256), 0, st, Xb, Rb, Wt, M, lam, G, Hm, Cr);
  } else {
    if (trunc)
      hipLaunchKernelGGL((normal_eq_kernel<true, 64>), neg, dim3(256), 0, st, Xb, Rb, Wt, M, lam, G, Hm, Cr);
    else
      hipLaunchKernelGGL((normal_eq_kernel<false, 64>), neg, dim3(256), 0, st, Xb, Rb, Wt, M, lam, G, Hm, Cr);
  }
  SPR_CHECK_LAUNCH();
  if (trunc) {
    const spr_status s = launch_eigen_factor(Cr, BH, d, out_rank, p.eig_clamp, Fr, gstat, st);
    if (s != SPR_OK) return s;
  }
  const size_t sm = size_t(d) * d * sizeof(double);
  const size_t tsm = (size_t(d) + 1) * ((out_rank + 3) & ~3) * sizeof(double);
  if (d == 128) {
    allow_lds(cholesky_solve_kernel<128>, sm);
    hipLaunchKernelGGL(cholesky_solve_kernel<128>, dim3(BH), dim3(1024), sm, st, G, Hm, family, gstat, !trunc, S, AB,
                       AC, fit_state, head_status);
    if (trunc) {
      allow_lds(truncate_kernel<128>, tsm);
      hipLaunchKernelGGL(truncate_kernel<128>, dim3(BH), dim3(256), tsm, st, Hm, G, Fr, out_rank);
      hipLaunchKernelGGL(fit_epilogue_kernel<128>, dim3(BH), dim3(1024), 0, st, Hm, S, AB, AC, fit_state, gstat,
                         head_status);
    }
  } else {
    allow_lds(cholesky_solve_kernel<64>, sm);
    hipLaunchKernelGGL(cholesky_solve_kernel<64>, dim3(BH), dim3(512), sm, st, G, Hm, family, gstat, !trunc, S, AB,
                       AC, fit_state, head_status);
    if (trunc) {
      allow_lds(truncate_kernel<64>, tsm);
      hipLaunchKernelGGL(truncate_kernel<64>, dim3(BH), dim3(256), tsm, st, Hm, G, Fr, out_rank);
      hipLaunchKernelGGL(fit_epilogue_kernel<64>, dim3(BH), dim3(512), 0, st, Hm, S, AB, AC, fit_state, gstat,
                         head_status);
    }
  }
  SPR_CHECK_LAUNCH();
  if (d == 128) {
    if (out_dtype == SPR_BF16) launch_apply<128, SPR_BF16>(desc, o_sp, part.q_perm, AB, AC, out, st);
    else launch_apply<128, SPR_F32>(desc, o_sp, part.q_perm, AB, AC, out, st);
  } else {
    if (out_dtype == SPR_BF16) launch_apply<64, SPR_BF16>(desc, o_sp, part.q_perm, AB, AC, out, st);
    else launch_apply<64, SPR_F32>(desc, o_sp, part.q_perm, AB, AC, out, st);
  }
  SPR_CHECK_LAUNCH();
  if (out_dtype == SPR_BF16)
    hipLaunchKernelGGL(probe_write_kernel<SPR_BF16>, dim3(M, BH), dim3(128), 0, st, o_probe, route.probe_idx, N, d, M, out);
  else
    hipLaunchKernelGGL(probe_write_kernel<SPR_F32>, dim3(M, BH), dim3(128), 0, st, o_probe, route.probe_idx, N, d, M, out);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

}  // namespace spr
