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

__global__ __launch_bounds__(256) void fit_prep_kernel(const float* __restrict__ o_sp, const float* __restrict__ o_probe,
                                                       const int* __restrict__ probe_idx, const double* __restrict__ probe_w,
                                                       const int* __restrict__ q_pos, int N, int Nv, int d, int M,
                                                       double std_eps, double* __restrict__ Xb, double* __restrict__ Rb,
                                                       double* __restrict__ S, double* __restrict__ Wt) {
  __shared__ double red[32];
  const int hd = blockIdx.x;
  const int* pidx = probe_idx + size_t(hd) * M;
  const double* pw = probe_w + size_t(hd) * M;
  double ws = 0.0;
  for (int p = threadIdx.x; p < M; p += blockDim.x) ws += pw[p];
  const double wsum = block_sum_d(ws, red);
  for (int p = threadIdx.x; p < M; p += blockDim.x) Wt[size_t(hd) * M + p] = double(M) * pw[p] / wsum;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    double mx = 0.0, mr = 0.0;
    for (int p = 0; p < M; ++p) {
      const int pos = q_pos[size_t(hd) * Nv + pidx[p]];
      const double x = o_sp[(size_t(hd) * N + pos) * d + c];
      const double r = double(o_probe[(size_t(hd) * M + p) * d + c]) - x;
      const double al = pw[p] / wsum;
      mx = fma(al, x, mx);
      mr = fma(al, r, mr);
      Xb[(size_t(hd) * M + p) * d + c] = x;
      Rb[(size_t(hd) * M + p) * d + c] = r;
    }
    double var = 0.0;
    for (int p = 0; p < M; ++p) {
      const double t = Xb[(size_t(hd) * M + p) * d + c] - mx;
      var = fma(pw[p] / wsum, t * t, var);
    }
    const double sd = sqrt(var + std_eps);
    for (int p = 0; p < M; ++p) {
      double* xp = Xb + (size_t(hd) * M + p) * d + c;
      *xp = (*xp - mx) / sd;
      Rb[(size_t(hd) * M + p) * d + c] -= mr;
    }
    S[(size_t(hd) * 4 + 0) * d + c] = mx;
    S[(size_t(hd) * 4 + 1) * d + c] = sd;
    S[(size_t(hd) * 4 + 2) * d + c] = mr;
  }
}

// G = Xb^T W Xb + lam I and H = Xb^T W Rb, 16 x 16 tiles, probes staged in LDS.
__global__ __launch_bounds__(256) void normal_eq_kernel(const double* __restrict__ Xb, const double* __restrict__ Rb,
                                                        const double* __restrict__ Wt, int d, int M, double lam,
                                                        double* __restrict__ G, double* __restrict__ Hm) {
  __shared__ double Xi[32][17], Xj[32][17], Rj[32][17], Ws[32];
  const int hd = blockIdx.y;
  const int tiles = d / 16;
  const int i0 = (blockIdx.x / tiles) * 16, j0 = (blockIdx.x % tiles) * 16;
  const int ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
  double g = 0.0, h = 0.0;
  for (int p0 = 0; p0 < M; p0 += 32) {
    for (int e = threadIdx.x; e < 32 * 16; e += 256) {
      const int pp = e >> 4, cc = e & 15, p = p0 + pp;
      const bool ok = p < M;
      Xi[pp][cc] = ok ? Xb[(size_t(hd) * M + p) * d + i0 + cc] : 0.0;
      Xj[pp][cc] = ok ? Xb[(size_t(hd) * M + p) * d + j0 + cc] : 0.0;
      Rj[pp][cc] = ok ? Rb[(size_t(hd) * M + p) * d + j0 + cc] : 0.0;
    }
    if (threadIdx.x < 32) Ws[threadIdx.x] = p0 + threadIdx.x < M ? Wt[size_t(hd) * M + p0 + threadIdx.x] : 0.0;
    __syncthreads();
    for (int pp = 0; pp < 32; ++pp) {
      const double wx = Ws[pp] * Xi[pp][ti];
      g = fma(wx, Xj[pp][tj], g);
      h = fma(wx, Rj[pp][tj], h);
    }
    __syncthreads();
  }
  if (i0 + ti == j0 + tj) g += lam;
  G[size_t(hd) * d * d + size_t(i0 + ti) * d + j0 + tj] = g;
  Hm[size_t(hd) * d * d + size_t(i0 + ti) * d + j0 + tj] = h;
}

// In-LDS fp64 Cholesky G = L L^T (right-looking), then B = L^-T L^-1 H with one thread per
// column of H.  A pivot <= 0 (possible only with lam = 0) gives B = 0: the mean-only
// correction, flagged in head_status.  Finally the affine map of the apply step.
__global__ __launch_bounds__(256) void cholesky_solve_kernel(const double* __restrict__ Gall, double* __restrict__ Hall,
                                                             const double* __restrict__ S, int d,
                                                             float* __restrict__ applyB, float* __restrict__ applyC,
                                                             double* __restrict__ fit_state, const int* __restrict__ gstat,
                                                             int* __restrict__ head_status) {
  extern __shared__ double Lm[];  // d x d row-major
  __shared__ int fail;
  const int hd = blockIdx.x;
  const double* Gm = Gall + size_t(hd) * d * d;
  double* Hm = Hall + size_t(hd) * d * d;
  for (int e = threadIdx.x; e < d * d; e += blockDim.x) Lm[e] = Gm[e];
  if (threadIdx.x == 0) fail = 0;
  __syncthreads();
  for (int k = 0; k < d; ++k) {
    const double pivot = Lm[k * d + k];
    if (!(pivot > 0.0)) {
      if (threadIdx.x == 0) fail = 1;
      break;  // uniform: every thread read the same pivot
    }
    const double lkk = sqrt(pivot);
    __syncthreads();
    for (int i = k + 1 + threadIdx.x; i < d; i += blockDim.x) Lm[i * d + k] /= lkk;
    __syncthreads();
    if (threadIdx.x == 0) Lm[k * d + k] = lkk;
    const int m = d - k - 1;
    for (int e = threadIdx.x; e < m * m; e += blockDim.x) {
      const int i = k + 1 + e / m, j = k + 1 + e % m;
      if (j <= i) Lm[i * d + j] -= Lm[i * d + k] * Lm[j * d + k];
    }
    __syncthreads();
  }
  __syncthreads();
  const bool failed = fail != 0;
  if (threadIdx.x < d) {
    const int j = threadIdx.x;
    if (failed) {
      for (int i = 0; i < d; ++i) Hm[size_t(i) * d + j] = 0.0;
    } else {
      for (int i = 0; i < d; ++i) {  // forward: L y = h
        double s = Hm[size_t(i) * d + j];
        for (int kk = 0; kk < i; ++kk) s -= Lm[i * d + kk] * Hm[size_t(kk) * d + j];
        Hm[size_t(i) * d + j] = s / Lm[i * d + i];
      }
      for (int i = d - 1; i >= 0; --i) {  // backward: L^T b = y
        double s = Hm[size_t(i) * d + j];
        for (int kk = i + 1; kk < d; ++kk) s -= Lm[kk * d + i] * Hm[size_t(kk) * d + j];
        Hm[size_t(i) * d + j] = s / Lm[i * d + i];
      }
    }
  }
  __syncthreads();
  const double* mx = S + (size_t(hd) * 4 + 0) * d;
  const double* sd = S + (size_t(hd) * 4 + 1) * d;
  const double* mr = S + (size_t(hd) * 4 + 2) * d;
  for (int e = threadIdx.x; e < d * d; e += blockDim.x) {
    const int i = e / d, j = e % d;
    applyB[size_t(hd) * d * d + e] = float((i == j ? 1.0 : 0.0) + Hm[e] / sd[i]);
  }
  if (threadIdx.x < d) {
    const int j = threadIdx.x;
    double c = mr[j];
    for (int i = 0; i < d; ++i) c -= mx[i] / sd[i] * Hm[size_t(i) * d + j];
    applyC[size_t(hd) * d + j] = float(c);
  }
  if (fit_state) {
    double* fs = fit_state + size_t(hd) * (3 * d + d * d);
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
      fs[c] = mx[c];
      fs[d + c] = sd[c];
      fs[2 * d + c] = mr[c];
    }
    for (int e = threadIdx.x; e < d * d; e += blockDim.x) fs[3 * d + e] = Hm[e];
  }
  if (threadIdx.x == 0) head_status[hd] = gstat[hd * 8 + 0] | (failed ? SPR_HS_CHOLESKY_FALLBACK : 0);
}

// O^hat rows for 64 group-major positions: corrected video rows scattered to their original
// row, text rows copied.  Thread = 4 rows x 8 columns; X tile stored transposed in LDS.
template <int D, int OUT_DT>
__global__ __launch_bounds__(256) void apply_kernel(const float* __restrict__ o_sp, const int* __restrict__ q_perm,
                                                    const float* __restrict__ applyB, const float* __restrict__ applyC,
                                                    int N, int Nv, void* __restrict__ out) {
  extern __shared__ float fsm[];
  float* Bs = fsm;               // [D][D]
  float* XT = fsm + D * D;       // [D][65]
  const int hd = blockIdx.y, row0 = blockIdx.x * 64;
  const float* Bm = applyB + size_t(hd) * D * D;
  for (int e = threadIdx.x * 4; e < D * D; e += 1024) *reinterpret_cast<float4*>(Bs + e) = *reinterpret_cast<const float4*>(Bm + e);
  for (int e = threadIdx.x; e < 64 * D; e += 256) {
    const int rr = e / D, c = e % D, pos = row0 + rr;
    XT[c * 65 + rr] = pos < N ? o_sp[(size_t(hd) * N + pos) * D + c] : 0.f;
  }
  __syncthreads();
  constexpr int CQ = D / 8;          // column blocks of 8
  constexpr int RQ = 256 / CQ;       // row groups
  constexpr int RPT = 64 / RQ;       // rows per thread
  const int cq = threadIdx.x % CQ, rq = threadIdx.x / CQ;
  float acc[RPT][8];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = applyC[size_t(hd) * D + cq * 8 + j];
  for (int k = 0; k < D; ++k) {
    float xr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) xr[i] = XT[k * 65 + rq * RPT + i];
    const float4 b0 = *reinterpret_cast<const float4*>(Bs + k * D + cq * 8);
    const float4 b1 = *reinterpret_cast<const float4*>(Bs + k * D + cq * 8 + 4);
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xr[i], bb[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int pos = row0 + rq * RPT + i;
    if (pos >= N) continue;
    size_t dst;
    if (pos < Nv) {
      dst = (size_t(hd) * N + q_perm[size_t(hd) * Nv + pos]) * D + cq * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) store_out<OUT_DT>(out, dst + j, acc[i][j]);
    } else {
      dst = (size_t(hd) * N + pos) * D + cq * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) store_out<OUT_DT>(out, dst + j, XT[(cq * 8 + j) * 65 + rq * RPT + i]);
    }
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
static void launch_apply(const spr_desc& desc, const float* o_sp, const int* q_perm, const float* B, const float* C,
                         void* out, hipStream_t st) {
  const size_t sm = size_t(D) * D * sizeof(float) + size_t(D) * 65 * sizeof(float);
  allow_lds(apply_kernel<D, OUT_DT>, sm);
  hipLaunchKernelGGL((apply_kernel<D, OUT_DT>), dim3(ceil_div(desc.N, 64), desc.B * desc.H), dim3(256), sm, st, o_sp,
                     q_perm, B, C, desc.N, desc.N - desc.n_text, out);
}

spr_status run_fit_correct(const spr_desc& desc, const spr_part_params& p, const spr_partition& part,
                           const spr_route& route, const float* o_sp, const float* o_probe, int M, double lam,
                           double std_eps, void* out, int out_dtype, double* fit_state, int* head_status, void* ws,
                           const Workspace& L, hipStream_t st) {
  (void)p;
  const int BH = desc.B * desc.H, d = desc.d, N = desc.N, Nv = N - desc.n_text;
  double* Xb = ws_ptr<double>(ws, L.fitX);
  double* Rb = ws_ptr<double>(ws, L.fitR);
  double* G = ws_ptr<double>(ws, L.fitG);
  double* Hm = ws_ptr<double>(ws, L.fitH);
  double* S = ws_ptr<double>(ws, L.fitS);
  double* Wt = ws_ptr<double>(ws, L.fitW);
  float* AB = ws_ptr<float>(ws, L.applyB);
  float* AC = ws_ptr<float>(ws, L.applyC);
  hipLaunchKernelGGL(fit_prep_kernel, dim3(BH), dim3(256), 0, st, o_sp, o_probe, route.probe_idx, route.probe_w,
                     part.q_pos, N, Nv, d, M, std_eps, Xb, Rb, S, Wt);
  hipLaunchKernelGGL(normal_eq_kernel, dim3((d / 16) * (d / 16), BH), dim3(256), 0, st, Xb, Rb, Wt, d, M, lam, G, Hm);
  SPR_CHECK_LAUNCH();
  const size_t sm = size_t(d) * d * sizeof(double);
  allow_lds(cholesky_solve_kernel, sm);
  hipLaunchKernelGGL(cholesky_solve_kernel, dim3(BH), dim3(256), sm, st, G, Hm, S, d, AB, AC, fit_state,
                     ws_ptr<int>(ws, L.gstat), head_status);
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
