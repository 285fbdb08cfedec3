// k-means of the response coordinates ("Partition the Support, Reconstruct the Residual",
// Sec. 4.1 for the K/V and query partitions, App. C.1 for the initialisation, Table C.1 for
// the limits) on gfx950.
//
// One Lloyd pass = four kernels:
//  screen   squared distances of every point to every centre from an MFMA cross term.
//           Coordinates are centred by the head's mean point and scaled by a power of two,
//           then split into fp16 hi + lo parts; x.c ~ hi.hi + hi.lo + lo.hi on
//           v_mfma_f32_16x16x32_f16.  A bound on the error of the screened distances decides,
//           per point, whether the nearest centre is certain; the rest go to a queue.
//  rescan   queued points: fp64 direct-difference distances to every centre (exact nearest,
//           ties to the lowest index), one wave per point.
//  accum    fp64 distance to the chosen centre (cost), label change count, and the Lloyd sums:
//           a wave walks its 64 points in order, one lane per coordinate, flushing a running sum
//           with fp64 atomics when the label changes.
//  finalize stopping rule (labels unchanged, relative cost decrease <= tol, or max_iters),
//           centre update (empty centres stay), and the fp16 split of the new centres.
// The control word per head (done flag, pass count, previous cost, largest centre norm, scale)
// lives on the device, so the host launches max_iters passes without synchronising and
// finished heads return immediately.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Coordinates are padded to RP = 64 (ranks up to 64) or 128 (rank 128, the raw 128-dimensional
// activations of the semantic partition) for the MFMA screening; the mean point is stored with
// stride RPMAX whatever the padding.
constexpr int RPMAX = 128;
constexpr int KC = 256;       // centres per LDS chunk
constexpr int CTRL = 8;       // doubles of control word per head
__host__ __device__ constexpr int crow(int rp) { return rp + 8; }  // LDS row stride (fp16), conflict free
__host__ __device__ constexpr int rpad(int r) { return r > 64 ? 128 : 64; }

enum { C_DONE = 0, C_PASSES = 1, C_JPREV = 2, C_CMAX = 3, C_SCALE = 4, C_AMAX = 5, C_STOPNOW = 6 };

__device__ __forceinline__ f16x8_t as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8_t, u); }

// Mean point mu and the power-of-two scale s with 2 max|x| s <= 2^14.  Row slices of the
// points are reduced by 64 blocks per head into fp64 sums (atomics) and a max (atomicMax on the
// bit pattern, monotone for non-negative doubles); km_stats_final_kernel divides and scales.
__global__ void km_stats_zero_kernel(double* __restrict__ mu, double* __restrict__ ctrl, int BH) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < BH * RPMAX) mu[i] = 0.0;
  if (i < BH) ctrl[i * CTRL + C_AMAX] = 0.0;
}

__global__ __launch_bounds__(256) void km_point_stats_kernel(const double* __restrict__ feat, int n, int r,
                                                             double* __restrict__ mu, double* __restrict__ ctrl) {
  __shared__ double ssum[256], smax[256];
  // EW threads per row (one coordinate each), 256 / EW rows at a time
  const int EW = r > 64 ? 128 : 64, NR = 256 / EW;
  const int hd = blockIdx.y, t = threadIdx.x, e = t % EW, r0 = t / EW;
  const int j0 = int(int64_t(n) * blockIdx.x / gridDim.x), j1 = int(int64_t(n) * (blockIdx.x + 1) / gridDim.x);
  double s = 0.0, m = 0.0;
  if (e < r)
    for (int j = j0 + r0; j < j1; j += NR) {
      const double x = feat[(size_t(hd) * n + j) * r + e];
      s += x;
      m = fmax(m, fabs(x));
    }
  ssum[t] = s;
  smax[t] = m;
  __syncthreads();
  if (t < EW) {
    double tot = 0.0;
    for (int q = 0; q < NR; ++q) tot += ssum[t + q * EW];
    if (t < r) atomicAdd(mu + size_t(hd) * RPMAX + t, tot);
  }
  if (t < 64) {
    double mx = fmax(fmax(smax[t], smax[t + 64]), fmax(smax[t + 128], smax[t + 192]));
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    if (t == 0)
      atomicMax(reinterpret_cast<unsigned long long*>(ctrl + hd * CTRL + C_AMAX),
                (unsigned long long)__double_as_longlong(mx));
  }
}

__global__ void km_stats_final_kernel(double* __restrict__ mu, double* __restrict__ ctrl, int n) {
  const int hd = blockIdx.x, e = threadIdx.x;
  mu[size_t(hd) * RPMAX + e] /= double(n);
  if (e == 0) {
    const double amax = ctrl[hd * CTRL + C_AMAX];
    double sc = 1.0;
    if (amax > 0.0) sc = ldexp(1.0, int(floor(log2(8192.0 / amax))));  // 2 amax sc <= 2^14
    ctrl[hd * CTRL + C_SCALE] = sc;
  }
}

// Scaled, centred fp16 hi/lo parts of every point and their norms.  RP / 8 lanes per point.
template <int RP>
__global__ __launch_bounds__(256) void km_point_prep_kernel(const double* __restrict__ feat, int n, int r,
                                                            const double* __restrict__ mu,
                                                            const double* __restrict__ ctrl,
                                                            _Float16* __restrict__ xh, _Float16* __restrict__ xl,
                                                            float* __restrict__ xnrm) {
  constexpr int LP = RP / 8;
  const int hd = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int j = idx / LP, cb = idx % LP;
  const bool valid = j < n;
  const double sc = ctrl[hd * CTRL + C_SCALE];
  double nrm = 0.0;
  if (valid) {
    _Float16 hv[8], lv[8];
    // r is a multiple of 8: a lane's eight coordinates are four aligned 16-byte loads
    double xr[8];
    const bool live = cb * 8 < r;
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const double2 t2 = live ? *reinterpret_cast<const double2*>(feat + (size_t(hd) * n + j) * r + cb * 8 + u)
                              : make_double2(0.0, 0.0);
      xr[u] = t2.x;
      xr[u + 1] = t2.y;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = cb * 8 + u;
      const double x = live ? (xr[u] - mu[size_t(hd) * RPMAX + e]) * sc : 0.0;
      const _Float16 h = _Float16(float(x));
      hv[u] = h;
      lv[u] = _Float16(float(x - double(h)));
      nrm = fma(x, x, nrm);
    }
    *reinterpret_cast<f16x8_t*>(xh + (size_t(hd) * n + j) * RP + cb * 8) =
        f16x8_t{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
    *reinterpret_cast<f16x8_t*>(xl + (size_t(hd) * n + j) * RP + cb * 8) =
        f16x8_t{lv[0], lv[1], lv[2], lv[3], lv[4], lv[5], lv[6], lv[7]};
  }
#pragma unroll
  for (int o = 1; o < LP; o <<= 1) nrm += __shfl_xor(nrm, o);
  if (valid && cb == 0) xnrm[size_t(hd) * n + j] = float(sqrt(nrm));
}

// fp16 split of the centres (same centring and scale as the points), their squared norms and
// the largest norm.  Element-parallel over the whole block of one head; n2s is LDS [C].
template <int RP>
__device__ void prep_centres(int hd, int C, int r, const double* __restrict__ cent, const double* __restrict__ mu,
                             double sc, _Float16* __restrict__ ch, _Float16* __restrict__ cl,
                             float* __restrict__ cn2, double* __restrict__ ctrl, double* n2s, double* red) {
  for (int m = threadIdx.x; m < C; m += blockDim.x) n2s[m] = 0.0;
  __syncthreads();
  for (int idx = threadIdx.x; idx < C * RP; idx += blockDim.x) {
    const int m = idx / RP, e = idx % RP;
    const double x = e < r ? (cent[(size_t(hd) * C + m) * r + e] - mu[size_t(hd) * RPMAX + e]) * sc : 0.0;
    const _Float16 h = _Float16(float(x));
    ch[(size_t(hd) * C + m) * RP + e] = h;
    cl[(size_t(hd) * C + m) * RP + e] = _Float16(float(x - double(h)));
    if (x != 0.0) atomicAdd(&n2s[m], x * x);
  }
  __syncthreads();
  double cmax = 0.0;
  for (int m = threadIdx.x; m < C; m += blockDim.x) {
    cn2[size_t(hd) * C + m] = float(n2s[m]);
    cmax = fmax(cmax, sqrt(n2s[m]));
  }
  for (int o = 32; o > 0; o >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tmax = 0.0;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) tmax = fmax(tmax, red[w]);
    ctrl[hd * CTRL + C_CMAX] = tmax;
  }
}

// Initial centres: C feature rows drawn uniformly with replacement by SplitMix64,
// counter ((head * 2 + stage) << 20) + m (App. C.1).
template <int RP>
__global__ __launch_bounds__(1024) void km_init_kernel(const double* __restrict__ feat, int n, int r, int C,
                                                      uint64_t seed, int stage, const double* __restrict__ mu,
                                                      double* __restrict__ cent, double* __restrict__ sums,
                                                      int* __restrict__ cnt, double* __restrict__ ctrl,
                                                      _Float16* __restrict__ ch, _Float16* __restrict__ cl,
                                                      float* __restrict__ cn2, int* __restrict__ rq_count,
                                                      int cent_given) {
  __shared__ double red[32];
  __shared__ double n2s[1024];
  const int hd = blockIdx.x;
  for (int idx = threadIdx.x; idx < C * r; idx += blockDim.x) {
    const int m = idx / r, e = idx % r;
    if (!cent_given) {
      const uint64_t ctr = ((uint64_t(hd) * 2ull + uint64_t(stage)) << 20) + uint64_t(m);
      const int j = int(splitmix64(seed, ctr) % uint64_t(n));
      cent[(size_t(hd) * C + m) * r + e] = feat[(size_t(hd) * n + j) * r + e];
    }
    sums[(size_t(hd) * C + m) * r + e] = 0.0;
  }
  for (int m = threadIdx.x; m < C; m += blockDim.x) cnt[size_t(hd) * C + m] = 0;
  __syncthreads();
  prep_centres<RP>(hd, C, r, cent, mu, ctrl[hd * CTRL + C_SCALE], ch, cl, cn2, ctrl, n2s, red);
  if (threadIdx.x == 0) {
    ctrl[hd * CTRL + C_DONE] = 0.0;
    ctrl[hd * CTRL + C_PASSES] = 0.0;
    ctrl[hd * CTRL + C_JPREV] = 0.0;
    rq_count[hd] = 0;
  }
}

// Screening pass.  A wave owns 64 points (4 tiles of 16); centres stream through LDS in
// chunks of 256.  The MFMA computes D^T tiles (16 centres x 16 points), so a lane holds four
// centres of one point and keeps that point's best value, its index and the second best.
template <int KS, int RP>
__global__ __launch_bounds__(256) void km_screen_kernel(int n, int C, const _Float16* __restrict__ xh,
                                                        const _Float16* __restrict__ xl,
                                                        const float* __restrict__ xnrm,
                                                        const _Float16* __restrict__ ch,
                                                        const _Float16* __restrict__ cl,
                                                        const float* __restrict__ cn2,
                                                        const double* __restrict__ ctrl, int* __restrict__ lab_new,
                                                        int* __restrict__ rq_count, int* __restrict__ rq_list) {
  constexpr int CROW = crow(RP);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  _Float16* Ch = reinterpret_cast<_Float16*>(smem);
  _Float16* Cl = Ch + KC * CROW;
  float* cns = reinterpret_cast<float*>(Cl + KC * CROW);
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, r16 = lane & 15;
  const int p0 = blockIdx.x * 256 + w * 64;
  f16x8_t bh[4][KS], bl[4][KS];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int j = p0 + pt * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 uh = make_uint4(0, 0, 0, 0), ul = make_uint4(0, 0, 0, 0);
      if (j < n) {
        uh = *reinterpret_cast<const uint4*>(xh + (size_t(hd) * n + j) * RP + ks * 32 + 8 * g);
        ul = *reinterpret_cast<const uint4*>(xl + (size_t(hd) * n + j) * RP + ks * 32 + 8 * g);
      }
      bh[pt][ks] = as_f16x8(uh);
      bl[pt][ks] = as_f16x8(ul);
    }
  }
  float b1[4], b2[4];
  int i1[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    b1[pt] = INFINITY;
    b2[pt] = INFINITY;
    i1[pt] = 0;
  }
  const _Float16* chh = ch + size_t(hd) * C * RP;
  const _Float16* cll = cl + size_t(hd) * C * RP;
  for (int c0 = 0; c0 < C; c0 += KC) {
    const int cc = min(KC, C - c0);
    __syncthreads();
    for (int e = t; e < KC * (RP / 8); e += 256) {
      const int row = e / (RP / 8), pc = e % (RP / 8);
      uint4 uh = make_uint4(0, 0, 0, 0), ul = make_uint4(0, 0, 0, 0);
      if (row < cc) {
        uh = *reinterpret_cast<const uint4*>(chh + size_t(c0 + row) * RP + pc * 8);
        ul = *reinterpret_cast<const uint4*>(cll + size_t(c0 + row) * RP + pc * 8);
      }
      *reinterpret_cast<uint4*>(Ch + row * CROW + pc * 8) = uh;
      *reinterpret_cast<uint4*>(Cl + row * CROW + pc * 8) = ul;
    }
    for (int e = t; e < KC; e += 256) cns[e] = e < cc ? cn2[size_t(hd) * C + c0 + e] : INFINITY;
    __syncthreads();
    const int nblk = (cc + 15) >> 4;
    for (int cb = 0; cb < nblk; ++cb) {
      f16x8_t ah[KS], al[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ah[ks] = as_f16x8(*reinterpret_cast<const uint4*>(Ch + (cb * 16 + r16) * CROW + ks * 32 + 8 * g));
        al[ks] = as_f16x8(*reinterpret_cast<const uint4*>(Cl + (cb * 16 + r16) * CROW + ks * 32 + 8 * g));
      }
      float cv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) cv[v] = cns[cb * 16 + 4 * g + v];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bh[pt][ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bl[pt][ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[ks], bh[pt][ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // branch-free running best / index / second best
          const float val = fmaf(-2.f, acc[v], cv[v]);
          const int m = c0 + cb * 16 + 4 * g + v;
          b2[pt] = fminf(b2[pt], fmaxf(b1[pt], val));
          i1[pt] = val < b1[pt] ? m : i1[pt];
          b1[pt] = fminf(b1[pt], val);
        }
      }
    }
  }
  const double cmax = ctrl[hd * CTRL + C_CMAX];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    // merge the four lanes of a point (their centre subsets are disjoint)
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ob1 = __shfl_xor(b1[pt], o), ob2 = __shfl_xor(b2[pt], o);
      const int oi = __shfl_xor(i1[pt], o);
      if (ob1 < b1[pt] || (ob1 == b1[pt] && oi < i1[pt])) {
        b2[pt] = fminf(ob2, b1[pt]);
        b1[pt] = ob1;
        i1[pt] = oi;
      } else {
        b2[pt] = fminf(b2[pt], ob1);
      }
    }
    const int j = p0 + pt * 16 + r16;
    if (g == 0 && j < n) {
      // bound on |screened - exact| squared distance (scaled units): cross-term error of
      // the split product with fp32 sums, plus fp32 rounding of norms and combination;
      // doubled for safety.  Decided when the runner-up is more than twice that away.
      const double xn = xnrm[size_t(hd) * n + j];
      const double tcross = (3.0 * RP * 5.960464477539063e-8 + 3.0 * 2.384185791015625e-7) * xn * cmax;
      const double E = 2.0 * (2.0 * tcross + 4.0 * 5.960464477539063e-8 * (xn + cmax) * (xn + cmax)) +
                       1e-12 * (xn + cmax) * (xn + cmax);
      const bool decided = double(b2[pt]) - double(b1[pt]) > 2.0 * E;
      lab_new[size_t(hd) * n + j] = decided ? i1[pt] : -1;
      if (!decided) {
        const int k = atomicAdd(rq_count + hd, 1);
        rq_list[size_t(hd) * n + k] = j;
      }
    }
  }
}

// fp64 nearest centre of every queued point, one wave per point (ties to the lowest index).
// The point sits in registers for ranks up to 64 and in the wave's LDS row (broadcast reads)
// for rank 128.
template <int R>
__global__ __launch_bounds__(256) void km_rescan_kernel(int n, int C, const double* __restrict__ feat,
                                                        const double* __restrict__ cent,
                                                        const double* __restrict__ ctrl,
                                                        const int* __restrict__ rq_count,
                                                        const int* __restrict__ rq_list, int* __restrict__ lab_new) {
  constexpr bool INLDS = R > 64;
  __shared__ double xs[INLDS ? 4 * R : 1];
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int cnt = rq_count[hd];
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int i = blockIdx.x * 4 + (threadIdx.x >> 6); i < cnt; i += nw) {
    const int j = rq_list[size_t(hd) * n + i];
    const double* f = feat + (size_t(hd) * n + j) * R;
    double xr[INLDS ? 1 : R];
    double* xw = xs + (INLDS ? (threadIdx.x >> 6) * R : 0);
    if constexpr (INLDS) {
      __builtin_amdgcn_wave_barrier();
      for (int e = lane; e < R; e += 64) xw[e] = f[e];
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll
      for (int e = 0; e < R; ++e) xr[e] = f[e];
    }
    const double* x = INLDS ? xw : xr;
    double best = INFINITY;
    int bi = 0;
    for (int m = lane; m < C; m += 64) {
      const double* c = cent + (size_t(hd) * C + m) * R;
      double dd = 0.0;
#pragma unroll
      for (int e = 0; e < R; ++e) {
        const double tdiff = x[e] - c[e];
        dd = fma(tdiff, tdiff, dd);
      }
      if (dd < best) {
        best = dd;
        bi = m;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ob < best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (lane == 0) lab_new[size_t(hd) * n + j] = bi;
  }
}

// Cost, label changes and Lloyd sums of the pass.  Each wave walks its 64 points in order with
// one lane per coordinate: it adds x to a running sum that is flushed (fp64 atomics) when the
// label changes, and (x - c_label)^2 to the lane's share of the cost.
template <int R>
__global__ __launch_bounds__(256) void km_accum_kernel(const double* __restrict__ feat, int n, int C,
                                                       const double* __restrict__ cent,
                                                       const int* __restrict__ lab_new, int* __restrict__ labels,
                                                       double* __restrict__ jpart, int* __restrict__ cpart,
                                                       const double* __restrict__ ctrl, double* __restrict__ sums,
                                                       int* __restrict__ cnt, int nblk) {
  __shared__ double red[32];
  __shared__ int64_t redi[32];
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const bool valid = j < n;
  int lab = 0, changed = 0;
  if (valid) {
    lab = lab_new[size_t(hd) * n + j];
    int* lp = labels + size_t(hd) * n + j;
    changed = (*lp != lab);
    *lp = lab;
  }
  // EPL coordinates per lane: lane + 64 q, q < EPL
  constexpr int EPL = (R + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int wbase = blockIdx.x * 256 + (threadIdx.x & ~63);
  const int L = valid ? lab : -1;
  int cur = __shfl(L, 0);
  double acc[EPL], cc[EPL], jsq = 0.0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + 64 * q;
    acc[q] = 0.0;
    cc[q] = (e < R && cur >= 0) ? cent[(size_t(hd) * C + cur) * R + e] : 0.0;
  }
  int run = 0;
  for (int p = 0; p < 64; ++p) {
    const int Lp = __shfl(L, p);
    if (Lp < 0) break;
    if (Lp != cur) {
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const int e = lane + 64 * q;
        if (e < R) atomicAdd(sums + (size_t(hd) * C + cur) * R + e, acc[q]);
        acc[q] = 0.0;
      }
      if (lane == 0) atomicAdd(cnt + size_t(hd) * C + cur, run);
      run = 0;
      cur = Lp;
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const int e = lane + 64 * q;
        if (e < R) cc[q] = cent[(size_t(hd) * C + cur) * R + e];
      }
    }
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + 64 * q;
      if (e < R) {
        const double x = feat[(size_t(hd) * n + wbase + p) * R + e];
        acc[q] += x;
        const double t = x - cc[q];
        jsq = fma(t, t, jsq);
      }
    }
    ++run;
  }
  if (run > 0) {
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + 64 * q;
      if (e < R) atomicAdd(sums + (size_t(hd) * C + cur) * R + e, acc[q]);
    }
    if (lane == 0) atomicAdd(cnt + size_t(hd) * C + cur, run);
  }
  const double jsum = block_sum_d(jsq, red);
  const int64_t csum = block_sum_i64(changed, redi);
  if (threadIdx.x == 0) {
    jpart[size_t(hd) * nblk + blockIdx.x] = jsum;
    cpart[size_t(hd) * nblk + blockIdx.x] = int(csum);
  }
}

// Stopping rule after a pass (one block per head): stop when the labels did not change, when
// the cost fell by at most tol relative to the previous pass, or at max_iters.  The decision is
// written to ctrl[C_STOPNOW]; km_update_kernel then moves the centres of heads that go on.
__global__ __launch_bounds__(256) void km_decide_kernel(int max_iters, double tol, int nblk,
                                                        const double* __restrict__ jpart,
                                                        const int* __restrict__ cpart, double* __restrict__ ctrl) {
  __shared__ double red[32];
  __shared__ int64_t redi[32];
  const int hd = blockIdx.x;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  double js = 0.0;
  int64_t cs = 0;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) {
    js += jpart[size_t(hd) * nblk + i];
    cs += cpart[size_t(hd) * nblk + i];
  }
  const double J = block_sum_d(js, red);
  const int64_t chg = block_sum_i64(cs, redi);
  if (threadIdx.x == 0) {
    const int passes = int(ctrl[hd * CTRL + C_PASSES]) + 1;
    const double Jprev = ctrl[hd * CTRL + C_JPREV];
    const bool stop = (passes > 1 && (chg == 0 || Jprev - J <= tol * Jprev)) || passes >= max_iters;
    ctrl[hd * CTRL + C_STOPNOW] = stop ? 1.0 : 0.0;
    ctrl[hd * CTRL + C_PASSES] = double(passes);
    ctrl[hd * CTRL + C_JPREV] = J;
    ctrl[hd * CTRL + C_CMAX] = 0.0;
  }
}

// Centre update (members' mean; empty centres stay), reset of the sums, and the fp16 split of
// the new centres for the next screening pass.  64 centres per block, one wave per centre row
// at a time; the largest centre norm is combined with atomicMax on its (non-negative) bits.
template <int RP>
__global__ __launch_bounds__(256) void km_update_kernel(int C, int r, double* __restrict__ cent,
                                                        double* __restrict__ sums, int* __restrict__ cnt,
                                                        double* __restrict__ ctrl, const double* __restrict__ mu,
                                                        _Float16* __restrict__ ch, _Float16* __restrict__ cl,
                                                        float* __restrict__ cn2, int* __restrict__ rq_count) {
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const bool stop = ctrl[hd * CTRL + C_STOPNOW] != 0.0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double sc = ctrl[hd * CTRL + C_SCALE];
  double cmax = 0.0;
  for (int m = blockIdx.x * 64 + w; m < min(C, blockIdx.x * 64 + 64); m += 4) {
    const size_t base = (size_t(hd) * C + m);
    const int k = cnt[base];
    double n2l = 0.0;
#pragma unroll
    for (int q = 0; q < RP / 64; ++q) {
      const int e = lane + 64 * q;
      double x = 0.0;
      if (e < r) {
        double c = cent[base * r + e];
        if (!stop && k > 0) {
          c = sums[base * r + e] / double(k);
          cent[base * r + e] = c;
        }
        sums[base * r + e] = 0.0;
        x = (c - mu[size_t(hd) * RPMAX + e]) * sc;
      }
      if (!stop) {
        const _Float16 h = _Float16(float(x));
        ch[base * RP + e] = h;
        cl[base * RP + e] = _Float16(float(x - double(h)));
        n2l = fma(x, x, n2l);
      }
    }
    if (!stop) {
      const double n2 = wave_sum_d(n2l);
      if (lane == 0) cn2[base] = float(n2);
      cmax = fmax(cmax, sqrt(n2));
    }
    if (lane == 0) cnt[base] = 0;
  }
  if (!stop && lane == 0 && cmax > 0.0)
    atomicMax(reinterpret_cast<unsigned long long*>(ctrl + hd * CTRL + C_CMAX),
              (unsigned long long)__double_as_longlong(cmax));
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    rq_count[hd] = 0;
    if (stop) ctrl[hd * CTRL + C_DONE] = 1.0;
  }
}

__global__ void copy_passes1_kernel(const double* ctrl, int BH, int* passes, int stride, int slot) {
  const int hd = blockIdx.x * blockDim.x + threadIdx.x;
  if (hd < BH) passes[hd * stride + slot] = int(ctrl[hd * CTRL + C_PASSES]);
}

void launch_copy_passes(const double* ctrl, int BH, int* passes, int stride, int slot, hipStream_t st) {
  hipLaunchKernelGGL(copy_passes1_kernel, dim3(ceil_div(BH, 256)), dim3(256), 0, st, ctrl, BH, passes, stride, slot);
}

bool kmeans_rank_supported(int r) { return r == 8 || r == 16 || r == 32 || r == 48 || r == 64 || r == 128; }

size_t kmeans_ws_bytes(int BH, int n, int C, int rmax) {
  size_t o = 0;
  auto take = [&](size_t b) { o += (b + 255) & ~size_t(255); };
  const int nblk = ceil_div(n, 256);
  take(size_t(BH) * C * rmax * 8);  // sums
  take(size_t(BH) * C * 4);         // counts
  take(size_t(BH) * n * 4);         // new labels
  take(size_t(BH) * nblk * 8);      // cost partials
  take(size_t(BH) * nblk * 4);      // change partials
  take(size_t(BH) * CTRL * 8);      // control words
  const int RP = rpad(rmax);
  take(size_t(BH) * RPMAX * 8);     // mean point
  take(size_t(BH) * n * RP * 2);    // point hi
  take(size_t(BH) * n * RP * 2);    // point lo
  take(size_t(BH) * n * 4);         // point norms
  take(size_t(BH) * C * RP * 2);    // centre hi
  take(size_t(BH) * C * RP * 2);    // centre lo
  take(size_t(BH) * C * 4);         // centre norms
  take(size_t(BH) * 4);             // queue counts
  take(size_t(BH) * n * 4);         // queue
  return o;
}

KmArgs kmeans_carve(void* ws, int BH, int n, int C, int rmax) {
  KmArgs a = {};
  char* w = static_cast<char*>(ws);
  size_t o = 0;
  auto take = [&](size_t b) {
    char* p = w + o;
    o += (b + 255) & ~size_t(255);
    return p;
  };
  const int nblk = ceil_div(n, 256);
  a.sums = reinterpret_cast<double*>(take(size_t(BH) * C * rmax * 8));
  a.cnt = reinterpret_cast<int*>(take(size_t(BH) * C * 4));
  a.lab_new = reinterpret_cast<int*>(take(size_t(BH) * n * 4));
  a.jpart = reinterpret_cast<double*>(take(size_t(BH) * nblk * 8));
  a.cpart = reinterpret_cast<int*>(take(size_t(BH) * nblk * 4));
  a.ctrl = reinterpret_cast<double*>(take(size_t(BH) * CTRL * 8));
  const int RP = rpad(rmax);
  a.mu = reinterpret_cast<double*>(take(size_t(BH) * RPMAX * 8));
  a.xh = take(size_t(BH) * n * RP * 2);
  a.xl = take(size_t(BH) * n * RP * 2);
  a.xnrm = reinterpret_cast<float*>(take(size_t(BH) * n * 4));
  a.ch = take(size_t(BH) * C * RP * 2);
  a.cl = take(size_t(BH) * C * RP * 2);
  a.cn2 = reinterpret_cast<float*>(take(size_t(BH) * C * 4));
  a.rq_count = reinterpret_cast<int*>(take(size_t(BH) * 4));
  a.rq_list = reinterpret_cast<int*>(take(size_t(BH) * n * 4));
  a.nblk = nblk;
  return a;
}

template <int R>
static void launch_pass(const KmArgs& a, hipStream_t st) {
  _Float16* xh = reinterpret_cast<_Float16*>(a.xh);
  _Float16* xl = reinterpret_cast<_Float16*>(a.xl);
  _Float16* ch = reinterpret_cast<_Float16*>(a.ch);
  _Float16* cl = reinterpret_cast<_Float16*>(a.cl);
  constexpr int KS = (R + 31) / 32, RP = rpad(R);
  const size_t sm = size_t(2) * KC * crow(RP) * sizeof(_Float16) + KC * sizeof(float);
  allow_lds(km_screen_kernel<KS, RP>, sm);
  hipLaunchKernelGGL((km_screen_kernel<KS, RP>), dim3(ceil_div(a.n, 256), a.BH), dim3(256), sm, st, a.n, a.C, xh, xl,
                     a.xnrm, ch, cl, a.cn2, a.ctrl, a.lab_new, a.rq_count, a.rq_list);
  hipLaunchKernelGGL(km_rescan_kernel<R>, dim3(16, a.BH), dim3(256), 0, st, a.n, a.C, a.feat, a.cent, a.ctrl,
                     a.rq_count, a.rq_list, a.lab_new);
  hipLaunchKernelGGL(km_accum_kernel<R>, dim3(a.nblk, a.BH), dim3(256), 0, st, a.feat, a.n, a.C, a.cent, a.lab_new,
                     a.labels, a.jpart, a.cpart, a.ctrl, a.sums, a.cnt, a.nblk);
  hipLaunchKernelGGL(km_decide_kernel, dim3(a.BH), dim3(256), 0, st, a.max_iters, a.tol, a.nblk, a.jpart, a.cpart,
                     a.ctrl);
  hipLaunchKernelGGL(km_update_kernel<RP>, dim3(ceil_div(a.C, 64), a.BH), dim3(256), 0, st, a.C, a.r, a.cent,
                     a.sums, a.cnt, a.ctrl, a.mu, ch, cl, a.cn2, a.rq_count);
}

template <int RP>
static void launch_prep(const KmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(km_point_prep_kernel<RP>, dim3(ceil_div(a.n * (RP / 8), 256), a.BH), dim3(256), 0, st, a.feat,
                     a.n, a.r, a.mu, a.ctrl, reinterpret_cast<_Float16*>(a.xh), reinterpret_cast<_Float16*>(a.xl),
                     a.xnrm);
  hipLaunchKernelGGL(km_init_kernel<RP>, dim3(a.BH), dim3(1024), 0, st, a.feat, a.n, a.r, a.C, a.seed, a.stage, a.mu,
                     a.cent, a.sums, a.cnt, a.ctrl, reinterpret_cast<_Float16*>(a.ch),
                     reinterpret_cast<_Float16*>(a.cl), a.cn2, a.rq_count, a.cent_given ? 1 : 0);
}

KmStatsTarget km_stats_target(const KmArgs& a) { return KmStatsTarget{a.mu, a.ctrl, RPMAX, CTRL, C_AMAX}; }

void kmeans_stats_zero(const KmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(km_stats_zero_kernel, dim3(ceil_div(a.BH * RPMAX, 256)), dim3(256), 0, st, a.mu, a.ctrl, a.BH);
}

spr_status run_kmeans(const KmArgs& a, hipStream_t st) {
  if (!kmeans_rank_supported(a.r)) return SPR_EUNSUPPORTED;
  if (!a.stats_given) {
    kmeans_stats_zero(a, st);
    hipLaunchKernelGGL(km_point_stats_kernel, dim3(64, a.BH), dim3(256), 0, st, a.feat, a.n, a.r, a.mu, a.ctrl);
  }
  hipLaunchKernelGGL(km_stats_final_kernel, dim3(a.BH), dim3(RPMAX), 0, st, a.mu, a.ctrl, a.n);
  if (a.r > 64) launch_prep<128>(a, st);
  else launch_prep<64>(a, st);
  SPR_CHECK_LAUNCH();
  for (int it = 0; it < a.max_iters; ++it) {
    switch (a.r) {
      case 128: launch_pass<128>(a, st); break;
      case 64: launch_pass<64>(a, st); break;
      case 48: launch_pass<48>(a, st); break;
      case 32: launch_pass<32>(a, st); break;
      case 16: launch_pass<16>(a, st); break;
      case 8: launch_pass<8>(a, st); break;
      default: return SPR_EUNSUPPORTED;
    }
    SPR_CHECK_LAUNCH();
  }
  return SPR_OK;
}

}  // namespace spr
