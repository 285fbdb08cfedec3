// k-means of the response coordinates ("Partition the Support, Reconstruct the Residual",
// Sec. 4.1 for the K/V and query partitions, App. C.1 for the initialisation, Table C.1 for
// the limits) on gfx950.
//
// One Lloyd pass:
//  screen   squared distances of every point to every centre from an MFMA cross term.
//           Coordinates are centred by the head's mean point and scaled by a power of two,
//           then split into fp16 hi + lo parts; x.c ~ hi.hi + hi.lo + lo.hi on
//           v_mfma_f32_32x32x16_f16.  A bound on the error of the screened distances decides,
//           per point, whether the nearest centre is certain; the rest go to a queue.
//  rescan   queued points: fp64 direct-difference distances to every centre (exact nearest,
//           ties to the lowest index).
//  sort     label histograms of 4096-point slices, a scan per head, a stable scatter: the
//           points of every new label in ascending index, and the count of changed labels.
//  reduce   one wave per centre: the Lloyd sums of its members (no atomics, a fixed order) and
//           their fp64 distances to the old centre (cost).
//  decide / update   stopping rule (labels unchanged, relative cost decrease <= tol, or
//           max_iters), centre update (empty centres stay), the fp16 split of the new centres.
// The final labels are compacted on the same sort (empty groups dropped, offsets, permutation).
// The control word per head (done flag, pass count, previous cost, largest centre norm, scale)
// lives on the device, so the host launches max_iters passes without synchronising and
// finished heads return immediately.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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
    // the mean point's eight coordinates (cb * 8 + 7 < RP <= RPMAX), loaded together
    double mv[8];
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const double2 m2 = *reinterpret_cast<const double2*>(mu + size_t(hd) * RPMAX + cb * 8 + u);
      mv[u] = m2.x;
      mv[u + 1] = m2.y;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double x = live ? (xr[u] - mv[u]) * sc : 0.0;
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

// Screening pass.  A wave owns 64 points (2 tiles of 32); centres stream through LDS in chunks
// of 256.  v_mfma_f32_32x32x16_f16 computes D^T tiles (32 centres x 32 points) as three split
// products (hi hi, hi lo, lo hi): lane l holds 16 centres (rows 8 q + 4 (l / 32) + i, q, i < 4) of
// point l % 32 and keeps that point's best value, its index and the second best; lanes l and
// l ^ 32 hold the other 16 centres of the same point and are merged at the end.
template <int KS, int RP>
__global__ __launch_bounds__(256) void km_screen_kernel(int n, int C, const _Float16* __restrict__ xh,
                                                        const _Float16* __restrict__ xl,
                                                        const float* __restrict__ xnrm,
                                                        const _Float16* __restrict__ ch,
                                                        const _Float16* __restrict__ cl,
                                                        const float* __restrict__ cn2,
                                                        const double* __restrict__ ctrl, int* __restrict__ lab_new,
                                                        int* __restrict__ rq_count, int* __restrict__ rq_list) {
  constexpr int CROW = crow(RP), K16 = RP / 16;  // LDS row stride, 16-column steps
  extern __shared__ __attribute__((aligned(16))) char smem[];
  _Float16* Ch = reinterpret_cast<_Float16*>(smem);
  _Float16* Cl = Ch + KC * CROW;
  float* cns = reinterpret_cast<float*>(Cl + KC * CROW);
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int p0 = blockIdx.x * 256 + w * 64;
  // B fragments: point p0 + 32 pt + l32, columns 16 ks + 8 h .. + 7 of the hi and lo slices
  f16x8_t bh[2][K16], bl[2][K16];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    const int j = p0 + pt * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < K16; ++ks) {
      uint4 uh = make_uint4(0, 0, 0, 0), ul = make_uint4(0, 0, 0, 0);
      if (j < n) {
        uh = *reinterpret_cast<const uint4*>(xh + (size_t(hd) * n + j) * RP + ks * 16 + 8 * h);
        ul = *reinterpret_cast<const uint4*>(xl + (size_t(hd) * n + j) * RP + ks * 16 + 8 * h);
      }
      bh[pt][ks] = as_f16x8(uh);
      bl[pt][ks] = as_f16x8(ul);
    }
  }
  // running best, its index and the second best per point tile; the index is kept as the
  // 32-centre block that last lowered the best (ib) and the register slot within it (iv)
  float b1[2], b2[2];
  int ib[2], iv[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    b1[pt] = INFINITY;
    b2[pt] = INFINITY;
    ib[pt] = iv[pt] = 0;
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
    const int nblk = (cc + 31) >> 5;
    for (int cb = 0; cb < nblk; ++cb) {
      // A fragments: centre c0 + 32 cb + l32, columns 16 ks + 8 h .. + 7
      f16x8_t ah[K16], al[K16];
#pragma unroll
      for (int ks = 0; ks < K16; ++ks) {
        ah[ks] = as_f16x8(*reinterpret_cast<const uint4*>(Ch + (cb * 32 + l32) * CROW + ks * 16 + 8 * h));
        al[ks] = as_f16x8(*reinterpret_cast<const uint4*>(Cl + (cb * 32 + l32) * CROW + ks * 16 + 8 * h));
      }
      float cv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 c4 = *reinterpret_cast<const float4*>(cns + cb * 32 + 8 * q + 4 * h);
        cv[4 * q] = c4.x; cv[4 * q + 1] = c4.y; cv[4 * q + 2] = c4.z; cv[4 * q + 3] = c4.w;
      }
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        f32x16_t acc = {};
#pragma unroll
        for (int ks = 0; ks < K16; ++ks) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[ks], bh[pt][ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[ks], bl[pt][ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[ks], bh[pt][ks], acc, 0, 0, 0);
        }
        // branch-free running best / slot / second best (centres in ascending index); with
        // b1 <= b2 the new second best is the median of b1, b2 and the value.  The slot v is an
        // inline constant of the select; the block is recorded once, when it lowered the best.
        const float b1_in = b1[pt];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float val = fmaf(-2.f, acc[v], cv[v]);
          b2[pt] = __builtin_amdgcn_fmed3f(b1[pt], b2[pt], val);
          iv[pt] = val < b1[pt] ? v : iv[pt];
          b1[pt] = fminf(b1[pt], val);
        }
        ib[pt] = b1[pt] < b1_in ? (c0 >> 5) + cb : ib[pt];
      }
    }
  }
  const double cmax = ctrl[hd * CTRL + C_CMAX];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    // centre of slot v of block ib: 32 ib + 8 (v / 4) + 4 h + v % 4
    int i1 = 32 * ib[pt] + 8 * (iv[pt] >> 2) + (iv[pt] & 3) + 4 * h;
    // merge the two lanes of a point (their centre subsets are disjoint)
    {
      const float ob1 = __shfl_xor(b1[pt], 32), ob2 = __shfl_xor(b2[pt], 32);
      const int oi = __shfl_xor(i1, 32);
      if (ob1 < b1[pt] || (ob1 == b1[pt] && oi < i1)) {
        b2[pt] = fminf(ob2, b1[pt]);
        b1[pt] = ob1;
        i1 = oi;
      } else {
        b2[pt] = fminf(b2[pt], ob1);
      }
    }
    const int j = p0 + pt * 32 + l32;
    bool queue = false;
    if (h == 0 && j < n) {
      // bound on |screened - exact| squared distance (scaled units): cross-term error of
      // the split product with fp32 sums, plus fp32 rounding of norms and combination;
      // doubled for safety.  Decided when the runner-up is more than twice that away.
      const double xn = xnrm[size_t(hd) * n + j];
      const double tcross = (3.0 * RP * 5.960464477539063e-8 + 3.0 * 2.384185791015625e-7) * xn * cmax;
      const double E = 2.0 * (2.0 * tcross + 4.0 * 5.960464477539063e-8 * (xn + cmax) * (xn + cmax)) +
                       1e-12 * (xn + cmax) * (xn + cmax);
      const bool decided = double(b2[pt]) - double(b1[pt]) > 2.0 * E;
      lab_new[size_t(hd) * n + j] = decided ? i1 : -1;
      queue = !decided;
    }
    // the undecided points of the wave join the rescan queue with one atomic
    const unsigned long long qm = __ballot(queue);
    if (qm) {
      int base = 0;
      if (lane == __ffsll((long long)qm) - 1) base = atomicAdd(rq_count + hd, __popcll(qm));
      base = __shfl(base, __ffsll((long long)qm) - 1);
      if (queue) rq_list[size_t(hd) * n + base + __popcll(qm & ((1ull << lane) - 1))] = j;
    }
  }
}

// fp64 nearest centre of every queued point (ties to the lowest index).  A block takes eight
// queued points at a time, staged in LDS; thread t walks centres t, t + 256, ..., reads each
// centre row once for the eight points and keeps eight direct-difference distances, summed
// over the coordinates in ascending order; the four waves' nearest centres are then merged.
template <int R>
__global__ __launch_bounds__(256) void km_rescan_kernel(int n, int C, const double* __restrict__ feat,
                                                        const double* __restrict__ cent,
                                                        const double* __restrict__ ctrl,
                                                        const int* __restrict__ rq_count,
                                                        const int* __restrict__ rq_list, int* __restrict__ lab_new) {
  constexpr int PP = 8;
  static_assert(R % 2 == 0, "pairs of coordinates");
  __shared__ __attribute__((aligned(16))) double xs[PP][R];
  __shared__ double rb[4][PP];
  __shared__ int ri[4][PP], jl[PP];
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int cnt = rq_count[hd];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i0 = blockIdx.x * PP; i0 < cnt; i0 += gridDim.x * PP) {
    const int np = min(PP, cnt - i0);
    __syncthreads();  // the previous points' rows and results are no longer read
    if (t < PP) jl[t] = t < np ? rq_list[size_t(hd) * n + i0 + t] : 0;
    __syncthreads();
    for (int e = t; e < PP * R; e += 256) {
      const int p = e / R;
      xs[p][e % R] = p < np ? feat[(size_t(hd) * n + jl[p]) * R + e % R] : 0.0;
    }
    __syncthreads();
    double best[PP];
    int bi[PP];
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      best[p] = INFINITY;
      bi[p] = 0;
    }
    for (int m = t; m < C; m += 256) {
      const double* c = cent + (size_t(hd) * C + m) * R;
      double dd[PP];
#pragma unroll
      for (int p = 0; p < PP; ++p) dd[p] = 0.0;
      for (int e = 0; e < R; e += 2) {
        const double2 ce = *reinterpret_cast<const double2*>(c + e);
#pragma unroll
        for (int p = 0; p < PP; ++p) {
          const double2 xv = *reinterpret_cast<const double2*>(&xs[p][e]);
          const double t0 = xv.x - ce.x;
          dd[p] = fma(t0, t0, dd[p]);
          const double t1 = xv.y - ce.y;
          dd[p] = fma(t1, t1, dd[p]);
        }
      }
#pragma unroll
      for (int p = 0; p < PP; ++p)
        if (dd[p] < best[p]) {
          best[p] = dd[p];
          bi[p] = m;
        }
    }
    auto better = [](double ob, int oi, double b, int i) { return ob < b || (ob == b && oi < i); };
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      for (int o = 32; o > 0; o >>= 1) {
        const double ob = __shfl_xor(best[p], o);
        const int oi = __shfl_xor(bi[p], o);
        if (better(ob, oi, best[p], bi[p])) {
          best[p] = ob;
          bi[p] = oi;
        }
      }
      if (lane == 0) {
        rb[w][p] = best[p];
        ri[w][p] = bi[p];
      }
    }
    __syncthreads();
    if (t < np) {
      double b = rb[0][t];
      int i = ri[0][t];
      for (int q = 1; q < 4; ++q)
        if (better(rb[q][t], ri[q][t], b, i)) {
          b = rb[q][t];
          i = ri[q][t];
        }
      lab_new[size_t(hd) * n + jl[t]] = i;
    }
  }
}

// Cost, label changes and Lloyd sums of the pass, without atomics on the sums: the points are
// counting-sorted by their new label (a histogram per slice of kSlicePts points, a scan per
// head, a stable scatter), then one wave per centre adds its members' coordinates, one lane per
// coordinate, in ascending point index, and their (x - c)^2 to the pass cost.  Every sum is
// thus formed in the same order on every run.
constexpr int kSlicePts = 4096;  // points per histogram / scatter block (1024 threads)

// Label histogram of one slice, its count of changed labels, and the labels of the pass (the
// compaction of the final labels passes no labels, ctrl or cpart).
__global__ __launch_bounds__(1024) void km_hist_kernel(int n, int C, const int* __restrict__ lab_new,
                                                       int* __restrict__ labels, const double* __restrict__ ctrl,
                                                       int* __restrict__ hist, int* __restrict__ cpart, int nsl) {
  __shared__ int h[1024];  // C <= 1024
  __shared__ int64_t redi[32];
  const int hd = blockIdx.y;
  if (ctrl && ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int t = threadIdx.x;
  if (t < C) h[t] = 0;
  __syncthreads();
  int changed = 0;
  const int j0 = blockIdx.x * kSlicePts;
  for (int i = t; i < kSlicePts; i += 1024) {
    const int j = j0 + i;
    if (j < n) {
      const int lab = lab_new[size_t(hd) * n + j];
      if (labels) {
        int* lp = labels + size_t(hd) * n + j;
        changed += *lp != lab;
        *lp = lab;
      }
      atomicAdd(&h[lab], 1);
    }
  }
  const int64_t cs = block_sum_i64(changed, redi);  // (its barriers also complete the histogram)
  if (t < C) hist[(size_t(hd) * nsl + blockIdx.x) * C + t] = h[t];
  if (t == 0 && cpart) cpart[size_t(hd) * nsl + blockIdx.x] = int(cs);
}

// Per head and centre: the member count, the first position of its members in the sorted order
// (centres ascending), and in place of each slice's count the position of that slice's first
// member.  One thread per centre.
__global__ __launch_bounds__(1024) void km_scan_kernel(int C, int nsl, const double* __restrict__ ctrl,
                                                       int* __restrict__ hist, int* __restrict__ cnt,
                                                       int* __restrict__ cstart) {
  __shared__ int scan[32];
  const int hd = blockIdx.x;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int c = threadIdx.x;
  int* hc = hist + size_t(hd) * nsl * C + c;
  int tot = 0;
  if (c < C)
    for (int b = 0; b < nsl; ++b) tot += hc[size_t(b) * C];
  int all;
  const int s0 = block_exscan_i(c < C ? tot : 0, scan, &all);
  if (c < C) {
    int run = s0;
    for (int b = 0; b < nsl; ++b) {
      const int v = hc[size_t(b) * C];
      hc[size_t(b) * C] = run;
      run += v;
    }
    cnt[size_t(hd) * C + c] = tot;
    cstart[size_t(hd) * C + c] = s0;
  }
}

// Compaction of the final labels: empty centres dropped and the others renumbered in ascending
// id (remap), group offsets, the group count and the empty-group status bit; in place of each
// slice's counts the position of the slice's first member of every group.
__global__ __launch_bounds__(1024) void km_compact_scan_kernel(int n, int C, int nsl, int* __restrict__ hist,
                                                               int* __restrict__ remap, int* __restrict__ off,
                                                               int* __restrict__ ngroups, int* __restrict__ gstat,
                                                               int empty_bit) {
  __shared__ int scan[32];
  const int hd = blockIdx.x, c = threadIdx.x;
  int* hc = hist + size_t(hd) * nsl * C + c;
  int tot = 0;
  if (c < C)
    for (int b = 0; b < nsl; ++b) tot += hc[size_t(b) * C];
  int ng, all;
  const int newid = block_exscan_i(c < C && tot > 0 ? 1 : 0, scan, &ng);
  const int s0 = block_exscan_i(c < C ? tot : 0, scan, &all);
  if (c < C) {
    int run = s0;
    for (int b = 0; b < nsl; ++b) {
      const int v = hc[size_t(b) * C];
      hc[size_t(b) * C] = run;
      run += v;
    }
    remap[size_t(hd) * C + c] = newid;
    if (tot > 0) off[size_t(hd) * (C + 1) + newid] = s0;
  }
  if (c == 0) {
    off[size_t(hd) * (C + 1) + ng] = n;
    ngroups[hd] = ng;
    if (ng < C) atomicOr(gstat + hd * 8 + 0, empty_bit);
  }
}

// Stable scatter of one slice: order[position] = point, members of a centre in ascending point
// index (for the compaction also the position of every point and its renumbered label).  Ranks
// inside a wave come from ballots, ranks across the 16 waves of a 1024-point chunk from
// per-wave counts in LDS.
__global__ __launch_bounds__(1024) void km_scatter_kernel(int n, int C, const int* __restrict__ lab_new,
                                                          const double* __restrict__ ctrl,
                                                          const int* __restrict__ hist, int nsl,
                                                          int* __restrict__ order, int* __restrict__ pos_of,
                                                          int* __restrict__ lab_c, const int* __restrict__ remap) {
  extern __shared__ int sc_sm[];
  int* cursor = sc_sm;      // [C]
  int* wcnt = sc_sm + C;    // [16][C]
  const int hd = blockIdx.y;
  if (ctrl && ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t < C) cursor[t] = hist[(size_t(hd) * nsl + blockIdx.x) * C + t];
  for (int e = t; e < 16 * C; e += 1024) wcnt[e] = 0;
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int j0 = blockIdx.x * kSlicePts;
  for (int c0 = 0; c0 < kSlicePts && j0 + c0 < n; c0 += 1024) {
    const int j = j0 + c0 + t;
    const bool valid = j < n;
    const int L = valid ? lab_new[size_t(hd) * n + j] : -1;
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
      order[size_t(hd) * n + pos] = j;
      if (pos_of) pos_of[size_t(hd) * n + j] = pos;
      if (lab_c) lab_c[size_t(hd) * n + j] = remap[size_t(hd) * C + L];
    }
    __syncthreads();
  }
}

// Sums and cost per centre, one wave per centre: members in sorted order, their loads issued
// PB at a time ahead of the additions.
template <int R>
__global__ __launch_bounds__(256) void km_reduce_kernel(const double* __restrict__ feat, int n, int C,
                                                        const double* __restrict__ cent,
                                                        const int* __restrict__ order, const int* __restrict__ cnt,
                                                        const int* __restrict__ cstart,
                                                        const double* __restrict__ ctrl, double* __restrict__ sums,
                                                        double* __restrict__ jpart) {
  constexpr int EPL = (R + 63) / 64, PB = 16;
  const int hd = blockIdx.y;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  const int c = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6)), lane = threadIdx.x & 63;
  if (c >= C) return;
  const int k = cnt[size_t(hd) * C + c];
  const int* od = order + size_t(hd) * n + cstart[size_t(hd) * C + c];
  const double* fh = feat + size_t(hd) * n * R;
  double acc[EPL], cc[EPL], jl = 0.0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + 64 * q;
    acc[q] = 0.0;
    cc[q] = e < R ? cent[(size_t(hd) * C + c) * R + e] : 0.0;
  }
  for (int i0 = 0; i0 < k; i0 += PB) {
    double xb[PB][EPL];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int jj = i0 + i < k ? od[i0 + i] : 0;
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const int e = lane + 64 * q;
        xb[i][q] = (e < R && i0 + i < k) ? fh[size_t(jj) * R + e] : 0.0;
      }
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      if (i0 + i >= k) break;
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const int e = lane + 64 * q;
        if (e < R) {
          acc[q] += xb[i][q];
          const double d = xb[i][q] - cc[q];
          jl = fma(d, d, jl);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + 64 * q;
    if (e < R) sums[(size_t(hd) * C + c) * R + e] = acc[q];
  }
  jl = wave_sum_d(jl);
  if (lane == 0) jpart[size_t(hd) * C + c] = jl;
}

// Stopping rule after a pass (one block per head): stop when the labels did not change, when
// the cost fell by at most tol relative to the previous pass, or at max_iters.  The decision is
// written to ctrl[C_STOPNOW]; km_update_kernel then moves the centres of heads that go on.
__global__ __launch_bounds__(256) void km_decide_kernel(int max_iters, double tol, int C,
                                                        const double* __restrict__ jpart, int nsl,
                                                        const int* __restrict__ cpart, double* __restrict__ ctrl) {
  __shared__ double red[32];
  __shared__ int64_t redi[32];
  const int hd = blockIdx.x;
  if (ctrl[hd * CTRL + C_DONE] != 0.0) return;
  double js = 0.0;
  int64_t cs = 0;
  for (int i = threadIdx.x; i < C; i += blockDim.x) js += jpart[size_t(hd) * C + i];
  for (int i = threadIdx.x; i < nsl; i += blockDim.x) cs += cpart[size_t(hd) * nsl + i];
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

// Centre update (members' mean; empty centres stay) and the fp16 split of the new centres for
// the next screening pass.  64 centres per block, one wave per centre row
// at a time; the largest centre norm is combined with atomicMax on its (non-negative) bits.
template <int RP>
__global__ __launch_bounds__(256) void km_update_kernel(int C, int r, double* __restrict__ cent,
                                                        const double* __restrict__ sums, const int* __restrict__ cnt,
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
  const int nsl = ceil_div(n, kSlicePts);
  take(size_t(BH) * C * rmax * 8);  // sums
  take(size_t(BH) * C * 4);         // counts
  take(size_t(BH) * n * 4);         // new labels
  take(size_t(BH) * C * 8);         // cost partials (per centre)
  take(size_t(BH) * nsl * 4);       // change partials (per slice)
  take(size_t(BH) * nsl * C * 4);   // slice histograms, then slice positions
  take(size_t(BH) * C * 4);         // first sorted position per centre
  take(size_t(BH) * n * 4);         // points sorted by label
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
  const int nsl = ceil_div(n, kSlicePts);
  a.sums = reinterpret_cast<double*>(take(size_t(BH) * C * rmax * 8));
  a.cnt = reinterpret_cast<int*>(take(size_t(BH) * C * 4));
  a.lab_new = reinterpret_cast<int*>(take(size_t(BH) * n * 4));
  a.jpart = reinterpret_cast<double*>(take(size_t(BH) * C * 8));
  a.cpart = reinterpret_cast<int*>(take(size_t(BH) * nsl * 4));
  a.hist = reinterpret_cast<int*>(take(size_t(BH) * nsl * C * 4));
  a.cstart = reinterpret_cast<int*>(take(size_t(BH) * C * 4));
  a.order = reinterpret_cast<int*>(take(size_t(BH) * n * 4));
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
  a.nsl = nsl;
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
  hipLaunchKernelGGL(km_rescan_kernel<R>, dim3(64, a.BH), dim3(256), 0, st, a.n, a.C, a.feat, a.cent, a.ctrl,
                     a.rq_count, a.rq_list, a.lab_new);
  hipLaunchKernelGGL(km_hist_kernel, dim3(a.nsl, a.BH), dim3(1024), 0, st, a.n, a.C, a.lab_new, a.labels, a.ctrl,
                     a.hist, a.cpart, a.nsl);
  hipLaunchKernelGGL(km_scan_kernel, dim3(a.BH), dim3(1024), 0, st, a.C, a.nsl, a.ctrl, a.hist, a.cnt, a.cstart);
  const size_t ssm = size_t(17) * a.C * sizeof(int);
  allow_lds(km_scatter_kernel, ssm);
  hipLaunchKernelGGL(km_scatter_kernel, dim3(a.nsl, a.BH), dim3(1024), ssm, st, a.n, a.C, a.lab_new, a.ctrl, a.hist,
                     a.nsl, a.order, nullptr, nullptr, nullptr);
  hipLaunchKernelGGL(km_reduce_kernel<R>, dim3(ceil_div(a.C, 4), a.BH), dim3(256), 0, st, a.feat, a.n, a.C, a.cent,
                     a.order, a.cnt, a.cstart, a.ctrl, a.sums, a.jpart);
  hipLaunchKernelGGL(km_decide_kernel, dim3(a.BH), dim3(256), 0, st, a.max_iters, a.tol, a.C, a.jpart, a.nsl,
                     a.cpart, a.ctrl);
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

spr_status launch_compact(const KmArgs& a, int* lab_c, int* perm, int* pos_of, int* off, int* ngroups, int* gstat,
                          int empty_bit, hipStream_t st) {
  // the pass scratch is free once the passes are done: slice histograms in hist, remap in cstart
  hipLaunchKernelGGL(km_hist_kernel, dim3(a.nsl, a.BH), dim3(1024), 0, st, a.n, a.C, a.labels, nullptr, nullptr,
                     a.hist, nullptr, a.nsl);
  hipLaunchKernelGGL(km_compact_scan_kernel, dim3(a.BH), dim3(1024), 0, st, a.n, a.C, a.nsl, a.hist, a.cstart, off,
                     ngroups, gstat, empty_bit);
  const size_t ssm = size_t(17) * a.C * sizeof(int);
  allow_lds(km_scatter_kernel, ssm);
  hipLaunchKernelGGL(km_scatter_kernel, dim3(a.nsl, a.BH), dim3(1024), ssm, st, a.n, a.C, a.labels, nullptr, a.hist,
                     a.nsl, perm, pos_of, lab_c, a.cstart);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
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
