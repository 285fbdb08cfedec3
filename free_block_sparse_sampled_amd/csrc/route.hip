// Routing and probe selection ("Partition the Support, Reconstruct the Residual",
// Sec. 4.3, App. B.3, App. A.2) on gfx950.
//
// The value-error score of App. B.3 expands, per (query group a, K/V group b), to
//   |G_b| s_ab = A^2 |G_b| |vbar_b|^2 - 2 A sum_j E_j (v_j . vbar_b) + sum_j E_j^2 |v_j|^2
// with A = e^{qbar_a kbar_b / sqrt d - m_a} and E_j = e^{qbar_a k_j / sqrt d - m_a}, so one
// pass over all (a, key) logits with segmented sums per (a, b) gives every score.  The shift m_a
// (the largest centroid logit of row a) multiplies a whole row by one positive factor and leaves
// the ranking unchanged.
//
// fp32 keys: that pass in fp64 (route_score_kernel), then the ranked prefix (route_select_kernel).
// bf16 keys: the pass on the bf16 matrix cores with a rigorous bound per score
// (route_score_fast_kernel), then route_resolve_kernel, which recomputes in fp64 exactly the
// scores the prefix and its order depend on; the outcome is that of the fp64 scores.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

// DPP lane moves and sums of doubles (all lanes of the rows involved active)
template <int CTRL>
__device__ __forceinline__ double dppd(double x) {
  const unsigned long long u = __double_as_longlong(x);
  const unsigned lo = __builtin_amdgcn_update_dpp(0, unsigned(u), CTRL, 0xF, 0xF, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0, unsigned(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((unsigned long long)lo | ((unsigned long long)hi << 32));
}
__device__ __forceinline__ double readlane_dbl(double x, int l) {
  const unsigned long long u = __double_as_longlong(x);
  const unsigned lo = __builtin_amdgcn_readlane(unsigned(u), l), hi = __builtin_amdgcn_readlane(unsigned(u >> 32), l);
  return __longlong_as_double((unsigned long long)lo | ((unsigned long long)hi << 32));
}
// sum over the 64 lanes (all active): DPP sums over each 16-lane row, then the four rows
__device__ __forceinline__ double wave_allsum_d(double x) {
  x += dppd<0xB1>(x);
  x += dppd<0x4E>(x);
  x += dppd<0x141>(x);
  x += dppd<0x140>(x);
  return (readlane_dbl(x, 0) + readlane_dbl(x, 16)) + (readlane_dbl(x, 32) + readlane_dbl(x, 48));
}

// Per key (group-major order), fp64: u_j = v_j . vbar_b(j), w_j = |v_j|^2, c_j = (vbar_b - v_j) . v_j
// and r_j = |vbar_b - v_j|^2.  d / 8 lanes per key, eight consecutive elements each (one 16-byte
// load for bf16), reduced across those lanes.
template <int DT>
__global__ __launch_bounds__(256) void vstat_kernel(const void* __restrict__ Vp, int N, int Nv, int d,
                                                    const int* __restrict__ kv_perm,
                                                    const int* __restrict__ kv_label,
                                                    const double* __restrict__ vbar, int Ck,
                                                    double* __restrict__ vstat) {
  const int hd = blockIdx.y;
  const int L = d >> 3;
  const int pos = blockIdx.x * (256 / L) + threadIdx.x / L, sub = threadIdx.x % L;
  double u = 0.0, w = 0.0, cr = 0.0, r = 0.0;
  if (pos < Nv) {
    const int b = kv_label[size_t(hd) * Nv + kv_perm[size_t(hd) * Nv + pos]];
    const double* vb = vbar + (size_t(hd) * Ck + b) * d + sub * 8;
    float x[8];
    load8<DT>(Vp, (int64_t(hd) * N + pos) * d + sub * 8, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const double xv = double(x[c]), dv = vb[c] - xv;
      u = fma(xv, vb[c], u);
      w = fma(xv, xv, w);
      cr = fma(dv, xv, cr);
      r = fma(dv, dv, r);
    }
  }
  // sums over the L = d / 8 lanes of a key (8 or 16 adjacent lanes: quad_perm [1,0,3,2],
  // [2,3,0,1], row_half_mirror, and row_mirror for 16)
  auto lsum = [L](double x) {
    x += dppd<0xB1>(x);
    x += dppd<0x4E>(x);
    x += dppd<0x141>(x);
    if (L == 16) x += dppd<0x140>(x);
    return x;
  };
  u = lsum(u);
  w = lsum(w);
  cr = lsum(cr);
  r = lsum(r);
  if (pos < Nv && sub == 0) {
    double* o = vstat + (size_t(hd) * Nv + pos) * 4;
    *reinterpret_cast<double2*>(o) = make_double2(u, w);
    *reinterpret_cast<double2*>(o + 2) = make_double2(cr, r);
  }
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// Centroid logits lbar_ab = qbar_a . kbar_b / sqrt d on the fp64 matrix cores.  One block per
// 64 query groups x 64 K/V groups of a head: the block's 64 key centroids are staged in LDS once
// (rows padded to D + 4 doubles) for its four waves; wave w owns query groups a0 + 16 w .. + 15
// (A fragments of qbar in registers: lane l holds qbar[a0 + 16 w + l % 16] at columns 4 ks + l / 16)
// and the block's four tiles of 16 K/V groups, each its own accumulation chain; lane l, slot v
// of tile t holds the logit of query group 16 w + l / 16 + 4 v and K/V group b0 + 16 t + l % 16.
template <int D>
constexpr size_t centroid_logits_smem() {
  return size_t(64) * (D + 4) * sizeof(double);
}
template <int D>
__global__ __launch_bounds__(256) void centroid_logits_kernel(const double* __restrict__ qbar,
                                                              const double* __restrict__ kbar,
                                                              const int* __restrict__ n_q,
                                                              const int* __restrict__ n_kv, int Cq, int Ck, int G,
                                                              double* __restrict__ lbar) {
  constexpr int KST = D + 4;  // LDS row stride (doubles)
  extern __shared__ __attribute__((aligned(16))) double kbs[];  // [64][KST]
  const int hd = blockIdx.z, hk = hd / G, a0 = blockIdx.x * 64, b0 = blockIdx.y * 64;  // query head, K/V head
  const int nq = n_q[hd], nkv = n_kv[hk];
  if (a0 >= nq || b0 >= nkv) return;
  // rows past the last K/V group repeat it (their logits are not stored)
  for (int e = threadIdx.x; e < 64 * D / 2; e += 256) {
    const int row = e / (D / 2), c2 = e % (D / 2);
    const double2 v2 =
        *reinterpret_cast<const double2*>(kbar + (size_t(hk) * Ck + min(b0 + row, nkv - 1)) * D + 2 * c2);
    *reinterpret_cast<double2*>(kbs + row * KST + 2 * c2) = v2;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r16 = lane & 15;
  const int aw = a0 + w * 16;
  if (aw >= nq) return;
  double qa[D / 4];
  {
    const int a = aw + r16;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) qa[ks] = a < nq ? qbar[(size_t(hd) * Cq + a) * D + ks * 4 + gq] : 0.0;
  }
  const double inv = 1.0 / sqrt(double(D));
  const double* kb = kbs + r16 * KST + gq;
  f64x4_t lg[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) lg[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      lg[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], kb[16 * t * KST + ks * 4], lg[t], 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int b = b0 + 16 * t + r16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int a = aw + gq + 4 * v;
      if (b < nkv && a < nq) lbar[(size_t(hd) * Cq + a) * Ck + b] = lg[t][v] * inv;
    }
  }
}

// The shift m_a = max_b lbar_ab of every query group, one wave per group.
__global__ __launch_bounds__(256) void logit_shift_kernel(const double* __restrict__ lbar,
                                                          const int* __restrict__ n_q,
                                                          const int* __restrict__ n_kv, int Cq, int Ck, int G,
                                                          double* __restrict__ shift) {
  const int hd = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= n_q[hd]) return;
  const int nkv = n_kv[hd / G];
  const double* row = lbar + (size_t(hd) * Cq + a) * Ck;
  double mx = -1.0e308;
  for (int b = lane; b < nkv; b += 64) mx = fmax(mx, row[b]);
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  if (lane == 0) shift[size_t(hd) * Cq + a] = mx;
}

// e^x in fp64 by Tang's table method: x = (64 n + j) ln2 / 64 + r with |r| <= ln2 / 128,
// e^x = 2^n 2^(j/64) e^r, e^r - 1 by its Taylor polynomial to degree 6 (truncation below 1e-19
// relative); ln2 / 64 in two parts (the split of ln2 whose high part has 32 trailing zero bits)
// so that n ln2_hi is exact.  T[j] = 2^(j/64).  About one ulp; arguments below -745 give 0.
__device__ __forceinline__ double exp_table(double x, const double* T) {
  constexpr double kInvL = 92.332482616893656877;        // 64 / ln2
  constexpr double kLhi = 6.93147180369123816490e-01 / 64;  // high part of ln2, / 64 (exact)
  constexpr double kLlo = 1.90821492927058770002e-10 / 64;  // ln2 - high part, / 64
  x = fmax(x, -746.0);
  const double n = __builtin_rint(x * kInvL);
  const int ni = int(n);
  double r = fma(-n, kLhi, x);
  r = fma(-n, kLlo, r);
  double p = fma(r, 1.0 / 720, 1.0 / 120);
  p = fma(p, r, 1.0 / 24);
  p = fma(p, r, 1.0 / 6);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p *= r;  // e^r - 1
  const double t = T[ni & 63];
  return ldexp(fma(t, p, t), ni >> 6);
}

// Scores of 64 query groups x 16 K/V groups.  The K/V groups are taken one at a time; their
// keys (contiguous in group-major order) are staged in LDS as fp64 in pieces of 64 and
// processed in 16-key tiles: logits on the fp64 matrix cores (same fragment layout as the
// centroid logits), then E = e^{logit - m_a} and the per-lane sums of E u and E^2 w in
// registers.  A key row is stored with column c at (c % 4) D / 4 + c / 4, so the D / 4 values a
// lane feeds to the products (columns 4 ks + l / 16) are contiguous and load before them.  Keys
// past a group's end are zero with u = w = 0 and add nothing.  At the end of a group the sums
// are reduced over the 16 lanes of each query group and the score is written.
constexpr int kScorePiece = 64;
template <int D>
constexpr size_t route_score_smem() {
  return (size_t(kScorePiece) * (D + 2) + 2 * kScorePiece + 64 + 16) * sizeof(double);
}
template <int DT, int D>
__global__ __launch_bounds__(256) void route_score_kernel(const void* __restrict__ Kp, int N, int Nv,
                                                          const double* __restrict__ qbar,
                                                          const double* __restrict__ lbar,
                                                          const double* __restrict__ vbar,
                                                          const int* __restrict__ kv_off,
                                                          const int* __restrict__ n_q,
                                                          const int* __restrict__ n_kv, int Cq, int Ck, int G,
                                                          const double* __restrict__ shift,
                                                          const double* __restrict__ vstat,
                                                          double* __restrict__ scores) {
  constexpr int PIECE = kScorePiece;
  constexpr int KSD = D + 2;  // key row stride in LDS (doubles)
  extern __shared__ double rs_sm[];
  double* Ks = rs_sm;                 // [PIECE][KSD]
  double* us = Ks + PIECE * KSD;      // [PIECE]
  double* wsv = us + PIECE;           // [PIECE]
  double* T = wsv + PIECE;            // [64] 2^(j/64)
  double* vns = T + 64;               // [16]
  const int hd = blockIdx.z, hk = hd / G;  // query head, its K/V head
  const int a0 = blockIdx.x * 64, b0 = blockIdx.y * 16;
  const int nq = n_q[hd], nkv = n_kv[hk];
  if (a0 >= nq || b0 >= nkv) return;
  const int b1 = min(b0 + 16, nkv);
  const int* off = kv_off + size_t(hk) * (Ck + 1);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r16 = lane & 15;
  if (threadIdx.x < 64) T[threadIdx.x] = exp2(double(threadIdx.x) / 64.0);
  double qa[D / 4];
  {
    const int a = a0 + w * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) qa[ks] = a < nq ? qbar[(size_t(hd) * Cq + a) * D + ks * 4 + gq] : 0.0;
  }
  double m_a[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int a = a0 + w * 16 + gq + 4 * v;
    m_a[v] = a < nq ? shift[size_t(hd) * Cq + a] : 0.0;
  }
  // |vbar_b|^2 of the block's groups: wave w takes groups b0 + 4 w .. + 3
  for (int k = 0; k < 4; ++k) {
    const int b = b0 + w * 4 + k;
    double x = 0.0;
    if (b < b1)
      for (int c = lane; c < D; c += 64) {
        const double y = vbar[(size_t(hk) * Ck + b) * D + c];
        x = fma(y, y, x);
      }
    x = wave_sum_d(x);
    if (lane == 0) vns[w * 4 + k] = x;
  }
  const double inv = 1.0 / sqrt(double(D));
  for (int b = b0; b < b1; ++b) {
    const int k0 = off[b], k1 = off[b + 1];
    double s1[4] = {0.0, 0.0, 0.0, 0.0}, s2[4] = {0.0, 0.0, 0.0, 0.0};
    for (int p0 = k0; p0 < k1; p0 += PIECE) {
      const int n = min(PIECE, k1 - p0);
      __syncthreads();
      for (int e = threadIdx.x; e < PIECE * (D / 8); e += 256) {
        const int jl = e / (D / 8), c8 = (e % (D / 8)) * 8;
        float x[8];
        if (jl < n) {
          load8<DT>(Kp, (int64_t(hk) * N + p0 + jl) * D + c8, x);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = 0.f;
        }
        // columns c8 .. c8 + 7 go to (c % 4) D / 4 + c / 4: two runs of 2 per residue class
        double* dst = Ks + jl * KSD + c8 / 4;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          *reinterpret_cast<double2*>(dst + m * (D / 4)) = make_double2(x[m], x[m + 4]);
      }
      if (threadIdx.x < PIECE) {
        const int jl = threadIdx.x;
        us[jl] = jl < n ? vstat[(size_t(hk) * Nv + p0 + jl) * 4 + 0] : 0.0;
        wsv[jl] = jl < n ? vstat[(size_t(hk) * Nv + p0 + jl) * 4 + 1] : 0.0;
      }
      __syncthreads();
      for (int t = 0; t * 16 < n; ++t) {
        const int jl = t * 16 + r16;
        const double* kr = Ks + jl * KSD + gq * (D / 4);
        double kb[D / 4];
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
          const double2 u = *reinterpret_cast<const double2*>(kr + 2 * i);
          kb[2 * i] = u.x;
          kb[2 * i + 1] = u.y;
        }
        // four independent accumulation chains keep the matrix pipe busy; summed pairwise
        f64x4_t l4[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) l4[h] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int ks = 0; ks < D / 4; ++ks)
          l4[ks & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], kb[ks], l4[ks & 3], 0, 0, 0);
        const f64x4_t lg = (l4[0] + l4[1]) + (l4[2] + l4[3]);
        const double uu = us[jl], ww = wsv[jl];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double E = exp_table(fma(lg[v], inv, -m_a[v]), T);
          s1[v] = fma(E, uu, s1[v]);
          s2[v] = fma(E * E, ww, s2[v]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      for (int o = 1; o < 16; o <<= 1) {
        s1[v] += __shfl_xor(s1[v], o);
        s2[v] += __shfl_xor(s2[v], o);
      }
    if (r16 == 0) {
      const double g = double(k1 - k0), vn = vns[b - b0];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int a = a0 + w * 16 + gq + 4 * v;
        if (a >= nq) continue;
        const double A = exp(lbar[(size_t(hd) * Cq + a) * Ck + b] - m_a[v]);
        scores[(size_t(hd) * Cq + a) * Ck + b] = A * A * vn - 2.0 * A * s1[v] / g + s2[v] / g;
      }
    }
  }
}

// ------------------------------------------------------------ bf16 scores with error bounds
// For bf16 keys the logits run on the bf16 matrix cores: qbar_a is split into three bf16
// slices (hi + mid + lo, each the rounding of what the previous slices leave), the keys are
// exact in bf16, and the three products accumulate in fp32.  Each pair is shifted by its own
// centroid logit, E'_j = e^{l_j - lbar_ab} = E_j / A, and the score is taken in centred form:
// with delta_j = 1 - E'_j, c_j = (vbar_b - v_j) . v_j and r_j = |vbar_b - v_j|^2,
//   g s_ab / A^2 = sum_j |vbar_b - E'_j v_j|^2 = sum_j r_j + 2 sum_j delta_j c_j + sum_j delta_j^2 |v_j|^2,
// the first sum fp64, the others fp32.  Nothing cancels.  A group of one key scores exactly 0
// (its centroid is its key) and is written so with a zero bound.  Each score comes with a bound on its
// distance to the exact score (same row factor), from:
//   - the logit: the hi slice takes one product per 32 columns (the first one seeded with the
//     mid and lo chain), so at most 2 (32 + 8) 2^-24 |qbar_a| max_j |k_j| for its products and
//     the fp32 sums that join them (every fp32 operation rounded, with a factor 2 for any
//     rounding mode of the matrix cores), 2 (2 d + 8) 2^-32 of the same for the mid and lo
//     chain, plus 2^-22 for the slices;
//   - the exponent argument: the fp32 scale (three roundings), the pair's shift and the fma;
//   - v_exp_f32 within 2^-21 relative;
//   - delta_j: within (relE + 2^-24)(E'_j + |delta_j|) of 1 - e^{x_j}, relE the relative error
//     of E'_j; the sums of |c_j| (E' + |delta|), |v_j|^2 |delta| (E' + |delta|) and
//     |v_j|^2 (E' + |delta|)^2 carry it to the two fp32 sums;
//   - the fp32 sums: at most g + 8 roundings on any path (g keys, four reduction levels),
//     each within 2^-24 of the sum of the magnitudes.
// A score whose sums overflow gets an infinite bound.
//
// A block takes 16 query groups per wave and 16 consecutive K/V groups, whose keys are
// contiguous; they pass through LDS in pieces of at most 64 keys of one group, double-buffered
// (the loads of the next piece are in flight while this one is computed), with the key norms
// formed while staging.  The sums of a group are reduced across the 16 lanes of each query
// group by DPP, and the scores and bounds of four groups are formed at once, one per lane.
// Blocks are ordered so that the query tiles sharing a K/V range run on one XCD (one L2).
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x4_t __attribute__((ext_vector_type(4)));
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum and maximum over 8 / 16 consecutive lanes (aligned): quad_perm [1,0,3,2] and [2,3,0,1],
// then row_half_mirror and row_mirror; every lane gets the result
__device__ __forceinline__ float lanes_sum8(float x) {
  x += dppf<0xB1>(x);
  x += dppf<0x4E>(x);
  return x + dppf<0x141>(x);
}
__device__ __forceinline__ float lanes_sum16(float x) {
  x = lanes_sum8(x);
  return x + dppf<0x140>(x);
}
// Sum over the 16 lanes of a row of x[my_v], my_v = (lane % 16) % 4, delivered to the lanes with
// that my_v: halves exchanged across lane bit 0 (quad_perm [1,0,3,2]) and bit 1 ([2,3,0,1]), then
// the four lanes of equal my_v summed by rotating the row by 4 and 8.
__device__ __forceinline__ float lanes_scatter_sum4(const float (&x)[4], int r16) {
  const bool b0 = r16 & 1, b1 = (r16 >> 1) & 1;
  float k0 = b0 ? x[1] : x[0], k1 = b0 ? x[3] : x[2];  // keep v = b0 and v = b0 + 2
  k0 += dppf<0xB1>(b0 ? x[0] : x[1]);
  k1 += dppf<0xB1>(b0 ? x[2] : x[3]);
  float z = b1 ? k1 : k0;  // keep v = b0 + 2 b1
  z += dppf<0x4E>(b1 ? k0 : k1);
  z += dppf<0x124>(z);  // row_ror:4
  return z + dppf<0x128>(z);  // row_ror:8
}
__device__ __forceinline__ float lanes_max16(float x) {
  x = fmaxf(x, dppf<0xB1>(x));
  x = fmaxf(x, dppf<0x4E>(x));
  x = fmaxf(x, dppf<0x141>(x));
  return fmaxf(x, dppf<0x140>(x));
}
constexpr int kFastPiece = 64;
constexpr int kFastWaves = 8;
template <int D>
constexpr size_t route_fast_buf() {
  return size_t(kFastPiece) * D * 2 + 3 * kFastPiece * 4;
}
template <int D>
constexpr size_t route_fast_smem() {
  return 2 * route_fast_buf<D>() + 16 * 8 + size_t(16) * 16 * kFastWaves * 8;
}
// blocks of the fast score kernel: one run of query tiles per (head, K/V range), eight runs
// side by side (one per XCD)
inline int64_t route_fast_blocks(int Cq, int Ck, int BH) {
  const int64_t TX = (Cq + 16 * kFastWaves - 1) / (16 * kFastWaves), TY = (Ck + 15) / 16;
  return 8 * TX * ((int64_t(BH) * TY + 7) / 8);
}
// qbar_a as three bf16 slices (hi, then mid = the rounding of what hi leaves, then lo) and its
// norm, one wave per query group.
template <int D>
__global__ __launch_bounds__(256) void qbar_split_kernel(const double* __restrict__ qbar, const int* __restrict__ n_q,
                                                         int Cq, __bf16* __restrict__ qsplit,
                                                         double* __restrict__ qnorm) {
  const int hd = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= n_q[hd]) return;
  double n2 = 0.0;
  __bf16* o = qsplit + (size_t(hd) * Cq + a) * 3 * D;
  for (int c = lane; c < D; c += 64) {
    const double x = qbar[(size_t(hd) * Cq + a) * D + c];
    const __bf16 h = __bf16(float(x));
    const double r1 = x - double(float(h));
    const __bf16 m = __bf16(float(r1));
    const double r2 = r1 - double(float(m));
    o[c] = h;
    o[D + c] = m;
    o[2 * D + c] = __bf16(float(r2));
    n2 = fma(x, x, n2);
  }
  n2 = wave_allsum_d(n2);
  if (lane == 0) qnorm[size_t(hd) * Cq + a] = sqrt(n2);
}
template <int D>
__global__ __launch_bounds__(kFastWaves * 64) void route_score_fast_kernel(const uint16_t* __restrict__ Kp, int N, int Nv,
                                                               const __bf16* __restrict__ qsplit,
                                                               const double* __restrict__ qnorm,
                                                               const double* __restrict__ lbar,
                                                               const double* __restrict__ vbar,
                                                               const int* __restrict__ kv_off,
                                                               const int* __restrict__ n_q,
                                                               const int* __restrict__ n_kv, int Cq, int Ck, int G,
                                                               int BH, const double* __restrict__ shift,
                                                               const double* __restrict__ vstat,
                                                               double* __restrict__ scores,
                                                               double* __restrict__ serr) {
  constexpr int PIECE = kFastPiece;
  constexpr int KS = D / 32;                   // 32-column steps
  constexpr int KPR = D / 8;                   // 16-byte pieces per key row
  constexpr int NTH = kFastWaves * 64, QT = 16 * kFastWaves;  // threads, query groups per block
  constexpr int KPT = PIECE * KPR / NTH;       // 16-byte pieces staged per thread
  constexpr size_t BUF = route_fast_buf<D>();
  extern __shared__ __attribute__((aligned(16))) char rf_sm[];
  double* p0s = reinterpret_cast<double*>(rf_sm + 2 * BUF);  // [16] sum_j r_j per group
  double* lbs = p0s + 16;                                    // [16][QT] lbar of the block's pairs
  const int TX = (Cq + QT - 1) / QT, TY = (Ck + 15) / 16;
  const int L = blockIdx.x, kq = L >> 3;
  const int tx = kq % TX, grp = (kq / TX) * 8 + (L & 7);
  if (grp >= BH * TY) return;
  const int hd = grp / TY, hk = hd / G, a0 = tx * QT, b0 = (grp % TY) * 16;
  const int nq = n_q[hd], nkv = n_kv[hk];
  if (a0 >= nq || b0 >= nkv) return;
  const int b1 = min(b0 + 16, nkv);
  const int* off = kv_off + size_t(hk) * (Ck + 1);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, gq = lane >> 4, r16 = lane & 15;
  const uint16_t* Kh = Kp + size_t(hk) * N * D;

  // A fragments (from qsplit): lane l holds query group a0 + 16 w + l % 16, columns
  // 32 ks + 8 (l / 16) .. + 7 of the three slices (zero past the last group)
  rbf16x8_t qh[KS], qm[KS], ql[KS];
  {
    const int a = a0 + w * 16 + r16;
    const uint4* qs4 = reinterpret_cast<const uint4*>(qsplit + (size_t(hd) * Cq + min(a, nq - 1)) * 3 * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 h = qs4[(0 * D + ks * 32 + gq * 8) / 8], m = qs4[(1 * D + ks * 32 + gq * 8) / 8],
            l = qs4[(2 * D + ks * 32 + gq * 8) / 8];
      if (a >= nq) h = m = l = make_uint4(0, 0, 0, 0);
      qh[ks] = __builtin_bit_cast(rbf16x8_t, h);
      qm[ks] = __builtin_bit_cast(rbf16x8_t, m);
      ql[ks] = __builtin_bit_cast(rbf16x8_t, l);
    }
  }
  // output slot v of lane l: query group a0 + 16 w + 4 (l / 16) + v, key l % 16 of the tile;
  // in the epilogue lane l forms the pair (query group slot v = l % 4, K/V group slot l % 16 / 4)
  const int my_v = r16 & 3, my_slot = r16 >> 2, my_a = a0 + w * 16 + gq * 4 + my_v;
  const double my_m = my_a < nq ? shift[size_t(hd) * Cq + my_a] : 0.0;
  const double my_qn = my_a < nq ? qnorm[size_t(hd) * Cq + my_a] : 0.0;
  // the block's centroid logits lbar_ab in LDS; the pair shifts (times log2 e, fp32) of the
  // lane's four query groups and group b
  for (int e = tid; e < 16 * QT; e += NTH) {
    const int bl = e % 16, al = e / 16;
    const int a = min(a0 + al, nq - 1), bg = min(b0 + bl, b1 - 1);
    lbs[bl * QT + al] = lbar[(size_t(hd) * Cq + a) * Ck + bg];
  }
  float m2[4];
  auto load_shift = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 4; ++v) m2[v] = float(lbs[(b - b0) * QT + w * 16 + gq * 4 + v] * 1.4426950408889634);
  };
  if (tid < 16) p0s[tid] = 0.0;

  // two register sets: the loads of a piece are issued two pieces before it is staged
  constexpr int KW = PIECE / 64;  // keys of a piece per lane of wave 0 (statistics)
  uint4 pk[2][KPT];
  double pu[2][KW], pw[2][KW], pr[2] = {0.0, 0.0};
  auto fetch = [&](auto set, int b, int p0) __attribute__((always_inline)) {
    constexpr int S = decltype(set)::value;
    const int n = min(PIECE, off[b + 1] - p0);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = tid + NTH * i, row = e / KPR, pc = e % KPR;
      pk[S][i] = make_uint4(0, 0, 0, 0);
      if (row < n) pk[S][i] = *reinterpret_cast<const uint4*>(Kh + size_t(p0 + row) * D + pc * 8);
    }
    if (tid < 64) {
      pr[S] = 0.0;
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int jl = tid + 64 * k;
        const double* st4 = vstat + (size_t(hk) * Nv + p0 + jl) * 4;
        pw[S][k] = jl < n ? st4[1] : 0.0;
        pu[S][k] = jl < n ? st4[2] : 0.0;
        pr[S] += jl < n ? st4[3] : 0.0;
      }
    }
  };
  // registers -> LDS buffer: key rows (16-byte piece p of row r at p ^ (r % KPR)), c, |v|^2,
  // |k|; the piece's sum of r_j is added to its group's (wave 0)
  auto put = [&](auto set, int bi, int bgrp) __attribute__((always_inline)) {
    constexpr int S = decltype(set)::value;
    uint16_t* K = reinterpret_cast<uint16_t*>(rf_sm + bi * BUF);
    float* F = reinterpret_cast<float*>(rf_sm + bi * BUF + size_t(PIECE) * D * 2);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = tid + NTH * i, row = e / KPR, pc = e % KPR;
      *reinterpret_cast<uint4*>(K + row * D + ((pc ^ (row % KPR)) * 8)) = pk[S][i];
      const uint32_t wd[4] = {pk[S][i].x, pk[S][i].y, pk[S][i].z, pk[S][i].w};
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(wd[j] << 16), hi = __uint_as_float(wd[j] & 0xFFFF0000u);
        sq = fmaf(lo, lo, fmaf(hi, hi, sq));
      }
      sq = KPR == 16 ? lanes_sum16(sq) : lanes_sum8(sq);
      if (pc == 0) F[2 * PIECE + row] = sqrtf(sq);
    }
    if (tid < 64) {
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        F[tid + 64 * k] = float(pu[S][k]);
        F[PIECE + tid + 64 * k] = float(pw[S][k]);
      }
      const double rs = wave_allsum_d(pr[S]);
      if (tid == 0) p0s[bgrp - b0] += rs;
    }
  };

  const float c2 = 1.4426950408889634f / sqrtf(float(D));
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // pieces: cur (in LDS buffer buf), nxt (register set of the other parity, loads in flight),
  // nn (loaded next); a piece position is (group, first key), group b1 once past the end
  auto advance = [&](int& pb, int& pp) {
    pp += PIECE;
    if (pp >= off[pb + 1]) {
      ++pb;
      pp = pb < b1 ? off[pb] : 0;
    }
  };
  int b = b0, p0 = off[b0];
  int nb = b, np0 = p0;
  advance(nb, np0);
  int nnb = nb, nnp0 = np0;
  if (nnb < b1) advance(nnb, nnp0);
  fetch(S0{}, b, p0);
  if (nb < b1) fetch(S1{}, nb, np0);
  __syncthreads();  // p0s cleared, lbs filled
  put(S0{}, 0, b);
  load_shift(b);
  __syncthreads();
  // per output slot: P1 = sum delta c, P2 = sum delta^2 |v|^2 and the three bound sums
  float P1[4], P2[4], B1[4], B2[4], B3[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) P1[v] = P2[v] = B1[v] = B2[v] = B3[v] = 0.f;
  float kmax = 0.f;
  float kP1 = 0.f, kP2 = 0.f, kB1 = 0.f, kB2 = 0.f, kB3 = 0.f, kK = 0.f;  // this lane's pair of the batch
  int slot = 0, gstart = b0, buf = 0;
  // one piece: set S held cur (staged), set S ^ 1 holds nxt; returns false after the last piece
  auto step = [&](auto set) __attribute__((always_inline)) -> bool {
    constexpr int S = decltype(set)::value;
    using SO = std::integral_constant<int, S ^ 1>;
    if (nnb < b1) fetch(set, nnb, nnp0);
    const int n = min(PIECE, off[b + 1] - p0);
    {
      const uint16_t* K = reinterpret_cast<const uint16_t*>(rf_sm + buf * BUF);
      const float* F = reinterpret_cast<const float*>(rf_sm + buf * BUF + size_t(PIECE) * D * 2);
      for (int t = 0; t * 16 < n; ++t) {
        const int jl = t * 16 + r16;
        rbf16x8_t kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kb[ks] = __builtin_bit_cast(rbf16x8_t,
                                      *reinterpret_cast<const uint4*>(K + jl * D + (((ks * 4 + gq) ^ (jl % KPR)) * 8)));
        // mid and lo slices in one chain, which then seeds the first hi product; the other hi
        // products start from zero
        const rf32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        rf32x4_t cml = zero, ch[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          cml = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm[ks], kb[ks], cml, 0, 0, 0);
          cml = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[ks], kb[ks], cml, 0, 0, 0);
        }
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) ch[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[ks], kb[ks], zero, 0, 0, 0);
        ch[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[0], kb[0], cml, 0, 0, 0);
        rf32x4_t lg = ch[0];
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) lg += ch[ks];
        const bool live = jl < n;
        const float cc = F[jl], ww = F[PIECE + jl], ac = fabsf(cc);
        if (live) kmax = fmaxf(kmax, F[2 * PIECE + jl]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float l = lg[v];
          const float E = live ? __builtin_amdgcn_exp2f(fmaf(l, c2, -m2[v])) : 1.f;
          const float dl = 1.f - E, ad = fabsf(dl), tt = E + ad;
          P1[v] = fmaf(dl, cc, P1[v]);
          P2[v] = fmaf(dl * dl, ww, P2[v]);
          B1[v] = fmaf(ac, tt, B1[v]);
          B2[v] = fmaf(ww * ad, tt, B2[v]);
          B3[v] = fmaf(ww * tt, tt, B3[v]);
        }
      }
    }
    if (p0 + PIECE >= off[b + 1]) {  // group b complete
      const float s1 = lanes_scatter_sum4(P1, r16), s2 = lanes_scatter_sum4(P2, r16),
                  s3 = lanes_scatter_sum4(B1, r16), s4 = lanes_scatter_sum4(B2, r16),
                  s5 = lanes_scatter_sum4(B3, r16);
      kmax = lanes_max16(kmax);
      if (my_slot == slot) {
        kP1 = s1;
        kP2 = s2;
        kB1 = s3;
        kB2 = s4;
        kB3 = s5;
        kK = kmax;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) P1[v] = P2[v] = B1[v] = B2[v] = B3[v] = 0.f;
      kmax = 0.f;
      ++slot;
      if (slot == 4 || b + 1 == b1) {
        const int bb = gstart + my_slot;
        if (my_slot < slot && my_a < nq) {
          constexpr double u = 0x1p-24;
          const int g_keys = off[bb + 1] - off[bb];
          const double g = double(g_keys), ig = 1.0 / g, R0 = p0s[bb - b0];
          const double Q1 = kP1, Q2 = kP2, C1 = kB1, C2 = kB2, C3 = kB3;
          const size_t at = (size_t(hd) * Cq + my_a) * Ck + bb;
          const double lb = lbs[(bb - b0) * QT + w * 16 + gq * 4 + my_v], A = exp(lb - my_m), A2 = A * A;
          double score = A2 * ((R0 + 2.0 * Q1 + Q2) * ig);
          // |qbar_a| |k_j| bounds |l_j| and the sum of the product magnitudes (norms from fp32 sums)
          const double C = my_qn * double(kK) * (1.0 + 1e-5);
          const double eps_l = 2.0 * (32 + 8) * u * C + 2.0 * (2 * D + 8) * 0x1p-32 * C + 0x1p-22 * C +
                               D * 0x1p-100 * double(kK);
          const double c2d = 1.4426950408889634 / sqrt(double(D)), m2d = fabs(lb * 1.4426950408889634);
          const double dx = eps_l * c2d * 1.001 + 6.0 * u * (C * c2d + m2d) * 1.001;
          const double y = dx * 0.69314718055994531;
          const double relE = (y < 0.5 ? y * (1.0 + y) : expm1(y)) * (1.0 + 0x1p-21) + 0x1p-21;
          const double nr = (g + 8.0) * u, re = relE + u;
          const double ep = (2.0 * (re + nr) * C1 + re * (2.0 * C2 + re * C3) + nr * fabs(Q2)) * 1.01;
          double err = A2 * (ep * ig * 1.001 + 1e-15 * (R0 + 2.0 * C1 + fabs(Q2)) * ig);
          if (!(fabs(score) <= 1.0e300) || !(err <= 1.0e300)) {
            score = 0.0;
            err = INFINITY;
          }
          if (g_keys == 1) score = err = 0.0;
          scores[at] = score;
          serr[at] = err;
        }
        slot = 0;
        gstart = b + 1;
      }
    }
    if (nb >= b1) return false;
    put(SO{}, buf ^ 1, nb);
    __syncthreads();
    buf ^= 1;
    if (nb != b) load_shift(nb);
    b = nb;
    p0 = np0;
    nb = nnb;
    np0 = nnp0;
    if (nnb < b1) advance(nnb, nnp0);
    return true;
  };
  while (step(S0{}) && step(S1{})) {
  }
}

// Bitonic network of one wave over P = 64 E entries held E per lane in rank order (lane l holds
// ranks l E .. l E + E - 1; strides below E are exchanges inside a lane, larger strides between
// lanes l and l ^ (stride / E)): key descending, ties to the lower id.  NP payload doubles per
// entry travel with it.
template <int E, int NP>
__device__ __forceinline__ void wave_sort_desc(double (&key)[E], int (&id)[E], double (&pl)[NP > 0 ? NP : 1][E],
                                               int lane) {
  constexpr int P = 64 * E;
  auto before = [](double s1, int i1, double s2, int i2) { return s1 > s2 || (s1 == s2 && i1 < i2); };
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride >= E; stride >>= 1) {  // between lanes
      const int pl_lane = lane ^ (stride / E);
      const bool low = lane < pl_lane, up = ((lane * E) & size) == 0;
#pragma unroll
      for (int t = 0; t < E; ++t) {
        const double os = __shfl(key[t], pl_lane);
        const int oi = __shfl(id[t], pl_lane);
        double op[NP > 0 ? NP : 1];
#pragma unroll
        for (int k = 0; k < NP; ++k) op[k] = __shfl(pl[k][t], pl_lane);
        const bool mine_first = before(key[t], id[t], os, oi);
        // the lower position keeps the entry that comes first in this block's direction
        const bool keep_mine = (low == up) ? mine_first : !mine_first;
        if (!keep_mine) {
          key[t] = os;
          id[t] = oi;
#pragma unroll
          for (int k = 0; k < NP; ++k) pl[k][t] = op[k];
        }
      }
    }
#pragma unroll
    for (int stride = E / 2; stride >= 1; stride >>= 1) {  // inside a lane
      if (stride >= size) continue;
#pragma unroll
      for (int t = 0; t < E; ++t) {
        const int u = t ^ stride;
        if (u > t) {
          const bool up = ((lane * E + t) & size) == 0;
          if (before(key[u], id[u], key[t], id[t]) == up) {
            const double ts = key[t];
            const int ti = id[t];
            key[t] = key[u]; id[t] = id[u];
            key[u] = ts; id[u] = ti;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
              const double tp = pl[k][t];
              pl[k][t] = pl[k][u];
              pl[k][u] = tp;
            }
          }
        }
      }
    }
  }
}

// Budgeted prefix of Sec. 4.3 from the ranked groups id (E per lane, rank order): the shortest
// prefix whose key count reaches Tk (at least one group, all groups when out of reach), written
// to out followed by the text group when n_text > 0, with the count, the routed pairs and the
// budget flag.
template <int E>
__device__ __forceinline__ void emit_prefix(const int (&id)[E], int nkv, const int* off, int64_t Tk, int lane,
                                            int n_text, int* out, int* cnt_out, int64_t ga, int64_t* pairs,
                                            int* gflag) {
  int loc[E], s = 0;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    loc[t] = lane * E + t < nkv ? off[id[t] + 1] - off[id[t]] : 0;
    s += loc[t];
  }
  int incl = s;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  int cum = incl - s, L = nkv;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int i = lane * E + t;
    cum += loc[t];
    if (i < nkv && cum >= Tk && cum - loc[t] < Tk) L = i + 1;  // unique crossing
  }
  for (int o = 32; o > 0; o >>= 1) L = min(L, __shfl_xor(L, o));
  int64_t keys = 0;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int i = lane * E + t;
    if (i < L) {
      out[i] = id[t];
      keys += loc[t];
    }
  }
  for (int o = 32; o > 0; o >>= 1) keys += __shfl_xor(keys, o);
  if (lane == 0) {
    int cnt = L;
    if (n_text > 0) out[cnt++] = nkv;
    *cnt_out = cnt;
    if (keys < Tk) atomicOr(gflag, SPR_HS_BUDGET_UNREACHED);
    atomicAdd(reinterpret_cast<unsigned long long*>(pairs), (unsigned long long)(ga * (keys + n_text)));
  }
}

// Budgeted prefix for one query group from fp64 scores, one wave per group.  The group past the
// last query group (index n_q) is the text query group, which selects every group.
template <int E>
__global__ __launch_bounds__(256) void route_select_kernel(const double* __restrict__ scores,
                                                           const int* __restrict__ kv_off,
                                                           const int* __restrict__ q_off,
                                                           const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                           int Cq, int Ck, int G, int n_text, int64_t Tk,
                                                           int* __restrict__ sel_cnt, int* __restrict__ sel_kv,
                                                           int64_t* __restrict__ pairs, int* __restrict__ gstat) {
  const int hd = blockIdx.y, hk = hd / G, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nq = n_q[hd], nkv = n_kv[hk];
  const int* off = kv_off + size_t(hk) * (Ck + 1);
  if (a > nq || (a == nq && n_text == 0)) return;
  int* out = sel_kv + (size_t(hd) * (Cq + 1) + a) * (Ck + 1);
  if (a == nq) {  // text query rows: every group
    for (int b = lane; b <= nkv; b += 64) out[b] = b;
    if (lane == 0) sel_cnt[size_t(hd) * (Cq + 1) + a] = nkv + 1;
    return;
  }
  double sc[E], none[1][E];
  int id[E];
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int i = lane * E + t;
    sc[t] = i < nkv ? scores[(size_t(hd) * Cq + a) * Ck + i] : -1.0e308;
    id[t] = i < nkv ? i : 0x7fffffff;
  }
  wave_sort_desc<E, 0>(sc, id, none, lane);
  const int64_t ga = q_off[size_t(hd) * (Cq + 1) + a + 1] - q_off[size_t(hd) * (Cq + 1) + a];
  emit_prefix<E>(id, nkv, off, Tk, lane, n_text, out, sel_cnt + size_t(hd) * (Cq + 1) + a, ga, pairs + hd,
                 gstat + hd * 8 + 0);
}

typedef unsigned int ru32x4_t __attribute__((ext_vector_type(4)));

// Routing of one query group from the bf16 scores and their bounds, one wave per group, in three
// phases with the fp64 rescoring between them (route_rescore_kernel, which reads the keys of a
// K/V group once for every query group that asked for it).  With I_b = [s_b - e_b, s_b + e_b]
// holding the exact score:
//   phase 0: scores whose bound is not finite or above 1e-3 of the row's largest score are
//            marked for rescoring;
//   phase 1: the groups are ranked by score, and lambda' is the smallest lower end among the
//            shortest ranked prefix holding Tk keys.  A group whose upper end is below lambda' is
//            preceded (in exact order) by groups holding at least Tk keys, so it is outside the
//            prefix; it ranks last (a stable partition through LDS).  Among the others, in rank
//            order, a group meets an earlier interval iff the smallest earlier lower end reaches
//            its upper end, and a later one iff the largest later upper end reaches its lower
//            end; such groups are marked for rescoring.  The ranking and the number of groups
//            that can be in the prefix are kept for phase 2;
//   phase 2: a group left with its bf16 score is disjoint from every other interval, so it sits
//            correctly against every score of the row; the rescored groups form runs of
//            consecutive ranks (a group between two overlapping intervals meets one of them),
//            which odd-even transposition passes put in order.  The ranking is then that of the
//            fp64 scores, and its prefix is the selection.
// Rescored entries are written back to `scores` with bound 0 between the phases.
template <int PHASE, int E, int D>
__global__ __launch_bounds__(256) void route_resolve_kernel(
    double* __restrict__ scores, double* __restrict__ serr, bool keep, const int* __restrict__ kv_off,
    const int* __restrict__ q_off, const int* __restrict__ n_q, const int* __restrict__ n_kv, int Cq, int Ck, int G,
    int n_text, int64_t Tk, unsigned long long* __restrict__ rbits, int* __restrict__ rorder, int* __restrict__ rnin,
    int* __restrict__ sel_cnt, int* __restrict__ sel_kv, int64_t* __restrict__ pairs, int* __restrict__ gstat) {
  __shared__ double part_val[4][64 * E];
  __shared__ int part_id[4][64 * E];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hd = blockIdx.y, hk = hd / G, a = blockIdx.x * 4 + w;
  const int nq = n_q[hd], nkv = n_kv[hk];
  const int* off = kv_off + size_t(hk) * (Ck + 1);
  if (a > nq || (a == nq && n_text == 0)) return;
  if (a == nq) {  // text query rows: every group
    if constexpr (PHASE == 2) {
      int* out = sel_kv + (size_t(hd) * (Cq + 1) + a) * (Ck + 1);
      for (int b = lane; b <= nkv; b += 64) out[b] = b;
      if (lane == 0) sel_cnt[size_t(hd) * (Cq + 1) + a] = nkv + 1;
    }
    return;
  }
  const size_t row = (size_t(hd) * Cq + a) * Ck;
  const int W = (Cq + 63) / 64;  // request words per K/V group
  auto request = [&](int b) {
    atomicOr(rbits + (size_t(hd) * Ck + b) * W + (a >> 6), 1ull << (a & 63));
  };
  int* ord = rorder + (size_t(hd) * Cq + a) * (64 * E);
  double sc[E], pl[1][E];  // score and its bound
  int id[E];
  if constexpr (PHASE < 2) {
    // coalesced loads: entry t of lane l is group t 64 + l (the ranking below does not depend on
    // where an entry starts, its order being a total one)
#pragma unroll
    for (int t = 0; t < E; ++t) {
      const int i = t * 64 + lane;
      sc[t] = i < nkv ? scores[row + i] : 0.0;
      pl[0][t] = i < nkv ? serr[row + i] : 0.0;
      id[t] = i < nkv ? i : 0x7fffffff;
    }
  }
  if constexpr (PHASE == 0) {
    // bounds that would overlap most of the row
    double rmax = 0.0;
#pragma unroll
    for (int t = 0; t < E; ++t)
      if (id[t] < nkv) rmax = fmax(rmax, fabs(sc[t]));
    for (int o = 32; o > 0; o >>= 1) rmax = fmax(rmax, __shfl_xor(rmax, o));
#pragma unroll
    for (int t = 0; t < E; ++t)
      if (id[t] < nkv && !(pl[0][t] <= 1e-3 * rmax)) request(id[t]);
    return;
  }
  if constexpr (PHASE == 1) {
    // rank by score; lambda' = the smallest lower end among the shortest ranked prefix holding Tk
    // keys.  Those groups hold at least Tk keys with lower ends >= lambda', so a group whose upper
    // end is below lambda' is outside the prefix (-inf when Tk is out of reach).  The bounds wait
    // in LDS by group (the ranking network carries only scores and groups).
#pragma unroll
    for (int t = 0; t < E; ++t) {
      part_val[w][t * 64 + lane] = pl[0][t];  // by group
      if (id[t] >= nkv) sc[t] = -1.0e308;
    }
    {
      double none[1][E];
      wave_sort_desc<E, 0>(sc, id, none, lane);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t = 0; t < E; ++t) pl[0][t] = id[t] < nkv ? part_val[w][id[t]] : 0.0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int sz[E], s_loc = 0;
#pragma unroll
    for (int t = 0; t < E; ++t) {
      sz[t] = id[t] < nkv ? off[id[t] + 1] - off[id[t]] : 0;
      s_loc += sz[t];
    }
    int incl = s_loc;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    double lam = INFINITY;
    {
      int cum = incl - s_loc;
#pragma unroll
      for (int t = 0; t < E; ++t) {
        if (id[t] < nkv && cum < Tk) lam = fmin(lam, sc[t] - pl[0][t]);  // ranks up to the crossing
        cum += sz[t];
      }
      for (int o = 32; o > 0; o >>= 1) lam = fmin(lam, __shfl_xor(lam, o));
      if (__shfl(incl, 63) < Tk) lam = -INFINITY;
    }
    // stable partition through LDS: the groups that can be in the prefix first, in rank order
    // (their scores and bounds are written out now for the others)
    bool in[E];
    int n_in_l = 0;
#pragma unroll
    for (int t = 0; t < E; ++t) {
      in[t] = id[t] < nkv && sc[t] + pl[0][t] >= lam;
      n_in_l += in[t] ? 1 : 0;
      if (keep && id[t] < nkv && !in[t]) serr[row + id[t]] = -(pl[0][t] + 1.0e-300);
    }
    int in_incl = n_in_l;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(in_incl, o);
      if (lane >= o) in_incl += y;
    }
    const int n_in = __shfl(in_incl, 63);
    {
      const int r_in0 = in_incl - n_in_l, r_out0 = n_in + (lane * E - (in_incl - n_in_l));
      double* vs = &part_val[w][0];
      int* is = &part_id[w][0];
      auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
      int r_in = r_in0, r_out = r_out0;
#pragma unroll
      for (int t = 0; t < E; ++t) {  // keys and ids
        const int dst = in[t] ? r_in++ : r_out++;
        vs[dst] = in[t] ? sc[t] : (id[t] < nkv ? -1.0e300 : -1.0e308);
        is[dst] = id[t];
      }
      wave_sync();
      double nk[E];
#pragma unroll
      for (int t = 0; t < E; ++t) {
        nk[t] = vs[lane * E + t];
        id[t] = is[lane * E + t];
      }
      wave_sync();
      r_in = r_in0;
      r_out = r_out0;
#pragma unroll
      for (int t = 0; t < E; ++t) vs[in[t] ? r_in++ : r_out++] = pl[0][t];  // bounds
      wave_sync();
#pragma unroll
      for (int t = 0; t < E; ++t) {
        sc[t] = nk[t];
        pl[0][t] = vs[lane * E + t];
        in[t] = lane * E + t < n_in;
      }
    }
    // overlaps among the groups that can be in the prefix: in rank order a group meets an
    // earlier interval iff the smallest earlier lower end reaches its upper end, a later one iff
    // the largest later upper end reaches its lower end
    double lmin = INFINITY, hmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < E; ++t)
      if (in[t]) {
        lmin = fmin(lmin, sc[t] - pl[0][t]);
        hmax = fmax(hmax, sc[t] + pl[0][t]);
      }
    double pmin = lmin, smax = hmax;
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(pmin, o), z = __shfl_down(smax, o);
      if (lane >= o) pmin = fmin(pmin, y);
      if (lane + o < 64) smax = fmax(smax, z);
    }
    double run_lo = __shfl_up(pmin, 1), run_hi = __shfl_down(smax, 1);
    if (lane == 0) run_lo = INFINITY;
    if (lane == 63) run_hi = -INFINITY;
    bool flag[E];
#pragma unroll
    for (int t = 0; t < E; ++t) {
      flag[t] = in[t] && pl[0][t] > 0.0 && run_lo <= sc[t] + pl[0][t];
      if (in[t]) run_lo = fmin(run_lo, sc[t] - pl[0][t]);
    }
#pragma unroll
    for (int t = E - 1; t >= 0; --t) {
      const double lo = sc[t] - pl[0][t], hi = sc[t] + pl[0][t];
      flag[t] = flag[t] || (in[t] && pl[0][t] > 0.0 && run_hi >= lo);
      if (in[t]) run_hi = fmax(run_hi, hi);
    }
#pragma unroll
    for (int t = 0; t < E; ++t) {
      if (flag[t]) request(id[t]);
      ord[lane * E + t] = id[t];
    }
    if (lane == 0) rnin[size_t(hd) * Cq + a] = n_in;
    return;
  }
  if constexpr (PHASE == 2) {
    const int n_in = rnin[size_t(hd) * Cq + a];
#pragma unroll
    for (int t = 0; t < E; ++t) {
      const int i = lane * E + t;
      id[t] = ord[i];
      const bool inn = i < n_in;
      sc[t] = inn ? scores[row + id[t]] : -1.0e300;
      pl[0][t] = inn ? serr[row + id[t]] : 0.0;
    }
    // odd-even transposition passes over the first n_in ranks until their ranking is that of
    // the scores (none swap when no score in the prefix candidates was rescored)
    auto before = [](double s1, int i1, double s2, int i2) { return s1 > s2 || (s1 == s2 && i1 < i2); };
    auto pass = [&](int parity) -> bool {
      bool sw_any = false;
#pragma unroll
      for (int t = 0; t + 1 < E; ++t)
        if (((lane * E + t) & 1) == parity && lane * E + t + 1 < n_in &&
            before(sc[t + 1], id[t + 1], sc[t], id[t])) {
          const double ts = sc[t], te = pl[0][t];
          const int ti = id[t];
          sc[t] = sc[t + 1]; pl[0][t] = pl[0][t + 1]; id[t] = id[t + 1];
          sc[t + 1] = ts; pl[0][t + 1] = te; id[t + 1] = ti;
          sw_any = true;
        }
      // the pair (last of this lane, first of the next lane)
      const double ns = __shfl_down(sc[0], 1), ne = __shfl_down(pl[0][0], 1);
      const int ni = __shfl_down(id[0], 1);
      const double ps = __shfl_up(sc[E - 1], 1), pe = __shfl_up(pl[0][E - 1], 1);
      const int pi = __shfl_up(id[E - 1], 1);
      const bool mine = lane < 63 && ((lane * E + E - 1) & 1) == parity && (lane + 1) * E < n_in &&
                        before(ns, ni, sc[E - 1], id[E - 1]);
      const bool take = __shfl_up(mine ? 1 : 0, 1) != 0 && lane > 0;
      if (mine) {
        sc[E - 1] = ns; pl[0][E - 1] = ne; id[E - 1] = ni;
        sw_any = true;
      }
      if (take) {
        sc[0] = ps; pl[0][0] = pe; id[0] = pi;
      }
      return __any(sw_any);
    };
    for (;;) {
      const bool s0 = pass(0);
      const bool s1 = pass(1);
      if (!s0 && !s1) break;
    }
    int* out = sel_kv + (size_t(hd) * (Cq + 1) + a) * (Ck + 1);
    const int64_t ga = q_off[size_t(hd) * (Cq + 1) + a + 1] - q_off[size_t(hd) * (Cq + 1) + a];
    emit_prefix<E>(id, nkv, off, Tk, lane, n_text, out, sel_cnt + size_t(hd) * (Cq + 1) + a, ga, pairs + hd,
                   gstat + hd * 8 + 0);
  }
}

// fp64 rescoring of the (query group, K/V group) pairs the resolve phases asked for, grouped by
// K/V group: block (b, head) reads the requests of its column of request bits (clearing them) and
// stages the group's keys and their statistics in LDS once.  The logits of 16 requests x 16 keys
// at a time are products on v_mfma_f64_16x16x4f64 (exact products of the bf16 keys with the fp64
// centroids, fp64 sums): lane l supplies centroid and key elements D/4 (l / 16) .. + D/4 - 1 and
// receives the logits of requests l / 16 + 4 v and key l % 16.  The four waves take the group's
// 16-key tiles in turn; the score expansion's two sums are reduced over the key lanes by DPP and
// over the waves in LDS.  A group of more keys than fit the 48 KB of LDS reads them from memory.
template <int D>
constexpr int rescore_keys() { return 49152 / (D * 2 + 16); }  // keys staged in LDS (48 KB)
template <int D>
__global__ __launch_bounds__(256) void route_rescore_kernel(
    unsigned long long* __restrict__ rbits, const void* __restrict__ Kp, int N, int Nv,
    const double* __restrict__ qbar, const double* __restrict__ lbar, const double* __restrict__ vbar,
    const double* __restrict__ shift, const double* __restrict__ vstat, const int* __restrict__ kv_off,
    const int* __restrict__ n_kv, int Cq, int Ck, int G, double* __restrict__ scores, double* __restrict__ serr) {
  constexpr int PC = D / 8;  // 16-byte pieces per key row
  constexpr int KR = rescore_keys<D>(), KSTR = PC + 1;  // key rows padded by 16 bytes in LDS
  constexpr int S = D / 4;   // elements per lane group (and matrix-core steps per tile)
  constexpr int SP = S / 8;  // their 16-byte pieces
  __shared__ __attribute__((aligned(16))) ru32x4_t ks[KR * KSTR];
  __shared__ double kst[KR][2];
  __shared__ double red[4][2][16];
  __shared__ int list[1024];
  __shared__ int nreq;
  const int b = blockIdx.x, hd = blockIdx.y, hk = hd / G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (b >= n_kv[hk]) return;
  const int W = (Cq + 63) / 64;
  unsigned long long* bits = rbits + (size_t(hd) * Ck + b) * W;
  if (threadIdx.x < 64) {  // wave 0: lane i takes request word i (W <= 16)
    unsigned long long m = lane < W ? bits[lane] : 0ull;
    if (m) bits[lane] = 0ull;
    const int c = __popcll(m);
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int k = incl - c;
    while (m) {
      list[k++] = lane * 64 + __ffsll((long long)m) - 1;
      m &= m - 1;
    }
    if (lane == 63) nreq = incl;
  }
  __syncthreads();
  const int n = nreq;
  if (n == 0) return;
  const int k0 = kv_off[size_t(hk) * (Ck + 1) + b], k1 = kv_off[size_t(hk) * (Ck + 1) + b + 1];
  const int nk = k1 - k0;
  const bool staged = nk <= KR;
  const ru32x4_t* Kg = static_cast<const ru32x4_t*>(Kp) + (int64_t(hk) * N + k0) * PC;
  if (staged) {
    for (int e = threadIdx.x; e < nk * PC; e += 256) ks[(e / PC) * KSTR + e % PC] = Kg[e];
    for (int j = threadIdx.x; j < nk; j += 256) {
      kst[j][0] = vstat[(size_t(hk) * Nv + k0 + j) * 4];
      kst[j][1] = vstat[(size_t(hk) * Nv + k0 + j) * 4 + 1];
    }
  }
  double vn = 0.0;  // |vbar_b|^2, the same for every request
  for (int c = lane; c < D; c += 64) {
    const double y = vbar[(size_t(hk) * Ck + b) * D + c];
    vn = fma(y, y, vn);
  }
  vn = wave_allsum_d(vn);
  __syncthreads();
  const double inv = 1.0 / sqrt(double(D));
  const int i16 = lane & 15, kq = lane >> 4;
  const int KT = (nk + 15) >> 4;  // 16-key tiles
  // row sums over the 16 lanes of a DPP row (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
  // row_mirror)
  auto rowsum = [](double x) {
    x += dppd<0xB1>(x);
    x += dppd<0x4E>(x);
    x += dppd<0x141>(x);
    return x + dppd<0x140>(x);
  };
  for (int rt = 0; rt < n; rt += 16) {
    // A fragments: centroid of request rt + l % 16 (zero past the last request)
    const int ra = rt + i16 < n ? list[rt + i16] : -1;
    double qa[S];
    {
      const double* qp = qbar + (size_t(hd) * Cq + (ra >= 0 ? ra : 0)) * D + S * kq;
#pragma unroll
      for (int e = 0; e < S; e += 2) {
        const double2 t2 = ra >= 0 ? *reinterpret_cast<const double2*>(qp + e) : make_double2(0.0, 0.0);
        qa[e] = t2.x;
        qa[e + 1] = t2.y;
      }
    }
    double mv[4], s1[4], s2[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = rt + kq + 4 * v;
      mv[v] = r < n ? shift[size_t(hd) * Cq + list[r]] : 0.0;
      s1[v] = s2[v] = 0.0;
    }
    for (int kt = w; kt < KT; kt += 4) {
      const int jl = kt * 16 + i16;
      const bool live = jl < nk;
      const int jc = live ? jl : nk - 1;
      ru32x4_t raw[SP];
#pragma unroll
      for (int t = 0; t < SP; ++t) raw[t] = staged ? ks[jc * KSTR + SP * kq + t] : Kg[int64_t(jc) * PC + SP * kq + t];
      f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int t = 0; t < SP; ++t) {
        const uint32_t wd[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[8 * t + 2 * h], double(__uint_as_float(wd[h] << 16)), acc,
                                                     0, 0, 0);
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[8 * t + 2 * h + 1],
                                                     double(__uint_as_float(wd[h] & 0xFFFF0000u)), acc, 0, 0, 0);
        }
      }
      double ux = 0.0, uy = 0.0;
      if (live) {
        ux = staged ? kst[jl][0] : vstat[(size_t(hk) * Nv + k0 + jl) * 4];
        uy = staged ? kst[jl][1] : vstat[(size_t(hk) * Nv + k0 + jl) * 4 + 1];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double Ej = live ? exp(fma(acc[v], inv, -mv[v])) : 0.0;
        s1[v] = fma(Ej, ux, s1[v]);
        s2[v] = fma(Ej * Ej, uy, s2[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      s1[v] = rowsum(s1[v]);
      s2[v] = rowsum(s2[v]);
      if (i16 == 0) {
        red[w][0][kq + 4 * v] = s1[v];
        red[w][1][kq + 4 * v] = s2[v];
      }
    }
    __syncthreads();
    if (threadIdx.x < 16 && rt + int(threadIdx.x) < n) {
      const int i = threadIdx.x, a = list[rt + i];
      const double t1 = (red[0][0][i] + red[1][0][i]) + (red[2][0][i] + red[3][0][i]);
      const double t2 = (red[0][1][i] + red[1][1][i]) + (red[2][1][i] + red[3][1][i]);
      const double g = double(nk);
      const size_t at = (size_t(hd) * Cq + a) * Ck + b;
      const double A = exp(lbar[at] - shift[size_t(hd) * Cq + a]);
      scores[at] = A * A * vn - 2.0 * A * t1 / g + t2 / g;
      serr[at] = 0.0;
    }
    __syncthreads();  // red is free again
  }
}

__global__ void zero_i64_kernel(int64_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Per head: rho_exec and the probe allocation m_a (largest remainder of M |G_a| / Nv;
// remainder ties to the larger group, then the lower id).
__global__ __launch_bounds__(1024) void route_finalize_kernel(const int* __restrict__ q_off,
                                                              const int* __restrict__ n_q, int Cq, int N, int Nv,
                                                              int n_text, int M, const int64_t* __restrict__ pairs,
                                                              double* __restrict__ rho, int* __restrict__ pstat) {
  __shared__ int buf[1024];
  __shared__ long long rem[1024];
  __shared__ int sz[1024];
  const int hd = blockIdx.x, t = threadIdx.x;
  const int nq = n_q[hd];
  const int* qo = q_off + size_t(hd) * (Cq + 1);
  // probes
  long long base = 0;
  if (t < nq) {
    sz[t] = qo[t + 1] - qo[t];
    base = (long long)M * sz[t] / Nv;
    rem[t] = (long long)M * sz[t] % Nv;
  }
  __syncthreads();
  int tb;
  block_exscan_i(int(base), buf, &tb);
  const int R = M - tb;
  int m = int(base);
  if (t < nq) {
    int rank = 0;
    for (int o = 0; o < nq; ++o) {
      const bool before = rem[o] > rem[t] || (rem[o] == rem[t] && (sz[o] > sz[t] || (sz[o] == sz[t] && o < t)));
      rank += before;
    }
    if (rank < R) ++m;
  }
  int mt;
  const int po = block_exscan_i(t < nq ? m : 0, buf, &mt);
  if (t < nq) {
    pstat[(size_t(hd) * Cq + t) * 2 + 0] = m;
    pstat[(size_t(hd) * Cq + t) * 2 + 1] = po;
  }
  if (t == 0) {
    const double Nd = double(N);
    rho[hd] = (double(pairs[hd]) + double(n_text) * Nd + double(M) * Nd) / (Nd * Nd);
  }
}

// Probe rows of one query group: the m_a members with the smallest d_i (ties to the lower
// row), listed nearest first at the group's probe offset; w_p = |G_a| / m_a (App. A.2).
__global__ __launch_bounds__(256) void probe_select_kernel(const int* __restrict__ q_off,
                                                           const int* __restrict__ q_perm,
                                                           const int* __restrict__ n_q, const double* __restrict__ qdist,
                                                           const int* __restrict__ pstat, int Cq, int Nv, int M,
                                                           int* __restrict__ probe_idx, double* __restrict__ probe_w) {
  const int hd = blockIdx.y, a = blockIdx.x;
  if (a >= n_q[hd]) return;
  const int m = pstat[(size_t(hd) * Cq + a) * 2 + 0], po = pstat[(size_t(hd) * Cq + a) * 2 + 1];
  if (m == 0) return;
  const int r0 = q_off[size_t(hd) * (Cq + 1) + a], r1 = q_off[size_t(hd) * (Cq + 1) + a + 1];
  const int* pm = q_perm + size_t(hd) * Nv;
  const double* dd = qdist + size_t(hd) * Nv;
  // the members' rows and distances in LDS (groups of up to kSelStage rows; larger ones rank
  // from memory)
  constexpr int kSelStage = 1024;
  __shared__ double sd[kSelStage];
  __shared__ int si[kSelStage];
  const int n = r1 - r0;
  const bool staged = n <= kSelStage;
  if (staged) {
    for (int e = threadIdx.x; e < n; e += 256) {
      const int i = pm[r0 + e];
      si[e] = i;
      sd[e] = dd[i];
    }
    __syncthreads();
  }
  for (int p = threadIdx.x; p < n; p += 256) {
    const int i = staged ? si[p] : pm[r0 + p];
    const double di = staged ? sd[p] : dd[i];
    int rank = 0;
    if (staged) {  // the members from LDS, eight at a time (broadcast reads)
#pragma unroll 8
      for (int o = 0; o < n; ++o) {
        const double dx = sd[o];
        const int io = si[o];
        rank += int(dx < di) | (int(dx == di) & int(io < i));
      }
    } else {
      for (int o = 0; o < n; ++o) {
        const int io = pm[r0 + o];
        const double dx = dd[io];
        rank += (dx < di) || (dx == di && io < i);
      }
    }
    if (rank < m) {
      probe_idx[size_t(hd) * M + po + rank] = i;
      probe_w[size_t(hd) * M + po + rank] = double(n) / double(m);
    }
  }
}

// Random and uniform probes (Table 4), one block of 1024 threads per head; weights Nv / M.
// Random: the M rows with the smallest draws splitmix64(seed ^ "probe", hd Nv + i), found by an
// 8-pass radix selection of the M-th smallest draw (8 bits per pass, most significant first);
// rows below it, and the first rows equal to it, are listed in ascending row.  Uniform: rows
// floor((2 i + 1) Nv / (2 M)).
constexpr uint64_t kProbeStream = 0x70726F6265ull;
__global__ __launch_bounds__(1024) void probe_plain_kernel(int mode, uint64_t seed, int Nv, int M,
                                                           int* __restrict__ probe_idx,
                                                           double* __restrict__ probe_w) {
  __shared__ int hist[256];
  __shared__ int buf[1024];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_need;
  const int hd = blockIdx.x, tid = threadIdx.x;
  int* out = probe_idx + size_t(hd) * M;
  double* ow = probe_w + size_t(hd) * M;
  const double wgt = double(Nv) / double(M);
  if (mode == SPR_PROBES_UNIFORM) {
    for (int i = tid; i < M; i += 1024) {
      out[i] = int((2 * int64_t(i) + 1) * Nv / (2 * int64_t(M)));
      ow[i] = wgt;
    }
    return;
  }
  const uint64_t sd = seed ^ kProbeStream, c0 = uint64_t(hd) * uint64_t(Nv);
  uint64_t prefix = 0;
  int need = M;  // rank (1-based) of the wanted draw among those matching the prefix
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t hi = pass == 0 ? 0ull : ~0ull << (shift + 8);
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < Nv; i += 1024) {
      const uint64_t k = splitmix64(sd, c0 + i);
      if ((k & hi) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, bin = 255;
      for (int b = 0; b < 256; ++b) {
        if (cum + hist[b] >= need) {
          bin = b;
          break;
        }
        cum += hist[b];
      }
      s_prefix = prefix | (uint64_t(bin) << shift);
      s_need = need - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    __syncthreads();
  }
  // prefix is the M-th smallest draw; take every smaller draw and the first `need` equal ones
  int base = 0, eq_seen = 0;
  for (int c = 0; c < Nv; c += 1024) {
    const int i = c + tid;
    uint64_t k = ~0ull;
    if (i < Nv) k = splitmix64(sd, c0 + i);
    const bool lt = i < Nv && k < prefix, eq = i < Nv && k == prefix;
    int n_eq;
    const int r_eq = block_exscan_i(eq ? 1 : 0, buf, &n_eq);
    const bool take = lt || (eq && eq_seen + r_eq < need);
    int n_take;
    const int pos = block_exscan_i(take ? 1 : 0, buf, &n_take);
    if (take) {
      out[base + pos] = i;
      ow[base + pos] = wgt;
    }
    base += n_take;
    eq_seen += n_eq;
  }
}

template <int DT>
static spr_status route_impl(const spr_desc& desc, const spr_part_params& p, const spr_partition& part, int M,
                             int64_t Tk, const spr_probe_options& probes, spr_route& out, void* ws,
                             const Workspace& L, hipStream_t st) {
  const int BH = desc.B * desc.H, d = desc.d, N = desc.N, Nv = N - desc.n_text;
  const int G = kv_group_size(desc), BHkv = BH / G;
  double* vstat = ws_ptr<double>(ws, L.vstat);
  double* shift = ws_ptr<double>(ws, L.shift);
  double* scores = out.scores ? out.scores : ws_ptr<double>(ws, L.scores);
  int* gstat = ws_ptr<int>(ws, L.gstat);
  int* pstat = ws_ptr<int>(ws, L.pstat);
  hipLaunchKernelGGL(vstat_kernel<DT>, dim3(ceil_div(Nv, 256 / (d / 8)), BHkv), dim3(256), 0, st, part.Vp, N, Nv, d,
                     part.kv_perm, part.kv_label, part.vbar, p.Ck, vstat);
  double* lbar = ws_ptr<double>(ws, L.lbar);
  const dim3 lgrid(ceil_div(p.Cq, 64), ceil_div(p.Ck, 64), BH), sgrid(ceil_div(p.Cq, 64), ceil_div(p.Ck, 16), BH);
  if (d == 128) {
    allow_lds(centroid_logits_kernel<128>, centroid_logits_smem<128>());
    hipLaunchKernelGGL(centroid_logits_kernel<128>, lgrid, dim3(256), centroid_logits_smem<128>(), st, part.qbar,
                       part.kbar, part.n_q, part.n_kv, p.Cq, p.Ck, G, lbar);
  } else {
    hipLaunchKernelGGL(centroid_logits_kernel<64>, lgrid, dim3(256), centroid_logits_smem<64>(), st, part.qbar,
                       part.kbar, part.n_q, part.n_kv, p.Cq, p.Ck, G, lbar);
  }
  hipLaunchKernelGGL(logit_shift_kernel, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, lbar, part.n_q, part.n_kv,
                     p.Cq, p.Ck, G, shift);
  hipLaunchKernelGGL(zero_i64_kernel, dim3(ceil_div(BH, 256)), dim3(256), 0, st, out.pairs, BH);
  const dim3 grid(ceil_div(p.Cq + 1, 4), BH);
  if constexpr (DT == SPR_BF16) {
    // bf16 keys: scores on the bf16 matrix cores with bounds, fp64 where the selection needs it
    double* serr = out.score_err ? out.score_err : ws_ptr<double>(ws, L.serr);
    const unsigned nblk = unsigned(route_fast_blocks(p.Cq, p.Ck, BH));
    __bf16* qsplit = ws_ptr<__bf16>(ws, L.qsplit);
    double* qnorm = ws_ptr<double>(ws, L.qnorm);
    if (d == 128)
      hipLaunchKernelGGL(qbar_split_kernel<128>, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, part.qbar, part.n_q,
                         p.Cq, qsplit, qnorm);
    else
      hipLaunchKernelGGL(qbar_split_kernel<64>, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, part.qbar, part.n_q,
                         p.Cq, qsplit, qnorm);
    auto fast = [&](auto kern, size_t smem) {
      allow_lds(kern, smem);
      hipLaunchKernelGGL(kern, dim3(nblk), dim3(kFastWaves * 64), smem, st, static_cast<const uint16_t*>(part.Kp), N, Nv,
                         qsplit, qnorm, lbar, part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, G, BH, shift,
                         vstat, scores, serr);
    };
    if (d == 128) fast(route_score_fast_kernel<128>, route_fast_smem<128>());
    else fast(route_score_fast_kernel<64>, route_fast_smem<64>());
    SPR_CHECK_LAUNCH();
    const bool keep = out.scores || out.score_err;
    // resolve in three phases with the fp64 rescoring of the requested pairs between them
    unsigned long long* rbits = ws_ptr<unsigned long long>(ws, L.rr_bits);
    int* rorder = ws_ptr<int>(ws, L.rr_order);
    int* rnin = ws_ptr<int>(ws, L.rr_nin);
    const int W = ceil_div(p.Cq, 64);
    const int64_t nbits = int64_t(BH) * p.Ck * W;
    hipLaunchKernelGGL(zero_i64_kernel, dim3(unsigned(ceil_div64(nbits, 256))), dim3(256), 0, st,
                       reinterpret_cast<int64_t*>(rbits), int(nbits));
    auto rescore = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(p.Ck, BH), dim3(256), 0, st, rbits, part.Kp, N, Nv, part.qbar, lbar, part.vbar,
                         shift, vstat, part.kv_off, part.n_kv, p.Cq, p.Ck, G, scores, serr);
    };
    auto phases = [&](auto k0, auto k1, auto k2, auto rk) {
      auto ph = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, scores, serr, keep, part.kv_off, part.q_off, part.n_q,
                           part.n_kv, p.Cq, p.Ck, G, desc.n_text, Tk, rbits, rorder, rnin, out.sel_cnt, out.sel_kv,
                           out.pairs, gstat);
      };
      ph(k0);
      rescore(rk);
      ph(k1);
      rescore(rk);
      ph(k2);
    };
#define SPR_RESOLVE(E, D)                                                                                 \
  phases(route_resolve_kernel<0, E, D>, route_resolve_kernel<1, E, D>, route_resolve_kernel<2, E, D>, \
         route_rescore_kernel<D>)
    if (d == 128) {
      if (p.Ck <= 64) SPR_RESOLVE(1, 128);
      else if (p.Ck <= 128) SPR_RESOLVE(2, 128);
      else if (p.Ck <= 256) SPR_RESOLVE(4, 128);
      else if (p.Ck <= 512) SPR_RESOLVE(8, 128);
      else SPR_RESOLVE(16, 128);
    } else {
      if (p.Ck <= 64) SPR_RESOLVE(1, 64);
      else if (p.Ck <= 128) SPR_RESOLVE(2, 64);
      else if (p.Ck <= 256) SPR_RESOLVE(4, 64);
      else if (p.Ck <= 512) SPR_RESOLVE(8, 64);
      else SPR_RESOLVE(16, 64);
    }
#undef SPR_RESOLVE
  } else {
    if (d == 128) {
      allow_lds(route_score_kernel<DT, 128>, route_score_smem<128>());
      hipLaunchKernelGGL((route_score_kernel<DT, 128>), sgrid, dim3(256), route_score_smem<128>(), st, part.Kp, N,
                         Nv, part.qbar, lbar, part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, G, shift, vstat,
                         scores);
    } else {
      allow_lds(route_score_kernel<DT, 64>, route_score_smem<64>());
      hipLaunchKernelGGL((route_score_kernel<DT, 64>), sgrid, dim3(256), route_score_smem<64>(), st, part.Kp, N,
                         Nv, part.qbar, lbar, part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, G, shift, vstat,
                         scores);
    }
    if (out.score_err) {
      const int64_t n = int64_t(BH) * p.Cq * p.Ck;
      hipLaunchKernelGGL(zero_i64_kernel, dim3(unsigned(ceil_div64(n, 256))), dim3(256), 0, st,
                         reinterpret_cast<int64_t*>(out.score_err), int(n));
    }
    SPR_CHECK_LAUNCH();
    auto sel = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, scores, part.kv_off, part.q_off, part.n_q, part.n_kv, p.Cq,
                         p.Ck, G, desc.n_text, Tk, out.sel_cnt, out.sel_kv, out.pairs, gstat);
    };
    if (p.Ck <= 64) sel(route_select_kernel<1>);
    else if (p.Ck <= 128) sel(route_select_kernel<2>);
    else if (p.Ck <= 256) sel(route_select_kernel<4>);
    else if (p.Ck <= 512) sel(route_select_kernel<8>);
    else sel(route_select_kernel<16>);
  }
  SPR_CHECK_LAUNCH();
  hipLaunchKernelGGL(route_finalize_kernel, dim3(BH), dim3(1024), 0, st, part.q_off, part.n_q, p.Cq, N, Nv,
                     desc.n_text, M, out.pairs, out.rho_exec, pstat);
  if (probes.mode == SPR_PROBES_STRATIFIED)
    hipLaunchKernelGGL(probe_select_kernel, dim3(p.Cq, BH), dim3(256), 0, st, part.q_off, part.q_perm, part.n_q,
                       part.qdist, pstat, p.Cq, Nv, M, out.probe_idx, out.probe_w);
  else
    hipLaunchKernelGGL(probe_plain_kernel, dim3(BH), dim3(1024), 0, st, probes.mode, probes.seed, Nv, M,
                       out.probe_idx, out.probe_w);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_route(const spr_desc& desc, const spr_part_params& p, const spr_partition& part, double rho, int M,
                     int64_t Tk, const spr_probe_options& probes, spr_route& out, void* ws, const Workspace& L,
                     hipStream_t st) {
  (void)rho;
  if (desc.dtype == SPR_BF16) return route_impl<SPR_BF16>(desc, p, part, M, Tk, probes, out, ws, L, st);
  return route_impl<SPR_F32>(desc, p, part, M, Tk, probes, out, ws, L, st);
}

}  // namespace spr
