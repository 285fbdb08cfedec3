// Internal helpers shared by the HIP translation units of libsparsepr.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparsepr.h"

namespace spr {

constexpr int kWave = 64;

// ----------------------------------------------------------------- element access
// bf16 values are handled as raw 16-bit patterns; widening to fp32 is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (DT == SPR_BF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

template <int DT>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float x) {
  if constexpr (DT == SPR_BF16) {
    // round to nearest even
    uint32_t u = __float_as_uint(x);
    uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    if ((u & 0x7F800000u) == 0x7F800000u) r = u;  // inf / nan pass through
    static_cast<uint16_t*>(base)[idx] = uint16_t(r >> 16);
  } else {
    static_cast<float*>(base)[idx] = x;
  }
}

// Eight consecutive elements starting at idx (a multiple of 8, 16-byte aligned rows) widened to
// fp32: one 16-byte load for bf16, two for fp32.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&x)[8]) {
  if constexpr (DT == SPR_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      x[2 * c] = __uint_as_float(w[c] << 16);
      x[2 * c + 1] = __uint_as_float(w[c] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// The same eight elements in their stored form (one 16-byte piece for bf16, two for fp32), for
// loads issued ahead of their use: widen8 turns them into fp32 once they are needed, so that the
// wait for the load falls there and not at the load.
template <int DT>
struct Raw8 {
  uint4 p[DT == SPR_BF16 ? 1 : 2];
};
template <int DT>
__device__ __forceinline__ Raw8<DT> load8_raw(const void* base, int64_t idx) {
  Raw8<DT> r;
  if constexpr (DT == SPR_BF16) {
    r.p[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  } else {
    r.p[0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
    r.p[1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx + 4);
  }
  return r;
}
template <int DT>
__device__ __forceinline__ void widen8(const Raw8<DT>& r, float (&x)[8]) {
  if constexpr (DT == SPR_BF16) {
    const uint32_t w[4] = {r.p[0].x, r.p[0].y, r.p[0].z, r.p[0].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      x[2 * c] = __uint_as_float(w[c] << 16);
      x[2 * c + 1] = __uint_as_float(w[c] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[8] = {r.p[0].x, r.p[0].y, r.p[0].z, r.p[0].w, r.p[1].x, r.p[1].y, r.p[1].z, r.p[1].w};
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = __uint_as_float(w[c]);
  }
}

template <int DT>
struct ElemSize {
  static constexpr int value = DT == SPR_BF16 ? 2 : 4;
};

// ----------------------------------------------------------------- head geometry
struct HeadGeom {
  int32_t B, H, N, Nv, d, n_text;
  int64_t sb, sh, sn;
  __host__ __device__ int64_t base(int hd) const { return int64_t(hd / H) * sb + int64_t(hd % H) * sh; }
};

inline HeadGeom make_geom(const spr_desc& d) {
  HeadGeom g;
  g.B = d.B; g.H = d.H; g.N = d.N; g.Nv = d.N - d.n_text; g.d = d.d; g.n_text = d.n_text;
  g.sb = d.sb; g.sh = d.sh; g.sn = d.sn;
  return g;
}

// Ranks of the k-means coordinates of a partition mode: raw activations have rank d.
inline int kv_coord_rank(const spr_part_params& p, int d) { return p.mode == SPR_PART_SEMANTIC ? d : p.rK; }
inline int q_coord_rank(const spr_part_params& p, int d) { return p.mode == SPR_PART_RESPONSE ? p.rQ : d; }

// Grouped-query attention: Hkv K/V heads, each shared by G = H / Hkv query heads (query head hd
// of the flattened index uses K/V head hd / G).
inline bool is_gqa(const spr_desc& d) { return d.Hkv > 0 && d.Hkv < d.H; }
inline int kv_heads(const spr_desc& d) { return is_gqa(d) ? d.Hkv : d.H; }
inline int kv_group_size(const spr_desc& d) { return d.H / kv_heads(d); }

// Geometry of k and v: Hkv heads with their own strides, or the geometry of q.
inline HeadGeom make_kv_geom(const spr_desc& d) {
  HeadGeom g = make_geom(d);
  if (is_gqa(d)) {
    g.H = d.Hkv;
    g.sb = d.ksb; g.sh = d.ksh; g.sn = d.ksn;
  }
  return g;
}

// ----------------------------------------------------------------- reductions
__device__ __forceinline__ double wave_sum_d(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max_f(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Deterministic block sum (fixed tree) of one double per thread; blockDim.x <= 1024.
__device__ inline double block_sum_d(double x, double* red /* [32] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_sum_d(x);
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    for (int i = 0; i < nw; ++i) t += red[i];
    red[0] = t;
  }
  __syncthreads();
  t = red[0];
  __syncthreads();
  return t;
}

__device__ inline int64_t block_sum_i64(int64_t x, int64_t* red /* [32] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  int64_t t = 0;
  if (threadIdx.x == 0) {
    for (int i = 0; i < nw; ++i) t += red[i];
    red[0] = t;
  }
  __syncthreads();
  t = red[0];
  __syncthreads();
  return t;
}

// Exclusive scan of one int per thread over the block (blockDim.x <= 1024); returns the
// exclusive prefix and writes the total to *total.  A scan inside each wave (lane shuffles),
// then the wave totals through buf (at least 16 entries): three barriers.
__device__ inline int block_exscan_i(int x, int* buf /* [>= 16] */, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (int(blockDim.x) + 63) >> 6;
  int incl = x;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __syncthreads();  // buf may still be read by a previous call
  if (lane == min(63, int(blockDim.x) - 1 - w * 64)) buf[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int v = buf[i];
    before += i < w ? v : 0;
    tot += v;
  }
  __syncthreads();  // buf is free again
  *total = tot;
  return before + incl - x;
}

// ----------------------------------------------------------------- SplitMix64
// Counter-based SplitMix64 (Steele, Lea & Flood 2014): output number `counter` of the
// generator seeded with `seed`.
__host__ __device__ inline uint64_t splitmix64(uint64_t seed, uint64_t counter) {
  uint64_t z = seed + (counter + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ----------------------------------------------------------------- workspace layout
// Every internal buffer of one operator invocation, as byte offsets into the caller's
// workspace.  Offsets are 256-byte aligned.
struct Workspace {
  size_t metric;     // double [BH][d][d]        M_K, later M_Q
  size_t ktilde;     // double [BH][Ck][d]       centred key centroids
  size_t phiK;       // double [BH][Nv][rK]      (unless the caller keeps them)
  size_t phiQ;       // double [BH][Nv][rQ]
  size_t km_cent;    // double [BH][Cmax][rmax]  k-means centres
  size_t km_lab;     // int    [BH][Nv]          uncompacted labels
  size_t km_region;  // k-means scratch (see kmeans_carve)
  size_t cbar;       // double [BH][Cq][rQ]      mean query coordinates c_a
  size_t vstat;      // double [BH][Nv][4]       v.vbar, |v|^2, (vbar - v).v, |vbar - v|^2 per key, Kp order
  size_t gstat;      // int    [2 BH][8]         flags per query head, then per K/V head
  size_t pstat;      // int    [BH][Cq][2]       probes per query group, prefix
  size_t shift;      // double [BH][Cq]          per-query-group exponent shift of the scores
  size_t lbar;       // double [BH][Cq][Ck]      centroid logits qbar_a . kbar_b / sqrt d
  size_t scores;     // double [BH][Cq][Ck]      (unless the caller keeps them)
  size_t serr;       // double [BH][Cq][Ck]      bounds of the bf16 scores (unless the caller keeps them)
  size_t qsplit;     // bf16   [BH][Cq][3][d]    qbar as hi, mid, lo bf16 slices (bf16 inputs)
  size_t qnorm;      // double [BH][Cq]          |qbar_a|
  size_t vh;         // fp16   [BHkv][N][d]      group-major values, scaled, in fp16 (bf16 inputs)
  size_t vamax;      // uint   [BHkv]            largest |v| per K/V head (bit pattern)
  size_t vscale;     // float  [2][BHkv]         2^e and 2^-e, the scaling of the fp16 values
  size_t pr_part;    // float  [BH][M][S][d+2]   split-K partials of the probe rows (probe call)
  size_t pr_vcopy;   // fp16 copy of v and its scales (probe call; see v_copy_bytes)
  size_t fitX;       // double [BH][M][d]        standardised probe features
  size_t fitR;       // double [BH][M][d]        centred probe residuals
  size_t fitG;       // double [BH][d][d]        normal matrix
  size_t fitH;       // double [BH][d][d]        right-hand sides, then B
  size_t fitS;       // double [BH][4][d]        mu_X, sd, mu_R, weights scratch
  size_t fitW;       // double [BH][M]           unit-mean weights
  size_t applyB;     // bf16   [BH][2][d][d]     E^T = (diag(1/sd) B)^T, high then low part
  size_t applyC;     // float  [BH][d]           mu_R - (mu_X / sd) B
  size_t fitF;       // double [BH][d][d]        factor of Rb^T W Rb for the output truncation
  size_t tiles;      // int    [BH][tmax][8]     block-sparse attention tiles (two row halves each)
  size_t ntiles;     // int    [BH]              tiles used per head
  size_t tile_prefix;  // int  [BH + 1]          exclusive prefix of ntiles
  size_t rr_bits;    // u64    [BH][Ck][Cq / 64]  fp64 rescoring requests of the routing resolve
  size_t rr_order;   // int    [BH][Cq][64 E]      ranking of each query group between resolve phases
  size_t rr_nin;     // int    [BH][Cq]            prefix candidates of each query group
  size_t pair_ov;    // uint16 [BH][Cq][Cq]     shared K/V groups of two query groups' selections
  size_t sel_bits;   // uint64 [BH][Cq][16]     selections as bitmaps over K/V groups
  size_t total;
  int tmax;          // tile capacity per head
  int nblk;          // k-means assign blocks per head
  int Cmax, rmax, splits;
};

constexpr int kAssignThreads = 256;
constexpr int kHalfRows = 64;  // query rows per half of a block-sparse attention tile

// Capacity of the per-head tile list: a query group of s > kHalfRows rows takes ceil(s / 2h)
// tiles (< s / 2h + 1), smaller groups go two to a tile, text rows take ceil(n_text / 2h).
inline int sparse_tile_capacity(int Cq, int Nv, int n_text) {
  const int h2 = 2 * kHalfRows;
  return Cq + (Nv + h2 - 1) / h2 + (n_text + h2 - 1) / h2 + 1;
}
constexpr int kProbeSplits = 16;

Workspace layout(const spr_desc& desc, const spr_part_params& p, int M);

}  // namespace spr

#define SPR_CHECK_LAUNCH()                          \
  do {                                              \
    if (hipGetLastError() != hipSuccess) return SPR_EHIP; \
  } while (0)
