// Flash-style attention kernels for the SparsePR operator on gfx950.
//
//  - block-sparse (Eq. (2) of "Partition the Support, Reconstruct the Residual", Sec. 3;
//    execution as in Sec. 4.3): one block per 64-row tile of a query group, keys streamed
//    from the concatenation of the group's selected K/V groups (ragged lengths, only the
//    last 64-key chunk is partial), row-wise renormalised online softmax;
//  - dense (Eq. (1)): the same kernel over one segment holding every key;
//  - probe rows (Sec. 4.2): gathered query rows against a contiguous key range (split-K),
//    partial (max, sum, unnormalised output) merged by a second kernel.
//
// bf16 inputs use MFMA: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (exact products, fp32
// sums), P rounded to fp16 and O^T += V^T P^T with v_mfma_f32_16x16x32_f16 (V converted from
// bf16 to fp16 while it is staged, transposed, into LDS).  Computing the transposes puts a
// query row's scores and its output columns in the same lane, so the softmax rescaling needs
// no cross-lane traffic.  fp32 inputs use a plain VALU kernel.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum { MODE_SPARSE = 0, MODE_DENSE = 1, MODE_PROBE = 2 };

constexpr int kChunk = 64;     // keys per LDS chunk
constexpr int kTileRows = 64;  // query rows per block (4 waves x 16)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  // query rows: SPARSE -> Qp [BH][N][d]; DENSE, PROBE -> original q with geometry g
  const void* q;
  const void* k;
  const void* v;
  HeadGeom g;
  // sparse routing
  const int* tile_off;   // [BH][Cq+2]
  const int* q_off;      // [BH][Cq+1]
  const int* n_q;
  const int* n_kv;
  const int* kv_off;     // [BH][Ck+1]
  const int* sel_cnt;    // [BH][Cq+1]
  const int* sel_kv;     // [BH][Cq+1][Ck+1]
  int Cq, Ck;
  // probes
  const int* probe_idx;  // [BH][M]
  int M, splits;
  float* part;           // [BH][M][splits][d + 2]
  // outputs
  float* o_sp;           // SPARSE: [BH][N][d]
  void* out;             // DENSE: [BH][N][d] contiguous
  int out_dtype;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// ------------------------------------------------------------------ tile geometry
struct TileInfo {
  int hd;
  int row0, nrows;  // rows [row0, row0 + nrows) of the query source (SPARSE / DENSE)
  int a;            // query group (SPARSE); probe tile base (PROBE)
  int key0, key1;   // DENSE / PROBE key range
  int split;
  bool valid;
};

template <int MODE>
__device__ inline TileInfo decode_tile(const AttnParams& P) {
  TileInfo t;
  t.hd = blockIdx.y;
  t.valid = true;
  t.split = 0;
  t.key0 = 0;
  t.key1 = P.g.N;
  t.a = 0;
  if constexpr (MODE == MODE_SPARSE) {
    const int hd = t.hd;
    const int nq = P.n_q[hd];
    const int ngt = nq + (P.g.n_text > 0 ? 1 : 0);
    const int* to = P.tile_off + size_t(hd) * (P.Cq + 2);
    const int tid = blockIdx.x;
    if (tid >= to[ngt]) {
      t.valid = false;
      return t;
    }
    int lo = 0, hi = ngt - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (to[mid] <= tid) lo = mid; else hi = mid - 1;
    }
    t.a = lo;
    const int ti = tid - to[lo];
    int g0, g1;
    if (lo < nq) {
      g0 = P.q_off[size_t(hd) * (P.Cq + 1) + lo];
      g1 = P.q_off[size_t(hd) * (P.Cq + 1) + lo + 1];
    } else {
      g0 = P.g.Nv;
      g1 = P.g.N;
    }
    t.row0 = g0 + ti * kTileRows;
    t.nrows = min(kTileRows, g1 - t.row0);
  } else if constexpr (MODE == MODE_DENSE) {
    t.row0 = blockIdx.x * kTileRows;
    t.nrows = min(kTileRows, P.g.N - t.row0);
  } else {
    t.row0 = blockIdx.x * kTileRows;  // probe slots
    t.nrows = min(kTileRows, P.M - t.row0);
    t.split = blockIdx.z;
    const int64_t N = P.g.N;
    t.key0 = int(N * t.split / P.splits);
    t.key1 = int(N * (t.split + 1) / P.splits);
  }
  return t;
}

// Build the segment table (start row and cumulative length) of a sparse tile's keys.
// Returns the total number of keys.
__device__ inline int build_segments(const AttnParams& P, const TileInfo& t, int* seg_start, int* seg_cum,
                                     int* scan) {
  const int hd = t.hd;
  const int cnt = P.sel_cnt[size_t(hd) * (P.Cq + 1) + t.a];
  const int* sel = P.sel_kv + (size_t(hd) * (P.Cq + 1) + t.a) * (P.Ck + 1);
  const int* off = P.kv_off + size_t(hd) * (P.Ck + 1);
  const int nkv = P.n_kv[hd];
  const int per = (cnt + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * per;
  int local = 0;
  for (int i = i0; i < min(i0 + per, cnt); ++i) {
    const int b = sel[i];
    int s, l;
    if (b < nkv) {
      s = off[b];
      l = off[b + 1] - s;
    } else {
      s = P.g.Nv;
      l = P.g.n_text;
    }
    seg_start[i] = s;
    seg_cum[i] = l;  // temporarily the length
    local += l;
  }
  int total;
  int run = block_exscan_i(local, scan, &total);
  for (int i = i0; i < min(i0 + per, cnt); ++i) {
    const int l = seg_cum[i];
    seg_cum[i] = run;
    run += l;
  }
  if (threadIdx.x == 0) seg_cum[cnt] = total;
  __syncthreads();
  return total;
}

__device__ __forceinline__ int seg_row(const int* seg_start, const int* seg_cum, int cnt, int pos) {
  int lo = 0, hi = cnt - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_cum[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return seg_start[lo] + (pos - seg_cum[lo]);
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int D, int MODE>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnParams P) {
  constexpr int KS = D + 8;   // Ks row stride (bf16 elements)
  constexpr int VS = kChunk + 4;  // Vt row stride (fp16 elements)
  constexpr int NT = D / 16;
  constexpr int KSTEPS = D / 32;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem_raw);
  _Float16* Vt = reinterpret_cast<_Float16*>(smem_raw + kChunk * KS * 2);
  int* rowidx = reinterpret_cast<int*>(smem_raw + kChunk * KS * 2 + D * VS * 2);
  int* seg_start = rowidx + kChunk;
  int* seg_cum = seg_start + (MODE == MODE_SPARSE ? 1040 : 0);
  int* scan = seg_cum + (MODE == MODE_SPARSE ? 1040 : 0);

  const TileInfo t = decode_tile<MODE>(P);
  if (!t.valid || t.nrows <= 0) return;
  const int hd = t.hd;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  // key source
  const uint16_t* Kb;
  const uint16_t* Vb;
  int64_t krs;  // key row stride (elements)
  if constexpr (MODE == MODE_SPARSE) {
    Kb = static_cast<const uint16_t*>(P.k) + size_t(hd) * P.g.N * D;
    Vb = static_cast<const uint16_t*>(P.v) + size_t(hd) * P.g.N * D;
    krs = D;
  } else {
    Kb = static_cast<const uint16_t*>(P.k) + P.g.base(hd);
    Vb = static_cast<const uint16_t*>(P.v) + P.g.base(hd);
    krs = P.g.sn;
  }
  int nseg = 0, total;
  if constexpr (MODE == MODE_SPARSE) {
    nseg = P.sel_cnt[size_t(hd) * (P.Cq + 1) + t.a];
    total = build_segments(P, t, seg_start, seg_cum, scan);
  } else {
    total = t.key1 - t.key0;
  }

  // query fragments: lane holds row r16 of this wave's 16 rows, dims ks*32 + 8g .. +7
  const int qslot = w * 16 + r16;
  const bool qvalid = qslot < t.nrows;
  bf16x8_t qf[KSTEPS];
  {
    const uint16_t* qrow = nullptr;
    if (qvalid) {
      if constexpr (MODE == MODE_SPARSE) {
        qrow = static_cast<const uint16_t*>(P.q) + (size_t(hd) * P.g.N + t.row0 + qslot) * D;
      } else if constexpr (MODE == MODE_DENSE) {
        qrow = static_cast<const uint16_t*>(P.q) + P.g.base(hd) + int64_t(t.row0 + qslot) * P.g.sn;
      } else {
        const int pr = P.probe_idx[size_t(hd) * P.M + t.row0 + qslot];
        qrow = static_cast<const uint16_t*>(P.q) + P.g.base(hd) + int64_t(pr) * P.g.sn;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qvalid) u = *reinterpret_cast<const uint4*>(qrow + ks * 32 + 8 * g);
      qf[ks] = as_bf16x8(u);
    }
  }
  const bool wave_active = (w * 16) < t.nrows;

  const float scale = kLog2e / sqrtf(float(D));
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t oacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) oacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (total + kChunk - 1) / kChunk;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int cbase = ch * kChunk;
    const int nvalid = min(kChunk, total - cbase);
    if (threadIdx.x < kChunk) {
      int row = -1;
      if (int(threadIdx.x) < nvalid) {
        if constexpr (MODE == MODE_SPARSE) row = seg_row(seg_start, seg_cum, nseg, cbase + threadIdx.x);
        else row = t.key0 + cbase + threadIdx.x;
      }
      rowidx[threadIdx.x] = row;
    }
    __syncthreads();
    // K chunk: 64 rows x D bf16, 16-byte pieces
    for (int e = threadIdx.x; e < kChunk * (D / 8); e += 256) {
      const int rr = e / (D / 8), cp = e % (D / 8);
      const int row = rowidx[rr];
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row >= 0) u = *reinterpret_cast<const uint4*>(Kb + int64_t(row) * krs + cp * 8);
      *reinterpret_cast<uint4*>(Ks + rr * KS + cp * 8) = u;
    }
    // V chunk, transposed and converted to fp16: 4 keys x 8 columns per item
    for (int e = threadIdx.x; e < (kChunk / 4) * (D / 8); e += 256) {
      const int kq = e % (kChunk / 4), dq = e / (kChunk / 4);
      _Float16 vv[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rowidx[kq * 4 + i];
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row >= 0) u = *reinterpret_cast<const uint4*>(Vb + int64_t(row) * krs + dq * 8);
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vv[i][2 * c] = _Float16(__uint_as_float(wv[c] << 16));
          vv[i][2 * c + 1] = _Float16(__uint_as_float(wv[c] & 0xFFFF0000u));
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f16x4_t pk = {vv[0][c], vv[1][c], vv[2][c], vv[3][c]};
        *reinterpret_cast<f16x4_t*>(Vt + (dq * 8 + c) * VS + kq * 4) = pk;
      }
    }
    __syncthreads();
    if (wave_active) {
      // S^T tiles: 4 x (16 keys x 16 rows)
      f32x4_t s[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const uint4 u = *reinterpret_cast<const uint4*>(Ks + (mt * 16 + r16) * KS + ks * 32 + 8 * g);
          s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u), qf[ks], s[mt], 0, 0, 0);
        }
      }
      // online softmax for row r16; this lane holds keys mt*16 + 4g + v
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = mt * 16 + 4 * g + v;
          const float x = key < nvalid ? s[mt][v] * scale : -INFINITY;
          s[mt][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float ls = 0.f;
      f16x8_t pf[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float pv = exp2f(s[mt][v] - m_new);
          ls += pv;
          pf[mt >> 1][(mt & 1) * 4 + v] = _Float16(pv);
        }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[nt] *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const _Float16* vrow = Vt + (nt * 16 + r16) * VS + h * 32 + 4 * g;
          const f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vrow);
          const f16x4_t hi = *reinterpret_cast<const f16x4_t*>(vrow + 16);
          const f16x8_t av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf[h], oacc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  if (!qvalid) return;
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  if constexpr (MODE == MODE_PROBE) {
    float* dst = P.part + ((size_t(hd) * P.M + t.row0 + qslot) * P.splits + t.split) * (D + 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<float4*>(dst + nt * 16 + 4 * g) = make_float4(oacc[nt][0], oacc[nt][1], oacc[nt][2], oacc[nt][3]);
    if (g == 0) {
      dst[D] = m_run;
      dst[D + 1] = lt;
    }
  } else {
    const float inv = 1.f / lt;
    if constexpr (MODE == MODE_SPARSE) {
      float* dst = P.o_sp + (size_t(hd) * P.g.N + t.row0 + qslot) * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<float4*>(dst + nt * 16 + 4 * g) =
            make_float4(oacc[nt][0] * inv, oacc[nt][1] * inv, oacc[nt][2] * inv, oacc[nt][3] * inv);
    } else {
      const size_t rowbase = (size_t(hd) * P.g.N + t.row0 + qslot) * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const size_t idx = rowbase + nt * 16 + 4 * g + v;
          if (P.out_dtype == SPR_BF16) store_out<SPR_BF16>(P.out, idx, oacc[nt][v] * inv);
          else store_out<SPR_F32>(P.out, idx, oacc[nt][v] * inv);
        }
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU kernel
// One wave per 64-row tile, one lane per query row; keys are read by all lanes at once.
template <int D, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams P) {
  __shared__ int seg_start[1040], seg_cum[1040], scan[1024];
  const TileInfo t = decode_tile<MODE>(P);
  if (!t.valid || t.nrows <= 0) return;
  const int hd = t.hd, lane = threadIdx.x;
  const float* Kb;
  const float* Vb;
  int64_t krs;
  if constexpr (MODE == MODE_SPARSE) {
    Kb = static_cast<const float*>(P.k) + size_t(hd) * P.g.N * D;
    Vb = static_cast<const float*>(P.v) + size_t(hd) * P.g.N * D;
    krs = D;
  } else {
    Kb = static_cast<const float*>(P.k) + P.g.base(hd);
    Vb = static_cast<const float*>(P.v) + P.g.base(hd);
    krs = P.g.sn;
  }
  int nseg = 0, total;
  if constexpr (MODE == MODE_SPARSE) {
    nseg = P.sel_cnt[size_t(hd) * (P.Cq + 1) + t.a];
    total = build_segments(P, t, seg_start, seg_cum, scan);
  } else {
    total = t.key1 - t.key0;
  }
  const bool valid = lane < t.nrows;
  float qv[D];
  {
    const float* qrow = nullptr;
    if (valid) {
      if constexpr (MODE == MODE_SPARSE) {
        qrow = static_cast<const float*>(P.q) + (size_t(hd) * P.g.N + t.row0 + lane) * D;
      } else if constexpr (MODE == MODE_DENSE) {
        qrow = static_cast<const float*>(P.q) + P.g.base(hd) + int64_t(t.row0 + lane) * P.g.sn;
      } else {
        const int pr = P.probe_idx[size_t(hd) * P.M + t.row0 + lane];
        qrow = static_cast<const float*>(P.q) + P.g.base(hd) + int64_t(pr) * P.g.sn;
      }
    }
    const float sc = 1.f / sqrtf(float(D));
#pragma unroll
    for (int c = 0; c < D; ++c) qv[c] = valid ? qrow[c] * sc : 0.f;
  }
  float m = -INFINITY, l = 0.f;
  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  for (int pos = 0; pos < total; ++pos) {
    int row;
    if constexpr (MODE == MODE_SPARSE) row = seg_row(seg_start, seg_cum, nseg, pos);
    else row = t.key0 + pos;
    const float* kr = Kb + int64_t(row) * krs;
    const float* vr = Vb + int64_t(row) * krs;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) s = fmaf(qv[c], kr[c], s);
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn);
    const float p = expf(s - mn);
    l = l * al + p;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = fmaf(o[c], al, p * vr[c]);
    m = mn;
  }
  if (!valid) return;
  if constexpr (MODE == MODE_PROBE) {
    float* dst = P.part + ((size_t(hd) * P.M + t.row0 + lane) * P.splits + t.split) * (D + 2);
#pragma unroll
    for (int c = 0; c < D; ++c) dst[c] = o[c];
    dst[D] = m * kLog2e;  // partials carry the max in log2 units like the MFMA kernel
    dst[D + 1] = l;
  } else if constexpr (MODE == MODE_SPARSE) {
    float* dst = P.o_sp + (size_t(hd) * P.g.N + t.row0 + lane) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) dst[c] = o[c] / l;
  } else {
    const size_t rowbase = (size_t(hd) * P.g.N + t.row0 + lane) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      if (P.out_dtype == SPR_BF16) store_out<SPR_BF16>(P.out, rowbase + c, o[c] / l);
      else store_out<SPR_F32>(P.out, rowbase + c, o[c] / l);
    }
  }
}

// Merge split-K partials: O = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m).
__global__ __launch_bounds__(256) void probe_merge_kernel(const float* __restrict__ part, int M, int splits, int D,
                                                          int BH, float* __restrict__ o_probe) {
  const int row = blockIdx.x;  // over BH * M
  if (row >= BH * M) return;
  const float* pr = part + size_t(row) * splits * (D + 2);
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, pr[s * (D + 2) + D]);
  float l = 0.f;
  for (int s = 0; s < splits; ++s) l += pr[s * (D + 2) + D + 1] * exp2f(pr[s * (D + 2) + D] - mx);
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += pr[s * (D + 2) + c] * exp2f(pr[s * (D + 2) + D] - mx);
    o_probe[size_t(row) * D + c] = acc / l;
  }
}

// ------------------------------------------------------------------ host drivers
template <int D, int MODE>
static size_t mfma_smem() {
  size_t s = size_t(kChunk) * (D + 8) * 2 + size_t(D) * (kChunk + 4) * 2 + kChunk * sizeof(int);
  if (MODE == MODE_SPARSE) s += (1040 * 2 + 1024) * sizeof(int);
  return s;
}

template <int D, int MODE>
static void launch_attn(const AttnParams& P, dim3 grid, int dtype, hipStream_t st) {
  if (dtype == SPR_BF16) {
    const size_t sm = mfma_smem<D, MODE>();
    allow_lds(attn_mfma_kernel<D, MODE>, sm);
    hipLaunchKernelGGL((attn_mfma_kernel<D, MODE>), grid, dim3(256), sm, st, P);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D, MODE>), grid, dim3(64), 0, st, P);
  }
}

template <int MODE>
static spr_status dispatch_d(const AttnParams& P, dim3 grid, int d, int dtype, hipStream_t st) {
  if (d == 128) launch_attn<128, MODE>(P, grid, dtype, st);
  else if (d == 64) launch_attn<64, MODE>(P, grid, dtype, st);
  else return SPR_EUNSUPPORTED;
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_attn_sparse(const spr_desc& desc, const spr_part_params& p, const spr_partition& part,
                           const spr_route& route, float* o_sp, void* ws, const Workspace& L, hipStream_t st) {
  (void)ws; (void)L;
  AttnParams P = {};
  P.q = part.Qp; P.k = part.Kp; P.v = part.Vp;
  P.g = make_geom(desc);
  P.tile_off = route.tile_off; P.q_off = part.q_off; P.n_q = part.n_q; P.n_kv = part.n_kv;
  P.kv_off = part.kv_off; P.sel_cnt = route.sel_cnt; P.sel_kv = route.sel_kv;
  P.Cq = p.Cq; P.Ck = p.Ck;
  P.o_sp = o_sp;
  const int Nv = desc.N - desc.n_text;
  const int max_tiles = p.Cq + ceil_div(Nv, kTileRows) + ceil_div(desc.n_text, kTileRows) + 1;
  return dispatch_d<MODE_SPARSE>(P, dim3(max_tiles, desc.B * desc.H), desc.d, desc.dtype, st);
}

spr_status run_probe_exact(const spr_desc& desc, const void* q, const void* k, const void* v, const int* probe_idx,
                           int M, float* o_probe, void* ws, const Workspace& L, hipStream_t st) {
  AttnParams P = {};
  P.q = q; P.k = k; P.v = v;
  P.g = make_geom(desc);
  P.probe_idx = probe_idx; P.M = M; P.splits = L.splits;
  P.part = ws_ptr<float>(ws, L.pr_part);
  const int BH = desc.B * desc.H;
  spr_status s = dispatch_d<MODE_PROBE>(P, dim3(ceil_div(M, kTileRows), BH, L.splits), desc.d, desc.dtype, st);
  if (s != SPR_OK) return s;
  hipLaunchKernelGGL(probe_merge_kernel, dim3(BH * M), dim3(128), 0, st, P.part, M, L.splits, desc.d, BH, o_probe);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_attn_dense(const spr_desc& desc, const void* q, const void* k, const void* v, void* out,
                          int out_dtype, hipStream_t st) {
  AttnParams P = {};
  P.q = q; P.k = k; P.v = v;
  P.g = make_geom(desc);
  P.out = out; P.out_dtype = out_dtype;
  return dispatch_d<MODE_DENSE>(P, dim3(ceil_div(desc.N, kTileRows), desc.B * desc.H), desc.d, desc.dtype, st);
}

}  // namespace spr
