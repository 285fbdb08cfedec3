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
#include <type_traits>

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
  int v_f16;             // v holds fp16 values (group-major fp16 copy of the values)
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

template <int MODE, int ROWS>
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
    t.row0 = g0 + ti * ROWS;
    t.nrows = min(ROWS, g1 - t.row0);
  } else if constexpr (MODE == MODE_DENSE) {
    t.row0 = blockIdx.x * ROWS;
    t.nrows = min(ROWS, P.g.N - t.row0);
  } else {
    t.row0 = blockIdx.x * ROWS;  // probe slots
    t.nrows = min(ROWS, P.M - t.row0);
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
// WAVES waves of 16 query rows share each 64-key chunk staged in LDS (K as bf16 rows, V
// transposed to fp16).  The global loads of chunk c+1 are issued into registers before the
// MFMAs of chunk c, and the row indices of chunk c+1 are resolved meanwhile, so memory latency
// overlaps compute.  Only the final chunk is masked.  The running maximum used for the
// exponentials is raised lazily: O and l are rescaled only when a row's maximum grows by more
// than 2^8, which keeps p <= 256 (exact range in fp16) and skips most rescales.
template <int D, int MODE, int WAVES, int RS, bool VF16>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(AttnParams P) {
  constexpr int NTH = WAVES * 64;
  constexpr int ROWS = WAVES * 16 * RS;
  constexpr int KS = D + 8;       // Ks row stride (bf16 elements)
  constexpr int VS = kChunk + 8;  // Vt row stride (fp16 elements; 16-byte aligned rows)
  constexpr int NT = D / 16;
  constexpr int KSTEPS = D / 32;
  constexpr int KPIECES = kChunk * (D / 8);              // 16-byte pieces of a K chunk
  constexpr int VITEMS = (kChunk / 4) * (D / 8);         // 4 keys x 8 columns items of a V chunk
  constexpr int KPT = (KPIECES + NTH - 1) / NTH;         // per thread
  constexpr int VPT = (VITEMS + NTH - 1) / NTH;
  constexpr float kRescale = 8.0f;                       // lazy rescale threshold (log2 units)
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem_raw);
  _Float16* Vt = reinterpret_cast<_Float16*>(smem_raw + kChunk * KS * 2);
  int* rowidx = reinterpret_cast<int*>(smem_raw + kChunk * KS * 2 + D * VS * 2);  // [2][kChunk]
  int* seg_start = rowidx + 2 * kChunk;
  int* seg_cum = seg_start + (MODE == MODE_SPARSE ? 1040 : 0);
  int* scan = seg_cum + (MODE == MODE_SPARSE ? 1040 : 0);

  const TileInfo t = decode_tile<MODE, ROWS>(P);
  if (!t.valid || t.nrows <= 0) return;
  const int hd = t.hd;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  const uint16_t* Kb;
  const uint16_t* Vb;
  int64_t krs;
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
  const int nchunks = (total + kChunk - 1) / kChunk;

  // query fragments: for row-set rs the lane holds row r16 of 16 rows, dims ks*32 + 8g .. +7
  bf16x8_t qf[RS][KSTEPS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int qslot = (w * RS + rs) * 16 + r16;
    const bool qvalid = qslot < t.nrows;
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
      qf[rs][ks] = as_bf16x8(u);
    }
  }
  const bool wave_active = (w * RS * 16) < t.nrows;
  const bool set1_active = RS > 1 && (w * RS * 16 + 16) < t.nrows;

  auto key_row = [&](int pos) -> int {
    if constexpr (MODE == MODE_SPARSE) return seg_row(seg_start, seg_cum, nseg, pos);
    else return t.key0 + pos;
  };
  // row indices of chunk 0
  if (threadIdx.x < kChunk) rowidx[threadIdx.x] = int(threadIdx.x) < min(kChunk, total) ? key_row(threadIdx.x) : -1;
  __syncthreads();

  uint4 kreg[KPT];
  uint4 vreg[VPT][4];
  auto load_chunk = [&](const int* ridx) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = threadIdx.x + i * NTH;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (e < KPIECES) {
        const int row = ridx[e / (D / 8)];
        if (row >= 0) kreg[i] = *reinterpret_cast<const uint4*>(Kb + int64_t(row) * krs + (e % (D / 8)) * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = threadIdx.x + i * NTH;
#pragma unroll
      for (int j = 0; j < 4; ++j) vreg[i][j] = make_uint4(0, 0, 0, 0);
      if (e < VITEMS) {
        const int kq = e % (kChunk / 4), dq = e / (kChunk / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = ridx[kq * 4 + j];
          if (row >= 0) vreg[i][j] = *reinterpret_cast<const uint4*>(Vb + int64_t(row) * krs + dq * 8);
        }
      }
    }
  };
  // V chunk stored transposed ([column][key], fp16).  Inside each 32-key half the key k sits at
  // position 8*((k % 16) / 4) + 4*(k / 16) + k % 4, so the eight keys that lane group g feeds to
  // one P V product ({4g..4g+3} and {16+4g..16+4g+3}) are one contiguous 16-byte read.
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (e < KPIECES) *reinterpret_cast<uint4*>(Ks + (e / (D / 8)) * KS + (e % (D / 8)) * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (e < VITEMS) {
        const int kq = e % (kChunk / 4), dq = e / (kChunk / 4);
        uint32_t wv[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (VF16) {
            wv[j][0] = vreg[i][j].x; wv[j][1] = vreg[i][j].y; wv[j][2] = vreg[i][j].z; wv[j][3] = vreg[i][j].w;
          } else {
            const uint32_t src[4] = {vreg[i][j].x, vreg[i][j].y, vreg[i][j].z, vreg[i][j].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const _Float16 lo = _Float16(__uint_as_float(src[c] << 16));
              const _Float16 hi = _Float16(__uint_as_float(src[c] & 0xFFFF0000u));
              wv[j][c] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
            }
          }
        }
        const int pos = (kq / 8) * 32 + 8 * (kq % 4) + 4 * ((kq % 8) / 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // columns 2c (low halves) and 2c + 1 (high halves) of the four keys
          const uint2 lo = make_uint2(__builtin_amdgcn_perm(wv[1][c], wv[0][c], 0x05040100u),
                                      __builtin_amdgcn_perm(wv[3][c], wv[2][c], 0x05040100u));
          const uint2 hi = make_uint2(__builtin_amdgcn_perm(wv[1][c], wv[0][c], 0x07060302u),
                                      __builtin_amdgcn_perm(wv[3][c], wv[2][c], 0x07060302u));
          *reinterpret_cast<uint2*>(Vt + (dq * 8 + 2 * c) * VS + pos) = lo;
          *reinterpret_cast<uint2*>(Vt + (dq * 8 + 2 * c + 1) * VS + pos) = hi;
        }
      }
    }
  };

  const float scale = kLog2e / sqrtf(float(D));
  float m_run[RS];
  f32x4_t oacc[RS][NT], lacc[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    m_run[rs] = -INFINITY;
    lacc[rs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[rs][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const f16x8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};

  // one chunk: S^T = K Q^T, online softmax, O^T += V^T P^T; row sums come from the same fp16
  // P through an MFMA against a tile of ones.  TAIL masks keys past the end.
  auto compute_chunk = [&](auto tail_tag, int nvalid) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    f32x4_t sacc[RS][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) sacc[rs][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + (mt * 16 + r16) * KS + ks * 32 + 8 * g));
        sacc[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], sacc[0][mt], 0, 0, 0);
        if (RS > 1 && set1_active)
          sacc[RS - 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[RS - 1][ks], sacc[RS - 1][mt], 0, 0, 0);
      }
    }
    f16x8_t pf[RS][2];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      if constexpr (TAIL) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (mt * 16 + 4 * g + v >= nvalid) sacc[rs][mt][v] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(sacc[rs][0][0], sacc[rs][0][1]), fmaxf(sacc[rs][0][2], sacc[rs][0][3]));
#pragma unroll
      for (int mt = 1; mt < 4; ++mt)
        mx = fmaxf(fmaxf(mx, fmaxf(sacc[rs][mt][0], sacc[rs][mt][1])), fmaxf(sacc[rs][mt][2], sacc[rs][mt][3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= scale;
      const bool grow = mx > m_run[rs] + kRescale;
      if (__builtin_expect(__any(grow), 0)) {
        __asm__ volatile("; rare rescale of the running output" ::);
        const float m_new = grow ? mx : m_run[rs];
        const float alpha = __builtin_amdgcn_exp2f(m_run[rs] - m_new);
        m_run[rs] = m_new;
        lacc[rs] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[rs][nt] *= alpha;
      }
      const float mneg = -m_run[rs];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          pf[rs][mt >> 1][(mt & 1) * 4 + v] = _Float16(__builtin_amdgcn_exp2f(fmaf(sacc[rs][mt][v], scale, mneg)));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[0][h], lacc[0], 0, 0, 0);
      if (RS > 1 && set1_active)
        lacc[RS - 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[RS - 1][h], lacc[RS - 1], 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f16x8_t av = __builtin_bit_cast(
            f16x8_t, *reinterpret_cast<const uint4*>(Vt + (nt * 16 + r16) * VS + h * 32 + 8 * g));
        oacc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf[0][h], oacc[0][nt], 0, 0, 0);
        if (RS > 1 && set1_active)
          oacc[RS - 1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf[RS - 1][h], oacc[RS - 1][nt], 0, 0, 0);
      }
    }
  };

  if (nchunks > 0) load_chunk(rowidx);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int cbase = ch * kChunk;
    const int nvalid = min(kChunk, total - cbase);
    store_chunk();
    int* ridx_next = rowidx + ((ch + 1) & 1) * kChunk;
    if (threadIdx.x < kChunk && ch + 1 < nchunks) {
      const int pos = cbase + kChunk + threadIdx.x;
      ridx_next[threadIdx.x] = pos < total ? key_row(pos) : -1;
    }
    __syncthreads();
    if (ch + 1 < nchunks) load_chunk(ridx_next);
    if (wave_active) {
      if (__builtin_expect(nvalid == kChunk, 1)) compute_chunk(std::false_type{}, nvalid);
      else compute_chunk(std::true_type{}, nvalid);
    }
    __syncthreads();
  }
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int qslot = (w * RS + rs) * 16 + r16;
    if (qslot >= t.nrows) continue;
    const float lt = lacc[rs][0];
    if constexpr (MODE == MODE_PROBE) {
      float* dst = P.part + ((size_t(hd) * P.M + t.row0 + qslot) * P.splits + t.split) * (D + 2);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<float4*>(dst + nt * 16 + 4 * g) =
            make_float4(oacc[rs][nt][0], oacc[rs][nt][1], oacc[rs][nt][2], oacc[rs][nt][3]);
      if (g == 0) {
        dst[D] = m_run[rs];
        dst[D + 1] = lt;
      }
    } else {
      const float inv = 1.f / lt;
      if constexpr (MODE == MODE_SPARSE) {
        float* dst = P.o_sp + (size_t(hd) * P.g.N + t.row0 + qslot) * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          *reinterpret_cast<float4*>(dst + nt * 16 + 4 * g) = make_float4(
              oacc[rs][nt][0] * inv, oacc[rs][nt][1] * inv, oacc[rs][nt][2] * inv, oacc[rs][nt][3] * inv);
      } else {
        const size_t rowbase = (size_t(hd) * P.g.N + t.row0 + qslot) * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const size_t idx = rowbase + nt * 16 + 4 * g + v;
            if (P.out_dtype == SPR_BF16) store_out<SPR_BF16>(P.out, idx, oacc[rs][nt][v] * inv);
            else store_out<SPR_F32>(P.out, idx, oacc[rs][nt][v] * inv);
          }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU kernel
// One wave per 64-row tile, one lane per query row; keys are read by all lanes at once.
template <int D, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams P) {
  __shared__ int seg_start[1040], seg_cum[1040], scan[1024];
  const TileInfo t = decode_tile<MODE, kTileRows>(P);
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
  size_t s = size_t(kChunk) * (D + 8) * 2 + size_t(D) * (kChunk + 8) * 2 + 2 * kChunk * sizeof(int);
  if (MODE == MODE_SPARSE) s += (1040 * 2 + 1024) * sizeof(int);
  return s;
}

// Block shapes of the MFMA kernel: waves per block and 16-row sets per wave (a wave with two
// sets reads each K and V fragment from LDS once for 32 rows).
#ifndef SPR_SPARSE_WAVES
#define SPR_SPARSE_WAVES 4
#endif
#ifndef SPR_SPARSE_RS
#define SPR_SPARSE_RS 1
#endif
#ifndef SPR_DENSE_WAVES
#define SPR_DENSE_WAVES 8
#endif
#ifndef SPR_DENSE_RS
#define SPR_DENSE_RS 1
#endif
template <int MODE>
constexpr int mfma_waves() { return MODE == MODE_SPARSE ? SPR_SPARSE_WAVES : MODE == MODE_DENSE ? SPR_DENSE_WAVES : 4; }
template <int MODE>
constexpr int mfma_rowsets() { return MODE == MODE_SPARSE ? SPR_SPARSE_RS : MODE == MODE_DENSE ? SPR_DENSE_RS : 1; }
template <int MODE>
constexpr int mfma_rows() { return 16 * mfma_waves<MODE>() * mfma_rowsets<MODE>(); }

template <int D, int MODE>
static void launch_attn(const AttnParams& P, dim3 grid, int dtype, hipStream_t st) {
  if (dtype == SPR_BF16) {
    constexpr int W = mfma_waves<MODE>(), RS = mfma_rowsets<MODE>();
    const size_t sm = mfma_smem<D, MODE>();
    if (MODE == MODE_SPARSE && P.v_f16) {
      allow_lds(attn_mfma_kernel<D, MODE, W, RS, true>, sm);
      hipLaunchKernelGGL((attn_mfma_kernel<D, MODE, W, RS, true>), grid, dim3(W * 64), sm, st, P);
    } else {
      allow_lds(attn_mfma_kernel<D, MODE, W, RS, false>, sm);
      hipLaunchKernelGGL((attn_mfma_kernel<D, MODE, W, RS, false>), grid, dim3(W * 64), sm, st, P);
    }
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
  AttnParams P = {};
  P.q = part.Qp; P.k = part.Kp; P.v = part.Vp;
  if (desc.dtype == SPR_BF16) {
    P.v = ws_ptr<void>(ws, L.vh);
    P.v_f16 = 1;
  }
  P.g = make_geom(desc);
  P.tile_off = route.tile_off; P.q_off = part.q_off; P.n_q = part.n_q; P.n_kv = part.n_kv;
  P.kv_off = part.kv_off; P.sel_cnt = route.sel_cnt; P.sel_kv = route.sel_kv;
  P.Cq = p.Cq; P.Ck = p.Ck;
  P.o_sp = o_sp;
  const int Nv = desc.N - desc.n_text;
  const int rows = desc.dtype == SPR_BF16 ? mfma_rows<MODE_SPARSE>() : kTileRows;
  const int max_tiles = p.Cq + ceil_div(Nv, rows) + ceil_div(desc.n_text, rows) + 1;
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
  const int rows = desc.dtype == SPR_BF16 ? mfma_rows<MODE_DENSE>() : kTileRows;
  return dispatch_d<MODE_DENSE>(P, dim3(ceil_div(desc.N, rows), desc.B * desc.H), desc.d, desc.dtype, st);
}

}  // namespace spr

namespace spr {
int sparse_rows_per_block(int dtype) { return dtype == SPR_BF16 ? mfma_rows<MODE_SPARSE>() : kTileRows; }
}  // namespace spr
