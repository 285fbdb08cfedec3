// Flash-style attention kernels for the SparsePR operator on gfx950.
//
//  - block-sparse (Eq. (2) of "Partition the Support, Reconstruct the Residual", Sec. 3;
//    execution as in Sec. 4.3).  A block holds two halves of up to 64 query rows.  A query
//    group with more than 64 rows fills both halves of its blocks; smaller groups are paired,
//    and the block streams the union of the two groups' selected K/V groups (groups selected
//    by both halves first, then those of one half only), each half skipping or masking keys it
//    did not select.  Either way every K/V chunk staged in LDS serves up to 128 query rows,
//    which is what bounds the kernel: with 64 rows per fetch it is limited by the traffic of
//    re-fetching K/V, not by the MFMA pipe.
//  - dense (Eq. (1)): the same kernel over one segment holding every key;
//  - probe rows (Sec. 4.2): gathered query rows against a contiguous key range (split-K),
//    partial (max, sum, unnormalised output) merged by a second kernel.
//
// bf16 inputs use MFMA: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (exact products, fp32
// sums), P rounded to fp16 and O^T += V^T P^T with v_mfma_f32_16x16x32_f16 (V staged,
// transposed, into LDS as fp16).  Computing the transposes puts a query row's scores and its
// output columns in the same lane, so the softmax rescaling needs no cross-lane traffic.
// fp32 inputs use a plain VALU kernel.
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
constexpr int kTileRows = 64;  // query rows per block of the fp32 kernel and the probe kernel
constexpr int kSegCap = 1040;  // segment table capacity (>= Ck + 1 groups)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  // query rows: SPARSE -> Qp [BH][N][d]; DENSE, PROBE -> original q with geometry g
  const void* q;
  const void* k;
  const void* v;
  HeadGeom g;
  HeadGeom gk;             // DENSE, PROBE: geometry of k and v (K/V head hd / G of query head hd)
  int G;                   // query heads per K/V head; SPARSE: Kp, Vp, n_kv, kv_off are per K/V head
  // sparse routing
  const int* tiles;        // [BH][tmax][8]: a0, row0, n0, a1, row1, n1 (row0 / row1 index Qp rows)
  const int* ntiles;       // [BH]
  const int* tile_prefix;  // [BH + 1]: tiles of the heads before each head; [BH] = all tiles
  int tmax, BH;
  const int* n_kv;       // [BH / G]
  const int* kv_off;     // [BH / G][Ck+1]
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
  int a0, row0, n0;  // half 0 (the only half of DENSE / PROBE tiles): query group, first row, rows
  int a1, row1, n1;  // half 1 (SPARSE)
  int key0, key1;    // DENSE / PROBE key range
  int split;
  bool pair;         // SPARSE: the halves hold two different query groups
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
  t.a0 = t.a1 = 0;
  t.row1 = t.n1 = 0;
  t.pair = false;
  if constexpr (MODE == MODE_SPARSE) {
    // Workgroups reach the 8 XCDs round-robin (block L on XCD L % 8), each XCD with its own L2.
    // Block L takes tile j = L / 8 of the contiguous share of XCD L % 8 in the head-major list
    // of all tiles, so one XCD works through a few heads at a time and its concurrent tiles
    // share those heads' K/V groups in its L2.
    const int total = P.tile_prefix[P.BH];
    const int per = (total + 7) >> 3;
    const int j = int(blockIdx.x) >> 3;
    const int n = (int(blockIdx.x) & 7) * per + j;
    if (j >= per || n >= total) {
      t.valid = false;
      return t;
    }
    int lo = 0, hi = P.BH;  // last head with tile_prefix[head] <= n
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (P.tile_prefix[mid] <= n) lo = mid;
      else hi = mid;
    }
    t.hd = lo;
    const int* td = P.tiles + (size_t(t.hd) * P.tmax + (n - P.tile_prefix[lo])) * 8;
    t.a0 = td[0]; t.row0 = td[1]; t.n0 = td[2];
    t.a1 = td[3]; t.row1 = td[4]; t.n1 = td[5];
    t.pair = t.n1 > 0 && t.a1 != t.a0;
  } else if constexpr (MODE == MODE_DENSE) {
    t.row0 = blockIdx.x * ROWS;
    t.n0 = min(ROWS, P.g.N - t.row0);
  } else {
    t.row0 = blockIdx.x * ROWS;  // probe slots
    t.n0 = min(ROWS, P.M - t.row0);
    t.split = blockIdx.z;
    const int64_t N = P.g.N;
    t.key0 = int(N * t.split / P.splits);
    t.key1 = int(N * (t.split + 1) / P.splits);
  }
  return t;
}

// Length of K/V group b of a K/V head (the text group when b == n_kv) and its first row in Kp.
__device__ __forceinline__ void kv_group(const AttnParams& P, const int* off, int nkv, int b, int* s, int* l) {
  if (b < nkv) {
    *s = off[b];
    *l = off[b + 1] - off[b];
  } else {
    *s = P.g.Nv;
    *l = P.g.n_text;
  }
}

// Lengths in seg_cum[0..nseg) -> exclusive prefix, total in seg_cum[nseg]; returns the total.
__device__ inline int prefix_lengths(int* seg_cum, int nseg, int* scan) {
  const int per = (nseg + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * per;
  int local = 0;
  for (int i = i0; i < min(i0 + per, nseg); ++i) local += seg_cum[i];
  int total;
  int run = block_exscan_i(local, scan, &total);
  for (int i = i0; i < min(i0 + per, nseg); ++i) {
    const int l = seg_cum[i];
    seg_cum[i] = run;
    run += l;
  }
  if (threadIdx.x == 0) seg_cum[nseg] = total;
  __syncthreads();
  return total;
}

// Segment table of one query group's selected K/V groups, in selection order (fp32 kernel).
__device__ inline int build_segments(const AttnParams& P, int hd, int a, int* seg_start, int* seg_cum, int* scan,
                                     int* nseg) {
  const int cnt = P.sel_cnt[size_t(hd) * (P.Cq + 1) + a];
  const int* sel = P.sel_kv + (size_t(hd) * (P.Cq + 1) + a) * (P.Ck + 1);
  const int* off = P.kv_off + size_t(hd / P.G) * (P.Ck + 1);
  const int nkv = P.n_kv[hd / P.G];
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) kv_group(P, off, nkv, sel[i], seg_start + i, seg_cum + i);
  __syncthreads();
  *nseg = cnt;
  return prefix_lengths(seg_cum, cnt, scan);
}

// Segment table of a sparse tile: every K/V group selected by either half, as runs of Kp rows
// with cumulative key counts and a 2-bit mask of the halves that selected them (bit h: half h).
// Groups selected by both halves come first, then half 0 alone, then half 1 alone, each run in
// ascending group id.  Returns the total number of keys.
__device__ inline int build_union_segments(const AttnParams& P, const TileInfo& t, int* seg_start, int* seg_cum,
                                           int* seg_cat, unsigned* bm /* [2][33] */, int* scan, int* nseg_out) {
  const int hd = t.hd, hk = hd / P.G;  // query head, its K/V head
  const int nkv = P.n_kv[hk];
  const int ng = nkv + (P.g.n_text > 0 ? 1 : 0);
  for (int i = threadIdx.x; i < 66; i += blockDim.x) bm[i] = 0u;
  __syncthreads();
  const int nh = t.pair ? 2 : 1;
  for (int h = 0; h < nh; ++h) {
    const size_t row = size_t(hd) * (P.Cq + 1) + (h ? t.a1 : t.a0);
    const int cnt = P.sel_cnt[row];
    const int* sel = P.sel_kv + row * (P.Ck + 1);
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
      const int b = sel[i];
      atomicOr(bm + h * 33 + (b >> 5), 1u << (b & 31));
    }
  }
  __syncthreads();
  auto cat_of = [&](int b) -> int {
    const unsigned bit = 1u << (b & 31);
    const int in0 = (bm[b >> 5] & bit) ? 1 : 0;
    const int in1 = t.pair ? ((bm[33 + (b >> 5)] & bit) ? 1 : 0) : in0;
    return in0 | (in1 << 1);
  };
  const int per = (ng + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * per;
  int c3 = 0, c1 = 0, c2 = 0;
  for (int b = i0; b < min(i0 + per, ng); ++b) {
    const int c = cat_of(b);
    c3 += c == 3;
    c1 += c == 1;
    c2 += c == 2;
  }
  // three counts (each <= 1025) packed in 11-bit fields share one scan
  int tot;
  const int ex = block_exscan_i(c3 | (c1 << 11) | (c2 << 22), scan, &tot);
  const int n3 = tot & 0x7ff, n1 = (tot >> 11) & 0x7ff, n2 = (tot >> 22) & 0x7ff;
  int o3 = ex & 0x7ff, o1 = n3 + ((ex >> 11) & 0x7ff), o2 = n3 + n1 + ((ex >> 22) & 0x7ff);
  const int* off = P.kv_off + size_t(hk) * (P.Ck + 1);
  for (int b = i0; b < min(i0 + per, ng); ++b) {
    const int c = cat_of(b);
    if (c == 0) continue;
    const int pos = c == 3 ? o3++ : c == 1 ? o1++ : o2++;
    kv_group(P, off, nkv, b, seg_start + pos, seg_cum + pos);
    seg_cat[pos] = c;
  }
  __syncthreads();
  *nseg_out = n3 + n1 + n2;
  return prefix_lengths(seg_cum, n3 + n1 + n2, scan);
}

__device__ __forceinline__ int seg_find(const int* seg_cum, int cnt, int pos) {
  int lo = 0, hi = cnt - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_cum[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ bf16 MFMA kernel
// WAVES waves of 16 query rows share each 64-key chunk staged in LDS (K as bf16 rows, V
// transposed to fp16).  The global loads of chunk c+1 are issued into registers before the
// MFMAs of chunk c, and the rows of chunk c+1 (with, for sparse tiles, a 64-bit mask per half
// of the keys that half selected) are resolved meanwhile, so memory latency overlaps compute.
// Full chunks run unmasked, empty ones are skipped.  The running maximum used for the
// exponentials is raised lazily: O and l are rescaled only when a row's maximum grows by more
// than 2^8, which keeps p <= 256 (exact range in fp16) and skips most rescales.
template <int D, int MODE, int WAVES, bool VF16>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(AttnParams P) {
  constexpr bool SPARSE = MODE == MODE_SPARSE;
  constexpr int NTH = WAVES * 64;
  constexpr int HW = SPARSE ? WAVES / 2 : WAVES;  // waves per row half
  constexpr int ROWS = WAVES * 16;
  // LDS tiles are unpadded; 16-byte pieces are XOR-swizzled so that the fragment reads of a
  // 16-lane group (and the staging writes) touch every bank once:
  //   K  [key][D]:   piece p of row r at p ^ (r % (D / 8))
  //   V^T[col][64]:  piece p of row r at p ^ ((r / 2) % 8)   (two 128-byte rows per bank line)
  constexpr int KS = D;           // Ks row stride (bf16 elements)
  constexpr int VS = kChunk;      // Vt row stride (fp16 elements)
  constexpr int KPR = D / 8;      // 16-byte pieces per K row
  constexpr int NT = D / 16;
  constexpr int KSTEPS = D / 32;
  constexpr int KPIECES = kChunk * (D / 8);              // 16-byte pieces of a K chunk
  constexpr int VITEMS = (kChunk / 4) * (D / 8);         // 4 keys x 8 columns items of a V chunk
  // threads [0, VTH) stage V (VPT items each), threads [VTH, NTH) stage K (up to KPT pieces each)
  constexpr int VPT = (VITEMS + NTH / 2 - 1) / (NTH / 2);
  constexpr int VTH = VITEMS / VPT;
  constexpr int KPT = (KPIECES + (NTH - VTH) - 1) / (NTH - VTH);
  constexpr int KTH = KPIECES / KPT;  // threads [VTH, VTH + KTH) stage K
  constexpr int NPRE = 4 * VPT > KPT ? 4 * VPT : KPT;  // 16-byte registers per stage
  static_assert(VTH * VPT == VITEMS && VTH % 64 == 0, "staging split (V)");
  static_assert(KTH * KPT == KPIECES && KTH % 64 == 0 && VTH + KTH <= NTH, "staging split (K)");
  constexpr float kRescale = 8.0f;                       // lazy rescale threshold (log2 units)
  static_assert(!SPARSE || HW * 16 == kHalfRows, "a sparse tile half is kHalfRows rows");
  constexpr int KBUF = kChunk * KS;  // bf16 elements of one K buffer
  constexpr int VBUF = D * VS;       // fp16 elements of one V buffer
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem_raw);                    // [2][KBUF]
  _Float16* Vt = reinterpret_cast<_Float16*>(smem_raw + 2 * KBUF * 2);     // [3][VBUF]
  int* rowidx = reinterpret_cast<int*>(smem_raw + 2 * KBUF * 2 + 3 * VBUF * 2);  // [8][kChunk]
  unsigned long long* cmask = reinterpret_cast<unsigned long long*>(rowidx + 8 * kChunk);  // [8][2]
  int* seg_start = reinterpret_cast<int*>(cmask + 16);
  int* seg_cum = seg_start + (SPARSE ? kSegCap : 0);
  int* seg_cat = seg_cum + (SPARSE ? kSegCap : 0);
  unsigned* bm = reinterpret_cast<unsigned*>(seg_cat + (SPARSE ? kSegCap : 0));
  int* scan = reinterpret_cast<int*>(bm + (SPARSE ? 66 : 0));

  const TileInfo t = decode_tile<MODE, ROWS>(P);
  if (!t.valid || t.n0 <= 0) return;
  const int hd = t.hd;
  // the wave index comes from a scalar register so that every per-wave decision is a scalar branch
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int half = SPARSE ? w / HW : 0;
  const int my_row0 = half ? t.row1 : t.row0;
  const int my_n = half ? t.n1 : t.n0;
  const int qslot = (w % HW) * 16 + r16;

  // K and V rows of the head are read through buffer resources with 32-bit byte offsets (the
  // host guarantees that a head's rows span less than 2 GiB)
  const uint16_t* Kb;
  const uint16_t* Vb;
  int row_bytes;
  if constexpr (SPARSE) {
    Kb = static_cast<const uint16_t*>(P.k) + size_t(hd / P.G) * P.g.N * D;
    Vb = static_cast<const uint16_t*>(P.v) + size_t(hd / P.G) * P.g.N * D;
    row_bytes = D * 2;
  } else {
    Kb = static_cast<const uint16_t*>(P.k) + P.gk.base(hd / P.G);
    Vb = static_cast<const uint16_t*>(P.v) + P.gk.base(hd / P.G);
    row_bytes = int(P.gk.sn) * 2;
  }
  const int head_bytes = (P.g.N - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kb, (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, (short)0, head_bytes, 0x00020000);
  int nseg = 0, total;
  if constexpr (SPARSE) total = build_union_segments(P, t, seg_start, seg_cum, seg_cat, bm, scan, &nseg);
  else total = t.key1 - t.key0;
  const int nchunks = (total + kChunk - 1) / kChunk;

  // query fragments: the lane holds row r16 of the wave's 16 rows, dims ks*32 + 8g .. +7
  bf16x8_t qf[KSTEPS];
  const bool qvalid = qslot < my_n;
  {
    const uint16_t* qrow = nullptr;
    if (qvalid) {
      if constexpr (SPARSE) {
        qrow = static_cast<const uint16_t*>(P.q) + (size_t(hd) * P.g.N + my_row0 + qslot) * D;
      } else if constexpr (MODE == MODE_DENSE) {
        qrow = static_cast<const uint16_t*>(P.q) + P.g.base(hd) + int64_t(my_row0 + qslot) * P.g.sn;
      } else {
        const int pr = P.probe_idx[size_t(hd) * P.M + my_row0 + qslot];
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
  const bool wave_active = (w % HW) * 16 < my_n;

  // Wave 0: Kp rows of chunk ch and, per half, the mask of keys that half attends to (ring of 8
  // slots).  Chunks are resolved in increasing order, so the segment holding the chunk's first
  // key is carried over from the previous chunk and only the segment starts inside the chunk are
  // visited.  Keys past the end get row 0 and no mask bit.
  int seg_cursor = 0;
  auto resolve = [&](int ch) __attribute__((always_inline)) {
    const int stage = ch & 7;
    const int p0 = ch * kChunk, pos = p0 + lane;
    int row = 0, cat = 0;
    if constexpr (SPARSE) {
      int sg = seg_cursor;
      for (int k = seg_cursor + 1; k < nseg; ++k) {
        const int start = __builtin_amdgcn_readfirstlane(seg_cum[k]);
        if (start > p0 + kChunk) break;
        if (pos >= start) sg = k;
        seg_cursor = k;
      }
      if (pos < total) {
        row = seg_start[sg] + (pos - seg_cum[sg]);
        cat = seg_cat[sg];
      }
    } else {
      if (pos < total) {
        row = t.key0 + pos;
        cat = 3;
      }
    }
    rowidx[stage * kChunk + lane] = row;
    const unsigned long long m0 = __ballot(cat & 1), m1 = __ballot(cat & 2);
    if (lane == 0) {
      cmask[stage * 2] = m0;
      cmask[stage * 2 + 1] = m1;
    }
  };
  // Staging of one chunk in registers: threads [0, VTH) hold VPT V items (4 keys x 8 columns
  // each), threads [VTH, VTH + KTH) hold KPT 16-byte pieces of K.  Two register sets and two LDS buffers
  // pipeline the chunks: while chunk c is computed, chunk c+1 sits in LDS and chunks c+2, c+3
  // are in flight.
  const bool stages_v = w * 64 < VTH;
  const int sidx = stages_v ? threadIdx.x : threadIdx.x - VTH;
  const bool stages_k = !stages_v && w * 64 - VTH < KTH;
  uint4 pre0[NPRE], pre1[NPRE];
  // Every thread issues exactly NPRE loads per chunk from straight-line code (no branch between
  // the loads of the two roles, which would make the loads of a set wait for each other): load
  // i reads row slot lslot[i] of the chunk at byte column lcol[i] through the wave's descriptor.
  // Roles with fewer pieces, and idle threads, load row slot 0 again.
  int lslot[NPRE], lcol[NPRE];
#pragma unroll
  for (int i = 0; i < NPRE; ++i) {
    if (stages_v) {
      const int e = sidx + (i / 4 < VPT ? i / 4 : 0) * VTH;
      lslot[i] = (e % (kChunk / 4)) * 4 + (i & 3);
      lcol[i] = (e / (kChunk / 4)) * 16;
    } else {
      const int e = stages_k ? sidx + (i < KPT ? i : 0) * KTH : 0;
      lslot[i] = e / KPR;
      lcol[i] = (e % KPR) * 16;
    }
  }
  const __amdgpu_buffer_rsrc_t lrsrc = stages_v ? vrsrc : krsrc;
  auto load_into = [&](uint4 (&pre)[NPRE], int ch) __attribute__((always_inline)) {
    const int* ridx = rowidx + (ch & 7) * kChunk;
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
      pre[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lrsrc, ridx[lslot[i]] * row_bytes + lcol[i], 0, 0));
  };
  // V chunk stored transposed ([column][key], fp16).  Inside each 32-key half the key k sits at
  // position 8*((k % 16) / 4) + 4*(k / 16) + k % 4, so the eight keys that lane group g feeds to
  // one P V product ({4g..4g+3} and {16+4g..16+4g+3}) are one contiguous 16-byte read.
  auto store_out_of = [&](const uint4 (&pre)[NPRE], int kbuf, int vbuf) __attribute__((always_inline)) {
    if (stages_v) {
      _Float16* V = Vt + vbuf * VBUF;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int e = sidx + i * VTH;
        const int kq = e % (kChunk / 4), dq = e / (kChunk / 4);
        uint32_t wv[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 u = pre[4 * i + j];
          if constexpr (VF16) {
            wv[j][0] = u.x; wv[j][1] = u.y; wv[j][2] = u.z; wv[j][3] = u.w;
          } else {
            const uint32_t src[4] = {u.x, u.y, u.z, u.w};
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
          // rows 2c and 2c + 1 (relative to dq * 8) share one swizzle
          const int row = dq * 8 + 2 * c;
          const int at = ((pos >> 3) ^ ((row >> 1) & 7)) * 8 + (pos & 7);
          *reinterpret_cast<uint2*>(V + row * VS + at) = lo;
          *reinterpret_cast<uint2*>(V + (row + 1) * VS + at) = hi;
        }
      }
    } else if (stages_k) {
      uint16_t* K = Ks + kbuf * KBUF;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int e = sidx + i * KTH;
        const int row = e / KPR;
        *reinterpret_cast<uint4*>(K + row * KS + ((e % KPR) ^ (row % KPR)) * 8) = pre[i];
      }
    }
  };

  auto load_to = [&](auto set, int ch) __attribute__((always_inline)) {
    if constexpr (decltype(set)::value) load_into(pre1, ch);
    else load_into(pre0, ch);
  };
  auto store_from = [&](auto set, int kbuf, int vbuf) __attribute__((always_inline)) {
    if constexpr (decltype(set)::value) store_out_of(pre1, kbuf, vbuf);
    else store_out_of(pre0, kbuf, vbuf);
  };

  const float scale = kLog2e / sqrtf(float(D));
  float m_run = -INFINITY;
  f32x4_t oacc[NT], lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) oacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f16x8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};

  // S^T = K Q^T of one chunk
  auto qk = [&](f32x4_t (&sacc)[4], int kbuf) __attribute__((always_inline)) {
    const uint16_t* K = Ks + kbuf * KBUF;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int row = mt * 16 + r16;
        const bf16x8_t kf = as_bf16x8(
            *reinterpret_cast<const uint4*>(K + row * KS + (((ks * 4 + g) ^ (row % KPR)) * 8)));
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
      }
    }
  };
  // Keys whose bit in m is clear get the score -inf (partial chunks only: tails and the seams
  // between the runs of a paired tile).
  auto apply_mask = [&](f32x4_t (&sacc)[4], unsigned long long m) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (!((m >> (mt * 16 + 4 * g + v)) & 1ull)) sacc[mt][v] = -INFINITY;
  };
  // Online softmax of one chunk's scores and O^T += V^T P^T; the row sums come from the same
  // fp16 P through an MFMA against a tile of ones.  P is formed with the running shift first; if
  // any p of the wave exceeds 2^8 (tested on the bit patterns, which order non-negative floats
  // and put inf and NaN above every finite value) the rare path forms the row maxima over the
  // four lanes of each row, raises the shift where it grew by more than 2^8, rescales O and l,
  // and forms P again.
  auto exps = [&](const f32x4_t (&sacc)[4], float (&pv)[16]) __attribute__((always_inline)) {
    const float mneg = -m_run;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) pv[mt * 4 + v] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][v], scale, mneg));
  };
  auto finish_pv = [&](const f32x4_t (&sacc)[4], float (&pv)[16], int vbuf, auto&& mid) __attribute__((always_inline)) {
    const _Float16* V = Vt + vbuf * VBUF;
    unsigned big = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) big = max(big, __float_as_uint(pv[i]));
    if (__builtin_expect(__any(big > 0x43800000u), 0)) {
      __asm__ volatile("; rare rescale of the running output" ::);
      float mx = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3]));
#pragma unroll
      for (int mt = 1; mt < 4; ++mt)
        mx = fmaxf(fmaxf(mx, fmaxf(sacc[mt][0], sacc[mt][1])), fmaxf(sacc[mt][2], sacc[mt][3]));
      mx *= scale;
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool grow = mx > m_run + kRescale;
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[nt] *= alpha;
      exps(sacc, pv);
    }
    f16x8_t pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = _Float16(pv[i]);
#pragma unroll
    for (int h = 0; h < 2; ++h) lacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[h], lacc, 0, 0, 0);
    mid();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f16x8_t av = __builtin_bit_cast(
            f16x8_t, *reinterpret_cast<const uint4*>(V + (nt * 16 + r16) * VS +
                                                      (((4 * h + g) ^ (((nt * 16 + r16) >> 1) & 7)) * 8)));
        oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf[h], oacc[nt], 0, 0, 0);
      }
    }
  };
  auto softmax_pv = [&](f32x4_t (&sacc)[4], int vbuf, auto&& mid) __attribute__((always_inline)) {
    float pv[16];
    exps(sacc, pv);
    finish_pv(sacc, pv, vbuf, mid);
  };
  // The scores of the next chunk on the matrix cores interleaved with the exponentials of this
  // chunk on the vector ALU (one K fragment read, one MFMA and two VALU operations per slot).
  auto qk_exps = [&](f32x4_t (&s_nxt)[4], int kbuf, const f32x4_t (&s_cur)[4], float (&pv)[16])
                     __attribute__((always_inline)) {
    qk(s_nxt, kbuf);
    exps(s_cur, pv);
    constexpr int AHEAD = 4;  // K fragment reads issued ahead of their MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < 4 * KSTEPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      if (i + AHEAD < 4 * KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
  };
  auto half_mask = [&](int c) __attribute__((always_inline)) -> unsigned long long {
    const unsigned long long mk = cmask[(c & 7) * 2 + half];
    const unsigned lo = __builtin_amdgcn_readfirstlane(unsigned(mk));
    const unsigned hi = __builtin_amdgcn_readfirstlane(unsigned(mk >> 32));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
  };

  // Pipeline over 64-key chunks.  Chunk x is staged in register set x & 1, then in K buffer
  // x & 1 and V buffer x % 3.  Step c computes the scores of chunk c+1 and the softmax and PV
  // product of chunk c (whose scores step c-1 computed), stores chunk c+2 into LDS, issues the
  // loads of chunk c+4 and resolves the rows of chunk c+5.  Loads, stores and row resolution
  // run for chunks past the end too (rows clamp to 0, masks are empty), so no branch skips a
  // load and every step keeps the same number of loads in flight.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (w == 0)
    for (int c = 0; c < 5; ++c) resolve(c);
  __syncthreads();
  load_to(S0{}, 0);
  load_to(S1{}, 1);
  store_from(S0{}, 0, 0);
  load_to(S0{}, 2);
  store_from(S1{}, 1, 1);
  load_to(S1{}, 3);
  __syncthreads();
  f32x4_t sa[4], sb[4];
  if (wave_active && half_mask(0) != 0ull) qk(sa, 0);
  __syncthreads();  // step 0 overwrites K buffer 0
  // The LDS staging of chunk c+2 runs inside the P V products of chunk c (its VALU and LDS
  // writes issue while the matrix cores work); the loads of chunk c+4 reuse its registers after.
  auto step = [&](auto set, int c, f32x4_t (&s_cur)[4], f32x4_t (&s_nxt)[4]) __attribute__((always_inline)) {
    auto stage = [&]() __attribute__((always_inline)) { store_from(set, c & 1, (c + 2) % 3); };
    // the dense and probe kernels convert V while staging, which needs the registers the
    // overlap would take: they stage first
    constexpr bool kLate = SPARSE;
    if constexpr (!kLate) {
      stage();
      load_to(set, c + 4);
    }
    auto mid = [&]() __attribute__((always_inline)) {
      if constexpr (kLate) stage();
    };
    if (w == 0) resolve(c + 5);
    bool staged = !kLate;
    if (wave_active) {
      const unsigned long long mn = half_mask(c + 1), m = half_mask(c);
      if (__builtin_expect(m != ~0ull, 0) && m != 0ull) apply_mask(s_cur, m);
      if (__builtin_expect(mn != 0ull && m != 0ull, 1)) {
        float pv[16];
        qk_exps(s_nxt, (c + 1) & 1, s_cur, pv);
        finish_pv(s_cur, pv, c % 3, mid);
        staged = true;
      } else if (mn != 0ull) {
        qk(s_nxt, (c + 1) & 1);
      } else if (m != 0ull) {
        softmax_pv(s_cur, c % 3, mid);
        staged = true;
      }
    }
    if constexpr (kLate) {
      if (!staged) stage();
      load_to(set, c + 4);
    }
    __syncthreads();
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(S0{}, c, sa, sb);
    step(S1{}, c + 1, sb, sa);
  }
  if (!qvalid) return;
  const float lt = lacc[0];
  if constexpr (MODE == MODE_PROBE) {
    float* dst = P.part + ((size_t(hd) * P.M + my_row0 + qslot) * P.splits + t.split) * (D + 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<float4*>(dst + nt * 16 + 4 * g) = make_float4(oacc[nt][0], oacc[nt][1], oacc[nt][2], oacc[nt][3]);
    if (g == 0) {
      dst[D] = m_run;
      dst[D + 1] = lt;
    }
  } else {
    const float inv = 1.f / lt;
    if constexpr (SPARSE) {
      float* dst = P.o_sp + (size_t(hd) * P.g.N + my_row0 + qslot) * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<float4*>(dst + nt * 16 + 4 * g) =
            make_float4(oacc[nt][0] * inv, oacc[nt][1] * inv, oacc[nt][2] * inv, oacc[nt][3] * inv);
    } else {
      const size_t rowbase = (size_t(hd) * P.g.N + my_row0 + qslot) * D;
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
// One wave per 64-row tile (for sparse tiles: one half of a tile), one lane per query row;
// keys are read by all lanes at once.
template <int D, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams P) {
  __shared__ int seg_start[kSegCap], seg_cum[kSegCap], scan[64];
  TileInfo t;
  int a = 0;
  if constexpr (MODE == MODE_SPARSE) {
    t.hd = blockIdx.y;
    t.key0 = 0;
    const int tile = blockIdx.x >> 1, half = blockIdx.x & 1;
    if (tile >= P.ntiles[t.hd]) return;
    const int* td = P.tiles + (size_t(t.hd) * P.tmax + tile) * 8 + 3 * half;
    a = td[0];
    t.row0 = td[1];
    t.n0 = td[2];
  } else {
    t = decode_tile<MODE, kTileRows>(P);
  }
  if (t.n0 <= 0) return;
  const int hd = t.hd, lane = threadIdx.x;
  const float* Kb;
  const float* Vb;
  int64_t krs;
  if constexpr (MODE == MODE_SPARSE) {
    Kb = static_cast<const float*>(P.k) + size_t(hd / P.G) * P.g.N * D;
    Vb = static_cast<const float*>(P.v) + size_t(hd / P.G) * P.g.N * D;
    krs = D;
  } else {
    Kb = static_cast<const float*>(P.k) + P.gk.base(hd / P.G);
    Vb = static_cast<const float*>(P.v) + P.gk.base(hd / P.G);
    krs = P.gk.sn;
  }
  int nseg = 0, total;
  if constexpr (MODE == MODE_SPARSE) {
    total = build_segments(P, hd, a, seg_start, seg_cum, scan, &nseg);
  } else {
    total = t.key1 - t.key0;
  }
  const bool valid = lane < t.n0;
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
    if constexpr (MODE == MODE_SPARSE) {
      const int sg = seg_find(seg_cum, nseg, pos);
      row = seg_start[sg] + (pos - seg_cum[sg]);
    } else {
      row = t.key0 + pos;
    }
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

// ------------------------------------------------------------------ sparse tiles
// Per head, the tile list of the block-sparse kernel: text rows first (they attend to every key,
// so their tiles are the longest), then each query group of more than kHalfRows rows in tiles of
// 2 kHalfRows rows, then the remaining (small) groups two to a tile.  A tile is
// {a0, row0, n0, a1, row1, n1}: the query group, first Qp row and row count of each half.
//
// A paired tile runs over the union of its two selections, so the small groups are paired by
// overlap (`ov`, the number of K/V groups two query groups both selected; null for ascending id
// order): a few rounds of mutual best matches (each unmatched group finds the unmatched group
// sharing the most K/V groups, ties to the lower rank; two groups that choose each other are
// paired), then the rest in ascending id order.  The pairing changes no row's result.
constexpr int kPairRounds = 4;
constexpr size_t kTilesLds = 128 * 1024;  // LDS for the small groups' overlaps
// Selections of the video query groups as bitmaps over K/V groups, one wave per query group.
constexpr int kOvTile = 32, kOvWords = 16;  // up to 1024 K/V groups
__global__ __launch_bounds__(256) void sel_bits_kernel(const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                       const int* __restrict__ sel_cnt, const int* __restrict__ sel_kv,
                                                       int Cq, int Ck, int G, int n_text,
                                                       unsigned long long* __restrict__ bits) {
  __shared__ unsigned long long wb[4][kOvWords];
  const int hd = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63, a = blockIdx.x * 4 + w;
  const int nq = n_q[hd], nkv = n_kv[hd / G];
  if (a >= nq) return;
  if (lane < kOvWords) wb[w][lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int* sl = sel_kv + (size_t(hd) * (Cq + 1) + a) * (Ck + 1);
  const int cnt = sel_cnt[size_t(hd) * (Cq + 1) + a] - (n_text > 0 ? 1 : 0);
  for (int k = lane; k < cnt; k += 64) {
    const int b = sl[k];
    if (b < nkv) atomicOr(&wb[w][b >> 6], 1ull << (b & 63));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < kOvWords) bits[(size_t(hd) * Cq + a) * kOvWords + lane] = wb[w][lane];
}
// Number of K/V groups two query groups both selected (saturated at 255), for every pair of video
// query groups of a head: blocks of 32 x 32 pairs.
__global__ __launch_bounds__(256) void pair_overlap_kernel(const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                           const unsigned long long* __restrict__ bits, int Cq,
                                                           int G, uint8_t* __restrict__ ov) {
  __shared__ unsigned long long bt[2 * kOvTile][kOvWords];
  const int hd = blockIdx.z, nq = n_q[hd], W = (n_kv[hd / G] + 63) / 64;
  const int a0 = blockIdx.x * kOvTile, c0 = blockIdx.y * kOvTile;
  if (a0 >= nq || c0 >= nq) return;
  for (int e = threadIdx.x; e < 2 * kOvTile * kOvWords; e += 256) {
    const int g = e / kOvWords, x = e % kOvWords;
    const int a = g < kOvTile ? a0 + g : c0 + g - kOvTile;
    bt[g][x] = a < nq ? bits[(size_t(hd) * Cq + a) * kOvWords + x] : 0ull;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kOvTile * kOvTile; e += 256) {
    const int i = e / kOvTile, j = e % kOvTile, a = a0 + i, c = c0 + j;
    if (a >= nq || c >= nq) continue;
    int v = 0;
    for (int x = 0; x < W; ++x) v += __popcll(bt[i][x] & bt[kOvTile + j][x]);
    ov[(size_t(hd) * Cq + a) * Cq + c] = uint8_t(min(v, 255));
  }
}
__global__ __launch_bounds__(1024) void sparse_tiles_kernel(const int* __restrict__ q_off, const int* __restrict__ n_q,
                                                            int Cq, int Nv, int n_text, int tmax,
                                                            const uint8_t* __restrict__ ov,
                                                            int* __restrict__ tiles, int* __restrict__ ntiles) {
  __shared__ int buf[1024], small_id[1024], partner[1024], best_of[1024];
  extern __shared__ uint8_t ovs[];  // [n_small][n_small] overlaps of the small groups, when they fit
  const int hd = blockIdx.x, t = threadIdx.x;
  const int nq = n_q[hd];
  const int* qo = q_off + size_t(hd) * (Cq + 1);
  int* out = tiles + size_t(hd) * tmax * 8;
  constexpr int H2 = 2 * kHalfRows;
  const int n_text_tiles = (n_text + H2 - 1) / H2;
  int s = 0;
  if (t < nq) s = qo[t + 1] - qo[t];
  const bool big = t < nq && s > kHalfRows, small = t < nq && !big;
  const int my_big_tiles = big ? (s + H2 - 1) / H2 : 0;
  int n_big_tiles, n_small;
  const int big_off = block_exscan_i(my_big_tiles, buf, &n_big_tiles);
  const int small_rank = block_exscan_i(small ? 1 : 0, buf, &n_small);
  auto put = [&](int tile, int h, int a, int row, int n) {
    if (tile >= tmax) return;  // cannot happen: tmax bounds the count
    int* d = out + size_t(tile) * 8 + 3 * h;
    d[0] = a;
    d[1] = row;
    d[2] = n;
  };
  for (int k = t; k < n_text_tiles; k += blockDim.x) {
    const int r = Nv + k * H2, n = min(H2, n_text - k * H2);
    put(k, 0, nq, r, min(kHalfRows, n));
    put(k, 1, nq, r + kHalfRows, max(0, n - kHalfRows));
  }
  if (big) {
    for (int k = 0; k < my_big_tiles; ++k) {
      const int r = qo[t] + k * H2, n = min(H2, s - k * H2);
      put(n_text_tiles + big_off + k, 0, t, r, min(kHalfRows, n));
      put(n_text_tiles + big_off + k, 1, t, r + kHalfRows, max(0, n - kHalfRows));
    }
  }
  // small groups by rank; partner[i] = rank of the paired group, -1 while unpaired
  if (small) small_id[small_rank] = t;
  if (t < n_small) partner[t] = -1;
  if (ov) {
    const uint8_t* ovh = ov + size_t(hd) * Cq * Cq;
    // the small groups' overlaps gathered into LDS when they fit
    const bool in_lds = size_t(n_small) * n_small <= kTilesLds;
    __syncthreads();  // small_id complete
    if (in_lds)  // row i by wave, columns by lane
      for (int i = t >> 6; i < n_small; i += blockDim.x >> 6) {
        const uint8_t* src = ovh + size_t(small_id[i]) * Cq;
        for (int j = t & 63; j < n_small; j += 64) ovs[i * n_small + j] = src[small_id[j]];
      }
    // four threads per group (adjacent lanes) split the candidates
    for (int round = 0; round < kPairRounds; ++round) {
      __syncthreads();
      for (int i0 = 0; i0 < n_small; i0 += 256) {
        const int i = i0 + (t >> 2), q = t & 3;
        int best = -1, bestv = -1;
        if (i < n_small && partner[i] < 0) {
          const uint8_t* row = ovh + size_t(small_id[i]) * Cq;
          // candidates j = q, q + 4, ... in batches of 8 (all loads of a batch issued first)
          for (int j0 = q; j0 < n_small; j0 += 32) {
            int vv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int j = j0 + 4 * u;
              vv[u] = j >= n_small ? -1 : in_lds ? int(ovs[i * n_small + j]) : int(row[small_id[j]]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int j = j0 + 4 * u;
              if (j < n_small && j != i && partner[j] < 0 && vv[u] > bestv) {
                bestv = vv[u];
                best = j;
              }
            }
          }
        }
        // best of the four (ties to the lower rank)
#pragma unroll
        for (int o = 1; o < 4; o <<= 1) {
          const int obv = __shfl_xor(bestv, o), ob = __shfl_xor(best, o);
          if (obv > bestv || (obv == bestv && ob >= 0 && (best < 0 || ob < best))) {
            bestv = obv;
            best = ob;
          }
        }
        if (i < n_small && q == 0) best_of[i] = best;
      }
      __syncthreads();
      if (t < n_small && partner[t] < 0 && best_of[t] >= 0 && best_of[best_of[t]] == t) partner[t] = best_of[t];
    }
  }
  __syncthreads();
  // matched pairs (listed by their lower rank), then the unmatched in rank order, two per tile
  const bool lead = t < n_small && partner[t] > t;
  const bool loose = t < n_small && partner[t] < 0;
  int n_pairs, n_loose;
  const int pair_rank = block_exscan_i(lead ? 1 : 0, buf, &n_pairs);
  const int loose_rank = block_exscan_i(loose ? 1 : 0, buf, &n_loose);
  const int base = n_text_tiles + n_big_tiles;
  if (lead) {
    const int a = small_id[t], c = small_id[partner[t]];
    put(base + pair_rank, 0, a, qo[a], qo[a + 1] - qo[a]);
    put(base + pair_rank, 1, c, qo[c], qo[c + 1] - qo[c]);
  }
  if (loose) {
    const int a = small_id[t];
    const int tile = base + n_pairs + loose_rank / 2;
    put(tile, loose_rank & 1, a, qo[a], qo[a + 1] - qo[a]);
    if ((loose_rank & 1) == 0 && loose_rank == n_loose - 1) put(tile, 1, a, qo[a], 0);  // no partner
  }
  if (t == 0) ntiles[hd] = min(tmax, base + n_pairs + (n_loose + 1) / 2);
}

// ------------------------------------------------------------------ host drivers
// Waves per block of the MFMA kernel: sparse tiles are two 64-row halves, dense and probe
// tiles 128 rows.
// Exclusive prefix of the per-head tile counts; prefix[BH] is the number of tiles of the call.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int* __restrict__ ntiles, int BH,
                                                           int* __restrict__ prefix) {
  __shared__ int buf[1024];
  int carry = 0;
  for (int base = 0; base < BH; base += 1024) {
    const int i = base + int(threadIdx.x);
    int tot;
    const int ex = block_exscan_i(i < BH ? ntiles[i] : 0, buf, &tot);
    if (i < BH) prefix[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) prefix[BH] = carry;
}

template <int MODE>
constexpr int mfma_waves() { return 8; }
template <int MODE>
constexpr int mfma_rows() { return 16 * mfma_waves<MODE>(); }

template <int D, int MODE>
static size_t mfma_smem() {
  size_t s = 2 * size_t(kChunk) * D * 2 + 3 * size_t(D) * kChunk * 2 + 8 * kChunk * sizeof(int) +
             16 * sizeof(unsigned long long);
  if (MODE == MODE_SPARSE) s += (3 * kSegCap + 66 + mfma_waves<MODE>() * 64) * sizeof(int);
  return s;
}

template <int D, int MODE>
static void launch_attn(const AttnParams& P, dim3 grid, int dtype, hipStream_t st) {
  if (dtype == SPR_BF16) {
    constexpr int W = mfma_waves<MODE>();
    constexpr bool VF16 = MODE == MODE_SPARSE;  // the sparse kernel reads the fp16 copy of V
    const size_t sm = mfma_smem<D, MODE>();
    allow_lds(attn_mfma_kernel<D, MODE, W, VF16>, sm);
    hipLaunchKernelGGL((attn_mfma_kernel<D, MODE, W, VF16>), grid, dim3(W * 64), sm, st, P);
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
  const int BH = desc.B * desc.H, Nv = desc.N - desc.n_text;
  int* tiles = ws_ptr<int>(ws, L.tiles);
  int* ntiles = ws_ptr<int>(ws, L.ntiles);
  // selection overlaps of every pair of query groups (for up to 1024 K/V groups), then the tiles
  uint8_t* ov = nullptr;
  if (p.Ck <= 64 * kOvWords) {
    ov = ws_ptr<uint8_t>(ws, L.pair_ov);
    unsigned long long* sbits = ws_ptr<unsigned long long>(ws, L.sel_bits);
    hipLaunchKernelGGL(sel_bits_kernel, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, part.n_q, part.n_kv,
                       route.sel_cnt, route.sel_kv, p.Cq, p.Ck, kv_group_size(desc), desc.n_text, sbits);
    const dim3 og(ceil_div(p.Cq, kOvTile), ceil_div(p.Cq, kOvTile), BH);
    hipLaunchKernelGGL(pair_overlap_kernel, og, dim3(256), 0, st, part.n_q, part.n_kv, sbits, p.Cq,
                       kv_group_size(desc), ov);
  }
  allow_lds(sparse_tiles_kernel, ov ? kTilesLds : 0);
  hipLaunchKernelGGL(sparse_tiles_kernel, dim3(BH), dim3(1024), ov ? kTilesLds : 0, st, part.q_off, part.n_q, p.Cq,
                     Nv, desc.n_text, L.tmax, ov, tiles, ntiles);
  int* tprefix = ws_ptr<int>(ws, L.tile_prefix);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, ntiles, BH, tprefix);
  SPR_CHECK_LAUNCH();
  AttnParams P = {};
  P.q = part.Qp; P.k = part.Kp; P.v = part.Vp;
  if (desc.dtype == SPR_BF16) P.v = ws_ptr<void>(ws, L.vh);
  P.g = make_geom(desc);
  P.gk = make_kv_geom(desc);
  P.G = kv_group_size(desc);
  P.tiles = tiles; P.ntiles = ntiles; P.tile_prefix = tprefix; P.tmax = L.tmax; P.BH = BH;
  P.n_kv = part.n_kv; P.kv_off = part.kv_off; P.sel_cnt = route.sel_cnt; P.sel_kv = route.sel_kv;
  P.Cq = p.Cq; P.Ck = p.Ck;
  P.o_sp = o_sp;
  // bf16: one block per tile, 1-D grid mapped onto the tile list (a multiple of 8 blocks, one
  // share per XCD); fp32: one block per tile half, grid (2 tmax, BH)
  const dim3 grid = desc.dtype == SPR_BF16 ? dim3(unsigned(8 * ceil_div64(int64_t(BH) * L.tmax, 8)))
                                           : dim3(2 * L.tmax, BH);
  return dispatch_d<MODE_SPARSE>(P, grid, desc.d, desc.dtype, st);
}

spr_status run_probe_exact(const spr_desc& desc, const void* q, const void* k, const void* v, const int* probe_idx,
                           int M, float* o_probe, void* ws, const Workspace& L, hipStream_t st) {
  AttnParams P = {};
  P.q = q; P.k = k; P.v = v;
  P.g = make_geom(desc);
  P.gk = make_kv_geom(desc);
  P.G = kv_group_size(desc);
  P.probe_idx = probe_idx; P.M = M; P.splits = L.splits;
  P.part = ws_ptr<float>(ws, L.pr_part);
  const int BH = desc.B * desc.H;
  const int rows = desc.dtype == SPR_BF16 ? mfma_rows<MODE_PROBE>() : kTileRows;
  spr_status s = dispatch_d<MODE_PROBE>(P, dim3(ceil_div(M, rows), BH, L.splits), desc.d, desc.dtype, st);
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
  P.gk = make_kv_geom(desc);
  P.G = kv_group_size(desc);
  P.out = out; P.out_dtype = out_dtype;
  const int rows = desc.dtype == SPR_BF16 ? mfma_rows<MODE_DENSE>() : kTileRows;
  return dispatch_d<MODE_DENSE>(P, dim3(ceil_div(desc.N, rows), desc.B * desc.H), desc.d, desc.dtype, st);
}

}  // namespace spr
