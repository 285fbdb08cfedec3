// Flash-style attention kernels for the SparsePR operator on gfx950.
//
//  - block-sparse (Eq. (2) of "Partition the Support, Reconstruct the Residual", Sec. 3;
//    execution as in Sec. 4.3).  A block holds two halves of up to 64 query rows.  A query
//    group with more than 64 rows fills both halves of its blocks; smaller groups are paired,
//    and the block streams the union of the two groups' selected K/V groups (groups selected
//    by both halves first, then those of one half only), each half skipping or masking keys it
//    did not select.  Either way every K/V chunk staged in LDS serves up to 128 query rows.
//  - dense (Eq. (1)): the same kernel over one run of every key;
//  - probe rows (Sec. 4.2): gathered query rows against a contiguous key range (split-K),
//    partial (max, sum, unnormalised output) merged by a second kernel.
//
// bf16 inputs use MFMA: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (exact products, fp32
// sums), P rounded to fp16 and O^T += V^T P^T with v_mfma_f32_32x32x16_f16 from an fp16 copy of
// V scaled by a power of two per K/V head (the scale is undone on the output).  Computing the
// transposes puts a query row's scores and its output columns in one lane.  fp32 inputs use a
// plain VALU kernel.
#include <mutex>
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
  // bf16: power-of-two factor per K/V head that undoes the scaling of the fp16 copy of V (null: 1)
  const float* vinv;
  __device__ float vscale_inv(int hk) const { return vinv ? vinv[hk] : 1.f; }
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// two floats rounded to bf16 (nearest even; inf and nan pass through), packed low then high
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) return u >> 16;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
  return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
}

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
    // Block L takes tile L of the head-major list of all tiles.  Workgroups reach the 8 XCDs
    // round-robin, so every XCD works on the same one or two heads at a time: their K/V stay in
    // the last-level cache the XCDs share, and tiles of unequal cost spread evenly over the XCDs
    // (contiguous shares of the list per XCD measured 7% slower on the long workload).
    const int total = P.tile_prefix[P.BH];
    const int n = int(blockIdx.x);
    if (n >= total) {
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
                                           uint8_t* seg_cat, unsigned* bm /* [2][33] */, int* scan,
                                           int* nseg_out, int* n3_out, int* n1_out) {
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
  // the counts of categories 3 and 1 (each <= 1025) share one scan in 16-bit fields, category 2
  // takes a second scan
  int tot, tot2;
  const int ex = block_exscan_i(c3 | (c1 << 16), scan, &tot);
  const int ex2 = block_exscan_i(c2, scan, &tot2);
  const int n3 = tot & 0xffff, n1 = tot >> 16, n2 = tot2;
  int o3 = ex & 0xffff, o1 = n3 + (ex >> 16), o2 = n3 + n1 + ex2;
  const int* off = P.kv_off + size_t(hk) * (P.Ck + 1);
  for (int b = i0; b < min(i0 + per, ng); ++b) {
    const int c = cat_of(b);
    if (c == 0) continue;
    const int pos = c == 3 ? o3++ : c == 1 ? o1++ : o2++;
    kv_group(P, off, nkv, b, seg_start + pos, seg_cum + pos);
    seg_cat[pos] = uint8_t(c);
  }
  __syncthreads();
  *nseg_out = n3 + n1 + n2;
  *n3_out = n3;
  *n1_out = n1;
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
// A block holds 128 query rows in four waves of 32 rows (for sparse tiles: two halves of two
// waves).  Every 64-key chunk is staged once in LDS for all four waves:
//  - K rows (bf16) by direct global-to-LDS loads, rows padded to D + 8 elements so that the
//    fragment reads of consecutive rows fall on different banks;
//  - V rows (fp16) by direct loads into unpadded rows whose 16-byte pieces are XOR-swizzled by
//    the row's residue mod 4; the P V operand is read with transposing LDS reads.
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16 (bf16, then fp16): a lane holds one
// query row's scores and output columns, so the softmax needs one cross-lane exchange (the two
// 32-lane halves hold the two halves of the keys) only when the running maximum is raised.
// Each step computes the scores of chunk c+1 interleaved with the exponentials of chunk c,
// then the P V products of chunk c, while the loads of K(c+2) and V(c+1) are in flight; one
// barrier per step.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __fp16 h4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
#define SPR_LDS __attribute__((address_space(3)))

// 16 bytes per lane from a buffer resource straight into LDS: lane l writes lds + 16 l
// (the LDS destination is given as a byte offset into the kernel's dynamic LDS)
extern __shared__ __attribute__((aligned(16))) char smem_raw[];
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, int lds_off, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SPR_LDS void*)((SPR_LDS char*)smem_raw + lds_off), 16, voffset, 0,
                                           0, 0);
#endif
}

template <int D>
struct Attn32Shape {
  static constexpr int KC = 64;              // keys per chunk
  static constexpr int PCS = D / 8;          // 16-byte pieces per row
  static constexpr int KSTR = PCS + 1;       // K row stride in pieces (padded)
  static constexpr int KLOADS = KC * KSTR / 64;  // wave-wide 1 KB loads per K chunk
  static constexpr int VLOADS = KC * PCS / 64;   // per V chunk
  static constexpr int KBUF = KC * KSTR * 16;    // bytes of one K buffer
  static constexpr int VBUF = KC * PCS * 16;     // bytes of one V buffer
  static constexpr int NT = D / 32;          // 32-column output tiles
  static constexpr int KS = D / 16;          // 16-column steps of the score product
  // XOR applied to the piece index of a V row with residue k mod 4: the four rows of one
  // transposing read (two pieces each) land on eight distinct 16-byte bank groups, and the
  // 32 lanes of a 32-column tile on sixteen
  static __device__ __forceinline__ int vswz(int k) { return D == 128 ? (0xAC60 >> (4 * k)) & 15 : 2 * k; }
};

constexpr int kRing = 4;  // chunk slots of the key-bias ring and of the row ring (sparse)

template <int D, int MODE>
static constexpr size_t attn32_smem() {
  using S = Attn32Shape<D>;
  size_t s = 2 * size_t(S::KBUF) + 2 * size_t(S::VBUF) + kRing * 2 * 64 * sizeof(float);
  if (MODE == MODE_SPARSE)
    s += kRing * 64 * sizeof(int) + 2 * kSegCap * sizeof(int) + kSegCap + 66 * sizeof(unsigned) + 32 * sizeof(int);
  return s;
}

template <int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn32_kernel(AttnParams P) {
  using S = Attn32Shape<D>;
  constexpr bool SPARSE = MODE == MODE_SPARSE;
  constexpr int KC = S::KC, NT = S::NT, KS = S::KS, VROW = D * 2;
  char* Kl = smem_raw;                                               // [2][KBUF]
  char* Vl = smem_raw + 2 * S::KBUF;                                 // [2][VBUF]
  float* kbias = reinterpret_cast<float*>(Vl + 2 * S::VBUF);         // [kRing][2][64]
  int* rowidx = reinterpret_cast<int*>(kbias + kRing * 2 * 64);      // [kRing][64]
  int* seg_start = rowidx + kRing * 64;                              // [kSegCap]
  int* seg_cum = seg_start + kSegCap;                                // [kSegCap]
  uint8_t* seg_cat = reinterpret_cast<uint8_t*>(seg_cum + kSegCap);  // [kSegCap]
  unsigned* bm = reinterpret_cast<unsigned*>(seg_cat + kSegCap);     // [66]
  int* scan = reinterpret_cast<int*>(bm + 66);                       // [32]

  const TileInfo t = decode_tile<MODE, 128>(P);
  if (!t.valid || t.n0 <= 0) return;
  const int hd = t.hd;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q32 = lane & 31, kg = lane >> 5;
  // this wave's 32 rows: sparse tiles give waves 0-1 to half 0 and waves 2-3 to half 1
  const int half = SPARSE ? (w >> 1) : 0;
  const int my_row0 = SPARSE ? (half ? t.row1 : t.row0) + 32 * (w & 1) : t.row0 + 32 * w;
  const int my_n = SPARSE ? (half ? t.n1 : t.n0) - 32 * (w & 1) : t.n0 - 32 * w;
  const bool wave_active = my_n > 0;
  const bool qvalid = q32 < my_n;

  // K rows through buffer resources with 32-bit byte offsets (a head's rows span < 2 GiB); V is
  // the contiguous fp16 copy [heads][N][D]
  const int hk = hd / P.G;
  const uint16_t* Kb;
  int krow_bytes;
  if constexpr (SPARSE) {
    Kb = static_cast<const uint16_t*>(P.k) + size_t(hk) * P.g.N * D;
    krow_bytes = D * 2;
  } else {
    Kb = static_cast<const uint16_t*>(P.k) + P.gk.base(hk);
    krow_bytes = int(P.gk.sn) * 2;
  }
  const _Float16* Vb = static_cast<const _Float16*>(P.v) + size_t(hk) * P.g.N * D;
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kb, (short)0, (P.g.N - 1) * krow_bytes + D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vb, (short)0, P.g.N * VROW, 0x00020000);

  // keys of the tile; a sparse tile's halves attend to keys [0, k31) (half 0: categories 3 and 1)
  // and [0, k3) with [k31, total) (half 1: categories 3 and 2)
  int nseg = 0, total, k3, k31;
  if constexpr (SPARSE) {
    int n3, n1;
    total = build_union_segments(P, t, seg_start, seg_cum, seg_cat, bm, scan, &nseg, &n3, &n1);
    k3 = seg_cum[n3];
    k31 = seg_cum[n3 + n1];
  } else {
    total = k3 = k31 = t.key1 - t.key0;
  }
  const int nchunks = (total + KC - 1) / KC;

  // query fragments (B operand of S^T = K Q^T): row q32, columns 16 s + 8 kg .. + 7
  uint4 qf[KS];
  {
    const uint16_t* qrow = nullptr;
    if (qvalid) {
      if constexpr (SPARSE) {
        qrow = static_cast<const uint16_t*>(P.q) + (size_t(hd) * P.g.N + my_row0 + q32) * D;
      } else if constexpr (MODE == MODE_DENSE) {
        qrow = static_cast<const uint16_t*>(P.q) + P.g.base(hd) + int64_t(my_row0 + q32) * P.g.sn;
      } else {
        const int pr = P.probe_idx[size_t(hd) * P.M + my_row0 + q32];
        qrow = static_cast<const uint16_t*>(P.q) + P.g.base(hd) + int64_t(pr) * P.g.sn;
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qvalid ? *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * kg) : make_uint4(0, 0, 0, 0);
  }

  // Wave 0 prepares each chunk two steps ahead (ring of kRing slots): per half, the bias of every
  // key (0 when the half attends to it, -inf otherwise, which also masks the keys past the end),
  // and for sparse tiles the Kp row of every key.  A sparse chunk's segments are found from the
  // segment holding its first key, carried over from the previous chunk.
  int seg_cursor = 0;
  auto prepare = [&](int ch) __attribute__((always_inline)) {
    const int slot = ch & (kRing - 1);
    const int pos = ch * KC + lane;
    int cat = pos < total ? 3 : 0;
    if constexpr (SPARSE) {
      int sg = seg_cursor, row = 0;
      for (int k = seg_cursor + 1; k < nseg; ++k) {
        const int start = __builtin_amdgcn_readfirstlane(seg_cum[k]);
        if (start > ch * KC + KC) break;
        if (pos >= start) sg = k;
        seg_cursor = k;
      }
      if (pos < total) {
        row = seg_start[sg] + (pos - seg_cum[sg]);
        cat = seg_cat[sg];
      }
      rowidx[slot * 64 + lane] = row;
    }
    kbias[(slot * 2) * 64 + lane] = (cat & 1) ? 0.f : -INFINITY;
    kbias[(slot * 2 + 1) * 64 + lane] = (cat & 2) ? 0.f : -INFINITY;
  };

  // Direct loads: wave w issues K loads j = 4 i + w and V loads j = 4 i + w (i < KQ, VQ); K loads
  // past 4 KQ (the padding makes KLOADS = 4 KQ + 1) go to wave 0.  Lane l of load j fills 16-byte
  // slot 64 j + l of its buffer: K slot s is piece s % KSTR of row s / KSTR (the padding piece
  // re-reads piece 0), V slot s holds piece (s % PCS) ^ vswz(row % 4) of row s / PCS.
  constexpr int KQ = S::KLOADS / 4, VQ = S::VLOADS / 4;
  static_assert(S::VLOADS == 4 * VQ && S::KLOADS == 4 * KQ + 1, "load split");
  auto kslot = [&](int j) __attribute__((always_inline)) -> int {  // row | byte column << 8
    const int s = 64 * j + lane, pc = s % S::KSTR;
    return (s / S::KSTR) | ((pc < S::PCS ? pc : 0) * 16) << 8;
  };
  int kslots[KQ];
#pragma unroll
  for (int i = 0; i < KQ; ++i) kslots[i] = kslot(4 * i + w);
  const int kslot_x = kslot(4 * KQ);
  constexpr int VRPL = 64 / S::PCS;  // V rows per load: 4 (D = 128) or 8 (D = 64)
  const int vrow_l = lane / S::PCS, vcol = ((lane % S::PCS) ^ S::vswz(vrow_l & 3)) * 16;
  const int klast = t.key1 - 1;
  // Dense and probe tiles address chunk ch through resources based at its first row, key0 + 64 ch,
  // whose range ends after row klast: every lane's offset is then the same in every chunk, and
  // the rows past klast of the last chunk read as zero (their bias masks them).  Sparse tiles read
  // each lane's row from the chunk's row list in LDS, all of a step's rows before its first load.
  int kvoff[KQ + 1], vvoff[VQ];
#pragma unroll
  for (int i = 0; i <= KQ; ++i) {
    const int sl = i < KQ ? kslots[i] : kslot_x;
    kvoff[i] = SPARSE ? (sl >> 8) : (sl & 255) * krow_bytes + (sl >> 8);
  }
#pragma unroll
  for (int i = 0; i < VQ; ++i) vvoff[i] = SPARSE ? vcol : (VRPL * (4 * i + w) + vrow_l) * VROW + vcol;
  auto chunk_k = [&](int ch) __attribute__((always_inline)) {
    const int rb = t.key0 + ch * KC;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(Kb + int64_t(rb) * (krow_bytes >> 1)), (short)0,
                                             max(0, (klast - rb) * krow_bytes + D * 2), 0x00020000);
  };
  auto chunk_v = [&](int ch) __attribute__((always_inline)) {
    const int rb = t.key0 + ch * KC;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(Vb + int64_t(rb) * D), (short)0, max(0, (klast + 1 - rb) * VROW),
                                             0x00020000);
  };
  // K of chunk kc into buffer kb, and with with_v V of chunk vc into buffer vb
  auto issue = [&](int kc, int kb, int vc, int vb, bool with_v) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      const int* kr = rowidx + (kc & (kRing - 1)) * 64;
      const int* vr = rowidx + (vc & (kRing - 1)) * 64;
      int krow[KQ + 1], vrow[VQ];
#pragma unroll
      for (int i = 0; i < KQ; ++i) krow[i] = kr[kslots[i] & 255];
      krow[KQ] = kr[kslot_x & 255];
#pragma unroll
      for (int i = 0; i < VQ; ++i) vrow[i] = with_v ? vr[VRPL * (4 * i + w) + vrow_l] : 0;
#pragma unroll
      for (int i = 0; i < KQ; ++i) lds_load16(krsrc, kb * S::KBUF + (4 * i + w) * 1024, krow[i] * krow_bytes + kvoff[i]);
      if (w == 0) lds_load16(krsrc, kb * S::KBUF + 4 * KQ * 1024, krow[KQ] * krow_bytes + kvoff[KQ]);
      if (with_v)
#pragma unroll
        for (int i = 0; i < VQ; ++i)
          lds_load16(vrsrc, 2 * S::KBUF + vb * S::VBUF + (4 * i + w) * 1024, vrow[i] * VROW + vvoff[i]);
    } else {
      const __amdgpu_buffer_rsrc_t rk = chunk_k(kc), rv = chunk_v(vc);
#pragma unroll
      for (int i = 0; i < KQ; ++i) lds_load16(rk, kb * S::KBUF + (4 * i + w) * 1024, kvoff[i]);
      if (w == 0) lds_load16(rk, kb * S::KBUF + 4 * KQ * 1024, kvoff[KQ]);
      if (with_v)
#pragma unroll
        for (int i = 0; i < VQ; ++i) lds_load16(rv, 2 * S::KBUF + vb * S::VBUF + (4 * i + w) * 1024, vvoff[i]);
    }
  };
  auto wait_loads = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

  // LDS read addresses.  K fragment of key row 32 tt + q32, columns 16 s + 8 kg: byte
  // (32 tt + q32) KSTR 16 + (2 s + kg) 16.  V transposing read of a 16-lane group: lane
  // i = 4 k + c supplies row R0 + k (R0 = 16 sg + 8 j + 4 kg) and columns 32 dt + 16 gg + 4 c .. + 3.
  const int kaddr = q32 * S::KSTR * 16 + kg * 16;
  int vaddr[NT];
  {
    const int i16 = lane & 15, gg = (lane >> 4) & 1, kk = i16 >> 2, cc = i16 & 3;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
      vaddr[dt] = (4 * kg + kk) * VROW + (((4 * dt + 2 * gg + (cc >> 1)) ^ S::vswz(kk)) * 16) + (cc & 1) * 8;
  }

  const float scale = kLog2e / sqrtf(float(D));
  float m_run = -INFINITY, lsum = 0.f;
  f32x16_t oacc[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) oacc[dt] = f32x16_t{};
  const f16x2_t ones2 = {_Float16(1.0f), _Float16(1.0f)};

  // scores of chunk c: the accumulators start from this half's key bias (score register r of tile
  // tt holds key 32 tt + 8 (r / 4) + 4 kg + r % 4); K fragment reads run two MFMAs ahead
  auto qk = [&](f32x16_t (&sacc)[2], int c) __attribute__((always_inline)) {
    const float* bias = kbias + ((c & (kRing - 1)) * 2 + half) * 64 + 4 * kg;
    const char* K = Kl + (c & 1) * S::KBUF + kaddr;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 b = *reinterpret_cast<const float4*>(bias + 32 * tt + 8 * j);
        sacc[tt][4 * j] = b.x; sacc[tt][4 * j + 1] = b.y; sacc[tt][4 * j + 2] = b.z; sacc[tt][4 * j + 3] = b.w;
      }
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(K + (32 * tt * S::KSTR + 2 * s) * 16)), as_bf16x8(qf[s]),
            sacc[tt], 0, 0, 0);
    }
  };
  // The running maximum is raised lazily: while every p of the wave stays <= 2^8 (exact range in
  // fp16; tested on the bit patterns, which order non-negative floats and put inf and NaN above
  // every finite value) the shift is kept; otherwise the rows whose maximum grew by more than
  // 2^8 take it as their new shift and O and l, which by then hold every earlier chunk, are
  // rescaled before the exponentials are formed again.
  auto exps = [&](const f32x16_t (&sacc)[2], f16x2_t (&pk)[16]) __attribute__((always_inline)) -> unsigned {
    const float mneg = -m_run;
    unsigned big = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 3][(2 * i) & 15], scale, mneg));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 3][(2 * i + 1) & 15], scale, mneg));
      big = max(big, max(__float_as_uint(p0), __float_as_uint(p1)));
      pk[i] = f16x2_t{_Float16(p0), _Float16(p1)};
    }
    return big;
  };
  auto rescale = [&](const f32x16_t (&sacc)[2]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[tt][r]);
    mx *= scale;
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool grow = mx > m_run + 8.0f;
    const float m_new = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) oacc[dt] *= alpha;
  };
  auto exps_settled = [&](const f32x16_t (&sacc)[2], f16x2_t (&pk)[16], unsigned big) __attribute__((always_inline)) {
    if (__builtin_expect(__any(big > 0x43800000u), 0)) {
      rescale(sacc);
      exps(sacc, pk);
    }
  };
  auto pv = [&](const f16x2_t (&pk)[16], int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) lsum = __builtin_amdgcn_fdot2(pk[i], ones2, lsum, false);
    const char* V = Vl + (c & 1) * S::VBUF;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      // B operand: p of keys 16 sg + 8 (j / 4) + 4 kg + j % 4, i.e. registers 8 (sg % 2) .. + 7 of tile sg / 2
      typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
      f16x8 b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[2 * j] = pk[4 * sg + j][0];
        b[2 * j + 1] = pk[4 * sg + j][1];
      }
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        const h4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPR_LDS h4_t*)(V + vaddr[dt] + (16 * sg) * VROW));
        const h4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPR_LDS h4_t*)(V + vaddr[dt] + (16 * sg + 8) * VROW));
        const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
        const f16x8 a = __builtin_bit_cast(f16x8, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, oacc[dt], 0, 0, 0);
      }
    }
  };

  // Steps: step c (one barrier) computes the scores of chunk c, then its exponentials interleaved
  // with the P V products of chunk c - 1, while K(c + 1) and V(c) load and wave 0 prepares chunk
  // c + 2.  Every wave takes part in all nchunks + 1 steps; it computes over the chunk runs its
  // half attends to (one run, or for half 1 of a paired tile the shared run and its own run)
  // and only loads in the other steps.  An empty key range (a probe split of fewer keys than
  // splits) leaves l = 0 and the shift at -inf.
  auto begin_step = [&](int c) __attribute__((always_inline)) {
    __syncthreads();  // K(c) and V(c - 1) are staged; every wave is done with K(c - 1) and V(c - 2)
    if (w == 0) prepare(c + 2);
    issue(c + 1, (c + 1) & 1, c, c & 1, true);
  };
  f32x16_t sacc[2];
  f16x2_t p_old[16];
  // chunks [lo, hi) in steps lo .. hi: a first step without P V products, straight steps with
  // them (the hot loop), and a last step with the P V products of chunk hi - 1 alone
  auto run = [&](int lo, int hi) __attribute__((always_inline)) {
    if (lo >= hi) return;
    begin_step(lo);
    qk(sacc, lo);
    exps_settled(sacc, p_old, exps(sacc, p_old));
    wait_loads();
    for (int c = lo + 1; c < hi; ++c) {
      begin_step(c);
      qk(sacc, c);
      f16x2_t p_new[16];
      const unsigned big = exps(sacc, p_new);
      pv(p_old, c - 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 64 / (4 * NT), 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 32 / (4 * NT), 0);
        if (i + 2 < 4 * NT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      exps_settled(sacc, p_new, big);
#pragma unroll
      for (int i = 0; i < 16; ++i) p_old[i] = p_new[i];
      wait_loads();
    }
    begin_step(hi);
    pv(p_old, hi - 1);
    wait_loads();
  };
  auto idle = [&](int lo, int hi) __attribute__((always_inline)) {
    for (int c = lo; c < hi; ++c) {
      begin_step(c);
      wait_loads();
    }
  };
  if (nchunks > 0) {
    if (w == 0)
      for (int c = 0; c < 2; ++c) prepare(c);
    __syncthreads();
    issue(0, 0, 0, 0, false);
    wait_loads();
    // this wave's chunk runs
    int lo0 = 0, hi0 = nchunks, lo1 = nchunks, hi1 = nchunks;
    if (SPARSE && half == 1 && t.pair) {
      // the shared run, then from the chunk holding key k31 (when half 1 has keys of its own)
      const int b = (k3 + KC - 1) / KC, c1 = k31 < total ? k31 / KC : nchunks;
      if (c1 > b) {
        hi0 = b;
        lo1 = c1;
      }
    } else if (SPARSE && t.pair) {
      hi0 = (k31 + KC - 1) / KC;
    }
    if (!wave_active) {
      hi0 = lo1 = hi1 = 0;
    }
    run(lo0, hi0);
    int st = hi0 > lo0 ? hi0 + 1 : 0;
    idle(st, lo1);
    run(lo1, hi1);
    st = hi1 > lo1 ? hi1 + 1 : max(st, lo1);
    idle(st, nchunks + 1);
  }
  if (!qvalid) return;
  // the two 32-lane halves hold the sums of the two halves of every chunk's keys
  const float lt = lsum + __shfl_xor(lsum, 32);
  // output column of register r of tile dt: 32 dt + 8 (r / 4) + 4 kg + r % 4
  if constexpr (MODE == MODE_PROBE) {
    float* dst = P.part + ((size_t(hd) * P.M + my_row0 + q32) * P.splits + t.split) * (D + 2);
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * j + 4 * kg) =
            make_float4(oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]);
    if (kg == 0) {
      dst[D] = m_run;
      dst[D + 1] = lt;
    }
  } else {
    const float inv = P.vscale_inv(hk) / lt;
    if constexpr (SPARSE) {
      float* dst = P.o_sp + (size_t(hd) * P.g.N + my_row0 + q32) * D;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(dst + 32 * dt + 8 * j + 4 * kg) =
              make_float4(oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv, oacc[dt][4 * j + 2] * inv,
                          oacc[dt][4 * j + 3] * inv);
    } else {
      const size_t rowbase = (size_t(hd) * P.g.N + my_row0 + q32) * D;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t idx = rowbase + 32 * dt + 8 * j + 4 * kg;
          const float x0 = oacc[dt][4 * j] * inv, x1 = oacc[dt][4 * j + 1] * inv;
          const float x2 = oacc[dt][4 * j + 2] * inv, x3 = oacc[dt][4 * j + 3] * inv;
          if (P.out_dtype == SPR_BF16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(P.out) + idx) =
                make_uint2(bf16_pair_rne(x0, x1), bf16_pair_rne(x2, x3));
          else
            *reinterpret_cast<float4*>(static_cast<float*>(P.out) + idx) = make_float4(x0, x1, x2, x3);
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

// Merge split-K partials: O = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m), times the factor that
// undoes the scaling of the fp16 copy of V (bf16 inputs).
__global__ __launch_bounds__(256) void probe_merge_kernel(const float* __restrict__ part, int M, int splits, int D,
                                                          int BH, int G, const float* __restrict__ vinv,
                                                          float* __restrict__ o_probe) {
  const int row = blockIdx.x;  // over BH * M
  if (row >= BH * M) return;
  const float* pr = part + size_t(row) * splits * (D + 2);
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, pr[s * (D + 2) + D]);
  float l = 0.f;
  for (int s = 0; s < splits; ++s) l += pr[s * (D + 2) + D + 1] * exp2f(pr[s * (D + 2) + D] - mx);
  const float f = vinv ? vinv[(row / M) / G] : 1.f;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += pr[s * (D + 2) + c] * exp2f(pr[s * (D + 2) + D] - mx);
    o_probe[size_t(row) * D + c] = acc / l * f;
  }
}

// ------------------------------------------------------------------ fp16 copy of V
// The P V products run in fp16, whose range is narrower than bf16's.  Every K/V head's V is
// scaled by 2^e, e chosen from its largest magnitude so that it lies in [2^14, 2^15) (e within
// [-100, 100]; a head of zeros, infinities or NaN keeps e = 0), and the output is multiplied by
// 2^-e.  Scaling by a power of two is exact; only magnitudes below 2^-24 of the head's largest
// lose bits to fp16 rounding.

// largest |v| per K/V head as a float bit pattern (non-negative patterns order like the values);
// grid (kAbsmaxBlocks, heads), amax cleared by v_amax_clear_kernel: each block strides over its
// head's 16-byte pieces and adds one atomic maximum, so a head sees kAbsmaxBlocks atomics
constexpr int kAbsmaxBlocks = 128;
__global__ __launch_bounds__(256) void v_absmax_kernel(const uint16_t* __restrict__ v, HeadGeom gk,
                                                       unsigned* __restrict__ amax) {
  __shared__ unsigned red[4];
  const int hk = blockIdx.y, per = gk.d / 8;
  const int64_t n = int64_t(gk.N) * per;
  unsigned m = 0;
  for (int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x; idx < n; idx += int64_t(gridDim.x) * 256) {
    const int row = int(idx / per), pc = int(idx % per);
    const uint4 u = *reinterpret_cast<const uint4*>(v + gk.base(hk) + int64_t(row) * gk.sn + pc * 8);
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const unsigned lo = (wv[c] << 16) & 0x7FFF0000u, hi = wv[c] & 0x7FFF0000u;
      m = max(m, max(lo, hi));
    }
  }
  for (int o = 32; o > 0; o >>= 1) m = max(m, unsigned(__shfl_xor(int(m), o)));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax + hk, max(max(red[0], red[1]), max(red[2], red[3])));
}
__global__ void v_amax_clear_kernel(unsigned* __restrict__ amax, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) amax[i] = 0u;
}
// scale[hk] = 2^e, scale[n + hk] = 2^-e
__global__ void v_scale_kernel(const unsigned* __restrict__ amax, int n, float* __restrict__ scale) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const unsigned a = amax[i];
  int e = 0;
  if (a != 0u && (a & 0x7F800000u) != 0x7F800000u) {
    const int E = int(a >> 23) - 127;  // floor(log2 a) for normal a; subnormals clamp below
    e = min(100, max(-100, 14 - E));
  }
  scale[i] = __uint_as_float(uint32_t(127 + e) << 23);
  scale[n + i] = __uint_as_float(uint32_t(127 - e) << 23);
}
// contiguous [heads][N][d] fp16 copy of v scaled by scale[hk]; grid (ceil(N d / 8 / 256), heads)
__global__ __launch_bounds__(256) void v_to_f16_kernel(const uint16_t* __restrict__ v, HeadGeom gk,
                                                       const float* __restrict__ scale, _Float16* __restrict__ vh) {
  const int hk = blockIdx.y, per = gk.d / 8;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(gk.N) * per) return;
  const int row = int(idx / per), pc = int(idx % per);
  const uint4 u = *reinterpret_cast<const uint4*>(v + gk.base(hk) + int64_t(row) * gk.sn + pc * 8);
  const float f = scale[hk];
  const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 o;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o[2 * c] = _Float16(__uint_as_float(wv[c] << 16) * f);
    o[2 * c + 1] = _Float16(__uint_as_float(wv[c] & 0xFFFF0000u) * f);
  }
  *reinterpret_cast<h8*>(vh + (size_t(hk) * gk.N + row) * gk.d + pc * 8) = o;
}

void launch_v_scale(const void* v, const HeadGeom& gk, int heads, unsigned* amax, float* scale, hipStream_t st) {
  hipLaunchKernelGGL(v_amax_clear_kernel, dim3(ceil_div(heads, 256)), dim3(256), 0, st, amax, heads);
  hipLaunchKernelGGL(v_absmax_kernel, dim3(kAbsmaxBlocks, heads), dim3(256), 0, st, static_cast<const uint16_t*>(v),
                     gk, amax);
  hipLaunchKernelGGL(v_scale_kernel, dim3(ceil_div(heads, 256)), dim3(256), 0, st, amax, heads, scale);
}

size_t v_copy_bytes(const spr_desc& desc) {
  if (desc.dtype != SPR_BF16) return 0;
  const size_t heads = size_t(desc.B) * kv_heads(desc);
  return ((heads * desc.N * desc.d * 2 + 255) & ~size_t(255)) + ((heads * 4 + 255) & ~size_t(255)) +
         ((2 * heads * 4 + 255) & ~size_t(255));
}

// scaled fp16 copy of v in ws (layout of v_copy_bytes); returns the inverse factors
static const float* make_v_copy(const spr_desc& desc, const void* v, void* ws, _Float16** vh, hipStream_t st) {
  const int heads = desc.B * kv_heads(desc);
  const HeadGeom gk = make_kv_geom(desc);
  char* base = static_cast<char*>(ws);
  *vh = reinterpret_cast<_Float16*>(base);
  base += (size_t(heads) * desc.N * desc.d * 2 + 255) & ~size_t(255);
  unsigned* amax = reinterpret_cast<unsigned*>(base);
  base += (size_t(heads) * 4 + 255) & ~size_t(255);
  float* scale = reinterpret_cast<float*>(base);
  launch_v_scale(v, gk, heads, amax, scale, st);
  const dim3 grid(unsigned(ceil_div64(int64_t(gk.N) * gk.d / 8, 256)), heads);
  hipLaunchKernelGGL(v_to_f16_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(v), gk, scale, *vh);
  return scale + heads;
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
// Number of K/V groups two query groups both selected, for every pair of video
// query groups of a head: blocks of 32 x 32 pairs.
__global__ __launch_bounds__(256) void pair_overlap_kernel(const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                           const unsigned long long* __restrict__ bits, int Cq,
                                                           int G, uint16_t* __restrict__ ov) {
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
    ov[(size_t(hd) * Cq + a) * Cq + c] = uint16_t(v);
  }
}
__global__ __launch_bounds__(1024) void sparse_tiles_kernel(const int* __restrict__ q_off, const int* __restrict__ n_q,
                                                            int Cq, int Nv, int n_text, int tmax,
                                                            const uint16_t* __restrict__ ov,
                                                            int* __restrict__ tiles, int* __restrict__ ntiles) {
  __shared__ int buf[1024], small_id[1024], partner[1024], best_of[1024];
  extern __shared__ uint16_t ovs[];  // [n_small][n_small] overlaps of the small groups, when they fit
  const int hd = blockIdx.x, t = threadIdx.x;
  const int nq = n_q[hd];
  const int* qo = q_off + size_t(hd) * (Cq + 1);
  int* out = tiles + size_t(hd) * tmax * 8;
  constexpr int H2 = 2 * kHalfRows;
  const int n_text_tiles = (n_text + H2 - 1) / H2;
  int s = 0;
  if (t < nq) s = qo[t + 1] - qo[t];
  // A group of more than one tile whose last tile would hold at most a half's rows keeps only its
  // full tiles and offers the rest, like a group of at most a half's rows, for pairing.
  const bool big = t < nq && s > kHalfRows;
  const bool rest = big && s > H2 && (s % H2) != 0 && (s % H2) <= kHalfRows;
  const bool small = t < nq && (!big || rest);
  const int my_big_tiles = big ? (rest ? s / H2 : (s + H2 - 1) / H2) : 0;
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
  // rows offered for pairing by group a: the whole group, or the rows past its full tiles
  auto item_row = [&](int a) {
    const int n = qo[a + 1] - qo[a];
    return n > kHalfRows ? qo[a] + (n / H2) * H2 : qo[a];
  };
  auto item_n = [&](int a) {
    const int n = qo[a + 1] - qo[a];
    return n > kHalfRows ? n % H2 : n;
  };
  // small groups by rank; partner[i] = rank of the paired group, -1 while unpaired
  if (small) small_id[small_rank] = t;
  if (t < n_small) partner[t] = -1;
  if (ov) {
    const uint16_t* ovh = ov + size_t(hd) * Cq * Cq;
    // the small groups' overlaps gathered into LDS when they fit
    const bool in_lds = size_t(n_small) * n_small * sizeof(uint16_t) <= kTilesLds;
    __syncthreads();  // small_id complete
    if (in_lds)  // row i by wave, columns by lane
      for (int i = t >> 6; i < n_small; i += blockDim.x >> 6) {
        const uint16_t* src = ovh + size_t(small_id[i]) * Cq;
        for (int j = t & 63; j < n_small; j += 64) ovs[i * n_small + j] = src[small_id[j]];
      }
    // four threads per group (adjacent lanes) split the candidates
    for (int round = 0; round < kPairRounds; ++round) {
      __syncthreads();
      for (int i0 = 0; i0 < n_small; i0 += 256) {
        const int i = i0 + (t >> 2), q = t & 3;
        int best = -1, bestv = -1;
        if (i < n_small && partner[i] < 0) {
          const uint16_t* row = ovh + size_t(small_id[i]) * Cq;
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
    put(base + pair_rank, 0, a, item_row(a), item_n(a));
    put(base + pair_rank, 1, c, item_row(c), item_n(c));
  }
  if (loose) {
    const int a = small_id[t];
    const int tile = base + n_pairs + loose_rank / 2;
    put(tile, loose_rank & 1, a, item_row(a), item_n(a));
    if ((loose_rank & 1) == 0 && loose_rank == n_loose - 1) put(tile, 1, a, item_row(a), 0);  // no partner
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

constexpr int kAttnRows = 128;  // query rows per block of the bf16 kernel

template <int D, int MODE>
static void launch_attn(const AttnParams& P, dim3 grid, int dtype, hipStream_t st) {
  if (dtype == SPR_BF16) {
    constexpr size_t sm = attn32_smem<D, MODE>();
    allow_lds(attn32_kernel<D, MODE>, sm);
    hipLaunchKernelGGL((attn32_kernel<D, MODE>), grid, dim3(256), sm, st, P);
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
  uint16_t* ov = nullptr;
  if (p.Ck <= 64 * kOvWords) {
    ov = ws_ptr<uint16_t>(ws, L.pair_ov);
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
  if (desc.dtype == SPR_BF16) {
    P.v = ws_ptr<void>(ws, L.vh);
    P.vinv = ws_ptr<float>(ws, L.vscale) + desc.B * kv_heads(desc);
  }
  P.g = make_geom(desc);
  P.gk = make_kv_geom(desc);
  P.G = kv_group_size(desc);
  P.tiles = tiles; P.ntiles = ntiles; P.tile_prefix = tprefix; P.tmax = L.tmax; P.BH = BH;
  P.n_kv = part.n_kv; P.kv_off = part.kv_off; P.sel_cnt = route.sel_cnt; P.sel_kv = route.sel_kv;
  P.Cq = p.Cq; P.Ck = p.Ck;
  P.o_sp = o_sp;
  // bf16: one block per tile, 1-D grid over the tile list (an upper bound; blocks past the
  // call's tiles return); fp32: one block per tile half, grid (2 tmax, BH)
  const dim3 grid = desc.dtype == SPR_BF16 ? dim3(unsigned(int64_t(BH) * L.tmax))
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
  if (desc.dtype == SPR_BF16) {
    _Float16* vh;
    P.vinv = make_v_copy(desc, v, ws_ptr<char>(ws, L.pr_vcopy), &vh, st);
    P.v = vh;
  }
  const int BH = desc.B * desc.H;
  const int rows = desc.dtype == SPR_BF16 ? kAttnRows : kTileRows;
  spr_status s = dispatch_d<MODE_PROBE>(P, dim3(ceil_div(M, rows), BH, L.splits), desc.d, desc.dtype, st);
  if (s != SPR_OK) return s;
  hipLaunchKernelGGL(probe_merge_kernel, dim3(BH * M), dim3(128), 0, st, P.part, M, L.splits, desc.d, BH, P.G, P.vinv,
                     o_probe);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_attn_dense(const spr_desc& desc, const void* q, const void* k, const void* v, void* out,
                          int out_dtype, void* ws, hipStream_t st) {
  AttnParams P = {};
  P.q = q; P.k = k; P.v = v;
  P.g = make_geom(desc);
  P.gk = make_kv_geom(desc);
  P.G = kv_group_size(desc);
  P.out = out; P.out_dtype = out_dtype;
  if (desc.dtype == SPR_BF16) {
    _Float16* vh;
    P.vinv = make_v_copy(desc, v, ws, &vh, st);
    P.v = vh;
  }
  const int rows = desc.dtype == SPR_BF16 ? kAttnRows : kTileRows;
  return dispatch_d<MODE_DENSE>(P, dim3(ceil_div(desc.N, rows), desc.B * desc.H), desc.d, desc.dtype, st);
}

// ------------------------------------------------------------------ allocation-free dense call
// Scratch of sparsepr_attn_dense_noalloc: a fixed array in device memory that every call on a
// device shares (the scaled fp16 copy of V and its per-head statistics).  Host code never uses the
// array's name as an address: the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

spr_status noalloc_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPR_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPR_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SPR_OK;
}

}  // namespace spr
