// Routing and probe selection ("Partition the Support, Reconstruct the Residual",
// Sec. 4.3, App. B.3, App. A.2) on gfx950.
//
// The value-error score of App. B.3 expands, per (query group a, K/V group b), to
//   |G_b| s_ab = A^2 |G_b| |vbar_b|^2 - 2 A sum_j E_j (v_j . vbar_b) + sum_j E_j^2 |v_j|^2
// with A = e^{qbar_a kbar_b / sqrt d - m_a} and E_j = e^{qbar_a k_j / sqrt d - m_a}, so one
// fp64 pass over all (a, key) logits with two segmented sums per (a, b) gives every score.
// The shift m_a (the largest centroid logit of row a) multiplies a whole row by one positive
// factor and leaves the ranking unchanged.
#include "common.hpp"
#include "stages.hpp"

namespace spr {

// Per key (group-major order): u_j = v_j . vbar_b(j) and w_j = |v_j|^2, fp64.  d / 8 lanes per
// key, eight consecutive elements each (one 16-byte load for bf16), reduced across those lanes.
template <int DT>
__global__ __launch_bounds__(256) void vstat_kernel(const void* __restrict__ Vp, int N, int Nv, int d,
                                                    const int* __restrict__ kv_perm,
                                                    const int* __restrict__ kv_label,
                                                    const double* __restrict__ vbar, int Ck,
                                                    double* __restrict__ vstat) {
  const int hd = blockIdx.y;
  const int L = d >> 3;
  const int pos = blockIdx.x * (256 / L) + threadIdx.x / L, sub = threadIdx.x % L;
  double u = 0.0, w = 0.0;
  if (pos < Nv) {
    const int b = kv_label[size_t(hd) * Nv + kv_perm[size_t(hd) * Nv + pos]];
    const double* vb = vbar + (size_t(hd) * Ck + b) * d + sub * 8;
    float x[8];
    load8<DT>(Vp, (int64_t(hd) * N + pos) * d + sub * 8, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u = fma(double(x[c]), vb[c], u);
      w = fma(double(x[c]), double(x[c]), w);
    }
  }
  for (int o = L >> 1; o > 0; o >>= 1) {
    u += __shfl_xor(u, o);
    w += __shfl_xor(w, o);
  }
  if (pos < Nv && sub == 0) {
    vstat[(size_t(hd) * Nv + pos) * 2 + 0] = u;
    vstat[(size_t(hd) * Nv + pos) * 2 + 1] = w;
  }
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// Centroid logits lbar_ab = qbar_a . kbar_b / sqrt d on the fp64 matrix cores.  One block per
// 64 query groups x 64 K/V groups of a head: wave w owns query groups a0 + 16 w .. + 15 (A
// fragments of qbar in registers: lane l holds qbar[a0 + 16 w + l % 16] at columns 4 ks + l / 16)
// and the block's four tiles of 16 K/V groups, each its own accumulation chain; lane l, slot v
// of tile t holds the logit of query group 16 w + l / 16 + 4 v and K/V group b0 + 16 t + l % 16.
template <int D>
__global__ __launch_bounds__(256) void centroid_logits_kernel(const double* __restrict__ qbar,
                                                              const double* __restrict__ kbar,
                                                              const int* __restrict__ n_q,
                                                              const int* __restrict__ n_kv, int Cq, int Ck, int G,
                                                              double* __restrict__ lbar) {
  const int hd = blockIdx.z, hk = hd / G, a0 = blockIdx.x * 64, b0 = blockIdx.y * 64;  // query head, K/V head
  const int nq = n_q[hd], nkv = n_kv[hk];
  if (a0 >= nq || b0 >= nkv) return;
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
  const double* kb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) kb[t] = kbar + (size_t(hk) * Ck + min(b0 + 16 * t + r16, nkv - 1)) * D + gq;
  f64x4_t lg[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) lg[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks)
#pragma unroll
    for (int t = 0; t < 4; ++t) lg[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], kb[t][ks * 4], lg[t], 0, 0, 0);
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
        us[jl] = jl < n ? vstat[(size_t(hk) * Nv + p0 + jl) * 2 + 0] : 0.0;
        wsv[jl] = jl < n ? vstat[(size_t(hk) * Nv + p0 + jl) * 2 + 1] : 0.0;
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

// Budgeted prefix of Sec. 4.3 for one query group, one wave per group: the n_kv scores sorted
// descending (ties to the lower group) by a bitonic network over P = 64 E entries held E per
// lane in rank order (lane l holds ranks l E .. l E + E - 1; strides below E are exchanges
// inside a lane, larger strides between lanes l and l ^ (stride / E)), then the shortest prefix
// whose key count reaches Tk (at least one group, all groups when out of reach).  The group past
// the last query group (index n_q) is the text query group, which selects every group.
template <int E>
__global__ __launch_bounds__(256) void route_select_kernel(const double* __restrict__ scores,
                                                           const int* __restrict__ kv_off,
                                                           const int* __restrict__ q_off,
                                                           const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                           int Cq, int Ck, int G, int n_text, int64_t Tk,
                                                           int* __restrict__ sel_cnt, int* __restrict__ sel_kv,
                                                           int64_t* __restrict__ pairs, int* __restrict__ gstat) {
  constexpr int P = 64 * E;
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
  double sc[E];
  int id[E];
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int i = lane * E + t;
    sc[t] = i < nkv ? scores[(size_t(hd) * Cq + a) * Ck + i] : -1.0e308;
    id[t] = i < nkv ? i : 0x7fffffff;
  }
  // "before" = larger score, then lower id
  auto before = [](double s1, int i1, double s2, int i2) { return s1 > s2 || (s1 == s2 && i1 < i2); };
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride >= E; stride >>= 1) {  // between lanes
      const int pl = lane ^ (stride / E);
      const bool low = lane < pl, up = ((lane * E) & size) == 0;
#pragma unroll
      for (int t = 0; t < E; ++t) {
        const double os = __shfl(sc[t], pl);
        const int oi = __shfl(id[t], pl);
        const bool mine_first = before(sc[t], id[t], os, oi);
        // the lower position keeps the entry that comes first in this block's direction
        const bool keep_mine = (low == up) ? mine_first : !mine_first;
        if (!keep_mine) {
          sc[t] = os;
          id[t] = oi;
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
          if (before(sc[u], id[u], sc[t], id[t]) == up) {
            const double ts = sc[t];
            const int ti = id[t];
            sc[t] = sc[u]; id[t] = id[u];
            sc[u] = ts; id[u] = ti;
          }
        }
      }
    }
  }
  // group sizes in ranked order and their running sum across the wave
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
    sel_cnt[size_t(hd) * (Cq + 1) + a] = cnt;
    if (keys < Tk) atomicOr(gstat + hd * 8 + 0, SPR_HS_BUDGET_UNREACHED);
    const int64_t ga = q_off[size_t(hd) * (Cq + 1) + a + 1] - q_off[size_t(hd) * (Cq + 1) + a];
    atomicAdd(reinterpret_cast<unsigned long long*>(pairs + hd), (unsigned long long)(ga * (keys + n_text)));
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
  for (int p = r0 + threadIdx.x; p < r1; p += 256) {
    const int i = pm[p];
    const double di = dd[i];
    int rank = 0;
    for (int o = r0; o < r1; ++o) {
      const int io = pm[o];
      const double dx = dd[io];
      rank += (dx < di) || (dx == di && io < i);
    }
    if (rank < m) {
      probe_idx[size_t(hd) * M + po + rank] = i;
      probe_w[size_t(hd) * M + po + rank] = double(r1 - r0) / double(m);
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
    hipLaunchKernelGGL(centroid_logits_kernel<128>, lgrid, dim3(256), 0, st, part.qbar, part.kbar, part.n_q,
                       part.n_kv, p.Cq, p.Ck, G, lbar);
    hipLaunchKernelGGL(logit_shift_kernel, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, lbar, part.n_q, part.n_kv,
                       p.Cq, p.Ck, G, shift);
    allow_lds(route_score_kernel<DT, 128>, route_score_smem<128>());
    hipLaunchKernelGGL((route_score_kernel<DT, 128>), sgrid, dim3(256), route_score_smem<128>(), st, part.Kp, N, Nv,
                       part.qbar, lbar,
                       part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, G, shift, vstat, scores);
  } else {
    hipLaunchKernelGGL(centroid_logits_kernel<64>, lgrid, dim3(256), 0, st, part.qbar, part.kbar, part.n_q,
                       part.n_kv, p.Cq, p.Ck, G, lbar);
    hipLaunchKernelGGL(logit_shift_kernel, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, lbar, part.n_q, part.n_kv,
                       p.Cq, p.Ck, G, shift);
    allow_lds(route_score_kernel<DT, 64>, route_score_smem<64>());
    hipLaunchKernelGGL((route_score_kernel<DT, 64>), sgrid, dim3(256), route_score_smem<64>(), st, part.Kp, N, Nv,
                       part.qbar, lbar,
                       part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, G, shift, vstat, scores);
  }
  SPR_CHECK_LAUNCH();
  hipLaunchKernelGGL(zero_i64_kernel, dim3(ceil_div(BH, 256)), dim3(256), 0, st, out.pairs, BH);
  {
    const dim3 grid(ceil_div(p.Cq + 1, 4), BH);
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
