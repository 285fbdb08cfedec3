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

// Per key (group-major order): u_j = v_j . vbar_b(j) and w_j = |v_j|^2, fp64.
template <int DT>
__global__ __launch_bounds__(256) void vstat_kernel(const void* __restrict__ Vp, int N, int Nv, int d,
                                                    const int* __restrict__ kv_perm,
                                                    const int* __restrict__ kv_label,
                                                    const double* __restrict__ vbar, int Ck,
                                                    double* __restrict__ vstat) {
  const int hd = blockIdx.y;
  const int pos = blockIdx.x * 256 + threadIdx.x;
  if (pos >= Nv) return;
  const int b = kv_label[size_t(hd) * Nv + kv_perm[size_t(hd) * Nv + pos]];
  const double* vb = vbar + (size_t(hd) * Ck + b) * d;
  const size_t base = (size_t(hd) * N + pos) * d;
  double u = 0.0, w = 0.0;
  for (int c = 0; c < d; ++c) {
    const double x = load_elem<DT>(Vp, base + c);
    u = fma(x, vb[c], u);
    w = fma(x, x, w);
  }
  vstat[(size_t(hd) * Nv + pos) * 2 + 0] = u;
  vstat[(size_t(hd) * Nv + pos) * 2 + 1] = w;
}

// m_a = max_b qbar_a . kbar_b / sqrt d, one wave per query group.
__global__ __launch_bounds__(256) void route_shift_kernel(const double* __restrict__ qbar,
                                                          const double* __restrict__ kbar,
                                                          const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                          int Cq, int Ck, int d, double* __restrict__ shift) {
  const int hd = blockIdx.y;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= n_q[hd]) return;
  const double* qa = qbar + (size_t(hd) * Cq + a) * d;
  const double inv = 1.0 / sqrt(double(d));
  double m = -1.0e308;
  for (int b = lane; b < n_kv[hd]; b += 64) {
    const double* kb = kbar + (size_t(hd) * Ck + b) * d;
    double s = 0.0;
    for (int c = 0; c < d; ++c) s = fma(qa[c], kb[c], s);
    m = fmax(m, s * inv);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  if (lane == 0) shift[size_t(hd) * Cq + a] = m;
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// Scores for a tile of 64 query groups x 16 K/V groups.  The keys of the 16 groups are
// contiguous in group-major order and stream through LDS in 64-key chunks.  Logits come from
// v_mfma_f64_16x16x4f64 (each wave: 16 query groups, A fragments of qbar kept in registers;
// lane l, slot v holds the logit of group (l / 16) + 4 v and key l % 16 of a 16-key tile);
// E u and E^2 w are added to per-(a, b) accumulators in LDS.
template <int DT, int D>
__global__ __launch_bounds__(256) void route_score_kernel(const void* __restrict__ Kp, int N, int Nv,
                                                          const double* __restrict__ qbar,
                                                          const double* __restrict__ kbar,
                                                          const double* __restrict__ vbar,
                                                          const int* __restrict__ kv_off,
                                                          const int* __restrict__ n_q,
                                                          const int* __restrict__ n_kv, int Cq, int Ck,
                                                          const double* __restrict__ shift,
                                                          const double* __restrict__ vstat,
                                                          double* __restrict__ scores) {
  constexpr int KSD = D + 4;  // key tile row stride (floats)
  extern __shared__ double sm[];
  const int hd = blockIdx.z;
  const int a0 = blockIdx.x * 64, b0 = blockIdx.y * 16;
  const int nq = n_q[hd], nkv = n_kv[hd];
  if (a0 >= nq || b0 >= nkv) return;
  const int b1 = min(b0 + 16, nkv);
  double* acc = sm;                                       // [64][16][2]
  float* Ks = reinterpret_cast<float*>(acc + 64 * 16 * 2);  // [64][KSD]
  __shared__ double us[64], wsv[64], shs[64];
  __shared__ int grp[64];
  const int* off = kv_off + size_t(hd) * (Ck + 1);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4, r16 = lane & 15;
  double qa[D / 4];
  {
    const int a = a0 + w * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) qa[ks] = a < nq ? qbar[(size_t(hd) * Cq + a) * D + ks * 4 + gq] : 0.0;
  }
  for (int e = threadIdx.x; e < 64 * 32; e += 256) acc[e] = 0.0;
  if (threadIdx.x < 64) {
    const int a = a0 + threadIdx.x;
    shs[threadIdx.x] = a < nq ? shift[size_t(hd) * Cq + a] : 0.0;
  }
  const double inv = 1.0 / sqrt(double(D));
  const int k0 = off[b0], k1 = off[b1];
  for (int kc = k0; kc < k1; kc += 64) {
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * D; e += 256) {
      const int jl = e / D, c = e % D, pos = kc + jl;
      Ks[jl * KSD + c] = pos < k1 ? load_elem<DT>(Kp, (size_t(hd) * N + pos) * D + c) : 0.f;
    }
    if (threadIdx.x < 64) {
      const int pos = kc + threadIdx.x;
      if (pos < k1) {
        us[threadIdx.x] = vstat[(size_t(hd) * Nv + pos) * 2 + 0];
        wsv[threadIdx.x] = vstat[(size_t(hd) * Nv + pos) * 2 + 1];
        int lo = b0, hi = b1 - 1;  // group of this key: last b with off[b] <= pos
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        grp[threadIdx.x] = lo - b0;
      } else {
        grp[threadIdx.x] = -1;
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
      const int jl = kt * 16 + r16;
      if (kc + kt * 16 >= k1) break;  // uniform
      f64x4_t lg = {0.0, 0.0, 0.0, 0.0};
      const float* kr = Ks + jl * KSD + gq;
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) lg = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], double(kr[ks * 4]), lg, 0, 0, 0);
      const int gb = grp[jl];
      if (gb >= 0) {
        const double uu = us[jl], ww = wsv[jl];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int al = w * 16 + gq + 4 * v;
          const double E = exp(lg[v] * inv - shs[al]);
          atomicAdd(&acc[(al * 16 + gb) * 2 + 0], E * uu);
          atomicAdd(&acc[(al * 16 + gb) * 2 + 1], E * E * ww);
        }
      }
    }
  }
  __syncthreads();
  // combine: s_ab = A^2 |vbar|^2 - 2 A S1 / |G| + S2 / |G|
  for (int e = threadIdx.x; e < 64 * 16; e += 256) {
    const int al = e >> 4, gb = e & 15, a = a0 + al, b = b0 + gb;
    if (a >= nq || b >= b1) continue;
    const double* qb = qbar + (size_t(hd) * Cq + a) * D;
    const double* kb = kbar + (size_t(hd) * Ck + b) * D;
    const double* vb = vbar + (size_t(hd) * Ck + b) * D;
    double l = 0.0, vn = 0.0;
    for (int c = 0; c < D; ++c) {
      l = fma(qb[c], kb[c], l);
      vn = fma(vb[c], vb[c], vn);
    }
    const double A = exp(l * inv - shs[al]);
    const double g = double(off[b + 1] - off[b]);
    const double sc = A * A * vn - 2.0 * A * acc[(al * 16 + gb) * 2 + 0] / g + acc[(al * 16 + gb) * 2 + 1] / g;
    scores[(size_t(hd) * Cq + a) * Ck + b] = sc;
  }
}

// Budgeted prefix of Sec. 4.3 for one query group: sort the n_kv scores descending (ties to
// the lower group) with a bitonic sort in LDS, then take the shortest prefix whose key count
// reaches Tk (at least one group, all groups when out of reach).  Block n_q handles the text
// query group, which selects every group.
__global__ __launch_bounds__(256) void route_select_kernel(const double* __restrict__ scores,
                                                           const int* __restrict__ kv_off,
                                                           const int* __restrict__ q_off,
                                                           const int* __restrict__ n_q, const int* __restrict__ n_kv,
                                                           int Cq, int Ck, int n_text, int64_t Tk,
                                                           int* __restrict__ sel_cnt, int* __restrict__ sel_kv,
                                                           int64_t* __restrict__ pairs, int* __restrict__ gstat) {
  __shared__ double ks[1024];
  __shared__ int ids[1024];
  __shared__ int buf[1024];
  __shared__ int Ls;
  const int hd = blockIdx.y, a = blockIdx.x;
  const int nq = n_q[hd], nkv = n_kv[hd];
  const int* off = kv_off + size_t(hd) * (Ck + 1);
  int* out = sel_kv + (size_t(hd) * (Cq + 1) + a) * (Ck + 1);
  if (a > nq || (a == nq && n_text == 0)) return;
  if (a == nq) {  // text query rows: every group
    for (int b = threadIdx.x; b <= nkv; b += 256) out[b] = b;
    if (threadIdx.x == 0) sel_cnt[size_t(hd) * (Cq + 1) + a] = nkv + 1;
    return;
  }
  int P = 1;
  while (P < nkv) P <<= 1;
  for (int i = threadIdx.x; i < P; i += 256) {
    ks[i] = i < nkv ? scores[(size_t(hd) * Cq + a) * Ck + i] : -1.0e308;
    ids[i] = i < nkv ? i : 0x7fffffff;
  }
  __syncthreads();
  // bitonic sort, "before" = larger score, then lower id
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P; i += 256) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const double si = ks[i], sj = ks[j];
          const int ii = ids[i], ij = ids[j];
          const bool j_before_i = (sj > si) || (sj == si && ij < ii);
          if (j_before_i == up) {
            ks[i] = sj; ks[j] = si;
            ids[i] = ij; ids[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  // prefix sums of group sizes in ranked order (4 consecutive ranks per thread)
  int loc[4];
  int s = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x * 4 + u;
    loc[u] = i < nkv ? off[ids[i] + 1] - off[ids[i]] : 0;
    s += loc[u];
  }
  buf[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int y = threadIdx.x >= o ? buf[threadIdx.x - o] : 0;
    __syncthreads();
    buf[threadIdx.x] += y;
    __syncthreads();
  }
  if (threadIdx.x == 0) Ls = nkv;
  __syncthreads();
  int cum = buf[threadIdx.x] - s;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x * 4 + u;
    cum += loc[u];
    if (i < nkv && cum >= Tk && cum - loc[u] < Tk) Ls = i + 1;  // unique crossing
  }
  __syncthreads();
  const int L = Ls;
  int64_t keys = 0;
  for (int i = threadIdx.x; i < L; i += 256) {
    out[i] = ids[i];
    keys += off[ids[i] + 1] - off[ids[i]];
  }
  __syncthreads();
  __shared__ int64_t red[32];
  keys = block_sum_i64(keys, red);
  if (threadIdx.x == 0) {
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

template <int DT>
static spr_status route_impl(const spr_desc& desc, const spr_part_params& p, const spr_partition& part, int M,
                             int64_t Tk, spr_route& out, void* ws, const Workspace& L, hipStream_t st) {
  const int BH = desc.B * desc.H, d = desc.d, N = desc.N, Nv = N - desc.n_text;
  double* vstat = ws_ptr<double>(ws, L.vstat);
  double* shift = ws_ptr<double>(ws, L.shift);
  double* scores = out.scores ? out.scores : ws_ptr<double>(ws, L.scores);
  int* gstat = ws_ptr<int>(ws, L.gstat);
  int* pstat = ws_ptr<int>(ws, L.pstat);
  hipLaunchKernelGGL(vstat_kernel<DT>, dim3(ceil_div(Nv, 256), BH), dim3(256), 0, st, part.Vp, N, Nv, d,
                     part.kv_perm, part.kv_label, part.vbar, p.Ck, vstat);
  hipLaunchKernelGGL(route_shift_kernel, dim3(ceil_div(p.Cq, 4), BH), dim3(256), 0, st, part.qbar, part.kbar,
                     part.n_q, part.n_kv, p.Cq, p.Ck, d, shift);
  SPR_CHECK_LAUNCH();
  const size_t smem = 64 * 16 * 2 * sizeof(double) + size_t(64) * (d + 4) * sizeof(float);
  const dim3 sgrid(ceil_div(p.Cq, 64), ceil_div(p.Ck, 16), BH);
  if (d == 128)
    hipLaunchKernelGGL((route_score_kernel<DT, 128>), sgrid, dim3(256), smem, st, part.Kp, N, Nv, part.qbar, part.kbar,
                       part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, shift, vstat, scores);
  else
    hipLaunchKernelGGL((route_score_kernel<DT, 64>), sgrid, dim3(256), smem, st, part.Kp, N, Nv, part.qbar, part.kbar,
                       part.vbar, part.kv_off, part.n_q, part.n_kv, p.Cq, p.Ck, shift, vstat, scores);
  SPR_CHECK_LAUNCH();
  hipLaunchKernelGGL(zero_i64_kernel, dim3(ceil_div(BH, 256)), dim3(256), 0, st, out.pairs, BH);
  hipLaunchKernelGGL(route_select_kernel, dim3(p.Cq + 1, BH), dim3(256), 0, st, scores, part.kv_off, part.q_off,
                     part.n_q, part.n_kv, p.Cq, p.Ck, desc.n_text, Tk, out.sel_cnt, out.sel_kv, out.pairs, gstat);
  SPR_CHECK_LAUNCH();
  hipLaunchKernelGGL(route_finalize_kernel, dim3(BH), dim3(1024), 0, st, part.q_off, part.n_q, p.Cq, N, Nv,
                     desc.n_text, M, out.pairs, out.rho_exec, pstat);
  hipLaunchKernelGGL(probe_select_kernel, dim3(p.Cq, BH), dim3(256), 0, st, part.q_off, part.q_perm, part.n_q,
                     part.qdist, pstat, p.Cq, Nv, M, out.probe_idx, out.probe_w);
  SPR_CHECK_LAUNCH();
  return SPR_OK;
}

spr_status run_route(const spr_desc& desc, const spr_part_params& p, const spr_partition& part, double rho, int M,
                     int64_t Tk, spr_route& out, void* ws, const Workspace& L, hipStream_t st) {
  (void)rho;
  if (desc.dtype == SPR_BF16) return route_impl<SPR_BF16>(desc, p, part, M, Tk, out, ws, L, st);
  return route_impl<SPR_F32>(desc, p, part, M, Tk, out, ws, L, st);
}

}  // namespace spr
