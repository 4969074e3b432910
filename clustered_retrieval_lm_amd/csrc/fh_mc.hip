// Monte-Carlo estimate of the two-stage sampler's distribution over the whole vocabulary
// (FlashHead paper, Appendix D.1 "Monte-Carlo Simulation"): the average, over N probe sets
// S_i drawn like the sampler's stage 1, of the full conditional p(v | h, S_i), the softmax of
// z / tau over the tokens of S_i (zero elsewhere); entries no S_i reaches are optionally
// clipped to the smallest non-zero estimate of the row.
//
// The conditional factors through per-cluster statistics.  With M_k = max_j z_kj / tau and
// Zc_k = sum_j exp(z_kj / tau - M_k), the probe set S contributes to token (k, j), k in S,
//   exp(z_kj / tau - M_k) * w_k(S),   w_k(S) = exp(M_k - m_S) / sum_{l in S} Zc_l exp(M_l - m_S),
// m_S = max_{l in S} M_l.  So each probe set adds p weights into a per-cluster accumulator
// A_k = sum_i [k in S_i] w_k(S_i) -- c values instead of a V-vector -- and one pass at the
// end expands est(k, j) = exp(z_kj / tau - M_k) A_k / N into vocabulary order.
//
// Kernels, in stream order (the centroid logits s come from the stage-1 scores, the token
// logits z, in tile order, from a dense pass over the tiles):
//   k_mc_stats   one thread per (row, cluster): M_k, Zc_k; clears A_k and the row minimum;
//   k_mc_prep, k_mc_grid, k_mc_pick   s / tau (fp32, the division the sampler's keys use)
//                and a prefilter threshold t0 per row (below);
//   k_mc_sets    one 1024-thread workgroup per (probe set i, row): the stage-1 keys
//                s / tau + G(seed, row, step = i, stream 0, k) (the sampler's own keys at
//                step i), the exact top-p, then one thread per kept cluster (ascending id)
//                adds w_k(S_i) into A (fp64 atomics: the order of the additions, and so the
//                last bits, vary by run);
//   k_mc_expand  one thread per (row, token slot): the estimate, scattered to out[row][C2T],
//                and the row's smallest non-zero estimate;
//   k_mc_clip    zeros replaced by that minimum (if clipping).
// Softmax statistics, weights and estimates are fp64.
//
// Prefilter.  The key of cluster k exceeds t with probability 1 - exp(-exp(s_k / tau - t)),
// so the expected number of keys above t is known per row.  t0 is the largest of 256 evenly
// spaced thresholds at which that expectation still reaches p + 8 sqrt(p) + 16 (a count below
// p is then more than seven standard deviations away); a probe set histograms only its keys >= t0
// (select_interval) instead of all c.  If fewer than p keys reach t0 -- a many-sigma event --
// the set falls back to the full selection, so the result is exact either way.
#include <hip/hip_runtime.h>

#include "fh_device.h"
#include "fh_internal.h"
#include "fh_select.h"

namespace fh {
namespace {

constexpr int kMcThreads = 256;

__device__ __forceinline__ int wave_sum_i32(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

__global__ __launch_bounds__(kMcThreads) void k_mc_stats(const float* z, int B, int c, int b, double tau,
                                                         double* M, double* Zc, double* A, uint64_t* minneg) {
  const int64_t i = (int64_t)blockIdx.x * kMcThreads + threadIdx.x;     // row * c + cluster
  if (i < (int64_t)B * c) {
    const float* zk = z + i * b;
    double m = -INFINITY;
    for (int j = 0; j < b; ++j) m = fmax(m, (double)zk[j] / tau);
    double s = 0.0;
    for (int j = 0; j < b; ++j) s += exp((double)zk[j] / tau - m);
    M[i] = m;
    Zc[i] = s;
    A[i] = 0.0;
  }
  if (i < B) minneg[i] = 0ull;
}

constexpr int kGrid = 256;      // candidate thresholds evaluated per row

// s / tau per cluster and the row's range [min - 3, max + 17] of possible keys (the Gumbel
// draws lie in [-ln(24 ln 2), -ln(-ln(1 - 2^-24))] ~ [-2.82, 16.7]).
__global__ __launch_bounds__(kSelThreads) void k_mc_prep(const float* s, int c, float tau, float* stau,
                                                         float* range) {
  __shared__ float rmin[kSelThreads / kWave], rmax[kSelThreads / kWave];
  const int r = blockIdx.x, tid = threadIdx.x, NT = blockDim.x, nw = NT >> 6, wave = tid >> 6;
  const float* sr = s + (size_t)r * c;
  float* ar = stau + (size_t)r * c;
  float lo = INFINITY, hi = -INFINITY;
  for (int k = tid; k < c; k += NT) {
    const float a = sr[k] / tau;
    ar[k] = a;
    lo = fminf(lo, a);
    hi = fmaxf(hi, a);
  }
  lo = wave_minmax_f32<false>(lo);
  hi = wave_minmax_f32<true>(hi);
  if ((tid & 63) == 0) { rmin[wave] = lo; rmax[wave] = hi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < nw; ++w) { lo = fminf(lo, rmin[w]); hi = fmaxf(hi, rmax[w]); }
    range[2 * r] = lo - 3.0f;
    range[2 * r + 1] = hi + 17.0f;
  }
}

__device__ __forceinline__ float grid_point(const float* range, int r, int j) {
  const float lo = range[2 * r], hi = range[2 * r + 1];
  return lo + (hi - lo) * ((float)j / (float)kGrid);
}

// grid (kGrid, B): the expected number of keys above candidate threshold j of row r.
__global__ __launch_bounds__(kMcThreads) void k_mc_grid(const float* stau, int c, const float* range, float* mu) {
  __shared__ float part[kMcThreads / kWave];
  const int j = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const float t = grid_point(range, r, j);
  const float* ar = stau + (size_t)r * c;
  float m = 0.0f;
  for (int k = tid; k < c; k += kMcThreads) m += -expm1f(-expf(ar[k] - t));
  m = wave_sum(m);
  if ((tid & 63) == 0) part[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) mu[(size_t)r * kGrid + j] = part[0] + part[1] + part[2] + part[3];
}

// One wave per row: the largest candidate threshold whose expectation reaches the target, as an
// order-preserving key (0: no filtering -- the target is out of reach or the range is not finite).
__global__ __launch_bounds__(kWave) void k_mc_pick(const float* range, const float* mu, int c, int p,
                                                   uint32_t* t0u) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const float target = (float)p + 8.0f * sqrtf((float)p) + 16.0f;
  int best = -1;
  for (int j = lane; j < kGrid; j += kWave)
    if (mu[(size_t)r * kGrid + j] >= target) best = j;
  for (int o = 32; o >= 1; o >>= 1) best = max(best, __shfl_xor(best, o, kWave));
  if (lane == 0) {
    const float lo = range[2 * r], hi = range[2 * r + 1];
    const bool ok = best >= 0 && target < (float)c && hi - lo < 1e30f;
    t0u[r] = ok ? ord_key(grid_point(range, r, best)) : 0u;
  }
}

// Block-wide max / sum of one double per thread; every thread gets the result.  The order of
// the additions is fixed (xor butterfly in each wave, then the waves in order).
template <bool MAX>
__device__ __forceinline__ double block_reduce_f64(double v, double* red) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double y = __shfl_xor(v, o, kWave);
    v = MAX ? fmax(v, y) : v + y;
  }
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < nw; ++w) r = MAX ? fmax(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

struct McParams {
  const float* stau;     // [B][c] centroid logits / tau
  const uint32_t* t0u;   // [B] prefilter threshold (order-preserving; 0: none)
  const double* M;       // [B][c]
  const double* Zc;      // [B][c]
  double* A;             // [B][c] accumulated weights
  int c, p;
  float tau;
  uint64_t seed;
  uint64_t set0;         // index of the first probe set of this launch
};

// Probe-set weights shared by both probe-set kernels: S holds the kept bitmap with its prefix
// offsets; thread q (q < p, strided) takes the q-th kept cluster in ascending id.
__device__ __forceinline__ void add_set_weights(const McParams& a, int r, const SelShared& S, double* red) {
  const int tid = threadIdx.x, NT = blockDim.x, c = a.c;
  const int nwords = (c + 31) >> 5;
  const double* Mr = a.M + (size_t)r * c;
  const double* Zr = a.Zc + (size_t)r * c;
  double* Ar = a.A + (size_t)r * c;
  int k0 = -1;
  double M0 = -INFINITY, Z0 = 0.0;
  if (tid < a.p) {
    k0 = kept_at(S, nwords, tid);
    M0 = Mr[k0];
    Z0 = Zr[k0];
  }
  double mloc = M0;
  for (int q = tid + NT; q < a.p; q += NT) mloc = fmax(mloc, Mr[kept_at(S, nwords, q)]);
  const double m = block_reduce_f64<true>(mloc, red);
  const double e0 = k0 >= 0 ? exp(M0 - m) : 0.0;
  double zl = Z0 * e0;
  for (int q = tid + NT; q < a.p; q += NT) {
    const int k = kept_at(S, nwords, q);
    zl += Zr[k] * exp(Mr[k] - m);
  }
  const double inv = 1.0 / block_reduce_f64<false>(zl, red);
  if (k0 >= 0) unsafeAtomicAdd(&Ar[k0], e0 * inv);
  for (int q = tid + NT; q < a.p; q += NT) {
    const int k = kept_at(S, nwords, q);
    unsafeAtomicAdd(&Ar[k], exp(Mr[k] - m) * inv);
  }
}

// Thread t holds the keys of clusters 4 (t + j NT) + e, j < KV, e < 4 (the four words of one
// Philox block), as order-preserving uint32.  512-thread workgroups at <= 128 registers let two
// probe sets share a CU, so one set's selection overlaps the other's key generation; above
// 16384 clusters the workgroup has 1024 threads.
template <int KV, int NT_>
__global__ __launch_bounds__(NT_, NT_ == 512 ? 4 : 1) void k_mc_sets(McParams a) {
  __shared__ SelShared S;
  __shared__ double red[kSelThreads / kWave];
  __shared__ int cnt_w[kSelThreads / kWave];
  __shared__ uint32_t max_w[kSelThreads / kWave];
  const int r = blockIdx.y, tid = threadIdx.x, NT = blockDim.x, c = a.c, wave = tid >> 6, nw = NT >> 6;
  const Rng g = make_rng(a.seed, a.set0 + blockIdx.x);
  const float* sr = a.stau + (size_t)r * c;
  const uint32_t t0 = a.t0u[r];
  uint32_t u[KV][4];
  int cnt = 0;
  uint32_t umax = 0u;
#pragma unroll
  for (int j = 0; j < KV; ++j) {
    const int id0 = 4 * (tid + j * NT);
    u[j][0] = u[j][1] = u[j][2] = u[j][3] = 0u;
    if (id0 < c) {
      const uint4 w = rng_block(g, (uint32_t)r, 0u, (uint32_t)id0 >> 2);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (id0 + e < c) {
          const uint32_t x = ord_key(gumbel_key(sr[id0 + e], ws[e]));
          u[j][e] = x;
          cnt += x >= t0;
          umax = max(umax, x);
        }
    }
  }
  for (int i = tid; i < kSelBins; i += NT) S.hist[i] = 0;
  for (int i = tid; i < kMaxWords; i += NT) S.bitmap[i] = 0u;
  cnt = wave_sum_i32(cnt);
  umax = wave_minmax_u32<true>(umax);
  if ((tid & 63) == 0) { cnt_w[wave] = cnt; max_w[wave] = umax; }
  __syncthreads();
  cnt = 0;
  umax = 0u;
  for (int w = 0; w < nw; ++w) { cnt += cnt_w[w]; umax = max(umax, max_w[w]); }
  uint32_t Tu;
  int Tid;
  if (t0 != 0u && cnt >= a.p) select_interval<KV>(u, c, S, t0, umax, a.p, cnt, Tu, Tid);
  else select_regs<KV>(u, c, a.p, S, Tu, Tid);
  mark_kept<KV>(u, c, Tu, Tid, S);
  add_set_weights(a, r, S, red);
}

constexpr int kListCap = 2048;     // candidate keys a probe set keeps in LDS
constexpr int kListThreads = 512;

// Keys recomputed from Philox on every call (the rare fallback of k_mc_sets_list).
struct PhiloxKeys {
  const float* sr;
  Rng g;
  uint32_t row;
  int c;
  template <class F>
  __device__ __forceinline__ void operator()(F&& f) const {
    for (int id4 = threadIdx.x; 4 * id4 < c; id4 += blockDim.x) {
      const uint4 w = rng_block(g, row, 0u, (uint32_t)id4);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = 4 * id4 + e;
        if (id < c) f(ord_key(gumbel_key(sr[id], ws[e])), id);
      }
    }
  }
};

// The candidate list in LDS.
struct ListKeys {
  const uint32_t* lu;
  const int* lid;
  int n;
  template <class F>
  __device__ __forceinline__ void operator()(F&& f) const {
    for (int i = threadIdx.x; i < n; i += blockDim.x) f(lu[i], lid[i]);
  }
};

// One probe set per workgroup, keys not held in registers: each key is computed once and, if
// it reaches the row's threshold t0, appended to an LDS list (wave-aggregated slots); the
// exact selection then runs over the list (keys below t0 cannot be kept when at least p keys
// reach t0).  If the list holds fewer than p keys or overflows, or the row has no threshold,
// the set recomputes its keys for every pass of the full selection instead.  Small register
// and LDS footprints let four probe sets share a CU.
__global__ __launch_bounds__(kListThreads, 8) void k_mc_sets_list(McParams a) {
  __shared__ SelShared S;
  __shared__ uint32_t lu[kListCap];
  __shared__ int lid[kListCap];
  __shared__ int nlist;
  __shared__ uint32_t max_w[kListThreads / kWave], min_w[kListThreads / kWave];
  __shared__ double red[kListThreads / kWave];
  const int r = blockIdx.y, tid = threadIdx.x, NT = blockDim.x, c = a.c, lane = tid & 63, wave = tid >> 6;
  const int nw = NT >> 6;
  const Rng g = make_rng(a.seed, a.set0 + blockIdx.x);
  const float* sr = a.stau + (size_t)r * c;
  const uint32_t t0 = a.t0u[r];
  if (tid == 0) nlist = 0;
  for (int i = tid; i < kSelBins; i += NT) S.hist[i] = 0;
  for (int i = tid; i < kMaxWords; i += NT) S.bitmap[i] = 0u;
  __syncthreads();
  uint32_t umax = 0u, umin = 0xFFFFFFFFu;
  const int nblk = (c + 3) >> 2;
  for (int b0 = 0; b0 < nblk; b0 += NT) {            // whole waves iterate together
    const int id4 = b0 + tid;
    uint32_t xs[4] = {0u, 0u, 0u, 0u};
    if (id4 < nblk) {
      const uint4 w = rng_block(g, (uint32_t)r, 0u, (uint32_t)id4);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * id4 + e < c) {
          xs[e] = ord_key(gumbel_key(sr[4 * id4 + e], ws[e]));
          umax = max(umax, xs[e]);
          umin = min(umin, xs[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool take = id4 < nblk && 4 * id4 + e < c && t0 != 0u && xs[e] >= t0;
      const uint64_t bal = __ballot(take);
      if (bal) {
        const int leader = __ffsll((unsigned long long)bal) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&nlist, __popcll(bal));
        base = __shfl(base, leader, kWave);
        if (take) {
          const int slot = base + lane_prefix(bal);
          if (slot < kListCap) { lu[slot] = xs[e]; lid[slot] = 4 * id4 + e; }
        }
      }
    }
  }
  umax = wave_minmax_u32<true>(umax);
  umin = wave_minmax_u32<false>(umin);
  if (lane == 0) { max_w[wave] = umax; min_w[wave] = umin; }
  __syncthreads();
  for (int w = 0; w < nw; ++w) { umax = max(umax, max_w[w]); umin = min(umin, min_w[w]); }
  const int n = nlist;
  uint32_t Tu;
  int Tid;
  if (t0 != 0u && n >= a.p && n <= kListCap) {
    const ListKeys keys{lu, lid, n};
    select_interval_each(keys, c, S, t0, umax, a.p, n, Tu, Tid);
    mark_kept_each(keys, c, Tu, Tid, S);
  } else {
    const PhiloxKeys keys{sr, g, (uint32_t)r, c};
    select_interval_each(keys, c, S, umin, umax, a.p, c, Tu, Tid);
    mark_kept_each(keys, c, Tu, Tid, S);
  }
  add_set_weights(a, r, S, red);
}

// grid (ceil(V / kMcThreads), B): a wave never spans two rows.
__global__ __launch_bounds__(kMcThreads) void k_mc_expand(const float* z, const int32_t* c2t, const double* M,
                                                          const double* A, int c, int b, int V, double tau,
                                                          double inv_n, double* out, uint64_t* minneg) {
  const int r = blockIdx.y;
  const int slot = blockIdx.x * kMcThreads + threadIdx.x;           // k b + j
  uint64_t key = 0ull;
  if (slot < V) {
    const int k = slot / b;
    const size_t rk = (size_t)r * c + k;
    const double Ak = A[rk];
    double est = 0.0;
    if (Ak > 0.0) est = exp((double)z[(size_t)r * V + slot] / tau - M[rk]) * Ak * inv_n;
    const int t = c2t[slot];
    if (t >= 0) out[(size_t)r * V + t] = est;      // empty slots of padded clusters are skipped
    // positive doubles order like their bit patterns: the smallest has the largest complement
    if (est > 0.0) key = ~(uint64_t)__double_as_longlong(est);
  }
  key = wave_max_u64(key);
  if ((threadIdx.x & 63) == 0 && key) atomicMax((unsigned long long*)&minneg[r], (unsigned long long)key);
}

__global__ __launch_bounds__(kMcThreads) void k_mc_clip(int V, const uint64_t* minneg, double* out) {
  const int r = blockIdx.y;
  const int t = blockIdx.x * kMcThreads + threadIdx.x;
  const uint64_t key = minneg[r];
  if (t < V && key) {
    double* o = out + (size_t)r * V + t;
    if (*o == 0.0) *o = __longlong_as_double((long long)~key);
  }
}

// Probe sets in launches of at most 2^20 workgroups along x.
template <class K>
hipError_t launch_sets(K kernel, int nt, const McParams& a, int B, int64_t n_sets, hipStream_t st) {
  McParams q = a;
  for (int64_t i0 = 0; i0 < n_sets; i0 += (int64_t)1 << 20) {
    const int64_t n = n_sets - i0 < ((int64_t)1 << 20) ? n_sets - i0 : ((int64_t)1 << 20);
    q.set0 = a.set0 + (uint64_t)i0;
    hipLaunchKernelGGL(kernel, dim3((unsigned)n, (unsigned)B), dim3(nt), 0, st, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

McWorkspace carve_mc_workspace(void* base, int B, int c, int b) {
  const Workspace fw = carve_workspace(nullptr, B, c, c);
  size_t off = (fw.bytes + 255) & ~(size_t)255;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = (off + n + 255) & ~(size_t)255;
    return base ? (char*)base + o : nullptr;
  };
  McWorkspace w;
  w.fw = carve_workspace(base, B, c, c);
  w.s = (float*)take((size_t)B * c * sizeof(float));
  w.stau = (float*)take((size_t)B * c * sizeof(float));
  w.t0u = (uint32_t*)take((size_t)B * sizeof(uint32_t));
  w.range = (float*)take((size_t)B * 2 * sizeof(float));
  w.mu = (float*)take((size_t)B * kGrid * sizeof(float));
  w.z = (float*)take((size_t)B * c * b * sizeof(float));
  w.M = (double*)take((size_t)B * c * sizeof(double));
  w.Zc = (double*)take((size_t)B * c * sizeof(double));
  w.A = (double*)take((size_t)B * c * sizeof(double));
  w.minneg = (uint64_t*)take((size_t)B * sizeof(uint64_t));
  w.token = (int32_t*)take((size_t)B * sizeof(int32_t));
  w.bytes = off;
  return w;
}

hipError_t launch_mc(const HeadShape& sh, int p, float tau, uint64_t seed, int64_t n_sets, int clip,
                     const int32_t* c2t, const McWorkspace& w, double* out, hipStream_t st) {
  const int B = sh.B, c = sh.c, b = sh.b, V = c * b;
  const int64_t nk = (int64_t)B * c;
  hipLaunchKernelGGL(k_mc_stats, dim3((unsigned)((nk + kMcThreads - 1) / kMcThreads)), dim3(kMcThreads), 0, st,
                     w.z, B, c, b, (double)tau, w.M, w.Zc, w.A, w.minneg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mc_prep, dim3((unsigned)B), dim3(kSelThreads), 0, st, w.s, c, tau, w.stau, w.range);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_mc_grid, dim3(kGrid, (unsigned)B), dim3(kMcThreads), 0, st, w.stau, c, w.range, w.mu);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_mc_pick, dim3((unsigned)B), dim3(kWave), 0, st, w.range, w.mu, c, p, w.t0u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  McParams a{w.stau, w.t0u, w.M, w.Zc, w.A, c, p, tau, seed, 0};
  // the candidate-list kernel when the expected candidates (the target of k_mc_pick) fit its
  // list with room to spare, else keys in registers
  const float target = (float)p + 8.0f * sqrtf((float)p) + 16.0f;
  if (target < (float)c && target <= 0.75f * (float)kListCap)
    e = launch_sets(k_mc_sets_list, kListThreads, a, B, n_sets, st);
  else if (c <= 4 * 512) e = launch_sets(k_mc_sets<1, 512>, 512, a, B, n_sets, st);
  else if (c <= 8 * 512) e = launch_sets(k_mc_sets<2, 512>, 512, a, B, n_sets, st);
  else if (c <= 16 * 512) e = launch_sets(k_mc_sets<4, 512>, 512, a, B, n_sets, st);
  else if (c <= 32 * 512) e = launch_sets(k_mc_sets<8, 512>, 512, a, B, n_sets, st);
  else e = launch_sets(k_mc_sets<8, 1024>, 1024, a, B, n_sets, st);
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)((V + kMcThreads - 1) / kMcThreads), (unsigned)B);
  hipLaunchKernelGGL(k_mc_expand, g, dim3(kMcThreads), 0, st, w.z, c2t, w.M, w.A, c, b, V, (double)tau,
                     1.0 / (double)n_sets, out, w.minneg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (clip) {
    hipLaunchKernelGGL(k_mc_clip, g, dim3(kMcThreads), 0, st, V, w.minneg, out);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace fh
