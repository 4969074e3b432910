// Offline balanced spherical k-means on the GPU (flashhead_build_clusters).
//
// Method: "FlashHead: Efficient Drop-In Replacement for the Classification Head in
// Language Model Inference", Section 3.1 (clustering the embedding matrix): spherical
// k-means over the normalised token embeddings, with an assignment step that gives every
// cluster exactly b = V / c members -- an over-full cluster keeps its b most similar
// members and the others move, greedily, to the most similar cluster that still has room.
// The steps the section leaves open are fixed as follows: k-means++ initialisation in the
// spherical metric (weights 2 - 2 cos, inverse CDF over the prefix sums in ascending id,
// draw m = Philox stream 2, row 0, step m, element 0); evicted tokens are placed in
// ascending token id; ties go to the smaller cluster or token id; the update is
// c_k = normalise(sum of the members' unit rows), a zero sum keeping the previous centroid.
//
// Everything is fp64 (unit rows, similarities, weights, sums), each reduction has a fixed
// order and the sorts are stable, so the result does not depend on scheduling.
#include <algorithm>

#include <hipcub/hipcub.hpp>

#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

namespace {

constexpr int kKmThreads = 256;
constexpr int kTopM = 16;                  // most similar clusters kept per evicted token
constexpr int kTile = 64;                  // similarity GEMM tile: tokens x clusters
constexpr int kKc = 16;                    // GEMM depth per LDS stage
constexpr int kMaxC = 32768;
constexpr int kRescanWG = 1024;            // workgroups of k_km_rescan

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;                                 // one butterfly: every lane holds the same value
}

// Monotone map of doubles onto uint64 (a > b implies key(a) > key(b)).
__device__ __forceinline__ uint64_t ord64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// (v, k) before (w, j): larger similarity first, then the smaller cluster id.
__device__ __forceinline__ bool sim_before(double v, int k, double w, int j) {
  return v > w || (v == w && k < j);
}

__device__ __forceinline__ double load_e(const void* E, int src_bf16, size_t i) {
  if (src_bf16) return (double)bf16_to_f32(reinterpret_cast<const uint16_t*>(E)[i]);
  return (double)reinterpret_cast<const float*>(E)[i];
}

// En[i] = E[i] / ||E[i]|| (a zero row stays zero); one wave per row.
__global__ __launch_bounds__(kKmThreads) void k_km_normalize(const void* E, int src_bf16, int V, int d, double* En,
                                                              double* nrm) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kKmThreads / 64) + (threadIdx.x >> 6);
  if (i >= V) return;
  double ss = 0.0;
  for (int j = lane; j < d; j += 64) {
    const double x = load_e(E, src_bf16, (size_t)i * d + j);
    ss = fma(x, x, ss);
  }
  const double n = sqrt(wave_sum_f64(ss));
  if (lane == 0) nrm[i] = n;
  for (int j = lane; j < d; j += 64) {
    const double x = load_e(E, src_bf16, (size_t)i * d + j);
    En[(size_t)i * d + j] = n > 0.0 ? x / n : 0.0;
  }
}

// k-means++ weights after draw m: w = max(2 - 2 e_i . e_new, 0) (m = 0) or the min of that
// and w (m > 0); the new centre's weight is 0.  One wave per token.
// D^2 weights of k-means++ after centre m: w_i = min(w_i, max(2 - 2 cos(e_i, e_new), 0)) (w_i
// itself for m = 0), 0 for the centre.  The cosine is the fp64 dot of the source rows (bf16 /
// fp32 values, exact products) over the product of their norms -- the same quantity as the dot
// of the normalised rows, from a quarter (bf16) or half (fp32) of their bytes.  One wave per
// token, 16-byte loads.
// Thread 0 also marks centre m used and primes chosen[m + 1] for the next draw's minimum.
template <int SRC_BF16>
__global__ __launch_bounds__(kKmThreads) void k_km_weights(const void* E, const double* nrm, int V, int d,
                                                          int32_t* chosen, int m, int c, double* w, uint8_t* used) {
  constexpr int EPC = SRC_BF16 ? 8 : 4;                // elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kKmThreads / 64) + (threadIdx.x >> 6);
  if (i >= V) return;
  const int nw = chosen[m];
  if (i == 0 && lane == 0) {
    used[nw] = 1;
    if (m + 1 < c) chosen[m + 1] = 0x7FFFFFFF;
  }
  const int nch = d / EPC;
  const uint4* x = reinterpret_cast<const uint4*>((const char*)E + (size_t)i * d * (SRC_BF16 ? 2 : 4));
  const uint4* y = reinterpret_cast<const uint4*>((const char*)E + (size_t)nw * d * (SRC_BF16 ? 2 : 4));
  double s = 0.0;
  for (int q = lane; q < nch; q += 64) {
    const uint4 a = x[q], b = y[q];
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (SRC_BF16) {
        s = fma((double)__uint_as_float(av[k] << 16), (double)__uint_as_float(bv[k] << 16), s);
        s = fma((double)__uint_as_float(av[k] & 0xFFFF0000u), (double)__uint_as_float(bv[k] & 0xFFFF0000u), s);
      } else {
        s = fma((double)__uint_as_float(av[k]), (double)__uint_as_float(bv[k]), s);
      }
    }
  }
  s = wave_sum_f64(s);
  if (lane == 0) {
    const double ni = nrm[i], nn = nrm[nw];
    const double dot = ni > 0.0 && nn > 0.0 ? s / (ni * nn) : 0.0;
    const double v = fmax(2.0 - 2.0 * dot, 0.0);
    double r = m == 0 ? v : fmin(w[i], v);
    if (i == nw) r = 0.0;
    w[i] = r;
  }
}

__global__ void k_km_first(int V, int first, int32_t* chosen, uint8_t* used) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) used[i] = i == first ? 1 : 0;
  if (i == 0) chosen[0] = first;
}

// Draw m: the first i with cum(w)_i >= u * total; when every weight is 0, the smallest id
// not chosen yet.  One workgroup: contiguous segments summed in order, then a sequential
// scan of the segment sums.
// The m-th draw by inverse CDF: the first token whose inclusive prefix sum of the weights
// (`cum`, ascending id) reaches u times the total (atomic minimum into chosen[m], which the
// previous k_km_weights set to INT_MAX); with a zero total, the smallest unused id.
__global__ __launch_bounds__(kKmThreads) void k_km_draw(const double* cum, int V, double u, int32_t* chosen, int m,
                                                        const uint8_t* used) {
  const int i = blockIdx.x * kKmThreads + threadIdx.x;
  if (i >= V) return;
  const double tot = cum[V - 1];
  if (tot > 0.0) {
    if (cum[i] >= u * tot) atomicMin(&chosen[m], i);
  } else if (i == 0) {                             // every token coincides with a centre (degenerate)
    int j = 0;
    while (j < V - 1 && used[j]) ++j;
    chosen[m] = j;
  }
}

// Cn[k] = En[chosen[k]].
__global__ __launch_bounds__(kKmThreads) void k_km_gather_rows(const double* En, const int32_t* rows, int n, int d,
                                                              double* out) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * (kKmThreads / 64) + (threadIdx.x >> 6);
  if (k >= n) return;
  const double* src = En + (size_t)rows[k] * d;
  for (int j = lane; j < d; j += 64) out[(size_t)k * d + j] = src[j];
}

// a[i] = argmax_k En_i . Cn_k (ties: the smaller k), sbest[i] its value.  64 tokens per
// workgroup, clusters in tiles of 64, each dot an fp64 fma chain in ascending depth.
__global__ __launch_bounds__(kKmThreads) void k_km_assign(const double* En, const double* Cn, int V, int c, int d,
                                                         int32_t* a, double* sbest) {
  __shared__ double As[kKc][kTile];
  __shared__ double Bs[kKc][kTile];
  __shared__ double bv[kTile][16];
  __shared__ int bi[kTile][16];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int tok0 = blockIdx.x * kTile;
  double best[4];
  int bidx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { best[i] = -INFINITY; bidx[i] = 0x7FFFFFFF; }
  const int lr = t >> 2, lc = (t & 3) * 4;
  for (int n0 = 0; n0 < c; n0 += kTile) {
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int k0 = 0; k0 < d; k0 += kKc) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = k0 + lc + q;
        As[lc + q][lr] = (tok0 + lr < V && kk < d) ? En[(size_t)(tok0 + lr) * d + kk] : 0.0;
        Bs[lc + q][lr] = (n0 + lr < c && kk < d) ? Cn[(size_t)(n0 + lr) * d + kk] : 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kKc; ++kk) {
        double av[4], bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { av[i] = As[kk][ty * 4 + i]; bw[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fma(av[i], bw[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n < c && sim_before(acc[i][j], n, best[i], bidx[i])) { best[i] = acc[i][j]; bidx[i] = n; }
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) { bv[ty * 4 + i][tx] = best[i]; bi[ty * 4 + i][tx] = bidx[i]; }
  __syncthreads();
  if (t < kTile && tok0 + t < V) {
    double v = bv[t][0];
    int k = bi[t][0];
    for (int q = 1; q < 16; ++q)
      if (sim_before(bv[t][q], bi[t][q], v, k)) { v = bv[t][q]; k = bi[t][q]; }
    a[tok0 + t] = k;
    sbest[tok0 + t] = v;
  }
}

__global__ void k_km_sort_keys(const double* sbest, int V, uint64_t* key, int32_t* ids) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) { key[i] = ord64(sbest[i] + 0.0); ids[i] = i; }   // +0: -0 and +0 tie
}

__global__ void k_km_gather_cluster(const int32_t* a, const int32_t* ids, int V, int32_t* key) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) key[i] = a[ids[i]];
}

__global__ void k_km_iota_cluster(const int32_t* a, int V, int32_t* key, int32_t* ids) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) { key[i] = a[i]; ids[i] = i; }
}

__global__ void k_km_zero(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void k_km_count(const int32_t* a, int V, int32_t* counts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) atomicAdd(&counts[a[i]], 1);
}

// Tokens sorted by (cluster, similarity desc, id asc): a token of rank >= b in its cluster
// is evicted.  room[k] = free slots left in cluster k.
__global__ void k_km_evict(const int32_t* sorted_ids, const int32_t* sorted_k, const int32_t* start,
                           const int32_t* counts, int V, int c, int b, uint8_t* flags, int32_t* room) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) {
    const int k = sorted_k[i];
    flags[sorted_ids[i]] = (i - start[k]) >= b ? 1 : 0;
  }
  if (i < c) room[i] = b - min(counts[i], b);
}

// For each evicted token, its kTopM most similar clusters (similarity desc, id asc), by
// the same fp64 fma chains as k_km_assign.  One wave per token; each lane keeps a sorted
// list of its own clusters, then the wave merges the 64 lists.
__global__ __launch_bounds__(kKmThreads) void k_km_topm(const double* En, const double* Cn, const int32_t* ev,
                                                       int n_ev, int c, int d, int32_t* top) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kKmThreads / 64) + (threadIdx.x >> 6);
  if (e >= n_ev) return;
  const double* x = En + (size_t)ev[e] * d;
  double lv[kTopM];
  int lk[kTopM];
#pragma unroll
  for (int q = 0; q < kTopM; ++q) { lv[q] = -INFINITY; lk[q] = 0x7FFFFFFF; }
  for (int k = lane; k < c; k += 64) {
    const double* y = Cn + (size_t)k * d;
    double s = 0.0;
    for (int j = 0; j < d; ++j) s = fma(x[j], y[j], s);
    if (sim_before(s, k, lv[kTopM - 1], lk[kTopM - 1])) {
      double v = s;
      int kk = k;
#pragma unroll
      for (int q = 0; q < kTopM; ++q) {          // insertion by compare-and-swap down the list
        if (sim_before(v, kk, lv[q], lk[q])) {
          const double tv = lv[q];
          const int tk = lk[q];
          lv[q] = v;
          lk[q] = kk;
          v = tv;
          kk = tk;
        }
      }
    }
  }
  for (int r = 0; r < kTopM; ++r) {                // merge: the best head wins, its lane pops
    double v = lv[0];
    int k = lk[0];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const double ov = __shfl_xor(v, m, kWave);
      const int ok = __shfl_xor(k, m, kWave);
      if (sim_before(ov, ok, v, k)) { v = ov; k = ok; }
    }
    if (lane == 0) top[(size_t)e * kTopM + r] = k < c ? k : -1;
    if (lk[0] == k) {
#pragma unroll
      for (int q = 0; q + 1 < kTopM; ++q) { lv[q] = lv[q + 1]; lk[q] = lk[q + 1]; }
      lv[kTopM - 1] = -INFINITY;
      lk[kTopM - 1] = 0x7FFFFFFF;
    }
  }
}

// Evicted tokens in ascending id, each to its most similar cluster with room: the first of
// its kTopM candidates with room.  One wave walks the tokens from `pos` in order; at a token
// whose candidates are all full it stops (*status = that position; n_ev when every token is
// placed), and the host has k_km_rescan + k_km_place settle that token against every
// cluster before the walk resumes.  `room` (global) carries the free slots between launches.
__global__ __launch_bounds__(64) void k_km_repair(const int32_t* ev, int n_ev, int pos, const int32_t* top,
                                                   int32_t* room_g, int c, int32_t* a, int32_t* status) {
  __shared__ uint16_t room[kMaxC];
  const int lane = threadIdx.x;
  for (int k = lane; k < c; k += 64) room[k] = (uint16_t)room_g[k];
  __syncthreads();
  int stop = n_ev;
  for (int e = pos; e < n_ev; ++e) {
    // lane q < kTopM looks at candidate q; the first with room wins
    const int kk = lane < kTopM ? top[(size_t)e * kTopM + lane] : -1;
    const bool ok = kk >= 0 && room[kk] > 0;
    const uint64_t bal = __ballot(ok);
    if (!bal) { stop = e; break; }
    const int q = __ffsll((unsigned long long)bal) - 1;
    const int k = __shfl(kk, q, kWave);
    if (lane == 0) {
      a[ev[e]] = k;
      room[k] = (uint16_t)(room[k] - 1);
    }
    __syncthreads();
  }
  __syncthreads();
  for (int k = lane; k < c; k += 64) room_g[k] = room[k];
  if (lane == 0) *status = stop;
}

// Token ev[pos] against every cluster with room: one wave per cluster (coalesced row dot),
// the best (similarity desc, id asc) of each workgroup to part_v / part_k.
__global__ __launch_bounds__(kKmThreads) void k_km_rescan(const double* En, const double* Cn, const int32_t* ev,
                                                          const int32_t* status, const int32_t* room, int c, int d,
                                                          double* part_v, int32_t* part_k) {
  __shared__ double wv[kKmThreads / 64];
  __shared__ int wk[kKmThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double* x = En + (size_t)ev[*status] * d;
  double v = -INFINITY;
  int kb = 0x7FFFFFFF;
  const int nwaves = gridDim.x * (kKmThreads / 64);
  for (int k = blockIdx.x * (kKmThreads / 64) + wave; k < c; k += nwaves) {
    if (room[k] <= 0) continue;                       // wave-uniform
    const double* y = Cn + (size_t)k * d;
    double s = 0.0;
    for (int j = lane; j < d; j += 64) s = fma(x[j], y[j], s);
    s = wave_sum_f64(s);
    if (sim_before(s, k, v, kb)) { v = s; kb = k; }
  }
  if (lane == 0) { wv[wave] = v; wk[wave] = kb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kKmThreads / 64; ++w)
      if (sim_before(wv[w], wk[w], v, kb)) { v = wv[w]; kb = wk[w]; }
    part_v[blockIdx.x] = v;
    part_k[blockIdx.x] = kb;
  }
}

// The rescan's winner: token ev[pos] takes it (total room equals the evicted count, so a
// cluster with room exists).
__global__ __launch_bounds__(64) void k_km_place(const double* part_v, const int32_t* part_k, int g,
                                                  const int32_t* ev, const int32_t* status, int c, int32_t* room,
                                                  int32_t* a) {
  const int lane = threadIdx.x;
  double v = -INFINITY;
  int kb = 0x7FFFFFFF;
  for (int i = lane; i < g; i += 64)
    if (sim_before(part_v[i], part_k[i], v, kb)) { v = part_v[i]; kb = part_k[i]; }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const double ov = __shfl_xor(v, m, kWave);
    const int ok = __shfl_xor(kb, m, kWave);
    if (sim_before(ov, ok, v, kb)) { v = ov; kb = ok; }
  }
  if (lane == 0 && kb >= 0 && kb < c) {
    a[ev[*status]] = kb;
    room[kb] -= 1;
  }
}

// Cn[k] = normalise(sum of En over members[k][0 .. b)), members in ascending id and summed
// in that order; a zero sum keeps Cn[k].  One wave per cluster.
__global__ __launch_bounds__(kKmThreads) void k_km_update(const double* En, const int32_t* members, int b, int c,
                                                         int d, double* Cn) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * (kKmThreads / 64) + (threadIdx.x >> 6);
  if (k >= c) return;
  const int32_t* mem = members + (size_t)k * b;
  double ss = 0.0;
  for (int j = lane; j < d; j += 64) {
    double s = 0.0;
    for (int q = 0; q < b; ++q) s += En[(size_t)mem[q] * d + j];
    ss = fma(s, s, ss);
  }
  const double n = sqrt(wave_sum_f64(ss));
  if (!(n > 0.0)) return;
  for (int j = lane; j < d; j += 64) {
    double s = 0.0;
    for (int q = 0; q < b; ++q) s += En[(size_t)mem[q] * d + j];
    Cn[(size_t)k * d + j] = s / n;
  }
}

__device__ __forceinline__ uint16_t km_bf16_rne(double x) {
  if (!(fabs(x) < 0x1p128)) {
    if (x != x) return 0x7FC0u;
    return x > 0 ? 0x7F80u : 0xFF80u;
  }
  int e;
  frexp(x, &e);
  const int qe = e - 8 > -133 ? e - 8 : -133;
  const double r = ldexp(rint(ldexp(x, -qe)), qe);
  if (fabs(r) >= 0x1p128) return x > 0 ? 0x7F80u : 0xFF80u;
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// The unit centroids as stored: Cn rounded once to fp32 or bf16.
__global__ void k_km_store_unit(const double* Cn, size_t n, int dst_bf16, void* out) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (dst_bf16) reinterpret_cast<uint16_t*>(out)[i] = km_bf16_rne(Cn[i]);
  else reinterpret_cast<float*>(out)[i] = (float)Cn[i];
}

struct KmWs {
  double *En, *Cn, *w, *sbest, *nrm;
  int32_t *a, *chosen, *ids, *ids2, *key32, *key32b, *counts, *start, *room, *ev, *n_ev, *top, *status, *part_k;
  double* part_v;
  uint64_t *key64, *key64b;
  uint8_t *used, *flags;
  void* tmp;
  size_t tmp_bytes, bytes;
};

size_t cub_tmp_bytes(int V, int c) {
  size_t s1 = 0, s2 = 0, s3 = 0, s4 = 0;
  // size queries only (null temporary storage): nothing is launched
  (void)hipcub::DeviceRadixSort::SortPairsDescending(nullptr, s1, (const uint64_t*)nullptr, (uint64_t*)nullptr,
                                                     (const int32_t*)nullptr, (int32_t*)nullptr, V);
  (void)hipcub::DeviceRadixSort::SortPairs(nullptr, s2, (const int32_t*)nullptr, (int32_t*)nullptr,
                                           (const int32_t*)nullptr, (int32_t*)nullptr, V);
  (void)hipcub::DeviceScan::ExclusiveSum(nullptr, s3, (const int32_t*)nullptr, (int32_t*)nullptr, c);
  (void)hipcub::DeviceSelect::Flagged(nullptr, s4, hipcub::CountingInputIterator<int32_t>(0),
                                      (const uint8_t*)nullptr, (int32_t*)nullptr, (int32_t*)nullptr, V);
  size_t s5 = 0;
  (void)hipcub::DeviceScan::InclusiveSum(nullptr, s5, (const double*)nullptr, (double*)nullptr, V);
  return std::max(std::max(std::max(s1, s2), std::max(s3, s4)), s5);
}

KmWs km_carve(void* base, int V, int d, int c) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  KmWs w{};
  char* p = (char*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? (void*)(p + off) : nullptr;
    off = up(off + bytes);
    return r;
  };
  w.En = (double*)take((size_t)V * d * 8);
  w.Cn = (double*)take((size_t)c * d * 8);
  w.w = (double*)take((size_t)V * 8);
  w.sbest = (double*)take((size_t)V * 8);
  w.nrm = (double*)take((size_t)V * 8);
  w.a = (int32_t*)take((size_t)V * 4);
  w.chosen = (int32_t*)take((size_t)c * 4);
  w.ids = (int32_t*)take((size_t)V * 4);
  w.ids2 = (int32_t*)take((size_t)V * 4);
  w.key32 = (int32_t*)take((size_t)V * 4);
  w.key32b = (int32_t*)take((size_t)V * 4);
  w.counts = (int32_t*)take((size_t)c * 4);
  w.start = (int32_t*)take((size_t)c * 4);
  w.room = (int32_t*)take((size_t)c * 4);
  w.ev = (int32_t*)take((size_t)V * 4);
  w.n_ev = (int32_t*)take(4);
  w.status = (int32_t*)take(4);
  w.part_v = (double*)take((size_t)kRescanWG * 8);
  w.part_k = (int32_t*)take((size_t)kRescanWG * 4);
  w.top = (int32_t*)take((size_t)V * kTopM * 4);
  w.key64 = (uint64_t*)take((size_t)V * 8);
  w.key64b = (uint64_t*)take((size_t)V * 8);
  w.used = (uint8_t*)take((size_t)V);
  w.flags = (uint8_t*)take((size_t)V);
  w.tmp_bytes = cub_tmp_bytes(V, c);
  w.tmp = take(w.tmp_bytes);
  w.bytes = off;
  return w;
}

inline int blocks(size_t n, int t) { return (int)((n + t - 1) / t); }

}  // namespace

size_t build_clusters_workspace_bytes(int V, int d, int c) { return km_carve(nullptr, V, d, c).bytes; }

hipError_t launch_build_clusters(int V, int d, int c, int src_bf16, const void* E, int iters, uint64_t seed, int unit,
                                 int dst_bf16, void* centroids, int32_t* c2t, void* ws_base, hipStream_t st) {
  const int b = V / c;
  KmWs w = km_carve(ws_base, V, d, c);
  const int wpb = kKmThreads / 64;             // one wave per row
  hipError_t e;
#define KM_CHECK()                              \
  do {                                          \
    e = hipGetLastError();                      \
    if (e != hipSuccess) return e;              \
  } while (0)
  hipLaunchKernelGGL(k_km_normalize, dim3(blocks(V, wpb)), dim3(kKmThreads), 0, st, E, src_bf16, V, d, w.En,
                     w.nrm);
  KM_CHECK();
  // ---- k-means++ (Philox stream 2, row 0, step m, element 0)
  auto uni = [&](int m) {
    const Rng g = make_rng(seed, (uint64_t)m);
    return (double)word_to_uniform(rng_word(g, 0u, 2u, 0u));
  };
  const double u0 = uni(0);
  int first = (int)floor(u0 * V);
  if (first > V - 1) first = V - 1;
  hipLaunchKernelGGL(k_km_first, dim3(blocks(V, 256)), dim3(256), 0, st, V, first, w.chosen, w.used);
  auto weights = [&](int m) {
    if (src_bf16)
      hipLaunchKernelGGL(k_km_weights<1>, dim3(blocks(V, wpb)), dim3(kKmThreads), 0, st, E, (const double*)w.nrm, V,
                         d, w.chosen, m, c, w.w, w.used);
    else
      hipLaunchKernelGGL(k_km_weights<0>, dim3(blocks(V, wpb)), dim3(kKmThreads), 0, st, E, (const double*)w.nrm, V,
                         d, w.chosen, m, c, w.w, w.used);
  };
  weights(0);
  KM_CHECK();
  for (int m = 1; m < c; ++m) {
    size_t tb = w.tmp_bytes;
    if ((e = hipcub::DeviceScan::InclusiveSum(w.tmp, tb, (const double*)w.w, w.sbest, V, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_km_draw, dim3(blocks(V, kKmThreads)), dim3(kKmThreads), 0, st, (const double*)w.sbest, V,
                       uni(m), w.chosen, m, (const uint8_t*)w.used);
    weights(m);
    KM_CHECK();
  }
  hipLaunchKernelGGL(k_km_gather_rows, dim3(blocks(c, wpb)), dim3(kKmThreads), 0, st, (const double*)w.En,
                     (const int32_t*)w.chosen, c, d, w.Cn);
  KM_CHECK();
  // ---- balanced assignment and update
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(k_km_assign, dim3(blocks(V, kTile)), dim3(kKmThreads), 0, st, (const double*)w.En,
                       (const double*)w.Cn, V, c, d, w.a, w.sbest);
    hipLaunchKernelGGL(k_km_sort_keys, dim3(blocks(V, 256)), dim3(256), 0, st, (const double*)w.sbest, V, w.key64,
                       w.ids);
    KM_CHECK();
    size_t tb = w.tmp_bytes;
    if ((e = hipcub::DeviceRadixSort::SortPairsDescending(w.tmp, tb, w.key64, w.key64b, w.ids, w.ids2, V, 0, 64,
                                                          st)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_km_gather_cluster, dim3(blocks(V, 256)), dim3(256), 0, st, (const int32_t*)w.a,
                       (const int32_t*)w.ids2, V, w.key32);
    KM_CHECK();
    tb = w.tmp_bytes;
    if ((e = hipcub::DeviceRadixSort::SortPairs(w.tmp, tb, w.key32, w.key32b, w.ids2, w.ids, V, 0, 32, st)) !=
        hipSuccess)
      return e;
    hipLaunchKernelGGL(k_km_zero, dim3(blocks(c, 256)), dim3(256), 0, st, w.counts, c);
    hipLaunchKernelGGL(k_km_count, dim3(blocks(V, 256)), dim3(256), 0, st, (const int32_t*)w.a, V, w.counts);
    KM_CHECK();
    tb = w.tmp_bytes;
    if ((e = hipcub::DeviceScan::ExclusiveSum(w.tmp, tb, w.counts, w.start, c, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_km_evict, dim3(blocks(V > c ? V : c, 256)), dim3(256), 0, st, (const int32_t*)w.ids,
                       (const int32_t*)w.key32b, (const int32_t*)w.start, (const int32_t*)w.counts, V, c, b, w.flags,
                       w.room);
    KM_CHECK();
    tb = w.tmp_bytes;
    if ((e = hipcub::DeviceSelect::Flagged(w.tmp, tb, hipcub::CountingInputIterator<int32_t>(0), w.flags, w.ev,
                                           w.n_ev, V, st)) != hipSuccess)
      return e;
    int n_ev = 0;
    if ((e = hipMemcpyAsync(&n_ev, w.n_ev, sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    if (n_ev > 0) {
      hipLaunchKernelGGL(k_km_topm, dim3(blocks(n_ev, wpb)), dim3(kKmThreads), 0, st, (const double*)w.En,
                         (const double*)w.Cn, (const int32_t*)w.ev, n_ev, c, d, w.top);
      const int g = blocks(c, kKmThreads / 64) < kRescanWG ? blocks(c, kKmThreads / 64) : kRescanWG;
      for (int pos = 0;;) {
        hipLaunchKernelGGL(k_km_repair, dim3(1), dim3(64), 0, st, (const int32_t*)w.ev, n_ev, pos,
                           (const int32_t*)w.top, w.room, c, w.a, w.status);
        KM_CHECK();
        if ((e = hipMemcpyAsync(&pos, w.status, sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
        if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
        if (pos >= n_ev) break;
        hipLaunchKernelGGL(k_km_rescan, dim3(g), dim3(kKmThreads), 0, st, (const double*)w.En, (const double*)w.Cn,
                           (const int32_t*)w.ev, (const int32_t*)w.status, (const int32_t*)w.room, c, d, w.part_v,
                           w.part_k);
        hipLaunchKernelGGL(k_km_place, dim3(1), dim3(64), 0, st, (const double*)w.part_v, (const int32_t*)w.part_k,
                           g, (const int32_t*)w.ev, (const int32_t*)w.status, c, w.room, w.a);
        KM_CHECK();
        ++pos;
      }
    }
    // members of every cluster in ascending token id
    hipLaunchKernelGGL(k_km_iota_cluster, dim3(blocks(V, 256)), dim3(256), 0, st, (const int32_t*)w.a, V, w.key32,
                       w.ids2);
    KM_CHECK();
    tb = w.tmp_bytes;
    if ((e = hipcub::DeviceRadixSort::SortPairs(w.tmp, tb, w.key32, w.key32b, w.ids2, w.ids, V, 0, 32, st)) !=
        hipSuccess)
      return e;
    hipLaunchKernelGGL(k_km_update, dim3(blocks(c, wpb)), dim3(kKmThreads), 0, st, (const double*)w.En,
                       (const int32_t*)w.ids, b, c, d, w.Cn);
    KM_CHECK();
  }
  // ---- outputs: C2T from the last assignment; centroids as stored
  if ((e = hipMemcpyAsync(c2t, w.ids, (size_t)V * sizeof(int32_t), hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return e;
  if (unit) {
    const size_t n = (size_t)c * d;
    hipLaunchKernelGGL(k_km_store_unit, dim3(blocks(n, 256)), dim3(256), 0, st, (const double*)w.Cn, n, dst_bf16,
                       centroids);
    KM_CHECK();
    return hipSuccess;
  }
#undef KM_CHECK
  return launch_centroids(d, c, b, src_bf16, dst_bf16, 0, E, c2t, centroids, st);
}

}  // namespace fh
