// Exact top-p selection by one workgroup (keys held in registers), shared by the probe
// selection kernels.  Ties go to the smaller id.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fh_device.h"

namespace fh {

constexpr int kSelThreads = 1024;

__device__ __forceinline__ int block_excl_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int t = sh[w];
      sh[w] = acc;
      acc += t;
    }
    sh[16] = acc;
  }
  __syncthreads();
  const int res = x - v + sh[wave];
  total = sh[16];
  __syncthreads();
  return res;
}

// Selection of the p largest of c keys by one workgroup of NT threads.  Thread t holds, in
// registers, the keys of ids 4 (t + j NT) + e (j < KV, e < 4) as order-preserving uint32 u
// (larger key <=> larger u; ties go to the smaller id).  The result is the boundary
// (Tu, Tid): a key is kept iff u > Tu, or u == Tu and id <= Tid.
//
// The candidate interval [ilo, ihi] (in u) starts as all keys (select_regs) or as a range
// known to hold the boundary (select_interval).  A pass histograms the
// candidates into 2048 bins and shrinks the interval to the bin holding the boundary; bins
// above it hold only larger keys and are kept.  The first two passes use bins linear in the
// key's float value between the interval's ends (a monotone map that spreads the keys near
// the boundary, so LDS atomics rarely collide); later passes use power-of-two-wide bins in
// u, each shrinking the u-span 2048-fold, so a single value is reached within three more
// passes.  Once at most kCand candidates remain they are ranked exactly by (u desc, id asc);
// a larger set of equal candidates is ordered by id through the bitmap below.
//
// The kept ids are then marked in a bitmap over [0, c); prefix popcounts of its words give
// the ascending-id rank of every kept cluster.
constexpr int kSelBins = 2048;
constexpr int kCand = 256;
constexpr int kMaxWords = 32768 / 32;

struct SelShared {
  int hist[kSelBins];
  uint32_t bitmap[kMaxWords];
  int woff[kMaxWords];
  uint32_t cu[kCand];
  int cid[kCand];
  int wtot[6][16];                         // per-wave partials, one slot per use
  uint32_t wred[6][16];
  int ncand;
  int bdig[3];
  uint32_t Tu;
  int Tid;
};

__device__ __forceinline__ float ord_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
}

// Both extremes over the block with one barrier.
__device__ __forceinline__ void block_minmax2(uint32_t& vmax, uint32_t& vmin, uint32_t* wmax, uint32_t* wmin) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  vmax = wave_minmax_u32<true>(vmax);
  vmin = wave_minmax_u32<false>(vmin);
  if ((threadIdx.x & 63) == 0) { wmax[wave] = vmax; wmin[wave] = vmin; }
  __syncthreads();
  vmax = wmax[0];
  vmin = wmin[0];
  for (int w = 1; w < nw; ++w) {
    vmax = wmax[w] > vmax ? wmax[w] : vmax;
    vmin = wmin[w] < vmin ? wmin[w] : vmin;
  }
}

// Exclusive prefix sum over the block (thread order); one barrier.  `wtot` must not be
// reused before the next barrier.
__device__ __forceinline__ int block_scan(int v, int* wtot, int& total) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int incl = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) wtot[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = wtot[w];
    off += w < wave ? t : 0;
    tot += t;
  }
  total = tot;
  return off + incl - v;
}

__device__ __forceinline__ int sel_bin(uint32_t u, bool flin, float lo_f, float inv, uint32_t ilo, int ushift) {
  if (flin) {
    const float t = (ord_to_float(u) - lo_f) * inv;
    return t >= 0.f ? (t < (float)(kSelBins - 1) ? (int)t : kSelBins - 1) : 0;
  }
  return (int)((u - ilo) >> ushift);
}

__device__ __forceinline__ int span_shift(uint32_t ilo, uint32_t ihi) {
  const uint32_t span = ihi - ilo;                 // bins needed: (span >> s) < kSelBins
  const int bits = span ? 32 - __clz(span) : 0;
  return bits > 11 ? bits - 11 : 0;
}

// Load the c keys (floats, global) into registers as ord keys; clears hist and bitmap.
template <int KV>
__device__ __forceinline__ void load_keys(const float* keys, int c, uint32_t (&u)[KV][4], SelShared& S) {
  const int NT = blockDim.x, tid = threadIdx.x;
  const bool al = (reinterpret_cast<uintptr_t>(keys) & 15) == 0;
#pragma unroll
  for (int j = 0; j < KV; ++j) {
    const int id0 = 4 * (tid + j * NT);
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (al && id0 + 4 <= c) {
      w = *reinterpret_cast<const uint4*>(keys + id0);
    } else if (id0 < c) {
      w.x = __float_as_uint(keys[id0]);
      if (id0 + 1 < c) w.y = __float_as_uint(keys[id0 + 1]);
      if (id0 + 2 < c) w.z = __float_as_uint(keys[id0 + 2]);
      if (id0 + 3 < c) w.w = __float_as_uint(keys[id0 + 3]);
    }
    u[j][0] = ord_key(__uint_as_float(w.x));
    u[j][1] = ord_key(__uint_as_float(w.y));
    u[j][2] = ord_key(__uint_as_float(w.z));
    u[j][3] = ord_key(__uint_as_float(w.w));
  }
  for (int i = tid; i < kSelBins; i += NT) S.hist[i] = 0;
  for (int i = tid; i < kMaxWords; i += NT) S.bitmap[i] = 0u;
}

// (Tu, Tid) = the need-th largest, by (u desc, id asc), of the keys `pick` accepts (at most
// kCand of them).  Expects S.ncand zero and a barrier since.
template <class Each, class Pick>
__device__ __forceinline__ void rank_candidates(const Each& each, const Pick& pick, int need, SelShared& S,
                                                uint32_t& Tu, int& Tid) {
  const int tid = threadIdx.x, NT = blockDim.x;
  each([&](uint32_t x, int id) {
    if (pick(x)) {
      const int slot = atomicAdd(&S.ncand, 1);
      if (slot < kCand) { S.cu[slot] = x; S.cid[slot] = id; }
    }
  });
  __syncthreads();
  const int n = S.ncand < kCand ? S.ncand : kCand;
  for (int t = tid; t < n; t += NT) {
    const uint32_t ut = S.cu[t];
    const int it = S.cid[t];
    int rank = 0;
    for (int q = 0; q < n; ++q) {
      const uint32_t uq = S.cu[q];
      rank += (uq > ut) || (uq == ut && S.cid[q] < it);
    }
    if (rank == need - 1) { S.Tu = ut; S.Tid = it; }
  }
  __syncthreads();
  Tu = S.Tu;
  Tid = S.Tid;
}

// The selection restricted to the keys in [ilo, ihi] (order-preserving values): every key
// above ihi is kept, and the `need` largest of the n_in keys in the interval complete the set
// (n_in >= need).  `each(f)` calls f(u, id) for every key this thread holds (id < c), in any
// order; every call of `each` must present the same keys.  Expects S.hist cleared (and a
// barrier since) and S.bitmap clear; leaves S.bitmap clear.
template <class Each>
__device__ __forceinline__ void select_interval_each(const Each& each, int c, SelShared& S, uint32_t ilo,
                                                     uint32_t ihi, int need, int n_in, uint32_t& Tu, int& Tid) {
  const int tid = threadIdx.x, NT = blockDim.x;
  for (int level = 0; level < 8 && n_in > kCand && n_in > need && ilo != ihi; ++level) {
    const float lo_f = ord_to_float(ilo), hi_f = ord_to_float(ihi);
    const float inv = (float)kSelBins / (hi_f - lo_f);
    const bool flin = level < 2 && inv > 0.f && inv < 3.0e38f;
    const int ushift = span_shift(ilo, ihi);
    if (level > 0) {
      for (int i = tid; i < kSelBins; i += NT) S.hist[i] = 0;
      __syncthreads();
    }
    each([&](uint32_t x, int) {
      if (x >= ilo && x <= ihi) atomicAdd(&S.hist[sel_bin(x, flin, lo_f, inv, ilo, ushift)], 1);
    });
    __syncthreads();
    // suffix counts from the top bin down: thread t owns bins 2047 - t*BPT - i
    const int bpt = kSelBins / NT;
    int local = 0;
    for (int i = 0; i < bpt; ++i) local += S.hist[kSelBins - 1 - tid * bpt - i];
    int tot;
    const int before = block_scan(local, S.wtot[level & 1], tot);
    if (before < need && before + local >= need) {
      int acc = before;
      for (int i = 0; i < bpt; ++i) {
        const int bin = kSelBins - 1 - tid * bpt - i;
        const int hc = S.hist[bin];
        if (acc + hc >= need) { S.bdig[0] = bin; S.bdig[1] = acc; S.bdig[2] = hc; break; }
        acc += hc;
      }
    }
    if (tid == 0) S.ncand = 0;
    __syncthreads();
    const int b = S.bdig[0];
    need -= S.bdig[1];
    n_in = S.bdig[2];
    if (n_in <= kCand) {                      // block-uniform: rank bin b's keys straight away
      rank_candidates(
          each, [&](uint32_t x) { return x >= ilo && x <= ihi && sel_bin(x, flin, lo_f, inv, ilo, ushift) == b; },
          need, S, Tu, Tid);
      return;
    }
    uint32_t bmax = 0u, bmin = 0xFFFFFFFFu;
    each([&](uint32_t x, int) {
      if (x >= ilo && x <= ihi && sel_bin(x, flin, lo_f, inv, ilo, ushift) == b) {
        bmax = max(bmax, x);
        bmin = min(bmin, x);
      }
    });
    block_minmax2(bmax, bmin, S.wred[2 + 2 * (level & 1)], S.wred[3 + 2 * (level & 1)]);
    ihi = bmax;
    ilo = bmin;
  }
  // every key with u > ihi is kept; `need` more come from the n_in keys in [ilo, ihi]
  if (n_in == need) {                         // the whole interval is kept
    Tu = ilo;
    Tid = 0x7FFFFFFF;
    return;
  }
  if (n_in <= kCand) {                        // rank the candidates exactly
    if (tid == 0) S.ncand = 0;
    __syncthreads();
    rank_candidates(each, [&](uint32_t x) { return x >= ilo && x <= ihi; }, need, S, Tu, Tid);
    return;
  }
  // many equal candidates (ilo == ihi): the need-th of them in id order, via the bitmap
  each([&](uint32_t x, int id) {
    if (x == ilo) atomicOr(&S.bitmap[id >> 5], 1u << (id & 31));
  });
  __syncthreads();
  const int nwords = (c + 31) >> 5;
  for (int w0 = 0; w0 < nwords; w0 += NT) {
    const int w = w0 + tid;
    const int pc = w < nwords ? __popc(S.bitmap[w]) : 0;
    int tot;
    const int before = block_scan(pc, S.wtot[2], tot) ;
    if (w < nwords && before < need && before + pc >= need) {
      uint32_t bits = S.bitmap[w];
      for (int k = before + 1; k < need; ++k) bits &= bits - 1u;
      S.Tid = (w << 5) + __ffs(bits) - 1;
    }
    need -= tot;
    __syncthreads();
  }
  for (int i = tid; i < kMaxWords; i += NT) S.bitmap[i] = 0u;
  __syncthreads();
  Tu = ilo;
  Tid = S.Tid;
}

// Keys held in registers: thread t holds ids 4 (t + j NT) + e, j < KV, e < 4.
template <int KV>
struct RegKeys {
  const uint32_t (&u)[KV][4];
  int c;
  template <class F>
  __device__ __forceinline__ void operator()(F&& f) const {
    const int tid = threadIdx.x, NT = blockDim.x;
#pragma unroll
    for (int j = 0; j < KV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = 4 * (tid + j * NT) + e;
        if (id < c) f(u[j][e], id);
      }
  }
};

template <int KV>
__device__ __forceinline__ void select_interval(const uint32_t (&u)[KV][4], int c, SelShared& S, uint32_t ilo,
                                                uint32_t ihi, int need, int n_in, uint32_t& Tu, int& Tid) {
  select_interval_each(RegKeys<KV>{u, c}, c, S, ilo, ihi, need, n_in, Tu, Tid);
}

template <int KV>
__device__ __forceinline__ void select_regs(const uint32_t (&u)[KV][4], int c, int p, SelShared& S,
                                            uint32_t& Tu, int& Tid) {
  const int tid = threadIdx.x, NT = blockDim.x;
  auto idof = [&](int j, int e) { return 4 * (tid + j * NT) + e; };
  uint32_t vmax = 0u, vmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < KV; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (idof(j, e) < c) { vmax = max(vmax, u[j][e]); vmin = min(vmin, u[j][e]); }
  block_minmax2(vmax, vmin, S.wred[0], S.wred[1]);
  select_interval<KV>(u, c, S, vmin, vmax, p, c, Tu, Tid);
}

// Word popcounts of S.bitmap turned into prefix offsets (S.woff), for kept_at.
__device__ __forceinline__ void bitmap_prefix(int c, SelShared& S) {
  const int tid = threadIdx.x, NT = blockDim.x;
  const int nwords = (c + 31) >> 5;
  int carry = 0;
  for (int w0 = 0; w0 < nwords; w0 += NT) {
    const int w = w0 + tid;
    const int pc = w < nwords ? __popc(S.bitmap[w]) : 0;
    int tot;
    const int before = block_scan(pc, S.wtot[4 + ((w0 / NT) & 1)], tot);
    if (w < nwords) S.woff[w] = carry + before;
    carry += tot;
  }
  __syncthreads();
}

// Mark the kept keys in the bitmap and turn its word popcounts into prefix offsets (woff).
template <int KV>
__device__ __forceinline__ void mark_kept(const uint32_t (&u)[KV][4], int c, uint32_t Tu, int Tid, SelShared& S) {
  const int tid = threadIdx.x, NT = blockDim.x;
#pragma unroll
  for (int j = 0; j < KV; ++j) {
    const int id0 = 4 * (tid + j * NT);
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int id = id0 + e;
      m |= (id < c && (u[j][e] > Tu || (u[j][e] == Tu && id <= Tid))) ? (1u << e) : 0u;
    }
    if (m) atomicOr(&S.bitmap[id0 >> 5], m << (id0 & 31));
  }
  __syncthreads();
  bitmap_prefix(c, S);
}

// The same for keys presented by `each` (as select_interval_each).
template <class Each>
__device__ __forceinline__ void mark_kept_each(const Each& each, int c, uint32_t Tu, int Tid, SelShared& S) {
  each([&](uint32_t x, int id) {
    if (x > Tu || (x == Tu && id <= Tid)) atomicOr(&S.bitmap[id >> 5], 1u << (id & 31));
  });
  __syncthreads();
  bitmap_prefix(c, S);
}

// Cluster id of ascending rank q among the kept ones (binary search over the word offsets).
__device__ __forceinline__ int kept_at(const SelShared& S, int nwords, int q) {
  int lo = 0, hi = nwords - 1;
  while (lo < hi) {                          // last word with woff <= q
    const int mid = (lo + hi + 1) >> 1;
    if (S.woff[mid] <= q) lo = mid; else hi = mid - 1;
  }
  uint32_t bits = S.bitmap[lo];
  for (int k = S.woff[lo]; k < q; ++k) bits &= bits - 1u;
  return (lo << 5) + __ffs(bits) - 1;
}

}  // namespace fh
