// FlashHead at one hidden state (B = 1): stage 1 and the fused selection + stage 2.
//
// "FlashHead: Efficient Drop-In Replacement for the Classification Head in Language Model
// Inference", Section 3.2: the centroid logits C h, the p clusters with the largest keys (the
// logits, or the logits / tau plus Gumbel noise: p draws without replacement), the logits of
// those clusters' tokens through the dense C2T map, and the argmax / Gumbel-max token.
//
// Three kernels per call, none of which waits for another workgroup:
//   k_b1_scores       streams C (one 4-row group per wave, every row load issued before any
//                     arithmetic) and writes the keys;
//   k_b1_stage2       every workgroup (one per CU) finds the same kept set from the keys,
//                     streams its share of the kept clusters' tiles and writes its best
//                     (key, token) candidate; the tiles of the clusters that are kept for
//                     certain are requested as soon as the boundary of the selection is known;
//   k_finalize_parts  reduces the per-workgroup candidates to the token.
//
// This file is compiled once per row format (FH_B1_RF = RF_F32, RF_BF16, RF_INT4); each object
// defines the two launchers of its format.
#include "fh_device.h"
#include "fh_internal.h"
#include "fh_rows.h"
#include "fh_select.h"

#ifndef FH_B1_RF
#error "compile with -DFH_B1_RF=0 (f32 rows), 1 (bf16 rows) or 2 (int4 rows)"
#endif

namespace fh {

struct B1Params {
  const void* h;
  const char* C;
  const uint16_t* c_scales;   // int4 centroids: their bf16 group scales
  int h_bf16, c, d, b, p;
  int cpad;             // key slots (a multiple of kB1Threads); the ones past c hold NaN
  int sample;
  float tau;
  Rng rng;
  float* keys;
  float* keys_out;      // optional copy of the keys (staged entry point)
  uint64_t* part;       // [gridDim.x] per-workgroup maxima of k_b1_stage2
  const int32_t* c2t;
  const char* tiles;
  const uint16_t* scales;
  int32_t* probe_out;
  float* logits_out;
  int32_t* tokens_out;
  int32_t* token;
};

// ------------------------------------------------------------------ stage 1

template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_b1_scores(B1Params a) {
  // key slots past c: quiet NaN, which every min, max and comparison of the selection ignores
  for (int i = a.c + blockIdx.x * kThreads + threadIdx.x; i < a.cpad; i += gridDim.x * kThreads)
    a.keys[i] = __uint_as_float(0x7FC00000u);
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int rb = row_bytes_of(RF, a.d);
  // h and the first rows are requested together; h is converted once both are in flight
  HRaw<RF, CH> hraw;
  load_h_raw<RF, CH>(hraw, a.h, a.h_bf16, a.d, lane);
  const int kfirst = wg * kRPI;
  RowGroup<RF, CH> g;
  if (kfirst < a.c) rows_load<RF, CH>(g, a.C, rb, kfirst, a.c, RF == RF_INT4 ? a.c_scales : nullptr, a.d >> 7, lane);
  HRegs<RF, CH> hr;
  unpack_h<RF, CH>(hr, hraw, a.h_bf16);
  for (int k0 = kfirst; k0 < a.c; k0 += nw * kRPI) {
    if (k0 != kfirst)
      rows_load<RF, CH>(g, a.C, rb, k0, a.c, RF == RF_INT4 ? a.c_scales : nullptr, a.d >> 7, lane);
    float s[kRPI];
    rows_dot<RF, CH>(g, hr, s);
    {                                            // lane i < kRPI: the key of row k0 + i
      const float si = lane_pick<kRPI>(s, lane);
      const int k = k0 + lane;
      if (lane < kRPI && k < a.c) {
        const float key = make_key(si, a.sample, a.tau, a.rng, 0u, 0u, (uint32_t)k);
        a.keys[k] = key;
        if (a.keys_out) a.keys_out[k] = key;
      }
    }
  }
}

// ------------------------------------------------------------------ selection + stage 2

// Key slots per thread of k_b1_stage2.
__host__ __device__ __forceinline__ int b1_slots(int c) { return b1_key_slots(c) / kB1Threads; }

constexpr int kS2MaxWords = 32768 / 64;
constexpr int kS2MaxCand = 64;             // keys the boundary bin may hold on the fast path
constexpr int kItemMax = 256;              // (cluster, row group) items one workgroup may own

struct S2Shared {
  int hist[kSelBins];
  // Bitmaps over the clusters, wave-major: bit l of w[wave NS + s] is cluster s 1024 + 64 wave + l.
  uint64_t words[kS2MaxWords];             // certain clusters (item mode, probe outputs) or all kept
  uint64_t bw[kS2MaxWords];                // the kept clusters of the boundary bin
  int pref[kS2MaxWords];                   // kept clusters before id-ordered word i (probe ids)
  float wmx[16], wmn[16];
  int wtot[16];
  int bnd[3];                              // boundary bin, keys above it, keys in it
  int ncand, nitems;
  float cx[kS2MaxCand];                    // the boundary bin's keys ...
  int cid[kS2MaxCand];                     // ... and clusters
  int items[kItemMax];                     // this workgroup's items: cluster << 8 | row group
  uint64_t wmax[16];
};

// Position of id-ordered word iw in a wave-major bitmap with NS slots.
template <int NS>
__device__ __forceinline__ int wm_index(int iw) { return (iw & 15) * NS + (iw >> 4); }

template <int NS>
__device__ __forceinline__ void wm_set(uint64_t* words, int k) {
  atomicOr((unsigned long long*)&words[((k >> 6) & 15) * NS + (k >> 10)], 1ull << (k & 63));
}

// Position of the (r + 1)-th set bit of v (0 <= r < popcount(v)): six halving steps.
__device__ __forceinline__ int nth_set_bit(uint64_t v, int r) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(v & ((1ull << w) - 1ull));
    const bool up = r >= c;
    r -= up ? c : 0;
    v = up ? v >> w : v;
    pos += up ? w : 0;
  }
  return pos;
}

// Cluster id of ascending rank q (wave-uniform) among the set bits of a wave-major bitmap;
// lane l scans the id-ordered words [l WPL, l WPL + WPL).  A rank past the last set bit gives 0.
template <int NS>
__device__ __forceinline__ int kept_rank_id(const uint64_t* words, int q) {
  constexpr int NW = NS * 16, WPL = NW >= 64 ? NW / 64 : 1;
  const int lane = threadIdx.x & 63;
  uint64_t wv[WPL];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < WPL; ++i) {
    const int iw = lane * WPL + i;
    wv[i] = iw < NW ? words[wm_index<NS>(iw)] : 0ull;
    cnt += __popcll(wv[i]);
  }
  const int incl = wave_incl_scan(cnt);
  const uint64_t hit = __ballot(incl > q);
  const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
  int id = 0;
  if (lane == L && hit) {
    int r = q - (incl - cnt);
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const int pc = __popcll(wv[i]);
      if (r >= 0 && r < pc) id = (lane * WPL + i) * 64 + nth_set_bit(wv[i], r);
      r -= pc;
    }
  }
  return __builtin_amdgcn_readlane(id, L);
}

// Set bits below cluster k (wave-uniform) in a wave-major bitmap: the ascending rank of k.
template <int NS>
__device__ __forceinline__ int kept_count_below(const uint64_t* words, int k) {
  constexpr int NW = NS * 16, WPL = NW >= 64 ? NW / 64 : 1;
  const int lane = threadIdx.x & 63;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < WPL; ++i) {
    const int iw = lane * WPL + i;
    if (iw < NW && iw <= (k >> 6)) {
      const uint64_t w = words[wm_index<NS>(iw)];
      cnt += __popcll(iw < (k >> 6) ? w : (w & ((1ull << (k & 63)) - 1ull)));
    }
  }
  return __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
}

// Selection and stage 2 for one hidden state in one kernel.  Every workgroup (1024 threads, one
// per CU) holds the c keys in registers (slot s of thread t: cluster 1024 s + t) and finds the
// same kept set, so no workgroup waits for another:
//  * one float-linear 2048-bin histogram between the key min and max locates the bin b holding
//    the p-th largest key; every key in a bin above b is kept for certain; wave 0 ranks the
//    keys of bin b exactly (key desc, id asc) and keeps the first p - above of them;
//  * the kept tiles are cut into items of NR rows, item (k, j) having the number
//    h = k * gpp + j (gpp items per cluster).  With 256 workgroups (p >= 256), workgroup g takes
//    the items with h % 256 == g: cluster k has an item there exactly when the thread holding
//    its key (t = k % 1024) satisfies (g - t * gpp) % 256 < gpp, so those threads list the
//    workgroup's certain items as soon as bin b is known, and the tile loads start before the
//    boundary keys are ranked, with no block-wide numbering of the kept clusters; wave 0 ranks
//    the boundary keys and takes the workgroup's items of the kept ones itself, so no other
//    wave waits for the ranking.  The number of items per workgroup is about p gpp / 256, the
//    kept clusters spreading over residues.
//  * with fewer workgroups (p < 256), with more items than a workgroup can list, or after the
//    general selection, the kept clusters are numbered 0 .. p-1 by ascending id (certain ones
//    first) and workgroup g takes the numbers g, g + G, ... (ranks from the kept bitmap).
// A boundary bin with more than kS2MaxCand keys (or all keys equal) sends the workgroup,
// block-uniformly, to the general selection (select_regs).  Each workgroup writes the packed
// maximum of its tokens to part[g].  Probe outputs are indexed by the ascending rank of the
// cluster among all kept ones.  NS: key slots per thread, NR: tile rows per item.
template <int RF, int CH, int NS, int NR>
__global__ __launch_bounds__(kB1Threads) void k_b1_stage2(B1Params a) {
  constexpr int NT = kB1Threads, NWAVE = NT / 64;
  constexpr int KV = NS >= 4 ? NS / 4 : 1;             // uint4 per thread of the general selection
  constexpr int NWID = NS * 16;                        // 64-bit bitmap words, padding included
  constexpr bool kEarlyH = CH * Fmt<RF>::EPC <= 32;    // h loads issued with the first tile rows
  __shared__ __align__(16) S2Shared Q;
  __shared__ SelShared S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, me = blockIdx.x;
  const int c = a.c, p = a.p;
  const bool want = a.probe_out || a.logits_out || a.tokens_out;
  const int gpp = (a.b + NR - 1) / NR;
  // items per workgroup by hash need 256 workgroups and few enough items to list
  bool itemized = G == kB1Workgroups && gpp <= kB1Workgroups &&                            // block-uniform
                  p * gpp <= (kItemMax / 4) * kB1Workgroups;
  // ---- keys; the slots past c hold NaN: ignored by min / max, never greater or equal
  float x[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) x[s] = a.keys[s * NT + tid];
  for (int i = tid; i < kSelBins; i += NT) Q.hist[i] = 0;
  for (int i = tid; i < NWID; i += NT) Q.bw[i] = 0ull;
  if (tid == 0) { Q.ncand = 0; Q.nitems = 0; }
  float mx = x[0], mn = x[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) { mx = fmaxf(mx, x[s]); mn = fminf(mn, x[s]); }
  mx = wave_minmax_f32<true>(mx);
  mn = wave_minmax_f32<false>(mn);
  if (lane == 0) { Q.wmx[wave] = mx; Q.wmn[wave] = mn; }
  __syncthreads();                                                          // 1
  float hi = Q.wmx[0], lo = Q.wmn[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) { hi = fmaxf(hi, Q.wmx[w]); lo = fminf(lo, Q.wmn[w]); }
  const float inv = (float)kSelBins / (hi - lo);
  bool fast = hi > lo && inv > 0.f && inv < 3.0e38f;                        // block-uniform
  const float off = -lo * inv;
  int bins[NS];
  if (fast) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {                 // NaN padding lands in bin 0
      bins[s] = (int)fminf(fmaxf(fmaf(x[s], inv, off), 0.f), (float)(kSelBins - 1));
      atomicAdd(&Q.hist[bins[s]], 1);
    }
    if (tid == 0 && NS * NT > c) atomicSub(&Q.hist[0], NS * NT - c);
  }
  __syncthreads();                                                          // 2
  // ---- boundary bin: wave w scans bins [2048 - 128 (w + 1), 2048 - 128 w) from the top
  const int top = kSelBins - 1 - 128 * wave - 2 * lane;
  int h_lo = 0, h_hi = 0, incl = 0;
  if (fast) {
    const int2 hh = *reinterpret_cast<const int2*>(&Q.hist[top - 1]);
    h_lo = hh.x;
    h_hi = hh.y;
    incl = wave_incl_scan(h_lo + h_hi);
    if (lane == 63) Q.wtot[wave] = incl;
  }
  __syncthreads();                                                          // 3
  if (fast) {
    int before = 0, bw = -1;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const int t = Q.wtot[w];
      if (bw < 0) {
        if (before + t >= p) bw = w;
        else before += t;
      }
    }
    if (wave == bw) {                       // the slice holding the p-th key resolves it
      const int cum = incl + before;
      const int L = __ffsll((unsigned long long)__ballot(cum >= p)) - 1;
      const int ex = cum - h_lo - h_hi;
      if (lane == L) {
        const bool upper = ex + h_hi >= p;
        Q.bnd[0] = upper ? top : top - 1;
        Q.bnd[1] = upper ? ex : ex + h_hi;
        Q.bnd[2] = upper ? h_hi : h_lo;
      }
    }
  }
  __syncthreads();                                                          // 4
  int b = 0, above = 0, inb = 0;
  if (fast) {
    b = Q.bnd[0];
    above = Q.bnd[1];
    inb = Q.bnd[2];
    fast = b > 0 && inb <= kS2MaxCand;
  }
  // ---- the keys of bin b compacted; this workgroup's items of the certain clusters listed by
  //      the threads that hold them; the certain bitmap when it is needed
  const int jme = (me - tid * gpp) & (kB1Workgroups - 1);     // this thread's row group, if < gpp
  if (fast) {
    const bool owner = itemized && jme < gpp;
    uint32_t wlo = 0u, whi = 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (owner && bins[s] > b) {
        const int pos = atomicAdd(&Q.nitems, 1);
        if (pos < kItemMax) Q.items[pos] = ((s * NT + tid) << 8) | jme;
      }
      if (want || !itemized) {
        const uint64_t m = __ballot(bins[s] > b);
        put_lane(wlo, (uint32_t)m, s);                               // the ballot into lane s
        put_lane(whi, (uint32_t)(m >> 32), s);
      }
      const uint64_t e = __ballot(bins[s] == b);
      if (e) {
        int base = 0;
        if (lane == __ffsll((unsigned long long)e) - 1) base = atomicAdd(&Q.ncand, __popcll(e));
        base = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(base, __ffsll((unsigned long long)e) - 1));
        const int pos = base + lane_prefix(e);
        if (bins[s] == b && pos < kS2MaxCand) { Q.cx[pos] = x[s]; Q.cid[pos] = s * NT + tid; }
      }
    }
    if ((want || !itemized) && lane < NS) Q.words[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
  }
  __syncthreads();                                                          // 5
  if (fast) fast = Q.ncand == inb;          // block-uniform
  int n_def = above;                        // rank numbers below n_def index Q.words, the rest Q.bw
  if (!fast) {                              // the general selection, then the full kept bitmap
    uint32_t u[KV][4];
    uint32_t Tu;
    int Tid;
    load_keys<KV>(a.keys, c, u, S);
    select_regs<KV>(u, c, p, S, Tu, Tid);
    const float T = ord_to_float(Tu);
    uint32_t wlo = 0u, whi = 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float v = NS < 32 ? x[s] : a.keys[s * NT + tid];     // 32 slots: not kept in registers
      const uint64_t m = __ballot(v > T) | __ballot(v == T && s * NT + tid <= Tid);
      put_lane(wlo, (uint32_t)m, s);                                 // the ballot into lane s
      put_lane(whi, (uint32_t)(m >> 32), s);
    }
    if (lane < NS) Q.words[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
    n_def = p;
    itemized = false;
  }
  if (itemized && Q.nitems > kItemMax) {   // block-uniform
    // more certain items than the list holds: number the kept clusters instead (the certain
    // bitmap from the keys again, the same bins)
    uint32_t wlo = 0u, whi = 0u;
    const float* kb = a.keys;
    asm volatile("" : "+s"(kb));            // fresh addresses here: none are kept from the first reads
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float v = kb[s * NT + tid];
      const int bn = (int)fminf(fmaxf(fmaf(v, inv, off), 0.f), (float)(kSelBins - 1));
      const uint64_t m = __ballot(bn > b && s * NT + tid < c);
      put_lane(wlo, (uint32_t)m, s);                                 // the ballot into lane s
      put_lane(whi, (uint32_t)(m >> 32), s);
    }
    if (lane < NS) Q.words[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
    itemized = false;
    __syncthreads();
  }
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  const int n1 = itemized ? Q.nitems : 0;  // this workgroup's items of certain clusters
  // ---- this wave's first item, when certain: requested while wave 0 ranks the boundary keys
  RowGroup<RF, CH, NR> g0;
  int tl0 = 0, k0 = -1;
  int bnd_id = 0, bnd_j = 0;                // wave 0, item mode: kept boundary clusters ...
  uint64_t bnd_mask = 0;                    // ... whose items this workgroup owns (lanes)
  HRaw<RF, CH> hraw;
  if constexpr (kEarlyH) load_h_raw<RF, CH>(hraw, a.h, a.h_bf16, a.d, lane);
  if (fast) {
    int q0 = -1, j00 = 0;
    if (itemized) {
      if (wave < n1) { q0 = Q.items[wave] >> 8; j00 = (Q.items[wave] & 255) * NR; }
    } else if (wave < (me < p ? (p - me + G - 1) / G : 0) * gpp) {
      const int qi = wave / gpp, q = me + qi * G;
      j00 = (wave - qi * gpp) * NR;
      if (q < above) q0 = kept_rank_id<NS>(Q.words, q);
    }
    if (q0 >= 0) {
      k0 = q0;
      const size_t row0 = (size_t)k0 * a.b;
      tl0 = (lane < NR && j00 + lane < a.b) ? a.c2t[row0 + j00 + lane] : 0;
      rows_load<RF, CH>(g0, a.tiles + row0 * rb, rb, j00, a.b, RF == RF_INT4 ? a.scales + row0 * spr : nullptr,
                        spr, lane);
    }
    if (wave == 0) {                        // rank the boundary keys; keep the first p - above
      const int n = inb;
      const int need = p - above;
      const bool act = lane < n;
      const float xt = act ? Q.cx[lane] : 0.f;
      const int it = act ? Q.cid[lane] : 0x7FFFFFFF;
      int rank = 0;
      for (int q = 0; q < n; ++q) {
        const float xq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xt), q));
        const int iq = __builtin_amdgcn_readlane(it, q);
        rank += (xq > xt || (xq == xt && iq < it)) ? 1 : 0;
      }
      const bool kept = act && rank < need;
      if (kept && (want || !itemized)) wm_set<NS>(Q.bw, it);
      // item mode: wave 0 itself takes this workgroup's items of kept boundary clusters
      bnd_id = it;
      bnd_j = (me - it * gpp) & (kB1Workgroups - 1);
      bnd_mask = __ballot(kept && itemized && bnd_j < gpp);
    }
  }
  // numbered mode and probe outputs need the kept boundary clusters in Q.bw; item mode
  // without probe outputs goes on without waiting for the ranking
  if (!itemized || want) __syncthreads();                                   // 6
  // ---- probe outputs: the kept clusters are Q.words | Q.bw (Q.bw is empty after the general
  //      selection); workgroup 0 writes their ids in ascending order
  if (want && me == 0 && a.probe_out) {
    int tot;
    const int pc = tid < NWID ? __popcll(Q.words[wm_index<NS>(tid)] | Q.bw[wm_index<NS>(tid)]) : 0;
    const int ex = block_scan(pc, Q.wtot, tot);
    if (tid < NWID) Q.pref[tid] = ex;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint64_t m = Q.words[wave * NS + s] | Q.bw[wave * NS + s];
      if ((m >> lane) & 1ull) a.probe_out[Q.pref[s * NWAVE + wave] + lane_prefix(m)] = s * NT + tid;
    }
  }
  // numbered mode: numbers below n_def are the ascending certain clusters (Q.words), the rest
  // the kept clusters of the boundary bin (Q.bw)
  const int nit = itemized ? n1 : (me < p ? (p - me + G - 1) / G : 0) * gpp;
  // ---- stage 2 on this workgroup's items
  HRegs<RF, CH> hr;
  if constexpr (kEarlyH) unpack_h<RF, CH>(hr, hraw, a.h_bf16);
  else load_h<RF, CH>(hr, a.h, a.h_bf16, a.d, lane);
  uint64_t bc = 0;
  // dot products, tokens and probe outputs of one item (cluster k, rows j0 .. j0 + NR - 1)
  auto item = [&](int k, int j0, int tl, const RowGroup<RF, CH, NR>& g) {
    float z[NR];
    rows_dot<RF, CH>(g, hr, z);
    const int qo = want ? kept_count_below<NS>(Q.words, k) + kept_count_below<NS>(Q.bw, k) : 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = j0 + i;
      if (j < a.b) {
        const int t = __builtin_amdgcn_readlane(tl, i);
        if (t >= 0) {                              // an empty slot (-1) is never chosen
          const float key = make_key(z[i], a.sample, a.tau, a.rng, 0u, 1u, (uint32_t)t);
          const uint64_t cnd = pack_cand(key, (uint32_t)t);
          bc = cnd > bc ? cnd : bc;
        }
        if (want && lane == 0) {
          if (a.logits_out) a.logits_out[(size_t)qo * a.b + j] = t >= 0 ? z[i] : -__builtin_huge_valf();
          if (a.tokens_out) a.tokens_out[(size_t)qo * a.b + j] = t;
        }
      }
    }
  };
  auto load_item = [&](int k, int j0, int& tl, RowGroup<RF, CH, NR>& g) {
    const size_t row0 = (size_t)k * a.b;
    tl = (lane < NR && j0 + lane < a.b) ? a.c2t[row0 + j0 + lane] : 0;
    rows_load<RF, CH>(g, a.tiles + row0 * rb, rb, j0, a.b, RF == RF_INT4 ? a.scales + row0 * spr : nullptr,
                      spr, lane);
  };
  for (int it = wave; it < nit; it += NWAVE) {
    if (it == wave && k0 >= 0) {
      item(k0, itemized ? (Q.items[it] & 255) * NR : (it - (it / gpp) * gpp) * NR, tl0, g0);
      continue;
    }
    int k, j0, tl;
    if (itemized) {
      k = Q.items[it] >> 8;
      j0 = (Q.items[it] & 255) * NR;
    } else {
      const int qi = it / gpp, q = me + qi * G;
      j0 = (it - qi * gpp) * NR;
      k = q < n_def ? kept_rank_id<NS>(Q.words, q) : kept_rank_id<NS>(Q.bw, q - n_def);
    }
    RowGroup<RF, CH, NR> g;
    load_item(k, j0, tl, g);
    item(k, j0, tl, g);
  }
  // item mode: wave 0 takes this workgroup's items of the kept boundary clusters
  for (uint64_t m = bnd_mask; m; m &= m - 1ull) {
    const int L = __builtin_ctzll(m);
    const int k = __builtin_amdgcn_readlane(bnd_id, L);
    const int j0 = __builtin_amdgcn_readlane(bnd_j, L) * NR;
    int tl;
    RowGroup<RF, CH, NR> g;
    load_item(k, j0, tl, g);
    item(k, j0, tl, g);
  }
  if (lane == 0) Q.wmax[wave] = bc;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = Q.wmax[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) m = Q.wmax[w] > m ? Q.wmax[w] : m;
    a.part[me] = m;
  }
}

// The token: the largest of the per-workgroup maxima part[0 .. n).  (Templated on the row
// format only so that each object of this file has its own copy.)
template <int RF>
__global__ __launch_bounds__(256) void k_finalize_parts(const uint64_t* part, int n, int32_t* token) {
  __shared__ uint64_t wm[4];
  const int tid = threadIdx.x;
  uint64_t m = 0;
  for (int i = tid; i < n; i += 256) m = part[i] > m ? part[i] : m;
  m = wave_max_u64(m);
  if ((tid & 63) == 0) wm[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    uint64_t r = wm[0];
    for (int w = 1; w < 4; ++w) r = wm[w] > r ? wm[w] : r;
    token[0] = (int32_t)cand_id(r);
  }
}

// ------------------------------------------------------------------ launchers (row format FH_B1_RF)

constexpr int kRF = FH_B1_RF;

// Chunk slots per lane: 1 .. 8 (int4 rows: 1 .. 4; the argument checks keep d within these).
#define FH_B1_DISPATCH_CH(CH, ...)                                \
  switch (CH) {                                                   \
    case 1: { constexpr int kCH = 1; __VA_ARGS__; } break;        \
    case 2: { constexpr int kCH = 2; __VA_ARGS__; } break;        \
    case 3: { constexpr int kCH = 3; __VA_ARGS__; } break;        \
    case 4: { constexpr int kCH = 4; __VA_ARGS__; } break;        \
    case 5: { constexpr int kCH = 5; __VA_ARGS__; } break;        \
    case 6: { constexpr int kCH = 6; __VA_ARGS__; } break;        \
    case 7: { constexpr int kCH = 7; __VA_ARGS__; } break;        \
    case 8: { constexpr int kCH = 8; __VA_ARGS__; } break;        \
    default: return hipErrorInvalidValue;                         \
  }
constexpr int kMaxCH = kRF == RF_INT4 ? 4 : 8;

static B1Params params_of(const B1Args& x) {
  B1Params a{};
  a.h = x.h; a.C = (const char*)x.C; a.c_scales = x.c_scales; a.h_bf16 = x.h_bf16;
  a.c = x.c; a.d = x.d; a.b = x.b; a.p = x.p; a.cpad = b1_key_slots(x.c);
  a.sample = x.sample; a.tau = x.tau; a.rng = make_rng(x.seed, x.step);
  a.keys = x.keys; a.keys_out = x.keys_out; a.part = x.part;
  a.c2t = x.c2t; a.tiles = (const char*)x.tiles; a.scales = x.scales;
  a.probe_out = x.probe_out; a.logits_out = x.logits_out; a.tokens_out = x.tokens_out; a.token = x.token;
  return a;
}

template <int CH>
static void launch_scores_ch(const B1Params& a, hipStream_t st) {
  if constexpr (CH <= kMaxCH) {
    const int groups = (a.c + kRPI - 1) / kRPI;          // one row group per wave
    const int wgs = (groups + 3) / 4;
    hipLaunchKernelGGL((k_b1_scores<kRF, CH>), dim3(wgs), dim3(kThreads), 0, st, a);
  }
}

// Two tile rows per item only where the kernel still holds them in registers (longer rows
// spill): fp32 rows up to 4 chunk slots, bf16 up to 3, int4 rows 1.
template <int CH>
constexpr bool kTwoRowsFit = kRF == RF_F32 ? CH <= 4 : kRF == RF_BF16 ? CH <= 3 : CH <= 1;

template <int CH, int S>
static void launch_stage2_s(const B1Params& a, int G, int nr, hipStream_t st) {
  if constexpr (kTwoRowsFit<CH>) {
    if (nr == 2) {
      hipLaunchKernelGGL((k_b1_stage2<kRF, CH, S, 2>), dim3(G), dim3(kB1Threads), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_b1_stage2<kRF, CH, S, 1>), dim3(G), dim3(kB1Threads), 0, st, a);
}

template <int CH>
static void launch_stage2_ch(const B1Params& a, hipStream_t st) {
  if constexpr (CH > kMaxCH) return;
  const int G = a.p < kB1Workgroups ? a.p : kB1Workgroups;
  const int n_my = (a.p + G - 1) / G;
  const int nr = n_my * a.b <= kB1Threads / 64 ? 1 : 2;     // one row per wave when that fills them
  const int slots = b1_slots(a.c);
  if (slots <= 2)       launch_stage2_s<CH, 2>(a, G, nr, st);
  else if (slots <= 4)  launch_stage2_s<CH, 4>(a, G, nr, st);
  else if (slots <= 8)  launch_stage2_s<CH, 8>(a, G, nr, st);
  else if (slots <= 16) launch_stage2_s<CH, 16>(a, G, nr, st);
  else                  launch_stage2_s<CH, 32>(a, G, nr, st);
  hipLaunchKernelGGL(k_finalize_parts<kRF>, dim3(1), dim3(256), 0, st, (const uint64_t*)a.part, G, a.token);
}

#if FH_B1_RF == 0
#define FH_B1_FN(name) name##_f32
#elif FH_B1_RF == 1
#define FH_B1_FN(name) name##_bf16
#else
#define FH_B1_FN(name) name##_int4
#endif

hipError_t FH_B1_FN(launch_b1_scores)(const B1Args& x, hipStream_t st) {
  const B1Params a = params_of(x);
  FH_B1_DISPATCH_CH(chunk_slots(kRF, x.d), launch_scores_ch<kCH>(a, st));
  return hipGetLastError();
}

hipError_t FH_B1_FN(launch_b1_stage2)(const B1Args& x, hipStream_t st) {
  const B1Params a = params_of(x);
  FH_B1_DISPATCH_CH(chunk_slots(kRF, x.d), launch_stage2_ch<kCH>(a, st));
  return hipGetLastError();
}

}  // namespace fh
