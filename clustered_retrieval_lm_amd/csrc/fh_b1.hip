// FlashHead at one hidden state (B = 1): stage 1 and the fused selection + stage 2.
//
// "FlashHead: Efficient Drop-In Replacement for the Classification Head in Language Model
// Inference", Section 3.2: the centroid logits C h, the p clusters with the largest keys (the
// logits, or the logits / tau plus Gumbel noise: p draws without replacement), the logits of
// those clusters' tokens through the dense C2T map, and the argmax / Gumbel-max token.
//
// Three kernels per call, none of which waits for another workgroup:
//   k_b1_scores       streams C (one 4-row group per wave, every row load issued before any
//                     arithmetic), writes the keys and, per group of g consecutive clusters
//                     (one workgroup), the group's m largest keys ranked: the candidate lists;
//   k_b1_stage2       every workgroup (one per CU) finds the same kept set from the lists (a
//                     few thousand entries instead of c keys; exact, with a fall-back to the
//                     selection over all keys when a list may be cut short), streams its share
//                     of the kept clusters' tiles and writes its best (key, token) candidate;
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
  int sample;
  float tau;
  Rng rng;
  float* keys;
  float* keys_out;      // optional copy of the keys (staged entry point)
  uint64_t* lst;        // candidate lists (B1Lists)
  int L, R;             // list entries (R of them real keys)
  int ng;               // groups: the lists are rank-major, entry (group, rank r) at r ng + group
  int use_list;         // the lists suit this p (else the selection runs over all keys)
  int fullable;         // m < g: a group's list may be cut short (its last entry is lst[16 w + 15])
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

// One workgroup of NWG waves per group of G = 4 NWG consecutive clusters: the keys, then the
// group's M = min(G, 16) largest in descending order (key desc, id asc): the entry of rank r goes to
// lst[r ngroups + group] (rank-major: a wave of the selection then holds one rank per list slot, and
// the waves holding ranks far down the lists skip the work of certain entries as a whole).
// The rank of an entry is the number of the group's entries that are larger as packed
// (ord key, ~id) values; every wave counts those among its own four and the counts meet in LDS.
template <int RF, int CH, int NWG>
__global__ __launch_bounds__(NWG * 64) void k_b1_scores(B1Params a) {
  constexpr int G = NWG * kRPI, M = G < 16 ? G : 16;
  __shared__ uint64_t pk[G];
  __shared__ int rk[G];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = row_bytes_of(RF, a.d);
  // h and the rows are requested together; h is converted once both are in flight
  HRaw<RF, CH> hraw;
  load_h_raw<RF, CH>(hraw, a.h, a.h_bf16, a.d, lane);
  const int k0 = blockIdx.x * G + wave * kRPI;
  RowGroup<RF, CH> g;
  rows_load<RF, CH>(g, a.C, rb, k0, a.c, RF == RF_INT4 ? a.c_scales : nullptr, a.d >> 7, lane);
  if (tid < G) rk[tid] = 0;
  HRegs<RF, CH> hr;
  unpack_h<RF, CH>(hr, hraw, a.h_bf16);
  float s[kRPI];
  rows_dot<RF, CH>(g, hr, s);
  {                                              // lane i < kRPI: the key of row k0 + i
    const float si = lane_pick<kRPI>(s, lane);
    const int k = k0 + lane;
    if (lane < kRPI) {
      uint64_t e = (uint64_t)(0xFFFFFFFFu - (uint32_t)k);      // past c: below every key
      if (k < a.c) {
        const float key = make_key(si, a.sample, a.tau, a.rng, 0u, 0u, (uint32_t)k);
        a.keys[k] = key;
        if (a.keys_out) a.keys_out[k] = key;
        e = pack_cand(key, (uint32_t)k);
      }
      pk[wave * kRPI + lane] = e;
    }
  }
  __syncthreads();
  if (lane < G) {                                // entries of this wave above entry `lane`
    const uint64_t x = pk[lane];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kRPI; ++i) n += pk[wave * kRPI + i] > x ? 1 : 0;
    if (n) atomicAdd(&rk[lane], n);
  }
  __syncthreads();
  if (tid < G) {
    const int r = rk[tid];
    if (r < M) a.lst[(size_t)r * gridDim.x + blockIdx.x] = pk[tid];
  }
}

// ------------------------------------------------------------------ selection + stage 2

constexpr int kS2MaxCand = 64;             // keys the boundary bin may hold on the fast path
constexpr int kItemMax = 256;              // (cluster, row group) items one workgroup may own

struct S2Shared {
  float wmx[16], wmn[16];
  int bnd[3];                              // boundary bin, entries above it, entries in it
  int ncand, nitems, full;
  float cx[kS2MaxCand];                    // the boundary bin's keys ...
  int cid[kS2MaxCand];                     // ... and clusters
  int items[kItemMax];                     // this workgroup's items: cluster << 8 | row group
  uint64_t wmax[16];
};

// The c keys of the workspace as the general selection takes them (re-read on every pass).
struct AllKeys {
  const float* keys;
  int c;
  template <class F>
  __device__ __forceinline__ void operator()(F&& f) const {
    for (int id = threadIdx.x; id < c; id += blockDim.x) f(ord_key(keys[id]), id);
  }
};

// Selection and stage 2 for one hidden state in one kernel.  Every workgroup (1024 threads, one
// per CU) finds the same kept set, so no workgroup waits for another:
//  * thread t holds list entries t + 1024 s (s < NL); one float-linear 2048-bin histogram
//    between the entries' min and max locates the bin b holding the p-th largest; every entry in
//    a bin above b is kept for certain; wave 0 ranks the entries of bin b exactly (key desc,
//    id asc) and keeps the first p - above of them.  The result is the top p of the c keys
//    unless a group whose list may be cut short (m < g) has its last entry in bin b or above:
//    then, and when bin b holds more than kS2MaxCand entries, the workgroup runs the general
//    selection over all c keys (select_interval_each), block-uniformly;
//  * the kept tiles are cut into items of NR rows, item (k, j) having the number
//    h = k * gpp + j (gpp items per cluster).  With 256 workgroups (p >= 256), workgroup g takes
//    the items with h % 256 == g: the thread holding cluster k's entry lists the workgroup's
//    items of k as soon as bin b is known, so the tile loads start before the boundary entries
//    are ranked, with no block-wide numbering of the kept clusters; wave 0 ranks the boundary
//    entries and takes the workgroup's items of the kept ones itself, so no other wave waits
//    for the ranking.  The number of items per workgroup is about p gpp / 256;
//  * with fewer workgroups (p < 256), with more items than a workgroup can list, after the
//    general selection, or with probe outputs, the kept clusters are marked in an id-ordered
//    bitmap whose prefix popcounts number them 0 .. p-1 by ascending id, and workgroup g takes
//    the numbers g, g + G, ...; probe outputs are written at each cluster's ascending rank.
// Each workgroup writes the packed maximum of its tokens to part[g].  NL: list slots per
// thread, NR: tile rows per item.
template <int RF, int CH, int NL, int NR>
__global__ __launch_bounds__(kB1Threads) void k_b1_stage2(B1Params a) {
  constexpr int NT = kB1Threads, NWAVE = NT / 64;
  constexpr bool kEarlyH = CH * Fmt<RF>::EPC <= 32;    // h loads issued with the first tile rows
  __shared__ __align__(16) S2Shared Q;
  __shared__ __align__(16) SelShared S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, me = blockIdx.x;
  const int c = a.c, p = a.p;
  const int nwords = (c + 31) >> 5;
  const bool want = a.probe_out || a.logits_out || a.tokens_out;
  const int gpp = (a.b + NR - 1) / NR;
  // items per workgroup by hash need 256 workgroups and few enough items to list
  bool itemized = G == kB1Workgroups && gpp <= kB1Workgroups &&                            // block-uniform
                  p * gpp <= (kItemMax / 4) * kB1Workgroups;
  bool fast = a.use_list != 0;                                                              // block-uniform
  // ---- list entries; past L, and the pads of a short last group, decode to NaN: ignored by
  //      min / max, never greater or equal, and counted in bin 0 only
  uint64_t e[NL];
  float x[NL];
#pragma unroll
  for (int s = 0; s < NL; ++s) {
    const int i = s * NT + tid;
    e[s] = (fast && i < a.L) ? a.lst[i] : 0ull;
  }
  for (int i = tid; i < kSelBins; i += NT) S.hist[i] = 0;
  for (int i = tid; i < kMaxWords; i += NT) S.bitmap[i] = 0u;
  if (tid == 0) { Q.ncand = 0; Q.nitems = 0; Q.full = 0; Q.bnd[0] = 0; Q.bnd[1] = 0; Q.bnd[2] = 0; }
#pragma unroll
  for (int s = 0; s < NL; ++s) x[s] = ord_to_float((uint32_t)(e[s] >> 32));
  float mx = x[0], mn = x[0];
#pragma unroll
  for (int s = 1; s < NL; ++s) { mx = fmaxf(mx, x[s]); mn = fminf(mn, x[s]); }
  mx = wave_minmax_f32<true>(mx);
  mn = wave_minmax_f32<false>(mn);
  if (lane == 0) { Q.wmx[wave] = mx; Q.wmn[wave] = mn; }
  __syncthreads();                                                          // 1
  float hi = Q.wmx[0], lo = Q.wmn[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) { hi = fmaxf(hi, Q.wmx[w]); lo = fminf(lo, Q.wmn[w]); }
  // the bins only need a map that is monotone in the key and the same in every thread, so the
  // hardware reciprocal serves
  const float inv = (float)kSelBins * __builtin_amdgcn_rcpf(hi - lo);
  fast = fast && hi > lo && inv > 0.f && inv < 3.0e38f;
  const float off = -lo * inv;
  // a NaN entry (a pad) falls in bin 0 (fmaxf returns the number): harmless, as the fast path
  // needs the boundary above bin 0, so bin 0 is never kept, ranked or counted above the boundary
  int bins[NL];
  if (fast) {
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      bins[s] = (int)fminf(fmaxf(fmaf(x[s], inv, off), 0.f), (float)(kSelBins - 1));
      atomicAdd(&S.hist[bins[s]], 1);
    }
  }
  __syncthreads();                                                          // 2
  // ---- boundary bin, found by wave 0 alone (one instruction costs a quarter of the issue slots it
  //      would take in every wave): lane l sums the 32 bins [2048 - 32 (l + 1), 2048 - 32 l), a
  //      scan from the top finds the slice holding the p-th entry, and a second scan over that
  //      slice's bins finds the bin.  No bin reaching p leaves bnd zero: the general selection.
  if (fast && wave == 0) {
    const int4* hp = reinterpret_cast<const int4*>(&S.hist[kSelBins - 32 * (lane + 1)]);
    int v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int4 q = hp[i];
      v += (q.x + q.y) + (q.z + q.w);
    }
    const int incl = wave_incl_scan(v);
    const int L = __ffsll((unsigned long long)__ballot(incl >= p)) - 1;
    if (L >= 0) {                           // wave-uniform
      const int before = L > 0 ? __builtin_amdgcn_readlane(incl, L - 1) : 0;
      const int bin = kSelBins - 32 * L - 1 - lane;
      const int hv = lane < 32 ? S.hist[bin > 0 ? bin : 0] : 0;
      const int incl2 = wave_incl_scan(hv) + before;
      const int J = __ffsll((unsigned long long)__ballot(lane < 32 && incl2 >= p)) - 1;
      if (lane == J) {
        Q.bnd[0] = bin;
        Q.bnd[1] = incl2 - hv;
        Q.bnd[2] = hv;
      }
    }
  }
  __syncthreads();                                                          // 3
  int b = 0, above = 0, inb = 0;
  if (fast) {
    b = Q.bnd[0];
    above = Q.bnd[1];
    inb = Q.bnd[2];
    fast = b > 0 && inb <= kS2MaxCand;
  }
  // ---- the entries of bin b compacted; this workgroup's items of the certain clusters listed by
  //      the threads that hold them; the certain clusters marked when numbering needs them; a
  //      group whose list may be cut short and whose last entry reaches bin b flagged
  const bool mark = want || !itemized;
  if (fast) {
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int id = (int)(0xFFFFFFFFu - (uint32_t)e[s]);
      const bool cert = bins[s] > b;
      if (a.fullable && bins[s] >= b && s * NT + tid >= a.L - a.ng) Q.full = 1;   // a group's last entry
      if (cert) {
        const int jme = (me - id * gpp) & (kB1Workgroups - 1);     // this workgroup's row group of id
        if (itemized && jme < gpp) {
          const int pos = atomicAdd(&Q.nitems, 1);
          if (pos < kItemMax) Q.items[pos] = (id << 8) | jme;
        }
        if (mark) atomicOr(&S.bitmap[id >> 5], 1u << (id & 31));
      }
      const uint64_t m = __ballot(bins[s] == b);
      if (m) {
        const int L0 = __ffsll((unsigned long long)m) - 1;
        int base = 0;
        if (lane == L0) base = atomicAdd(&Q.ncand, __popcll(m));
        base = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(base, L0));
        const int pos = base + lane_prefix(m);
        if (bins[s] == b && pos < kS2MaxCand) { Q.cx[pos] = x[s]; Q.cid[pos] = id; }
      }
    }
  }
  __syncthreads();                                                          // 4
  if (fast) fast = Q.ncand == inb && !Q.full;          // block-uniform
  if (!fast) {                              // the general selection over all c keys
    for (int i = tid; i < kSelBins; i += NT) S.hist[i] = 0;
    for (int i = tid; i < kMaxWords; i += NT) S.bitmap[i] = 0u;
    const AllKeys keys{a.keys, c};
    uint32_t vmax = 0u, vmin = 0xFFFFFFFFu;
    keys([&](uint32_t u, int) { vmax = max(vmax, u); vmin = min(vmin, u); });
    block_minmax2(vmax, vmin, S.wred[0], S.wred[1]);
    uint32_t Tu;
    int Tid;
    select_interval_each(keys, c, S, vmin, vmax, p, c, Tu, Tid);
    mark_kept_each(keys, c, Tu, Tid, S);    // the kept bitmap and its prefix offsets
    itemized = false;
  } else if (itemized && Q.nitems > kItemMax) {        // block-uniform
    // more certain items than the list holds: number the kept clusters instead
    if (!want) {
#pragma unroll
      for (int s = 0; s < NL; ++s)
        if (bins[s] > b) {
          const int id = (int)(0xFFFFFFFFu - (uint32_t)e[s]);
          atomicOr(&S.bitmap[id >> 5], 1u << (id & 31));
        }
    }
    itemized = false;
  }
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  const int n1 = itemized ? Q.nitems : 0;  // this workgroup's items of certain clusters
  // ---- this wave's first item: requested while wave 0 ranks the boundary entries
  RowGroup<RF, CH, NR> g0;
  int tl0 = 0, k0 = -1;
  int bnd_id = 0, bnd_j = 0;                // wave 0, item mode: kept boundary clusters ...
  uint64_t bnd_mask = 0;                    // ... whose items this workgroup owns (lanes)
  HRaw<RF, CH> hraw;
  if constexpr (kEarlyH) load_h_raw<RF, CH>(hraw, a.h, a.h_bf16, a.d, lane);
  if (fast) {
    if (itemized && wave < n1) {
      k0 = Q.items[wave] >> 8;
      const int j00 = (Q.items[wave] & 255) * NR;
      const size_t row0 = (size_t)k0 * a.b;
      tl0 = (lane < NR && j00 + lane < a.b) ? a.c2t[row0 + j00 + lane] : 0;
      rows_load<RF, CH>(g0, a.tiles + row0 * rb, rb, j00, a.b, RF == RF_INT4 ? a.scales + row0 * spr : nullptr,
                        spr, lane);
    }
    if (wave == 0) {                        // rank the boundary entries; keep the first p - above
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
      if (kept && !(itemized && !want)) atomicOr(&S.bitmap[it >> 5], 1u << (it & 31));
      // item mode: wave 0 itself takes this workgroup's items of kept boundary clusters
      bnd_id = it;
      bnd_j = (me - it * gpp) & (kB1Workgroups - 1);
      bnd_mask = __ballot(kept && itemized && bnd_j < gpp);
    }
  }
  // numbering and probe outputs need the whole kept bitmap and its prefix offsets (the general
  // selection built both); item mode without probe outputs goes on without waiting for the ranking
  if (fast && (!itemized || want)) {        // block-uniform
    __syncthreads();                                                        // 5
    bitmap_prefix(c, S);
  }
  // ---- probe outputs: workgroup 0 writes the kept ids in ascending order
  if (want && me == 0 && a.probe_out) {
    for (int w = tid; w < nwords; w += NT) {
      uint32_t bits = S.bitmap[w];
      int o = S.woff[w];
      while (bits) {
        a.probe_out[o++] = (w << 5) + __ffs(bits) - 1;
        bits &= bits - 1u;
      }
    }
  }
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
    const int qo = want ? S.woff[k >> 5] + __popc(S.bitmap[k >> 5] & ((1u << (k & 31)) - 1u)) : 0;
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
      item(k0, (Q.items[it] & 255) * NR, tl0, g0);
      continue;
    }
    int k, j0, tl;
    if (itemized) {
      k = Q.items[it] >> 8;
      j0 = (Q.items[it] & 255) * NR;
    } else {
      const int qi = it / gpp, q = me + qi * G;
      j0 = (it - qi * gpp) * NR;
      k = kept_at(S, nwords, q);
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

// The token: the largest of the per-workgroup maxima part[0 .. n), n <= 256, by one wave (each lane
// reduces four of them, then a butterfly of lane shuffles: no barrier).  (Templated on the row format
// only so that each object of this file has its own copy.)
template <int RF>
__global__ __launch_bounds__(64) void k_finalize_parts(const uint64_t* part, int n, int32_t* token) {
  const int lane = threadIdx.x;
  uint64_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = lane + 64 * q < n ? part[lane + 64 * q] : 0ull;     // all loads first
  uint64_t m = v[0] > v[1] ? v[0] : v[1];
  const uint64_t m2 = v[2] > v[3] ? v[2] : v[3];
  m = wave_max_u64(m > m2 ? m : m2);
  if (lane == 0) token[0] = (int32_t)cand_id(m);
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

// Thresholds of the list path: a group with m < g keeps on average lambda = g p / c of the p
// clusters, and its list is cut short only when it keeps all m = 16 (for lambda <= 4 about once
// in 10^5 groups); lists of more than 8192 entries are not held in registers.
static B1Params params_of(const B1Args& x) {
  B1Params a{};
  a.h = x.h; a.C = (const char*)x.C; a.c_scales = x.c_scales; a.h_bf16 = x.h_bf16;
  a.c = x.c; a.d = x.d; a.b = x.b; a.p = x.p;
  a.sample = x.sample; a.tau = x.tau; a.rng = make_rng(x.seed, x.step);
  a.keys = x.keys; a.keys_out = x.keys_out; a.part = x.part;
  const B1Lists l = b1_lists(x.c, x.c_slots);
  a.lst = x.lst; a.L = l.L; a.R = l.R; a.ng = l.ngroups;
  a.fullable = l.m < l.g;
  a.use_list = (l.m == l.g || (long)l.g * x.p <= 4L * x.c) && l.R >= x.p && l.L <= 8192;
  a.c2t = x.c2t; a.tiles = (const char*)x.tiles; a.scales = x.scales;
  a.probe_out = x.probe_out; a.logits_out = x.logits_out; a.tokens_out = x.tokens_out; a.token = x.token;
  return a;
}

template <int CH>
static void launch_scores_ch(const B1Params& a, const B1Lists& l, hipStream_t st) {
  if constexpr (CH <= kMaxCH) {
    if constexpr (CH <= 3) {
      if (l.g == 64) {
        hipLaunchKernelGGL((k_b1_scores<kRF, CH, 16>), dim3(l.ngroups), dim3(1024), 0, st, a);
        return;
      }
    }
    if (l.g == 32) hipLaunchKernelGGL((k_b1_scores<kRF, CH, 8>), dim3(l.ngroups), dim3(512), 0, st, a);
    else           hipLaunchKernelGGL((k_b1_scores<kRF, CH, 4>), dim3(l.ngroups), dim3(256), 0, st, a);
  }
}

// Two tile rows per item only where the kernel still holds them in registers (longer rows
// spill): fp32 rows up to 4 chunk slots, bf16 up to 3, int4 rows 1.
template <int CH>
constexpr bool kTwoRowsFit = kRF == RF_F32 ? CH <= 4 : kRF == RF_BF16 ? CH <= 3 : CH <= 1;

template <int CH, int NL>
static void launch_stage2_nl(const B1Params& a, int G, int nr, hipStream_t st) {
  if constexpr (kTwoRowsFit<CH>) {
    if (nr == 2) {
      hipLaunchKernelGGL((k_b1_stage2<kRF, CH, NL, 2>), dim3(G), dim3(kB1Threads), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_b1_stage2<kRF, CH, NL, 1>), dim3(G), dim3(kB1Threads), 0, st, a);
}

template <int CH>
static void launch_stage2_ch(const B1Params& a, hipStream_t st) {
  if constexpr (CH > kMaxCH) return;
  const int G = a.p < kB1Workgroups ? a.p : kB1Workgroups;
  const int n_my = (a.p + G - 1) / G;
  const int nr = n_my * a.b <= kB1Threads / 64 ? 1 : 2;     // one row per wave when that fills them
  if (!a.use_list || a.L <= 2 * kB1Threads) launch_stage2_nl<CH, 2>(a, G, nr, st);
  else if (a.L <= 4 * kB1Threads)           launch_stage2_nl<CH, 4>(a, G, nr, st);
  else                                      launch_stage2_nl<CH, 8>(a, G, nr, st);
  hipLaunchKernelGGL(k_finalize_parts<kRF>, dim3(1), dim3(64), 0, st, (const uint64_t*)a.part, G, a.token);
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
  const B1Lists l = b1_lists(x.c, x.c_slots);
  FH_B1_DISPATCH_CH(chunk_slots(kRF, x.d), launch_scores_ch<kCH>(a, l, st));
  return hipGetLastError();
}

hipError_t FH_B1_FN(launch_b1_stage2)(const B1Args& x, hipStream_t st) {
  const B1Params a = params_of(x);
  FH_B1_DISPATCH_CH(chunk_slots(kRF, x.d), launch_stage2_ch<kCH>(a, st));
  return hipGetLastError();
}

}  // namespace fh
