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
//                     certain are requested before the rest of the selection is resolved;
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
  int cpad;             // key slots (a multiple of kB1Threads); the ones past c hold -inf
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
  // key slots past c: -inf is never kept (every real key is finite)
  for (int i = a.c + blockIdx.x * kThreads + threadIdx.x; i < a.cpad; i += gridDim.x * kThreads)
    a.keys[i] = -__builtin_huge_valf();
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
constexpr int kSegCap = 128;               // middle keys one wave may hold
constexpr int kS2RankMax = 64;             // keys one wave ranks exactly
constexpr int kSubBits = 9;                // sub-histogram of the middle keys: 512 bins
constexpr int kSubBins = 1 << kSubBits;
constexpr int kSampBins = 128;             // histogram of wave 0's keys (the threshold sample)

struct S2Shared {
  // Bitmaps over the clusters, wave-major: bit l of w[wave NS + s] is cluster s 1024 + 64 wave + l.
  uint64_t words[kS2MaxWords];             // clusters with keys >= T_hi (kept for certain)
  uint64_t bw[kS2MaxWords];                // the other kept clusters
  uint64_t fullw[kS2MaxWords];             // all kept clusters (probe outputs; the general selection)
  int pref[kS2MaxWords];                   // kept clusters before id-ordered word i (probe ids)
  __align__(16) int sub[kSubBins];         // middle keys per sub-bin of [T_lo, T_hi)
  int samp[kSampBins];
  float cx[16 * kSegCap];                  // middle keys, wave w's at [w kSegCap, (w + 1) kSegCap) ...
  int cid[16 * kSegCap];                   // ... and their clusters
  float cx2[kS2RankMax];                   // the middle keys of the boundary sub-bin ...
  int cid2[kS2RankMax];                    // ... and their clusters
  int nhi[16], nmid[16];
  int wtot[16];
  float thr[2];                            // T_hi, T_lo
  int ncand2;
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

// One wave: of the n <= 64 keys (cx, cid) in LDS, sets the `need` largest (ties to the smaller
// cluster id) in the wave-major bitmap bw.  Exact: ranks by all pairwise comparisons.
template <int NS>
__device__ __forceinline__ void rank_keep(const float* cx, const int* cid, int n, int need, uint64_t* bw) {
  const int lane = threadIdx.x & 63;
  const bool act = lane < n;
  const float xt = act ? cx[lane] : 0.f;
  const int it = act ? cid[lane] : 0x7FFFFFFF;
  int rank = 0;
  for (int q = 0; q < n; ++q) {
    const float xq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xt), q));
    const int iq = __builtin_amdgcn_readlane(it, q);
    rank += (xq > xt || (xq == xt && iq < it)) ? 1 : 0;
  }
  if (act && rank < need) wm_set<NS>(bw, it);
}

// One wave: in a histogram of 512 bins (lane l: bins [8 l, 8 l + 8)), the bin holding the
// need-th largest item counted from the top (the bins above it hold fewer than need items,
// with it at least need).  Returns (wave-uniform) the bin, the items above it and the items
// in it; bin -1 if the histogram holds fewer than need items.
__device__ __forceinline__ int3 wave_boundary_bin(const int* hist, int need) {
  const int lane = threadIdx.x & 63;
  const int4* hv = reinterpret_cast<const int4*>(hist) + 2 * lane;
  const int4 v0 = hv[0], v1 = hv[1];
  const int n[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  int t = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += n[j];
  const int in = wave_incl_scan(t);
  int cum = __builtin_amdgcn_readlane(in, 63) - in;        // items in the lanes above this one
  const bool mine = cum < need && cum + t >= need;
  int3 r = make_int3(-1, 0, 0);
  if (mine) {
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      if (r.x < 0 && cum + n[j] >= need) r = make_int3(8 * lane + j, cum, n[j]);
      cum += n[j];
    }
  }
  const uint64_t who = __ballot(mine);
  if (!who) return make_int3(-1, 0, 0);
  const int L = __ffsll((unsigned long long)who) - 1;
  return make_int3(__builtin_amdgcn_readlane(r.x, L), __builtin_amdgcn_readlane(r.y, L),
                   __builtin_amdgcn_readlane(r.z, L));
}

// Selection and stage 2 for one hidden state in one kernel.  Every workgroup (1024 threads, one
// per CU) holds the c keys in registers (slot s of thread t: cluster 1024 s + t) and finds the
// same kept set:
//  1. wave 0 estimates two thresholds from a 128-bin histogram of its own c/16 keys: about
//     0.7 p keys of all lie at or above T_hi, and p with a margin at or above T_lo;
//  2. one pass over the keys: those >= T_hi go into a bitmap (N_hi of them), those in
//     [T_lo, T_hi) into per-wave LDS lists and a 512-bin histogram of their order-preserving
//     codes (N_mid); if N_hi <= p <= N_hi + N_mid, the clusters >= T_hi are kept for certain
//     and the tiles of this workgroup's share of them are requested at once;
//  3. every wave finds the sub-bin of the 512 holding the (p - N_hi)-th middle key; the middle
//     keys above it are kept, and wave 0 ranks the <= 64 in it exactly (key desc, id asc) while
//     the other waves' tile loads are in flight.
// Kept clusters are numbered 0 .. p-1: the certain ones by ascending id, then the others by
// ascending id; workgroup g takes the numbers g, g + G, ...  Thresholds that miss (fewer than
// p keys >= T_lo, more than p >= T_hi, a full list) or a boundary sub-bin with more than 64 keys
// send the workgroup, block-uniformly and before any tile load, to the general selection
// (select_regs), after which every kept cluster comes from one bitmap.  Each workgroup writes the packed maximum of its tokens to
// part[g].  Probe outputs are indexed by the ascending rank of the cluster among all kept ones.
// NS: key slots per thread, NR: tile rows per wave step.
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
  // ---- keys (slots past c hold -inf)
  float x[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) x[s] = a.keys[s * NT + tid];
  for (int i = tid; i < NWID; i += NT) Q.bw[i] = 0ull;
  for (int i = tid; i < kSubBins; i += NT) Q.sub[i] = 0;
  if (tid < kSampBins) Q.samp[tid] = 0;
  if (tid == 0) Q.ncand2 = 0;
  __syncthreads();                                                          // 1
  // ---- 1. thresholds from wave 0's keys
  if (wave == 0) {
    float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf();
    int n0 = 0;                                          // wave 0's real keys (a closed form)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int left = c - s * NT;
      n0 += left >= 64 ? 64 : (left > 0 ? left : 0);
      if (s * NT + tid < c) { mx = fmaxf(mx, x[s]); mn = fminf(mn, x[s]); }
    }
    mx = wave_minmax_f32<true>(mx);
    mn = wave_minmax_f32<false>(mn);
    // sample ranks: k_hi ~ 0.7 p n0 / c; k_lo ~ 1.4 p n0 / c plus three standard deviations
    const float ps = (float)p * (float)n0 / (float)c;
    const int khi = (int)(0.7f * ps);
    const int klo = (int)ceilf(1.4f * ps + 3.0f * sqrtf(ps) + 2.0f);
    float thi = __builtin_huge_valf(), tlo = -3.4028235e38f;      // +inf / the lowest finite
    if (mx > mn) {
      const float scale = (float)kSampBins / (mx - mn);
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (s * NT + tid < c) atomicAdd(&Q.samp[min((int)((x[s] - mn) * scale), kSampBins - 1)], 1);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // lane l: bins 2 l, 2 l + 1; counts from the top
      const int h0 = Q.samp[2 * lane], h1 = Q.samp[2 * lane + 1];
      const int in = wave_incl_scan(h0 + h1);
      const int above = __builtin_amdgcn_readlane(in, 63) - in;   // sample keys in bins above 2 l + 1
      // T_hi: the upper edge of the bin where the count from the top reaches khi (fewer than khi
      // sample keys lie at or above it); T_lo: the lower edge of the bin where it reaches klo
      if (khi >= 1) {
        const bool in1 = above < khi && above + h1 >= khi;
        const bool in0 = above + h1 < khi && above + h1 + h0 >= khi;
        if (in1) thi = mn + (float)(2 * lane + 2) / scale;
        if (in0) thi = mn + (float)(2 * lane + 1) / scale;
      }
      if (klo < n0) {
        const bool in1 = above < klo && above + h1 >= klo;
        const bool in0 = above + h1 < klo && above + h1 + h0 >= klo;
        if (in1) tlo = mn + (float)(2 * lane + 1) / scale;
        if (in0) tlo = mn + (float)(2 * lane) / scale;
      }
      thi = wave_minmax_f32<false>(thi);
      tlo = wave_minmax_f32<true>(tlo);
    }
    if (lane == 0) { Q.thr[0] = thi; Q.thr[1] = tlo; }
  }
  __syncthreads();                                                          // 2
  // ---- 2. one pass: certain keys into the bitmap, middle keys into lists and the sub-histogram
  const float T_hi = Q.thr[0], T_lo = Q.thr[1];
  const uint32_t olo = ord_key(T_lo);
  const uint32_t span = ord_key(T_hi) - olo;
  const int shift = span > (uint32_t)kSubBins ? 32 - __clz((int)((span - 1u) >> kSubBits)) : 0;
  {
    uint32_t wlo = 0u, whi = 0u;
    int nh = 0, nm = 0;                                  // wave-uniform
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float v = x[s];
      const bool hi = v >= T_hi;
      const uint64_t mh = __ballot(hi);
      put_lane(wlo, (uint32_t)mh, s);                                 // the ballot into lane s
      put_lane(whi, (uint32_t)(mh >> 32), s);
      nh += __popcll(mh);
      const bool mid = v >= T_lo && !hi;                 // never the -inf padding
      const uint64_t mm = __ballot(mid);
      if (mm) {
        if (mid) {
          const int pos = nm + lane_prefix(mm);
          if (pos < kSegCap) { Q.cx[wave * kSegCap + pos] = v; Q.cid[wave * kSegCap + pos] = s * NT + tid; }
          atomicAdd(&Q.sub[(int)((ord_key(v) - olo) >> shift)], 1);
        }
        nm += __popcll(mm);
      }
    }
    if (lane < NS) Q.words[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
    if (lane == 0) { Q.nhi[wave] = nh; Q.nmid[wave] = nm; }
  }
  __syncthreads();                                                          // 3
  int n_hi = 0, n_mid = 0;
  bool full = false;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    n_hi += Q.nhi[w];
    n_mid += Q.nmid[w];
    full = full || Q.nmid[w] > kSegCap;
  }
  // the keys >= T_hi are kept for certain only if there are at most p of them and the middle
  // keys complete them to at least p; the middle keys of the boundary sub-bin must fit one wave
  bool fast = n_hi <= p && p <= n_hi + n_mid && !full;                   // block-uniform
  int3 bb = make_int3(-1, 0, 0);
  if (fast && p > n_hi) {
    bb = wave_boundary_bin(Q.sub, p - n_hi);
    fast = bb.x >= 0 && bb.z <= kS2RankMax;
  }
  if (!fast) {
    // the exact selection over all keys; every kept cluster goes to Q.bw
    uint32_t u[KV][4];
    uint32_t Tu;
    int Tid;
    load_keys<KV>(a.keys, c, u, S);
    select_regs<KV>(u, c, p, S, Tu, Tid);
    const float T = ord_to_float(Tu);
    uint32_t wlo = 0u, whi = 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float v = a.keys[s * NT + tid];
      const uint64_t m = __ballot(v > T) | __ballot(v == T && s * NT + tid <= Tid);
      put_lane(wlo, (uint32_t)m, s);                                 // the ballot into lane s
      put_lane(whi, (uint32_t)(m >> 32), s);
    }
    if (lane < NS) Q.bw[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
    n_hi = 0;
  }
  const int n_def = n_hi;                   // numbers below n_def index Q.words, the rest Q.bw
  const int n_my = me < p ? (p - me + G - 1) / G : 0;
  const int gpp = (a.b + NR - 1) / NR;
  const int nit = n_my * gpp;
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  // ---- this wave's first tile rows, when certain: resolved and requested now
  RowGroup<RF, CH, NR> g0;
  int tl0 = 0, k0 = -1;
  HRaw<RF, CH> hraw;
  if constexpr (kEarlyH) load_h_raw<RF, CH>(hraw, a.h, a.h_bf16, a.d, lane);
  if (fast && wave < nit) {
    const int qi = wave / gpp, j0 = (wave - qi * gpp) * NR;
    const int q = me + qi * G;
    if (q < n_def) {
      k0 = kept_rank_id<NS>(Q.words, q);
      const size_t row0 = (size_t)k0 * a.b;
      tl0 = (lane < NR && j0 + lane < a.b) ? a.c2t[row0 + j0 + lane] : 0;
      rows_load<RF, CH>(g0, a.tiles + row0 * rb, rb, j0, a.b, RF == RF_INT4 ? a.scales + row0 * spr : nullptr,
                        spr, lane);
    }
  }
  // ---- 3. the kept middle keys: above the boundary sub-bin, and the ranked ones in it
  if (fast && p > n_hi) {
    const int nmine = Q.nmid[wave];          // wave w marks its own list
    for (int i = lane; i < nmine; i += 64) {
      const float v = Q.cx[wave * kSegCap + i];
      const int sb = (int)((ord_key(v) - olo) >> shift);
      if (sb > bb.x) {
        wm_set<NS>(Q.bw, Q.cid[wave * kSegCap + i]);
      } else if (sb == bb.x) {
        const int pos = atomicAdd(&Q.ncand2, 1);
        Q.cx2[pos] = v;
        Q.cid2[pos] = Q.cid[wave * kSegCap + i];
      }
    }
    __syncthreads();
    if (wave == 0) rank_keep<NS>(Q.cx2, Q.cid2, bb.z, p - n_hi - bb.y, Q.bw);
  }
  __syncthreads();                                                          // 4
  // ---- probe outputs: the full kept bitmap gives every cluster its ascending rank
  const uint64_t* fw = Q.fullw;
  if (want) {
    for (int i = tid; i < NWID; i += NT) Q.fullw[i] = (n_def ? Q.words[i] : 0ull) | Q.bw[i];   // n_def = 0: words unused
    __syncthreads();
    if (me == 0 && a.probe_out) {
      int tot2;
      const int pc = tid < NWID ? __popcll(fw[wm_index<NS>(tid)]) : 0;
      const int ex = block_scan(pc, Q.wtot, tot2);
      if (tid < NWID) Q.pref[tid] = ex;
      __syncthreads();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint64_t m = fw[wave * NS + s];
        if ((m >> lane) & 1ull) a.probe_out[Q.pref[s * NWAVE + wave] + lane_prefix(m)] = s * NT + tid;
      }
    }
  }
  // ---- stage 2 on this workgroup's clusters
  HRegs<RF, CH> hr;
  if constexpr (kEarlyH) unpack_h<RF, CH>(hr, hraw, a.h_bf16);
  else load_h<RF, CH>(hr, a.h, a.h_bf16, a.d, lane);
  uint64_t bc = 0;
  for (int it = wave; it < nit; it += NWAVE) {
    const int qi = it / gpp, j0 = (it - qi * gpp) * NR;
    const int q = me + qi * G;
    int k, tl;
    RowGroup<RF, CH, NR> g;
    if (it == wave && k0 >= 0) {
      k = k0;
      tl = tl0;
      g = g0;
    } else {
      k = q < n_def ? kept_rank_id<NS>(Q.words, q) : kept_rank_id<NS>(Q.bw, q - n_def);
      const size_t row0 = (size_t)k * a.b;
      tl = (lane < NR && j0 + lane < a.b) ? a.c2t[row0 + j0 + lane] : 0;
      rows_load<RF, CH>(g, a.tiles + row0 * rb, rb, j0, a.b, RF == RF_INT4 ? a.scales + row0 * spr : nullptr,
                        spr, lane);
    }
    float z[NR];
    rows_dot<RF, CH>(g, hr, z);
    const int qo = want ? kept_count_below<NS>(fw, k) : 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = j0 + i;
      if (j < a.b) {
        const int t = __builtin_amdgcn_readlane(tl, i);
        const float key = make_key(z[i], a.sample, a.tau, a.rng, 0u, 1u, (uint32_t)t);
        const uint64_t cnd = pack_cand(key, (uint32_t)t);
        bc = cnd > bc ? cnd : bc;
        if (want && lane == 0) {
          if (a.logits_out) a.logits_out[(size_t)qo * a.b + j] = z[i];
          if (a.tokens_out) a.tokens_out[(size_t)qo * a.b + j] = t;
        }
      }
    }
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

template <int CH, int S>
static void launch_stage2_s(const B1Params& a, int G, int nr, hipStream_t st) {
  if (nr == 1) hipLaunchKernelGGL((k_b1_stage2<kRF, CH, S, 1>), dim3(G), dim3(kB1Threads), 0, st, a);
  else         hipLaunchKernelGGL((k_b1_stage2<kRF, CH, S, 2>), dim3(G), dim3(kB1Threads), 0, st, a);
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
