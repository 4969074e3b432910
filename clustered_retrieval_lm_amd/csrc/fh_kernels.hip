// FlashHead kernels for gfx950 (CDNA4, wave64).
//
// Stage 1  k_scores_gemv / k_mfma<EPI_KEYS>  centroid logits C h -> probe keys
// Select   k_select                           per-row top-p on order-preserving uint32 keys
// Stage 2  k_tiles_probe (B == 1)             streams the kept clusters' contiguous tiles
//          k_tiles_mask  (B > 1)              min(c, 8192) workgroups loop over the list of clusters kept
//                                             by any row (each kept tile read once)
// Token    k_finalize                         packed (key, ~id) maxima -> token ids
// Dense    k_dense_gemv / k_mfma<EPI_ARGMAX>  the full-vocabulary comparator
// Offline  k_pack / k_check_counts            cluster-major tiles, optional int4 groups
//
// Method: "FlashHead: Efficient Drop-In Replacement for the Classification Head in
// Language Model Inference", Section 3.2 (two-stage retrieval, dense C2T).
#include <atomic>

#include "fh_device.h"
#include "fh_internal.h"
#include "fh_rows.h"
#include "fh_select.h"

namespace fh {


// ------------------------------------------------------------------ stage 1, row GEMV

struct ScoreParams {
  const void* h;
  const char* C;
  const uint16_t* c_scales;   // int4 centroids: their bf16 group scales
  int h_bf16, B, c, d;
  int sample;
  float tau;
  Rng rng;
  float* keys;
  float* keys_out;
  uint64_t* mask;
  int W;
  uint32_t* kflag;
  int32_t* nkept;
};

template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_scores_gemv(ScoreParams a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int wg = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int rb = row_bytes_of(RF, a.d);
  // h and the first rows are requested together; h is converted once both are in flight
  HRaw<RF, CH> hraw;
  load_h_raw<RF, CH>(hraw, (const char*)a.h + (size_t)r * a.d * (a.h_bf16 ? 2 : 4), a.h_bf16, a.d, lane);
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
        const float key = make_key(si, a.sample, a.tau, a.rng, (uint32_t)r, 0u, (uint32_t)k);
        a.keys[(size_t)r * a.c + k] = key;
        if (a.keys_out) a.keys_out[(size_t)r * a.c + k] = key;
      }
    }
    if (a.mask && r == 0) {                      // the selection's per-cluster state, cleared
      for (int j = lane; j < kRPI * a.W; j += kWave) {
        const int k = k0 + j / a.W;
        if (k < a.c) a.mask[(size_t)k * a.W + j % a.W] = 0ull;
      }
      if (lane < kRPI && k0 + lane < a.c) a.kflag[k0 + lane] = 0u;
      if (k0 == 0 && lane == 0) *a.nkept = 0;
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA GEMM
// S[n][m] = sum_k H[n][k] M[m][k] with v_mfma_f32_16x16x32_bf16: A = 16 rows of M
// (lane l: row l % 16, k = 8 (l / 16) .. +7), B = 16 rows of H (same lane map),
// D lane l: column n = l % 16, rows m = 4 (l / 16) + i.
//
// A workgroup of kMfmaWaves waves owns MT 16-row tiles of M at a time (32 to 64 rows) and NT
// 16-row tiles of H (up to 64 rows); its waves split K by pairs of K-steps (32 columns each):
// wave w takes the steps 2w, 2w + 1, 2w + 16, 2w + 17, ...  A wave issues the loads of up to
// GS of its K-steps (the whole range at d = 1024 and NT = 4) before any MFMA, so a tile costs
// about one memory round trip.  With
// NACC > 1 a wave rotates NACC accumulators per tile over its K-steps, shortening the rounding
// chain, and sums them by a tree at the end; the partial tiles of the 8 waves are summed in
// LDS by a fixed 3-level tree.  Roundings on the path of one product: <= 6 per MFMA (32 exact
// bf16 products and the accumulator, a tree of depth 6) times ceil(steps per wave / NACC),
// + log2(NACC), + 3; a wave takes at most 2 ceil(d / 512) steps.
constexpr int kMfmaWaves = 8;
// Every workgroup reads all of its H rows once per group: a CU streams about 24 KB/us, so the
// launch takes the smallest MT (2..4) whose groups fit on the CUs in one round.
constexpr int kMfmaMaxMT = 4;
constexpr int kMfmaThreads = kMfmaWaves * 64;

enum { EPI_KEYS = 0, EPI_ARGMAX = 1 };

struct MfmaParams {
  const uint16_t* H;
  const uint16_t* M;
  int B, rows, d;
  int sample;
  float tau;
  Rng rng;
  float* keys;        // EPI_KEYS: [B][rows]
  float* keys_out;
  uint64_t* mask;
  int W;
  uint32_t* kflag;    // EPI_KEYS, B > 1: the selection's per-cluster flags (cleared here)
  int32_t* nkept;
  uint64_t* best;     // EPI_ARGMAX: [B]
  float* logits;      // EPI_ARGMAX: [B][rows], may be null
};

template <int NT, int MT, int EPI>
__global__ __launch_bounds__(kMfmaThreads) void k_mfma(MfmaParams a) {
  constexpr int NW = kMfmaWaves;
  constexpr int NACC = NT == 1 ? 4 : NT == 2 ? 2 : 1;
  // K-steps per load group.  A CU keeps only about 64 KB of loads in flight, so a workgroup's
  // C and H bytes take several memory round trips whatever the grouping; with one H tile
  // (B <= 16) the group holds every step of the wave (up to 36 16-byte words of loads per lane,
  // a multiple of NACC so that step j always feeds accumulator j % NACC) and its loads queue
  // behind each other without an MFMA phase between them (int4 B = 16: 16.7 us instead of 19.4);
  // with more H tiles, groups of 2 - 4 steps measured faster (Qwen B = 64: 14.0 against 15.3)
  constexpr int GS0 = 36 / (MT + NT);
  constexpr int GS = NT == 1 ? (GS0 - GS0 % NACC > NACC ? GS0 - GS0 % NACC : NACC) : MT + NT <= 6 ? 4 : 2;
  __shared__ f32x4_t red[NW][MT * NT][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.y * 64;
  const int kq = (lane >> 4) * 8;
  const int nsteps = a.d / 32;
  const int ngroups = (a.rows + 16 * MT - 1) / (16 * MT);
  // workgroups start their K range at different even steps, so the ones running together read
  // different lines of H first
  const int rot = (nsteps & 1) ? 0 : (2 * (int)(blockIdx.x % 8u) * ((nsteps + 15) / 16)) % nsteps;
  const uint16_t* hp[NT];
  bool hv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + 16 * t + (lane & 15);
    hv[t] = n < a.B;
    hp[t] = a.H + (size_t)(hv[t] ? n : 0) * a.d + kq;
  }
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  uint64_t bc[NT];                                   // EPI_ARGMAX: best candidate per H tile
#pragma unroll
  for (int t = 0; t < NT; ++t) bc[t] = 0;
  for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int m0 = grp * 16 * MT;
    const uint16_t* mp[MT];
    bool mv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int mr = m0 + 16 * mt + (lane & 15);
      mv[mt] = mr < a.rows;
      mp[mt] = a.M + (size_t)(mv[mt] ? mr : 0) * a.d + kq;
    }
    f32x4_t acc[NACC][MT][NT];
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[q][mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the j-th K-step of this wave is 2 (wave + 8 (j / 2)) + j % 2: the two halves of each
    // 128-byte line of a row are read by one wave, back to back
    for (int j0 = 0; 2 * (wave + NW * (j0 >> 1)) < nsteps; j0 += GS) {
      uint4 av[GS][MT], bv[GS][NT];
#pragma unroll
      for (int u = 0; u < GS; ++u) {                 // every load of the group first
        const int j = j0 + u;
        int st = 2 * (wave + NW * (j >> 1)) + (j & 1);
        st = st < nsteps ? st + rot : 0;             // past the end: a valid address, masked below
        const int ko = (st >= nsteps ? st - nsteps : st) * 32;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[u][mt] = ld16_stream(mp[mt] + ko);
#pragma unroll
        for (int t = 0; t < NT; ++t) bv[u][t] = ld16(hp[t] + ko);
      }
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        const int j = j0 + u;
        if (2 * (wave + NW * (j >> 1)) + (j & 1) >= nsteps) continue;      // wave-uniform
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, mv[mt] ? av[u][mt] : z4);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint4 bb = hv[t] ? bv[u][t] : z4;
            acc[u % NACC][mt][t] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, bb), acc[u % NACC][mt][t], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t v = acc[0][mt][t];
        if constexpr (NACC == 2) v = v + acc[1][mt][t];
        if constexpr (NACC == 4) v = (v + acc[1][mt][t]) + (acc[2][mt][t] + acc[3][mt][t]);
        red[wave][mt * NT + t][lane] = v;
      }
    __syncthreads();
    for (int tile = wave; tile < MT * NT; tile += NW) {   // wave w finishes tiles w, w + 8
      const int mt = tile / NT, t = tile % NT;
      const f32x4_t v = ((red[0][tile][lane] + red[1][tile][lane]) + (red[2][tile][lane] + red[3][tile][lane])) +
                        ((red[4][tile][lane] + red[5][tile][lane]) + (red[6][tile][lane] + red[7][tile][lane]));
      const int n = n0 + 16 * t + (lane & 15);
      const int mb = m0 + 16 * mt + 4 * (lane >> 4);
      if (n < a.B) {
        // the four elements m = mb .. mb + 3 (mb % 4 == 0) share one Philox block
        const uint4 wb = a.sample ? rng_block(a.rng, (uint32_t)n, EPI == EPI_KEYS ? 0u : 1u, (uint32_t)mb >> 2)
                                  : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t wv[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mb + i;
          if (m < a.rows) {
            const float key = a.sample ? sample_key(v[i], a.tau, wv[i]) : v[i] + 0.0f;
            if (EPI == EPI_KEYS) {
              a.keys[(size_t)n * a.rows + m] = key;
              if (a.keys_out) a.keys_out[(size_t)n * a.rows + m] = key;
            } else {
              const uint64_t cnd = pack_cand(key, (uint32_t)m);
#pragma unroll
              for (int tt = 0; tt < NT; ++tt)
                if (tt == t) bc[tt] = cnd > bc[tt] ? cnd : bc[tt];
              if (a.logits) a.logits[(size_t)n * a.rows + m] = v[i];
            }
          }
        }
      }
    }
    if (EPI == EPI_KEYS && a.mask && blockIdx.y == 0) {   // the selection's per-cluster state, cleared
      for (int j = threadIdx.x; j < 16 * MT * a.W; j += kMfmaThreads) {
        const int m = m0 + j / a.W;
        if (m < a.rows) a.mask[(size_t)m * a.W + j % a.W] = 0ull;
      }
      if (threadIdx.x < 16 * MT && m0 + (int)threadIdx.x < a.rows) a.kflag[m0 + threadIdx.x] = 0u;
      if (m0 == 0 && threadIdx.x == 0) *a.nkept = 0;
    }
    __syncthreads();
  }
  if (EPI == EPI_ARGMAX && wave < MT * NT) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {                 // the H tiles this wave finished
      if (t != wave % NT && (MT * NT <= NW || NW % NT == 0)) continue;     // wave-uniform
      uint64_t b = bc[t];
      uint64_t o = __shfl_xor(b, 16, kWave);
      b = o > b ? o : b;
      o = __shfl_xor(b, 32, kWave);
      b = o > b ? o : b;
      const int n = n0 + 16 * t + lane;
      if (lane < 16 && n < a.B && b) atomicMax((unsigned long long*)&a.best[(size_t)n * kBestStride], (unsigned long long)b);
    }
  }
}


// ------------------------------------------------------------------ probe selection
// k_select: one 1024-thread workgroup per row of keys, held in registers as order-preserving
// uint32; select_regs finds the p-th largest (ties to the smaller id) and the kept ids are
// written in ascending order (prefix popcounts of a bitmap over the clusters).

// KV: key blocks of four per thread, the smallest power of two with 4 KV NT >= c.
template <int KV>
__global__ __launch_bounds__(kSelThreads) void k_select(const float* keys, int c, int p, int32_t* probes,
                                                        int32_t* probe_out, uint64_t* mask, int W,
                                                        uint64_t* best, uint32_t* kflag, int32_t* klist,
                                                        int32_t* nkept) {
  __shared__ SelShared S;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  uint32_t u[KV][4];
  uint32_t Tu;
  int Tid;
  load_keys<KV>(keys + (size_t)r * c, c, u, S);
  select_regs<KV>(u, c, p, S, Tu, Tid);
  mark_kept<KV>(u, c, Tu, Tid, S);
  const int nwords = (c + 31) >> 5;
  for (int q = tid; q < p; q += kSelThreads) {
    const int k = kept_at(S, nwords, q);
    probes[(size_t)r * p + q] = k;
    if (probe_out) probe_out[(size_t)r * p + q] = k;
    if (mask) {
      atomicOr((unsigned long long*)&mask[(size_t)k * W + (r >> 6)], 1ull << (r & 63));
      // the first row to keep k lists it (slots claimed once per wave)
      const bool first = atomicOr(&kflag[k], 1u) == 0u;
      const uint64_t bal = __ballot(first);
      if (bal) {
        const int leader = __ffsll((unsigned long long)bal) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(nkept, __popcll(bal));
        base = __shfl(base, leader, kWave);
        if (first) klist[base + lane_prefix(bal)] = k;
      }
    }
  }
  if (tid == 0) best[(size_t)r * kBestStride] = 0ull;
}

// ------------------------------------------------------------------ stage 2

struct TileParams {
  const int32_t* klist;   // B > 1: the clusters kept by any row ...
  const int32_t* nkept;   // ... and their count
  const void* h;
  int h_bf16, B, d, c, b, p;
  const int32_t* probes;
  const int32_t* c2t;
  const char* tiles;
  const uint16_t* scales;
  int sample;
  float tau;
  Rng rng;
  float* logits_out;
  int32_t* tokens_out;
  uint64_t* best;
  const uint64_t* mask;
  int W;
};

// B == 1: workgroup q streams the tile of the q-th kept cluster.
template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_tiles_probe(TileParams a) {
  __shared__ uint64_t wmax[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = blockIdx.x;
  const int k = a.probes[q];
  if ((unsigned)k >= (unsigned)a.c) return;   // only if the workspace holds no probe list
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  const char* tile = a.tiles + (size_t)k * a.b * rb;
  const uint16_t* sc = RF == RF_INT4 ? a.scales + (size_t)k * a.b * spr : nullptr;
  HRegs<RF, CH> hr;
  load_h<RF, CH>(hr, a.h, a.h_bf16, a.d, lane);
  uint64_t bc = 0;
  for (int j0 = wave * kRPI; j0 < a.b; j0 += 4 * kRPI) {
    RowGroup<RF, CH> g;
    rows_load<RF, CH>(g, tile, rb, j0, a.b, sc, spr, lane);
    float z[kRPI];
    rows_dot<RF, CH>(g, hr, z);
    {                                            // lane i < kRPI: the token of row j0 + i
      const float zi = lane_pick<kRPI>(z, lane);
      const int j = j0 + lane;
      if (lane < kRPI && j < a.b) {
        const int t = a.c2t[(size_t)k * a.b + j];
        if (t >= 0) {                              // an empty slot (-1) is never chosen
          const float key = make_key(zi, a.sample, a.tau, a.rng, 0u, 1u, (uint32_t)t);
          const uint64_t cnd = pack_cand(key, (uint32_t)t);
          bc = cnd > bc ? cnd : bc;
        }
        if (a.logits_out) a.logits_out[(size_t)q * a.b + j] = t >= 0 ? zi : -__builtin_huge_valf();
        if (a.tokens_out) a.tokens_out[(size_t)q * a.b + j] = t;
      }
    }
  }
  bc = wave_max_u64(bc);
  if (lane == 0) wmax[wave] = bc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = wmax[0];
    for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
    atomicMax((unsigned long long*)&a.best[0], (unsigned long long)m);
  }
}

// B > 1: workgroup k serves every row whose probe set holds cluster k; each tile row
// group is read from HBM once and reused from registers for those rows.
// SAMPLE: the token keys carry Gumbel noise (the greedy instantiation leaves out the Philox
// code and its registers).
template <int RF, int CH, bool SAMPLE, bool HB = false>
__global__ __launch_bounds__(kThreads) void k_tiles_mask(TileParams a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  const int hsz = a.h_bf16 ? 2 : 4;
  const bool want = a.logits_out || a.tokens_out;
  __shared__ uint64_t wbest[2][4];
  // SAMPLE: the 4 waves' logits and tokens of the tile rows for one hidden row meet in LDS, and
  // wave 0 draws the 16 Gumbel keys on 16 lanes (one Philox evaluation per token, instead of each
  // wave running it with 4 of its lanes active)
  __shared__ float zbuf[2][4 * kRPI];
  __shared__ int tbuf[2][4 * kRPI];
  int par = 0;
  // workgroup g takes entries g, g + G, ... of the list of clusters kept by any row
  const int nk = *a.nkept;
  for (int e = blockIdx.x; e < nk; e += gridDim.x) {
    const int k = a.klist[e];
    const uint64_t* mk = a.mask + (size_t)k * a.W;
    const uint64_t m0 = mk[0];
    const char* tile = a.tiles + (size_t)k * a.b * rb;
    const uint16_t* sc = RF == RF_INT4 ? a.scales + (size_t)k * a.b * spr : nullptr;
    // every wave runs the same (block, row) sequence: the barrier below is reached uniformly
    for (int base = 0; base < a.b; base += 4 * kRPI) {
      const int j0 = base + wave * kRPI;            // may lie past the tile: no candidates
      RowGroup<RF, CH> g;
      rows_load<RF, CH>(g, tile, rb, j0, a.b, sc, spr, lane);
      int tj[kRPI];
#pragma unroll
      for (int i = 0; i < kRPI; ++i) tj[i] = (j0 + i < a.b) ? a.c2t[(size_t)k * a.b + j0 + i] : 0;
      for (int wi = 0; wi < a.W; ++wi) {
        uint64_t bits = wi == 0 ? m0 : mk[wi];
        while (bits) {
          const int r = wi * 64 + __builtin_ctzll(bits);
          bits &= bits - 1ull;
          if (r >= a.B) continue;                   // only if the workspace holds no masks
          // fp32 and int4 row words are opaque per hidden row: their conversions are redone for
          // each row instead of being hoisted out of this loop (which would hold every converted
          // element of the four rows in registers; measured slower).  bf16 rows with bf16 h are
          // dotted as raw words, with nothing to hoist, and left to the scheduler
          if (!(RF == RF_BF16 && HB)) {
#pragma unroll
            for (int i = 0; i < kRPI; ++i)
#pragma unroll
              for (int q = 0; q < CH; ++q) {
                asm volatile("" : "+v"(g.w[i][q].x), "+v"(g.w[i][q].y), "+v"(g.w[i][q].z), "+v"(g.w[i][q].w));
                asm volatile("" : "+v"(g.sc[i][q]));
              }
          }
          float z[kRPI];
          rows_dot_stream<RF, CH, kRPI, HB>(g, (const char*)a.h + (size_t)r * a.d * hsz, a.h_bf16, a.d, lane, z);
          // position of k in row r's ascending probe list (probe outputs only)
          int lo = 0;
          if (want) {
            const int32_t* pr = a.probes + (size_t)r * a.p;
            int hi = a.p;
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if (pr[mid] < k) lo = mid + 1; else hi = mid;
            }
          }
          uint64_t bc = 0;
          {                                          // lane i < kRPI: the token of row j0 + i
            const float zi = lane_pick<kRPI>(z, lane);
            const int t = lane_pick<kRPI>(tj, lane);
            const int j = j0 + lane;
            if (SAMPLE && lane < kRPI) {             // past the tile: no token
              zbuf[par][wave * kRPI + lane] = zi;
              tbuf[par][wave * kRPI + lane] = j < a.b ? t : -1;
            }
            if (lane < kRPI && j < a.b) {
              if (!SAMPLE && t >= 0) {               // an empty slot (-1) is never chosen
                const float key = make_key(zi, false, a.tau, a.rng, (uint32_t)r, 1u, (uint32_t)t);
                bc = pack_cand(key, (uint32_t)t);
              }
              const size_t o = ((size_t)r * a.p + lo) * a.b + j;
              if (a.logits_out) a.logits_out[o] = t >= 0 ? zi : -__builtin_huge_valf();
              if (a.tokens_out) a.tokens_out[o] = t;
            }
          }
          if constexpr (SAMPLE) {
            __syncthreads();
            if (wave == 0) {
              uint64_t c = 0;
              if (lane < 4 * kRPI) {
                const int t = tbuf[par][lane];
                if (t >= 0) {                        // an empty slot (-1) is never chosen
                  const float key = make_key(zbuf[par][lane], true, a.tau, a.rng, (uint32_t)r, 1u, (uint32_t)t);
                  c = pack_cand(key, (uint32_t)t);
                }
              }
              c = wave_max_u64(c);
              if (lane == 0) atomicMax((unsigned long long*)&a.best[(size_t)r * kBestStride], (unsigned long long)c);
            }
            par ^= 1;
            continue;
          }
          // the four waves' maxima for row r meet in LDS: one atomic per (cluster, row)
          bc = wave_max_u64(bc);
          if (lane == 0) wbest[par][wave] = bc;
          __syncthreads();
          if (threadIdx.x == 0) {
            uint64_t m = wbest[par][0];
            for (int w = 1; w < 4; ++w) m = wbest[par][w] > m ? wbest[par][w] : m;
            atomicMax((unsigned long long*)&a.best[(size_t)r * kBestStride], (unsigned long long)m);
          }
          par ^= 1;
        }
      }
    }
  }
}

// Decodes the per-row maxima and clears them, so the workspace holds zero maxima
// between calls.
__global__ void k_finalize(uint64_t* best, int32_t* token, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) {
    token[i] = (int32_t)cand_id(best[(size_t)i * kBestStride]);
    best[(size_t)i * kBestStride] = 0ull;
  }
}

__global__ void k_fill_u64(uint64_t* p, int n, uint64_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------ dense comparator

struct DenseParams {
  const void* h;
  const char* E;
  const uint16_t* scales;     // int4 rows: their bf16 group scales [V][d/128]
  int h_bf16, B, V, d;
  int sample;
  float tau;
  Rng rng;
  uint64_t* best;
  float* logits;
};

template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_dense_gemv(DenseParams a) {
  __shared__ uint64_t wmax[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int wg = blockIdx.x * 4 + wave;
  const int nw = gridDim.x * 4;
  const int rb = row_bytes_of(RF, a.d);
  HRegs<RF, CH> hr;
  load_h<RF, CH>(hr, (const char*)a.h + (size_t)r * a.d * (a.h_bf16 ? 2 : 4), a.h_bf16, a.d, lane);
  uint64_t bc = 0;
  for (int t0 = wg * kRPI; t0 < a.V; t0 += nw * kRPI) {
    RowGroup<RF, CH> g;
    rows_load<RF, CH>(g, a.E, rb, t0, a.V, RF == RF_INT4 ? a.scales : nullptr, a.d >> 7, lane);
    float z[kRPI];
    rows_dot<RF, CH>(g, hr, z);
    {                                            // lane i < kRPI: the token t0 + i
      const float zi = lane_pick<kRPI>(z, lane);
      const int t = t0 + lane;
      if (lane < kRPI && t < a.V) {
        const float key = make_key(zi, a.sample, a.tau, a.rng, (uint32_t)r, 1u, (uint32_t)t);
        const uint64_t cnd = pack_cand(key, (uint32_t)t);
        bc = cnd > bc ? cnd : bc;
        if (a.logits) a.logits[(size_t)r * a.V + t] = zi;
      }
    }
  }
  bc = wave_max_u64(bc);
  if (lane == 0) wmax[wave] = bc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = wmax[0];
    for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
    atomicMax((unsigned long long*)&a.best[(size_t)r * kBestStride], (unsigned long long)m);
  }
}

// ------------------------------------------------------------------ offline packing

struct PackParams {
  const char* E;
  const int32_t* c2t;
  char* tiles;
  uint16_t* scales;
  uint32_t* counts;
  uint32_t* bad;
  int V, d, rows, src_bf16, dst_fmt;
};

__global__ __launch_bounds__(kThreads) void k_pack(PackParams a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int ssz = a.src_bf16 ? 2 : 4;
  for (int row = gw; row < a.rows; row += nw) {
    const int t = a.c2t[row];
    if (t >= a.V) {
      if (lane == 0) atomicOr(a.bad, 1u);
      continue;
    }
    if (t < 0) {                                   // an empty slot of a padded cluster: a zero row
      if (lane == 0) atomicAdd(&a.counts[a.V], 1u);
      const int rbytes = a.dst_fmt == RF_F32 ? 4 * a.d : a.dst_fmt == RF_BF16 ? 2 * a.d : a.d / 2;
      uint32_t* dst = (uint32_t*)(a.tiles + (size_t)row * rbytes);
      for (int e = lane; e < rbytes / 4; e += kWave) dst[e] = 0u;
      if (a.dst_fmt == RF_INT4)
        for (int gi = lane; gi < (a.d >> 7); gi += kWave) a.scales[(size_t)row * (a.d >> 7) + gi] = 0;
      continue;
    }
    if (lane == 0) atomicAdd(&a.counts[t], 1u);
    const char* src = a.E + (size_t)t * a.d * ssz;
    auto val = [&](int e) -> float {
      return a.src_bf16 ? bf16_to_f32(((const uint16_t*)src)[e]) : ((const float*)src)[e];
    };
    if (a.dst_fmt == RF_F32) {
      float* dst = (float*)a.tiles + (size_t)row * a.d;
      for (int e = lane; e < a.d; e += kWave) dst[e] = val(e);
    } else if (a.dst_fmt == RF_BF16) {
      uint16_t* dst = (uint16_t*)a.tiles + (size_t)row * a.d;
      for (int e = lane; e < a.d; e += kWave)
        dst[e] = a.src_bf16 ? ((const uint16_t*)src)[e] : f32_to_bf16_rne(val(e));
    } else {
      uint8_t* dst = (uint8_t*)a.tiles + (size_t)row * (a.d / 2);
      const int ng = a.d >> 7;
      for (int gi = 0; gi < ng; ++gi) {
        const float x0 = val(gi * 128 + 2 * lane), x1 = val(gi * 128 + 2 * lane + 1);
        const float amax = wave_max_f32(fmaxf(fabsf(x0), fabsf(x1)));
        const uint16_t sb = f32_to_bf16_rne(amax / 7.0f);
        const float s = bf16_to_f32(sb);
        int q0 = 0, q1 = 0;
        if (s != 0.f) {
          q0 = (int)fminf(fmaxf(rintf(x0 / s), -7.f), 7.f);
          q1 = (int)fminf(fmaxf(rintf(x1 / s), -7.f), 7.f);
        }
        dst[gi * 64 + lane] = (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
        if (lane == 0) a.scales[(size_t)row * ng + gi] = sb;
      }
    }
  }
}

// Rows [rows][d] of bf16 values to int4 groups of 128 (the k_pack rule): nibbles
// [rows][d/2] and bf16 scales [rows][d/128].  One wave per row.
__global__ __launch_bounds__(kThreads) void k_quant_int4_rows(const uint16_t* src, int rows, int d, uint8_t* q,
                                                              uint16_t* scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* x = src + (size_t)row * d;
  const int ng = d >> 7;
  for (int gi = 0; gi < ng; ++gi) {
    const float x0 = bf16_to_f32(x[gi * 128 + 2 * lane]), x1 = bf16_to_f32(x[gi * 128 + 2 * lane + 1]);
    const float amax = wave_max_f32(fmaxf(fabsf(x0), fabsf(x1)));
    const uint16_t sb = f32_to_bf16_rne(amax / 7.0f);
    const float s = bf16_to_f32(sb);
    int q0 = 0, q1 = 0;
    if (s != 0.f) {
      q0 = (int)fminf(fmaxf(rintf(x0 / s), -7.f), 7.f);
      q1 = (int)fminf(fmaxf(rintf(x1 / s), -7.f), 7.f);
    }
    q[(size_t)row * (d / 2) + gi * 64 + lane] = (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
    if (lane == 0) scales[(size_t)row * ng + gi] = sb;
  }
}

// The tokens of C2T are exactly 0 .. n - 1, each once, n = V minus the empty slots (counts[V]).
__global__ void k_check_counts(const uint32_t* counts, int V, uint32_t* bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = V - (int)counts[V];
  if (i < V && counts[i] != (i < n ? 1u : 0u)) atomicOr(bad, 2u);
}

// ------------------------------------------------------------------ cluster centroids
// C[k] = mean of the b rows E[C2T[k][j]] (or, for unit centroids, the normalised sum of
// the normalised rows), accumulated in fp64 and rounded once to the stored dtype.

// Round a double to bf16, nearest even, by rounding at the bf16 quantum of its binade.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  if (!(fabs(x) < 0x1p128)) {            // inf, NaN or beyond the bf16 range
    if (x != x) return 0x7FC0u;
    return x > 0 ? 0x7F80u : 0xFF80u;
  }
  int e;
  frexp(x, &e);                           // |x| = m 2^e, 0.5 <= m < 1
  const int qe = e - 8 > -133 ? e - 8 : -133;
  const double r = ldexp(rint(ldexp(x, -qe)), qe);   // exact scaling, ties to even
  if (fabs(r) >= 0x1p128) return x > 0 ? 0x7F80u : 0xFF80u;
  return (uint16_t)(__float_as_uint((float)r) >> 16);   // r has <= 8 significant bits
}

struct CentroidParams {
  const char* E;
  const int32_t* c2t;
  void* out;
  int d, b, src_bf16, dst_bf16, unit;
};

__global__ __launch_bounds__(kThreads) void k_centroids(CentroidParams a) {
  __shared__ double inv_norm[256];       // b <= 256
  __shared__ double red[kThreads / kWave];
  const int k = blockIdx.x, tid = threadIdx.x;
  const int esz = a.src_bf16 ? 2 : 4;
  auto val = [&](int row, int e) -> double {
    const char* src = a.E + ((size_t)row * a.d + e) * esz;
    return a.src_bf16 ? (double)bf16_to_f32(*(const uint16_t*)src) : (double)*(const float*)src;
  };
  const int32_t* rows = a.c2t + (size_t)k * a.b;
  int nmem = 0;                          // members: the slots that are not empty (-1)
  for (int j = 0; j < a.b; ++j) nmem += rows[j] >= 0 ? 1 : 0;
  if (a.unit) {
    for (int j = 0; j < a.b; ++j) {
      if (rows[j] < 0) {
        if (tid == 0) inv_norm[j] = 0.0;
        continue;
      }
      double ss = 0.0;
      for (int e = tid; e < a.d; e += kThreads) { const double v = val(rows[j], e); ss += v * v; }
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
      if ((tid & 63) == 0) red[tid >> 6] = ss;
      __syncthreads();
      if (tid == 0) {
        const double t = (red[0] + red[1]) + (red[2] + red[3]);
        inv_norm[j] = t > 0.0 ? 1.0 / sqrt(t) : 0.0;
      }
      __syncthreads();
    }
  }
  double nsq = 0.0;
  for (int pass = 0; pass < (a.unit ? 2 : 1); ++pass) {
    double scale = 1.0;
    if (a.unit && pass == 1) {
      if ((tid & 63) == 0) red[tid >> 6] = nsq;
      __syncthreads();
      const double t = (red[0] + red[1]) + (red[2] + red[3]);
      scale = t > 0.0 ? 1.0 / sqrt(t) : 0.0;
    }
    for (int e = tid; e < a.d; e += kThreads) {
      double sum = 0.0;
      for (int j = 0; j < a.b; ++j) {
        if (rows[j] < 0) continue;
        sum += a.unit ? val(rows[j], e) * inv_norm[j] : val(rows[j], e);
      }
      if (a.unit && pass == 0) { nsq += sum * sum; continue; }
      const double m = a.unit ? sum * scale : (nmem ? sum / (double)nmem : 0.0);
      const size_t o = (size_t)k * a.d + e;
      if (a.dst_bf16) ((uint16_t*)a.out)[o] = f64_to_bf16_rne(m);
      else ((float*)a.out)[o] = (float)m;
    }
    if (a.unit && pass == 0) {
      for (int m = 32; m >= 1; m >>= 1) nsq += __shfl_xor(nsq, m, kWave);
    }
  }
}

// ------------------------------------------------------------------ host launchers

Workspace carve_workspace(void* base, int B, int c, int p) {
  // Regions stage 1 touches come first, so their offsets do not depend on p.
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  Workspace w{};
  w.W = (B + 63) / 64;
  size_t off = 0;
  char* b = (char*)base;
  w.keys = (float*)(b ? b + off : nullptr);
  off = up(off + (B == 1 ? (size_t)b1_key_slots(c) : (size_t)B * c) * sizeof(float));
  w.lst = nullptr;
  if (B == 1) {
    w.lst = (uint64_t*)(b ? b + off : nullptr);
    off = up(off + ((size_t)c + 64) * sizeof(uint64_t));
  }

  w.mask = nullptr;
  w.kflag = nullptr;
  w.klist = nullptr;
  w.nkept = nullptr;
  if (B > 1) {
    w.mask = (uint64_t*)(b ? b + off : nullptr);
    off = up(off + (size_t)c * w.W * sizeof(uint64_t));
    w.kflag = (uint32_t*)(b ? b + off : nullptr);
    off = up(off + (size_t)c * sizeof(uint32_t));
    w.klist = (int32_t*)(b ? b + off : nullptr);
    off = up(off + (size_t)c * sizeof(int32_t));
    w.nkept = (int32_t*)(b ? b + off : nullptr);
    off = up(off + sizeof(int32_t));
  }
  w.best = (uint64_t*)(b ? b + off : nullptr);
  off = up(off + (size_t)B * kBestStride * sizeof(uint64_t));
  w.part = (uint64_t*)(b ? b + off : nullptr);
  off = up(off + (size_t)kB1Workgroups * sizeof(uint64_t));
  w.probes = (int32_t*)(b ? b + off : nullptr);
  off = up(off + (size_t)B * p * sizeof(int32_t));
  w.bytes = off;
  return w;
}

size_t dense_workspace_bytes(int B) { return (((size_t)B * kBestStride * sizeof(uint64_t)) + 255) & ~(size_t)255; }

int max_chunk_slots(int fmt) { return fmt == RF_INT4 ? 4 : 8; }

int chunk_slots(int fmt, int d) {
  const long cpr = (long)row_bytes_of(fmt, d) / 16;
  return (int)((cpr + 63) / 64);
}

#define FH_DISPATCH_CH(CH, ...)                                   \
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

#define FH_DISPATCH_CH_INT4(CH, ...)                              \
  switch (CH) {                                                   \
    case 1: { constexpr int kCH = 1; __VA_ARGS__; } break;        \
    case 2: { constexpr int kCH = 2; __VA_ARGS__; } break;        \
    case 3: { constexpr int kCH = 3; __VA_ARGS__; } break;        \
    case 4: { constexpr int kCH = 4; __VA_ARGS__; } break;        \
    default: return hipErrorInvalidValue;                         \
  }

static bool use_mfma(const HeadShape& s, int fmt) {
  return s.B > 1 && s.h_bf16 && fmt == RF_BF16 && (s.d % 32) == 0;
}

// Compute units of the current device, looked up once per device.
static int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int NT, int EPI>
static void launch_mfma_nt(const MfmaParams& p, int mt, dim3 grid, hipStream_t st) {
  if (mt == 2)      hipLaunchKernelGGL((k_mfma<NT, 2, EPI>), grid, dim3(kMfmaThreads), 0, st, p);
  else if (mt == 3) hipLaunchKernelGGL((k_mfma<NT, 3, EPI>), grid, dim3(kMfmaThreads), 0, st, p);
  else              hipLaunchKernelGGL((k_mfma<NT, 4, EPI>), grid, dim3(kMfmaThreads), 0, st, p);
}

template <int EPI>
static hipError_t launch_mfma(const MfmaParams& p, int max_wg, hipStream_t st) {
  const int cus = device_cus();
  int mt = 2;
  while (mt < kMfmaMaxMT && (p.rows + 16 * mt - 1) / (16 * mt) > cus) ++mt;
  const int ngroups = (p.rows + 16 * mt - 1) / (16 * mt);
  const int nb = (p.B + 63) / 64;
  dim3 grid(ngroups < max_wg ? ngroups : max_wg, nb);
  const int nt = p.B >= 64 ? 4 : (p.B + 15) / 16;
  switch (nt) {
    case 1: launch_mfma_nt<1, EPI>(p, mt, grid, st); break;
    case 2: launch_mfma_nt<2, EPI>(p, mt, grid, st); break;
    case 3: launch_mfma_nt<3, EPI>(p, mt, grid, st); break;
    default: launch_mfma_nt<4, EPI>(p, mt, grid, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_scores(const HeadShape& s, const void* h, const void* C, const Sampling& smp,
                         const Workspace& ws, float* keys_out, hipStream_t st) {
  const Rng rng = make_rng(smp.seed, smp.step);
  const uint16_t* c_scales =
      s.c_fmt == RF_INT4 ? (const uint16_t*)((const char*)C + int4_scales_offset(s.c, s.d)) : nullptr;
  if (s.B == 1) {   // the same kernel the fused B = 1 forward runs
    B1Args a{};
    a.h = h; a.C = C; a.c_scales = c_scales; a.h_bf16 = s.h_bf16; a.c = s.c; a.d = s.d; a.b = s.b;
    a.sample = smp.sample; a.tau = smp.tau; a.seed = smp.seed; a.step = smp.step;
    a.keys = ws.keys; a.keys_out = keys_out; a.lst = ws.lst; a.c_slots = chunk_slots(s.c_fmt, s.d);
    return s.c_fmt == RF_F32 ? launch_b1_scores_f32(a, st)
         : s.c_fmt == RF_BF16 ? launch_b1_scores_bf16(a, st) : launch_b1_scores_int4(a, st);
  }
  if (use_mfma(s, s.c_fmt)) {
    MfmaParams p{};
    p.H = (const uint16_t*)h;
    p.M = (const uint16_t*)C;
    p.B = s.B; p.rows = s.c; p.d = s.d;
    p.sample = smp.sample; p.tau = smp.tau; p.rng = rng;
    p.keys = ws.keys; p.keys_out = keys_out; p.mask = ws.mask; p.W = ws.W; p.kflag = ws.kflag; p.nkept = ws.nkept;
    return launch_mfma<EPI_KEYS>(p, 1 << 30, st);
  }
  ScoreParams a{h, (const char*)C, c_scales, s.h_bf16, s.B, s.c, s.d, smp.sample, smp.tau, rng,
                ws.keys, keys_out, ws.mask, ws.W, ws.kflag, ws.nkept};
  const int groups = (s.c + kRPI - 1) / kRPI;
  int wgs = (groups + 3) / 4;
  if (wgs > 4096) wgs = 4096;
  dim3 grid(wgs, s.B);
  const int ch = chunk_slots(s.c_fmt, s.d);
  if (s.c_fmt == RF_F32) {
    FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_scores_gemv<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a));
  } else if (s.c_fmt == RF_BF16) {
    FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_scores_gemv<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a));
  } else {
    FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_scores_gemv<RF_INT4, kCH>), grid, dim3(kThreads), 0, st, a));
  }
  return hipGetLastError();
}

hipError_t launch_select(const HeadShape& s, int p, const Workspace& ws, int32_t* probe_out, hipStream_t st) {
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(s.B), dim3(kSelThreads), 0, st, (const float*)ws.keys, s.c, p, ws.probes,
                       probe_out, ws.mask, ws.W, ws.best, ws.kflag, ws.klist, ws.nkept);
  };
  if (s.c <= 4 * kSelThreads) go(k_select<1>);
  else if (s.c <= 8 * kSelThreads) go(k_select<2>);
  else if (s.c <= 16 * kSelThreads) go(k_select<4>);
  else go(k_select<8>);
  return hipGetLastError();
}

hipError_t launch_tiles(const HeadShape& s, int p, const void* h, const int32_t* c2t, const void* tiles,
                        const uint16_t* scales, const Sampling& smp, const Workspace& ws,
                        float* logits_out, int32_t* tokens_out, int32_t* token, hipStream_t st) {
  TileParams a{};
  a.h = h; a.h_bf16 = s.h_bf16; a.B = s.B; a.d = s.d; a.c = s.c; a.b = s.b; a.p = p;
  a.probes = ws.probes; a.c2t = c2t; a.tiles = (const char*)tiles; a.scales = scales;
  a.sample = smp.sample; a.tau = smp.tau; a.rng = make_rng(smp.seed, smp.step);
  a.logits_out = logits_out; a.tokens_out = tokens_out; a.best = ws.best; a.mask = ws.mask; a.W = ws.W;
  a.klist = ws.klist; a.nkept = ws.nkept;
  const int ch = chunk_slots(s.e_fmt, s.d);
  const bool b1 = s.B == 1;
  const dim3 grid(b1 ? p : (s.c < kMaskWorkgroups ? s.c : kMaskWorkgroups));
  if (s.e_fmt == RF_F32) {
    if (b1) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_probe<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a)); }
    else if (smp.sample) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_F32, kCH, true>), grid, dim3(kThreads), 0, st, a)); }
    else    { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_F32, kCH, false>), grid, dim3(kThreads), 0, st, a)); }
  } else if (s.e_fmt == RF_BF16) {
    if (b1) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_probe<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a)); }
    else if (s.h_bf16 && smp.sample) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_BF16, kCH, true, true>), grid, dim3(kThreads), 0, st, a)); }
    else if (s.h_bf16) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_BF16, kCH, false, true>), grid, dim3(kThreads), 0, st, a)); }
    else if (smp.sample) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_BF16, kCH, true>), grid, dim3(kThreads), 0, st, a)); }
    else    { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_BF16, kCH, false>), grid, dim3(kThreads), 0, st, a)); }
  } else {
    if (b1) { FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_tiles_probe<RF_INT4, kCH>), grid, dim3(kThreads), 0, st, a)); }
    else if (smp.sample) { FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_tiles_mask<RF_INT4, kCH, true>), grid, dim3(kThreads), 0, st, a)); }
    else    { FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_tiles_mask<RF_INT4, kCH, false>), grid, dim3(kThreads), 0, st, a)); }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_finalize, dim3((s.B + 255) / 256), dim3(256), 0, st, ws.best, token, s.B);
  return hipGetLastError();
}

hipError_t launch_stage2_b1(const HeadShape& s, int p, const void* h, const int32_t* c2t, const void* tiles,
                            const uint16_t* scales, const Sampling& smp, const Workspace& ws, int32_t* probe_out,
                            float* logits_out, int32_t* tokens_out, int32_t* token, hipStream_t st) {
  B1Args a{};
  a.h = h; a.h_bf16 = s.h_bf16; a.c = s.c; a.d = s.d; a.b = s.b; a.p = p;
  a.sample = smp.sample; a.tau = smp.tau; a.seed = smp.seed; a.step = smp.step;
  a.keys = ws.keys; a.part = ws.part; a.lst = ws.lst; a.c_slots = chunk_slots(s.c_fmt, s.d);
  a.c2t = c2t; a.tiles = tiles; a.scales = scales;
  a.probe_out = probe_out; a.logits_out = logits_out; a.tokens_out = tokens_out; a.token = token;
  return s.e_fmt == RF_F32 ? launch_b1_stage2_f32(a, st)
       : s.e_fmt == RF_BF16 ? launch_b1_stage2_bf16(a, st) : launch_b1_stage2_int4(a, st);
}

hipError_t launch_dense(const HeadShape& s, int V, const void* h, const void* E, const Sampling& smp,
                        uint64_t* best, int32_t* token, float* logits, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_u64, dim3((s.B * kBestStride + 255) / 256), dim3(256), 0, st, best, s.B * kBestStride,
                     (uint64_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const Rng rng = make_rng(smp.seed, smp.step);
  if (use_mfma(s, s.e_fmt)) {
    MfmaParams p{};
    p.H = (const uint16_t*)h; p.M = (const uint16_t*)E;
    p.B = s.B; p.rows = V; p.d = s.d;
    p.sample = smp.sample; p.tau = smp.tau; p.rng = rng;
    p.best = best; p.logits = logits;
    e = launch_mfma<EPI_ARGMAX>(p, 2048, st);
  } else {
    const uint16_t* sc =
        s.e_fmt == RF_INT4 ? (const uint16_t*)((const char*)E + int4_scales_offset((size_t)V, (size_t)s.d)) : nullptr;
    DenseParams a{h, (const char*)E, sc, s.h_bf16, s.B, V, s.d, smp.sample, smp.tau, rng, best, logits};
    const int groups = (V + kRPI - 1) / kRPI;
    int wgs = (groups + 3) / 4;
    if (wgs > 2048) wgs = 2048;
    dim3 grid(wgs, s.B);
    const int ch = chunk_slots(s.e_fmt, s.d);
    if (s.e_fmt == RF_F32) {
      FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_dense_gemv<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a));
    } else if (s.e_fmt == RF_BF16) {
      FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_dense_gemv<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a));
    } else {
      FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_dense_gemv<RF_INT4, kCH>), grid, dim3(kThreads), 0, st, a));
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_finalize, dim3((s.B + 255) / 256), dim3(256), 0, st, best, token, s.B);
  return hipGetLastError();
}

hipError_t launch_centroids(int d, int c, int b, int src_bf16, int dst_bf16, int unit, const void* E,
                            const int32_t* c2t, void* out, hipStream_t st) {
  CentroidParams a{(const char*)E, c2t, out, d, b, src_bf16, dst_bf16, unit};
  hipLaunchKernelGGL(k_centroids, dim3(c), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quant_int4_rows(const uint16_t* src, int rows, int d, uint8_t* q, uint16_t* scales,
                                  hipStream_t st) {
  hipLaunchKernelGGL(k_quant_int4_rows, dim3((rows + 3) / 4), dim3(kThreads), 0, st, src, rows, d, q, scales);
  return hipGetLastError();
}

hipError_t launch_pack(int V, int d, int c, int b, int src_bf16, int dst_fmt, const void* E, const int32_t* c2t,
                       void* tiles, uint16_t* scales, uint32_t* counts, uint32_t* bad, hipStream_t st) {
  PackParams a{(const char*)E, c2t, (char*)tiles, scales, counts, bad, V, d, c * b, src_bf16, dst_fmt};
  int wgs = (c * b + 3) / 4;
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(k_pack, dim3(wgs), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_check_counts, dim3((V + 255) / 256), dim3(256), 0, st, (const uint32_t*)counts, V, bad);
  return hipGetLastError();
}

}  // namespace fh
