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
#include "fh_device.h"
#include "fh_internal.h"
#include "fh_select.h"

namespace fh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRPI = 4;          // rows per wave per row-dot step
constexpr int kB1Threads = 1024; // workgroup size of the B = 1 select + tiles kernel
constexpr int kB1Workgroups = 256;
constexpr int kThreads = 256;    // 4 waves
constexpr int kMaskWorkgroups = 8192;  // k_tiles_mask: workgroups looping over the kept clusters

__host__ __device__ __forceinline__ int row_bytes_of(int fmt, int d) {
  return fmt == RF_F32 ? 4 * d : fmt == RF_BF16 ? 2 * d : d / 2;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 16-byte load (non-temporal: rows of C, tiles and E are read once per call).
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ row dot products

template <int RF, int CH, int NR = kRPI>
struct RowGroup {
  uint4 w[NR][CH];
  uint32_t sc[NR][CH];      // int4: bf16 bits of the group scale (converted at the dot)
};

// Load rows [j0, j0 + NR) (those < nrows) of a matrix with row stride rb bytes.
template <int RF, int CH, int NR>
__device__ __forceinline__ void rows_load(RowGroup<RF, CH, NR>& g, const char* base, int rb, int j0, int nrows,
                                          const uint16_t* scales, int spr, int lane) {
  const int cpr = rb >> 4;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int j = j0 + r;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = lane + kWave * i;
      const bool ok = j < nrows && q < cpr;
      g.w[r][i] = ok ? ld16_stream(base + (size_t)j * rb + (size_t)q * 16) : make_uint4(0u, 0u, 0u, 0u);
      g.sc[r][i] = (RF == RF_INT4 && ok) ? (uint32_t)scales[(size_t)j * spr + (q >> 2)] : 0u;
    }
  }
}

// Full dot products of the loaded rows with h (every lane receives every sum).
template <int RF, int CH, int NR>
__device__ __forceinline__ void rows_dot(const RowGroup<RF, CH, NR>& g, const HRegs<RF, CH>& hr, float (&out)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) acc = chunk_dot<RF>(g.w[r][i], hr.v[i], acc, __uint_as_float(g.sc[r][i] << 16));
    out[r] = wave_sum(acc);
  }
}

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
// D lane l: column n = l % 16, rows m = 4 (l / 16) + i.  A workgroup owns one 16-row tile
// of M at a time and 64 rows of H; its 4 waves split K (k-steps w, w + 4, ...) and their
// partial tiles are summed in LDS in wave order.

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

template <int NT, int EPI>
__global__ __launch_bounds__(kThreads) void k_mfma(MfmaParams a) {
  __shared__ f32x4_t red[4][NT][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.y * 64;
  const int kq = (lane >> 4) * 8;
  const int nsteps = a.d / 32;
  const int ntiles = (a.rows + 15) / 16;
  const uint16_t* hp[NT];
  bool hv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + 16 * t + (lane & 15);
    hv[t] = n < a.B;
    hp[t] = a.H + (size_t)(hv[t] ? n : 0) * a.d + kq;
  }
  uint64_t bc = 0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int m0 = tile * 16;
    const int mr = m0 + (lane & 15);
    const bool mv = mr < a.rows;
    const uint16_t* mp = a.M + (size_t)(mv ? mr : 0) * a.d + kq;
    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this wave's K steps s = wave, wave + 4, ... in groups of GS: the loads of a group are
    // all issued (from valid addresses, masked afterwards) before its MFMAs, so one memory
    // latency is paid per group instead of per step; the MFMA order is unchanged
    constexpr int GS = NT >= 3 ? 2 : 4;             // steps per group (register budget)
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (int s0 = wave; s0 < nsteps; s0 += 4 * GS) {
      uint4 av[GS], bv[GS][NT];
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        const int s = s0 + 4 * u;
        const int ko = s < nsteps ? s * 32 : 0;
        av[u] = ld16(mp + ko);
#pragma unroll
        for (int t = 0; t < NT; ++t) bv[u][t] = ld16(hp[t] + ko);
      }
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        const bool ok = s0 + 4 * u < nsteps;
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, ok && mv ? av[u] : z4);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (!ok) continue;                        // wave-uniform
          const uint4 b = hv[t] ? bv[u][t] : z4;
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, b), acc[t], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave < NT) {
      const int t = wave;
      const f32x4_t v = ((red[0][t][lane] + red[1][t][lane]) + red[2][t][lane]) + red[3][t][lane];
      const int n = n0 + 16 * t + (lane & 15);
      const int mb = m0 + 4 * (lane >> 4);
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
              bc = cnd > bc ? cnd : bc;
              if (a.logits) a.logits[(size_t)n * a.rows + m] = v[i];
            }
          }
        }
      }
    }
    if (EPI == EPI_KEYS && a.mask && blockIdx.y == 0) {
      for (int j = threadIdx.x; j < 16 * a.W; j += kThreads) {
        const int m = m0 + j / a.W;
        if (m < a.rows) a.mask[(size_t)m * a.W + j % a.W] = 0ull;
      }
      if (threadIdx.x < 16 && m0 + (int)threadIdx.x < a.rows) a.kflag[m0 + threadIdx.x] = 0u;
      if (m0 == 0 && threadIdx.x == 0) *a.nkept = 0;
    }
    __syncthreads();
  }
  if (EPI == EPI_ARGMAX && wave < NT) {
    uint64_t o = __shfl_xor(bc, 16, kWave);
    bc = o > bc ? o : bc;
    o = __shfl_xor(bc, 32, kWave);
    bc = o > bc ? o : bc;
    const int n = n0 + 16 * wave + lane;
    if (lane < 16 && n < a.B) atomicMax((unsigned long long*)&a.best[(size_t)n * kBestStride], (unsigned long long)bc);
  }
}

// Eight consecutive elements of h (bf16 or fp32 storage) from byte address src as floats;
// zeros if !ok (src must still be a readable address: the load is unconditional).
__device__ __forceinline__ void h_piece8(float (&hv)[8], const char* src, int h_bf16, bool ok) {
  const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
  if (h_bf16) {
    const uint4 x = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {x.x & m, x.y & m, x.z & m, x.w & m};
#pragma unroll
    for (int j = 0; j < 4; ++j) { hv[2 * j] = bf16_lo(w[j]); hv[2 * j + 1] = bf16_hi(w[j]); }
  } else {
    const uint4 x = reinterpret_cast<const uint4*>(src)[0];
    const uint4 y = reinterpret_cast<const uint4*>(src)[1];
    const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) hv[j] = __uint_as_float(w[j] & m);
  }
}

// rows_dot with h read from memory (L2) piece by piece instead of held in registers: the same
// fused multiply-adds in the same order per row, so the results are bitwise those of rows_dot
// with load_h.  For kernels that dot the same rows with many hidden states.
template <int RF, int CH, int NR>
__device__ __forceinline__ void rows_dot_stream(const RowGroup<RF, CH, NR>& g, const void* h, int h_bf16, int d,
                                                int lane, float (&out)[NR]) {
  constexpr int EPC = Fmt<RF>::EPC;
  const int esz = h_bf16 ? 2 : 4;
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int e0 = (lane + kWave * i) * EPC;
    const bool ok = e0 < d;
    const char* src = (const char*)h + (ok ? (size_t)e0 * esz : 0);
    if (RF == RF_F32) {
      float hv[4];
      const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
      if (h_bf16) {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        hv[0] = bf16_lo(x.x & m); hv[1] = bf16_hi(x.x & m); hv[2] = bf16_lo(x.y & m); hv[3] = bf16_hi(x.y & m);
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        hv[0] = __uint_as_float(x.x & m); hv[1] = __uint_as_float(x.y & m);
        hv[2] = __uint_as_float(x.z & m); hv[3] = __uint_as_float(x.w & m);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = chunk_dot<RF_F32>(g.w[r][i], hv, acc[r], 0.f);
    } else if (RF == RF_BF16) {
      float hv[8];
      h_piece8(hv, src, h_bf16, ok);
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = chunk_dot<RF_BF16>(g.w[r][i], hv, acc[r], 0.f);
    } else {
      float s[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) s[r] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {             // word j of the row chunk: elements 8 j .. 8 j + 7
        float hv[8];
        h_piece8(hv, src + (size_t)8 * j * esz, h_bf16, ok);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const uint32_t wj = j == 0 ? g.w[r][i].x : j == 1 ? g.w[r][i].y : j == 2 ? g.w[r][i].z : g.w[r][i].w;
#pragma unroll
          for (int k = 0; k < 8; ++k) s[r] = fmaf(nib(wj, k), hv[k], s[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = fmaf(__uint_as_float(g.sc[r][i] << 16), s[r], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) out[r] = wave_sum(acc[r]);
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

// ------------------------------------------------------------------ B = 1 fused path
// Three kernels per call.  k_b1_scores streams C (one 4-row group per wave, all row loads
// issued before any arithmetic) and writes the keys.  k_b1_stage2: every workgroup finds
// the same kept set from the keys, scores its share of the kept clusters' tiles and writes
// its best candidate; k_finalize_parts reduces those to the token.  No workgroup ever
// waits for another.

struct B1Params {
  const void* h;
  const char* C;
  const uint16_t* c_scales;   // int4 centroids: their bf16 group scales
  int h_bf16, c, d, b, p;
  int cpad;             // keys padded with NaN up to this count
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

template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_b1_scores(B1Params a) {
  for (int i = a.c + blockIdx.x * kThreads + threadIdx.x; i < a.cpad; i += gridDim.x * kThreads)
    a.keys[i] = __uint_as_float(0x7FC00000u);      // quiet NaN padding for k_b1_stage2
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


// Shared state of k_b1_stage2.  Keys live in registers: slot s of thread t holds the key of
// cluster s * 1024 + t, so one wave ballot covers 64 consecutive clusters and the kept set
// is written as 64-bit words without atomics.
// Key slots per thread of k_b1_stage2: the power of two >= c / 1024 (at least 2).  At B = 1
// the workspace keys are padded to kB1Threads * slots with quiet NaNs, which every min, max
// and comparison of the selection ignores.
__host__ __device__ __forceinline__ int b1_key_slots(int c) {
  int s = 2;
  while (s * kB1Threads < c) s *= 2;
  return s;
}

constexpr int kS2MaxWords = 32768 / 64;
constexpr int kS2MaxCand = 64;             // keys the boundary bin may hold on the fast path

struct S2Shared {
  int hist[kSelBins];
  // Bitmaps over the clusters, wave-major: bit l of w[wave NS + s] is cluster s 1024 + 64 wave + l.
  uint64_t words[kS2MaxWords];             // clusters certainly kept (or all kept, general path)
  uint64_t fullw[kS2MaxWords];             // all kept clusters (probe outputs only)
  int pref[kS2MaxWords];                   // kept clusters before id-ordered word i (probe ids)
  float wmx[16], wmn[16];
  int wtot[16];
  int bnd[3];                              // boundary bin, keys above it, keys in it
  int ncand;
  float cx[kS2MaxCand];                    // the boundary bin's keys ...
  int cid[kS2MaxCand];                     // ... and clusters
  int bk[kS2MaxCand];                      // boundary clusters that are kept, ascending id
  uint64_t wmax[16];
};

// Position of id-ordered word iw in a wave-major bitmap with NS slots.
template <int NS>
__device__ __forceinline__ int wm_index(int iw) { return (iw & 15) * NS + (iw >> 4); }

// Cluster id of ascending rank q (wave-uniform) among the set bits of a wave-major bitmap;
// lane l scans the id-ordered words [l WPL, l WPL + WPL).
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
  const int L = __ffsll((unsigned long long)hit) - 1;
  int id = 0;
  if (lane == L) {
    int r = q - (incl - cnt);
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const int pc = __popcll(wv[i]);
      if (r >= 0 && r < pc) {
        uint64_t bits = wv[i];
        for (int k = 0; k < r; ++k) bits &= bits - 1ull;
        id = (lane * WPL + i) * 64 + __ffsll((unsigned long long)bits) - 1;
      }
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

// Selection and stage 2 for one row in one kernel.  Every workgroup (1024 threads, one per
// CU) reads the c keys and finds the same kept set, so no workgroup waits for another:
//  * one float-linear 2048-bin histogram between the key min and max locates the bin b
//    holding the p-th largest key; every key in a bin above b is certainly kept;
//  * the clusters are numbered 0 .. p-1 in this order: the certain ones by ascending id,
//    then the kept keys of bin b by ascending id; workgroup g takes the numbers g, g + G, ..;
//  * the certain clusters are resolved and their tile loads issued while wave 0 ranks the
//    keys of bin b exactly (key desc, id asc) to pick the p - above of them that are kept.
// A boundary bin with more than kS2MaxCand keys (or all keys equal) sends the workgroup to
// the general selection (select_regs), after which every cluster is resolved from the full
// kept bitmap.  Each workgroup writes the packed maximum of its tokens to part[g];
// k_finalize_parts turns the maxima into the token.  Probe outputs are indexed by the
// ascending rank of the cluster among all kept ones.  NS: key slots per thread, NR: tile rows
// per wave step.
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
  // ---- keys; the slots past c hold NaN: ignored by min / max, never greater or equal
  float x[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) x[s] = a.keys[s * NT + tid];
  for (int i = tid; i < kSelBins; i += NT) Q.hist[i] = 0;
  if (tid == 0) Q.ncand = 0;
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
  // ---- the certain clusters (bins above b) as a bitmap; the keys of bin b compacted
  if (fast) {
    uint32_t wlo = 0u, whi = 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint64_t m = __ballot(bins[s] > b);
      put_lane(wlo, (uint32_t)m, s);                                 // the ballot into lane s
      put_lane(whi, (uint32_t)(m >> 32), s);
      const uint64_t e = __ballot(bins[s] == b);
      if (e) {
        int base = 0;
        if (lane == __ffsll((unsigned long long)e) - 1) base = atomicAdd(&Q.ncand, __popcll(e));
        base = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(base, __ffsll((unsigned long long)e) - 1));
        const int pos = base + lane_prefix(e);
        if (bins[s] == b && pos < kS2MaxCand) { Q.cx[pos] = x[s]; Q.cid[pos] = s * NT + tid; }
      }
    }
    if (lane < NS) Q.words[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
  }
  __syncthreads();                                                          // 5
  if (fast) fast = Q.ncand == inb;          // block-uniform
  int n_def = above;                        // numbers below n_def index Q.words
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
      const float v = a.keys[s * NT + tid];
      const uint64_t m = __ballot(v > T) | __ballot(v == T && s * NT + tid <= Tid);
      put_lane(wlo, (uint32_t)m, s);                                 // the ballot into lane s
      put_lane(whi, (uint32_t)(m >> 32), s);
    }
    if (lane < NS) Q.words[wave * NS + lane] = ((uint64_t)whi << 32) | wlo;
    n_def = p;
  }
  const int n_my = me < p ? (p - me + G - 1) / G : 0;
  const int gpp = (a.b + NR - 1) / NR;
  const int nit = n_my * gpp;
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  // this wave's first tile rows, when certain: resolved and loaded while wave 0 ranks
  RowGroup<RF, CH, NR> g0;
  int tl0 = 0, k0 = -1;
  HRaw<RF, CH> hraw;
  if constexpr (kEarlyH) load_h_raw<RF, CH>(hraw, a.h, a.h_bf16, a.d, lane);
  if (fast) {
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
      int pos = 0;
      for (int q = 0; q < n; ++q) {
        const int rq = __builtin_amdgcn_readlane(rank, q);
        const int iq = __builtin_amdgcn_readlane(it, q);
        pos += (rq < need && iq < it) ? 1 : 0;
      }
      if (kept) Q.bk[pos] = it;
    }
    if (wave < nit) {
      const int qi = wave / gpp, j0 = (wave - qi * gpp) * NR;
      const int q = me + qi * G;
      if (q < above) {
        k0 = kept_rank_id<NS>(Q.words, q);
        const size_t row0 = (size_t)k0 * a.b;
        tl0 = (lane < NR && j0 + lane < a.b) ? a.c2t[row0 + j0 + lane] : 0;
        rows_load<RF, CH>(g0, a.tiles + row0 * rb, rb, j0, a.b, RF == RF_INT4 ? a.scales + row0 * spr : nullptr,
                          spr, lane);
      }
    }
  }
  __syncthreads();                                                          // 6
  // ---- probe outputs: the full kept bitmap gives every cluster its ascending rank
  const uint64_t* fw = fast ? Q.fullw : Q.words;
  if (want) {
    if (fast) {
      for (int i = tid; i < NWID; i += NT) Q.fullw[i] = Q.words[i];
      __syncthreads();
      if (tid < p - above) {
        const int k = Q.bk[tid];
        atomicOr((unsigned long long*)&Q.fullw[(((k >> 6) & 15) * NS) + (k >> 10)], 1ull << (k & 63));
      }
      __syncthreads();
    }
    if (me == 0 && a.probe_out) {
      int tot;
      const int pc = tid < NWID ? __popcll(fw[wm_index<NS>(tid)]) : 0;
      const int ex = block_scan(pc, Q.wtot, tot);
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
      k = q < n_def ? kept_rank_id<NS>(Q.words, q) : Q.bk[q - n_def];
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

// The token of the fused B = 1 path: the largest of the per-workgroup maxima part[0 .. n).
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
        const float key = make_key(zi, a.sample, a.tau, a.rng, 0u, 1u, (uint32_t)t);
        const uint64_t cnd = pack_cand(key, (uint32_t)t);
        bc = cnd > bc ? cnd : bc;
        if (a.logits_out) a.logits_out[(size_t)q * a.b + j] = zi;
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
template <int RF, int CH, bool SAMPLE>
__global__ __launch_bounds__(kThreads) void k_tiles_mask(TileParams a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  const int hsz = a.h_bf16 ? 2 : 4;
  const bool want = a.logits_out || a.tokens_out;
  __shared__ uint64_t wbest[2][4];
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
          // the row words are opaque per hidden row: their conversions are redone for each row
          // instead of being hoisted out of this loop (which would hold every converted element
          // of the four rows in registers)
#pragma unroll
          for (int i = 0; i < kRPI; ++i)
#pragma unroll
            for (int q = 0; q < CH; ++q) {
              asm volatile("" : "+v"(g.w[i][q].x), "+v"(g.w[i][q].y), "+v"(g.w[i][q].z), "+v"(g.w[i][q].w));
              asm volatile("" : "+v"(g.sc[i][q]));
            }
          float z[kRPI];
          rows_dot_stream<RF, CH>(g, (const char*)a.h + (size_t)r * a.d * hsz, a.h_bf16, a.d, lane, z);
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
            if (lane < kRPI && j < a.b) {
              const float key = make_key(zi, SAMPLE, a.tau, a.rng, (uint32_t)r, 1u, (uint32_t)t);
              bc = pack_cand(key, (uint32_t)t);
              const size_t o = ((size_t)r * a.p + lo) * a.b + j;
              if (a.logits_out) a.logits_out[o] = zi;
              if (a.tokens_out) a.tokens_out[o] = t;
            }
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
    rows_load<RF, CH>(g, a.E, rb, t0, a.V, nullptr, 0, lane);
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
    if (t < 0 || t >= a.V) {
      if (lane == 0) atomicOr(a.bad, 1u);
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

__global__ void k_check_counts(const uint32_t* counts, int V, uint32_t* bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V && counts[i] != 1u) atomicOr(bad, 2u);
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
  if (a.unit) {
    for (int j = 0; j < a.b; ++j) {
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
      for (int j = 0; j < a.b; ++j) sum += a.unit ? val(rows[j], e) * inv_norm[j] : val(rows[j], e);
      if (a.unit && pass == 0) { nsq += sum * sum; continue; }
      const double m = a.unit ? sum * scale : sum / (double)a.b;
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
  off = up(off + (B == 1 ? (size_t)b1_key_slots(c) * kB1Threads : (size_t)B * c) * sizeof(float));
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

template <int RF, int CH>
static void launch_b1_scores(const B1Params& a, int c, hipStream_t st) {
  const int groups = (c + kRPI - 1) / kRPI;          // one row group per wave
  const int wgs = (groups + 3) / 4;
  hipLaunchKernelGGL((k_b1_scores<RF, CH>), dim3(wgs), dim3(kThreads), 0, st, a);
}

template <int RF, int CH, int S>
static void launch_b1_stage2_s(const B1Params& a, int G, int nr, hipStream_t st) {
  if (nr == 1) hipLaunchKernelGGL((k_b1_stage2<RF, CH, S, 1>), dim3(G), dim3(kB1Threads), 0, st, a);
  else         hipLaunchKernelGGL((k_b1_stage2<RF, CH, S, 2>), dim3(G), dim3(kB1Threads), 0, st, a);
}

template <int RF, int CH>
static void launch_b1_stage2(const B1Params& a, int c, int p, int b, hipStream_t st) {
  const int G = p < kB1Workgroups ? p : kB1Workgroups;
  const int n_my = (p + G - 1) / G;
  const int nr = n_my * b <= kB1Threads / 64 ? 1 : 2;     // one row per wave when that fills them
  const int slots = (c + kB1Threads - 1) / kB1Threads;
  if (slots <= 2)       launch_b1_stage2_s<RF, CH, 2>(a, G, nr, st);
  else if (slots <= 4)  launch_b1_stage2_s<RF, CH, 4>(a, G, nr, st);
  else if (slots <= 8)  launch_b1_stage2_s<RF, CH, 8>(a, G, nr, st);
  else if (slots <= 16) launch_b1_stage2_s<RF, CH, 16>(a, G, nr, st);
  else                  launch_b1_stage2_s<RF, CH, 32>(a, G, nr, st);
  hipLaunchKernelGGL(k_finalize_parts, dim3(1), dim3(256), 0, st, (const uint64_t*)a.part, G, a.token);
}

static bool use_mfma(const HeadShape& s, int fmt) {
  return s.B > 1 && s.h_bf16 && fmt == RF_BF16 && (s.d % 32) == 0;
}

template <int NT, int EPI>
static void launch_mfma_nt(const MfmaParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((k_mfma<NT, EPI>), grid, dim3(kThreads), 0, st, p);
}

template <int EPI>
static hipError_t launch_mfma(const MfmaParams& p, int max_wg, hipStream_t st) {
  const int ntiles = (p.rows + 15) / 16;
  const int nb = (p.B + 63) / 64;
  dim3 grid(ntiles < max_wg ? ntiles : max_wg, nb);
  const int nt = p.B >= 64 ? 4 : (p.B + 15) / 16;
  switch (nt) {
    case 1: launch_mfma_nt<1, EPI>(p, grid, st); break;
    case 2: launch_mfma_nt<2, EPI>(p, grid, st); break;
    case 3: launch_mfma_nt<3, EPI>(p, grid, st); break;
    default: launch_mfma_nt<4, EPI>(p, grid, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_scores(const HeadShape& s, const void* h, const void* C, const Sampling& smp,
                         const Workspace& ws, float* keys_out, hipStream_t st) {
  const Rng rng = make_rng(smp.seed, smp.step);
  const uint16_t* c_scales =
      s.c_fmt == RF_INT4 ? (const uint16_t*)((const char*)C + int4_scales_offset(s.c, s.d)) : nullptr;
  if (s.B == 1) {   // the same kernel the fused B = 1 forward runs
    B1Params a{};
    a.h = h; a.C = (const char*)C; a.c_scales = c_scales; a.h_bf16 = s.h_bf16; a.c = s.c; a.d = s.d;
    a.sample = smp.sample; a.tau = smp.tau; a.rng = rng;
    a.keys = ws.keys; a.keys_out = keys_out; a.cpad = b1_key_slots(s.c) * kB1Threads;
    const int ch = chunk_slots(s.c_fmt, s.d);
    if (s.c_fmt == RF_F32) {
      FH_DISPATCH_CH(ch, (launch_b1_scores<RF_F32, kCH>(a, s.c, st)));
    } else if (s.c_fmt == RF_BF16) {
      FH_DISPATCH_CH(ch, (launch_b1_scores<RF_BF16, kCH>(a, s.c, st)));
    } else {
      FH_DISPATCH_CH_INT4(ch, (launch_b1_scores<RF_INT4, kCH>(a, s.c, st)));
    }
    return hipGetLastError();
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
  B1Params a{};
  a.h = h; a.h_bf16 = s.h_bf16; a.c = s.c; a.d = s.d; a.b = s.b; a.p = p;
  a.sample = smp.sample; a.tau = smp.tau; a.rng = make_rng(smp.seed, smp.step);
  a.keys = ws.keys; a.part = ws.part;
  a.c2t = c2t; a.tiles = (const char*)tiles; a.scales = scales;
  a.probe_out = probe_out; a.logits_out = logits_out; a.tokens_out = tokens_out; a.token = token;
  const int ch = chunk_slots(s.e_fmt, s.d);
  if (s.e_fmt == RF_F32) {
    FH_DISPATCH_CH(ch, (launch_b1_stage2<RF_F32, kCH>(a, s.c, p, s.b, st)));
  } else if (s.e_fmt == RF_BF16) {
    FH_DISPATCH_CH(ch, (launch_b1_stage2<RF_BF16, kCH>(a, s.c, p, s.b, st)));
  } else {
    FH_DISPATCH_CH_INT4(ch, (launch_b1_stage2<RF_INT4, kCH>(a, s.c, p, s.b, st)));
  }
  return hipGetLastError();
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
    DenseParams a{h, (const char*)E, s.h_bf16, s.B, V, s.d, smp.sample, smp.tau, rng, best, logits};
    const int groups = (V + kRPI - 1) / kRPI;
    int wgs = (groups + 3) / 4;
    if (wgs > 2048) wgs = 2048;
    dim3 grid(wgs, s.B);
    const int ch = chunk_slots(s.e_fmt, s.d);
    if (s.e_fmt == RF_F32) {
      FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_dense_gemv<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a));
    } else {
      FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_dense_gemv<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a));
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
