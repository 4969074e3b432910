// FlashHead kernels for gfx950 (CDNA4, wave64).
//
// Stage 1  k_scores_gemv / k_mfma<EPI_KEYS>  centroid logits C h -> probe keys
// Select   k_select                           per-row top-p on order-preserving uint32 keys
// Stage 2  k_tiles_probe (B == 1)             streams the kept clusters' contiguous tiles
//          k_tiles_mask  (B > 1)              one workgroup per cluster kept by any row
// Token    k_finalize                         packed (key, ~id) maxima -> token ids
// Dense    k_dense_gemv / k_mfma<EPI_ARGMAX>  the full-vocabulary comparator
// Offline  k_pack / k_check_counts            cluster-major tiles, optional int4 groups
//
// Method: "FlashHead: Efficient Drop-In Replacement for the Classification Head in
// Language Model Inference", Section 3.2 (two-stage retrieval, dense C2T).
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRPI = 4;          // rows per wave per row-dot step
constexpr int kThreads = 256;    // 4 waves

__host__ __device__ __forceinline__ int row_bytes_of(int fmt, int d) {
  return fmt == RF_F32 ? 4 * d : fmt == RF_BF16 ? 2 * d : d / 2;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// ------------------------------------------------------------------ row dot products

template <int RF, int CH>
struct RowGroup {
  uint4 w[kRPI][CH];
  float sc[kRPI][CH];
};

// Load rows [j0, j0 + kRPI) (those < nrows) of a matrix with row stride rb bytes.
template <int RF, int CH>
__device__ __forceinline__ void rows_load(RowGroup<RF, CH>& g, const char* base, int rb, int j0, int nrows,
                                          const uint16_t* scales, int spr, int lane) {
  const int cpr = rb >> 4;
#pragma unroll
  for (int r = 0; r < kRPI; ++r) {
    const int j = j0 + r;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = lane + kWave * i;
      const bool ok = j < nrows && q < cpr;
      g.w[r][i] = ok ? ld16(base + (size_t)j * rb + (size_t)q * 16) : make_uint4(0u, 0u, 0u, 0u);
      g.sc[r][i] = (RF == RF_INT4 && ok) ? bf16_to_f32(scales[(size_t)j * spr + (q >> 2)]) : 0.f;
    }
  }
}

// Full dot products of the loaded rows with h (every lane receives every sum).
template <int RF, int CH>
__device__ __forceinline__ void rows_dot(const RowGroup<RF, CH>& g, const HRegs<RF, CH>& hr, float (&out)[kRPI]) {
#pragma unroll
  for (int r = 0; r < kRPI; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) acc = chunk_dot<RF>(g.w[r][i], hr.v[i], acc, g.sc[r][i]);
    out[r] = wave_sum(acc);
  }
}

// ------------------------------------------------------------------ stage 1, row GEMV

struct ScoreParams {
  const void* h;
  const char* C;
  int h_bf16, B, c, d;
  int sample;
  float tau;
  Rng rng;
  float* keys;
  float* keys_out;
  uint64_t* mask;
  int W;
};

template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_scores_gemv(ScoreParams a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int wg = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int rb = row_bytes_of(RF, a.d);
  HRegs<RF, CH> hr;
  load_h<RF, CH>(hr, (const char*)a.h + (size_t)r * a.d * (a.h_bf16 ? 2 : 4), a.h_bf16, a.d, lane);
  for (int k0 = wg * kRPI; k0 < a.c; k0 += nw * kRPI) {
    RowGroup<RF, CH> g;
    rows_load<RF, CH>(g, a.C, rb, k0, a.c, nullptr, 0, lane);
    float s[kRPI];
    rows_dot<RF, CH>(g, hr, s);
#pragma unroll
    for (int i = 0; i < kRPI; ++i) {
      const int k = k0 + i;
      if (lane == i && k < a.c) {
        const float key = make_key(s[i], a.sample, a.tau, a.rng, (uint32_t)r, 0u, (uint32_t)k);
        a.keys[(size_t)r * a.c + k] = key;
        if (a.keys_out) a.keys_out[(size_t)r * a.c + k] = key;
      }
    }
    if (a.mask && r == 0) {
      for (int j = lane; j < kRPI * a.W; j += kWave) {
        const int k = k0 + j / a.W;
        if (k < a.c) a.mask[(size_t)k * a.W + j % a.W] = 0ull;
      }
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
    for (int s = wave; s < nsteps; s += 4) {
      const int ko = s * 32;
      const uint4 av = mv ? ld16(mp + ko) : make_uint4(0u, 0u, 0u, 0u);
      const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 bv = hv[t] ? ld16(hp[t] + ko) : make_uint4(0u, 0u, 0u, 0u);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, bv), acc[t], 0, 0, 0);
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mb + i;
          if (m < a.rows) {
            if (EPI == EPI_KEYS) {
              const float key = make_key(v[i], a.sample, a.tau, a.rng, (uint32_t)n, 0u, (uint32_t)m);
              a.keys[(size_t)n * a.rows + m] = key;
              if (a.keys_out) a.keys_out[(size_t)n * a.rows + m] = key;
            } else {
              const float key = make_key(v[i], a.sample, a.tau, a.rng, (uint32_t)n, 1u, (uint32_t)m);
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
    }
    __syncthreads();
  }
  if (EPI == EPI_ARGMAX && wave < NT) {
    uint64_t o = __shfl_xor(bc, 16, kWave);
    bc = o > bc ? o : bc;
    o = __shfl_xor(bc, 32, kWave);
    bc = o > bc ? o : bc;
    const int n = n0 + 16 * wave + lane;
    if (lane < 16 && n < a.B) atomicMax((unsigned long long*)&a.best[n], (unsigned long long)bc);
  }
}

// ------------------------------------------------------------------ probe selection
// One 1024-thread workgroup per row.  Thread t holds keys [t kpt, (t+1) kpt) as
// order-preserving uint32.  Four 8-bit radix passes from the top find T, the p-th largest
// key; then every key > T is kept and, of the keys == T, the ones with the smallest ids.
// Kept ids are written in ascending order (block scans over the per-thread chunks).

constexpr int kSelThreads = 1024;
constexpr int kSelMaxPerThread = 32;   // c <= 32768

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

__global__ __launch_bounds__(kSelThreads) void k_select(const float* keys, int c, int p, int32_t* probes,
                                                        int32_t* probe_out, uint64_t* mask, int W,
                                                        uint64_t* best) {
  __shared__ int hist[256];
  __shared__ int scan_sh[17];
  __shared__ int sh_digit, sh_above;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int kpt = (c + kSelThreads - 1) / kSelThreads;
  const int lo = tid * kpt;
  const float* kr = keys + (size_t)r * c;
  uint32_t u[kSelMaxPerThread];
#pragma unroll
  for (int i = 0; i < kSelMaxPerThread; ++i) u[i] = (i < kpt && lo + i < c) ? ord_key(kr[lo + i]) : 0u;
  uint32_t prefix = 0, pmask = 0;
  int need = p;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    if (tid == 0) { sh_digit = 0; sh_above = 0; }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelMaxPerThread; ++i) {
      if (i < kpt && lo + i < c && (u[i] & pmask) == prefix) atomicAdd(&hist[(u[i] >> shift) & 255u], 1);
    }
    __syncthreads();
    const int v = tid < 256 ? hist[255 - tid] : 0;
    int tot;
    const int ex = block_excl_scan(v, scan_sh, tot);
    if (tid < 256 && ex < need && ex + v >= need) {
      sh_digit = 255 - tid;
      sh_above = ex;
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    pmask |= 0xFFu << shift;
    need -= sh_above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < kSelMaxPerThread; ++i) {
    if (i < kpt && lo + i < c) {
      n_gt += u[i] > T;
      n_eq += u[i] == T;
    }
  }
  int tot;
  const int eq_before = block_excl_scan(n_eq, scan_sh, tot);
  const int take_eq = min(max(need - eq_before, 0), n_eq);
  int pos = block_excl_scan(n_gt + take_eq, scan_sh, tot);
  int32_t* pr = probes + (size_t)r * p;
  int eq_seen = 0;
#pragma unroll
  for (int i = 0; i < kSelMaxPerThread; ++i) {
    if (i < kpt && lo + i < c) {
      bool take = u[i] > T;
      if (u[i] == T) {
        take = eq_seen < take_eq;
        ++eq_seen;
      }
      if (take && pos < p) {
        const int k = lo + i;
        pr[pos] = k;
        if (probe_out) probe_out[(size_t)r * p + pos] = k;
        if (mask) atomicOr((unsigned long long*)&mask[(size_t)k * W + (r >> 6)], 1ull << (r & 63));
        ++pos;
      }
    }
  }
  if (tid == 0) best[r] = 0ull;
}

// ------------------------------------------------------------------ stage 2

struct TileParams {
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
#pragma unroll
    for (int i = 0; i < kRPI; ++i) {
      const int j = j0 + i;
      if (lane == i && j < a.b) {
        const int t = a.c2t[(size_t)k * a.b + j];
        const float key = make_key(z[i], a.sample, a.tau, a.rng, 0u, 1u, (uint32_t)t);
        const uint64_t cnd = pack_cand(key, (uint32_t)t);
        bc = cnd > bc ? cnd : bc;
        if (a.logits_out) a.logits_out[(size_t)q * a.b + j] = z[i];
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
template <int RF, int CH>
__global__ __launch_bounds__(kThreads) void k_tiles_mask(TileParams a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = blockIdx.x;
  const uint64_t* mk = a.mask + (size_t)k * a.W;
  bool any = false;
  for (int wi = 0; wi < a.W; ++wi) any |= mk[wi] != 0ull;
  if (!any) return;
  const int rb = row_bytes_of(RF, a.d);
  const int spr = a.d >> 7;
  const int hsz = a.h_bf16 ? 2 : 4;
  const char* tile = a.tiles + (size_t)k * a.b * rb;
  const uint16_t* sc = RF == RF_INT4 ? a.scales + (size_t)k * a.b * spr : nullptr;
  for (int j0 = wave * kRPI; j0 < a.b; j0 += 4 * kRPI) {
    RowGroup<RF, CH> g;
    rows_load<RF, CH>(g, tile, rb, j0, a.b, sc, spr, lane);
    int tj[kRPI];
#pragma unroll
    for (int i = 0; i < kRPI; ++i) tj[i] = (j0 + i < a.b) ? a.c2t[(size_t)k * a.b + j0 + i] : 0;
    for (int wi = 0; wi < a.W; ++wi) {
      uint64_t bits = mk[wi];
      while (bits) {
        const int r = wi * 64 + __builtin_ctzll(bits);
        bits &= bits - 1ull;
        if (r >= a.B) continue;                   // only if the workspace holds no masks
        HRegs<RF, CH> hr;
        load_h<RF, CH>(hr, (const char*)a.h + (size_t)r * a.d * hsz, a.h_bf16, a.d, lane);
        float z[kRPI];
        rows_dot<RF, CH>(g, hr, z);
        // position of k in row r's ascending probe list
        const int32_t* pr = a.probes + (size_t)r * a.p;
        int lo = 0, hi = a.p;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (pr[mid] < k) lo = mid + 1; else hi = mid;
        }
        uint64_t bc = 0;
#pragma unroll
        for (int i = 0; i < kRPI; ++i) {
          const int j = j0 + i;
          if (lane == i && j < a.b) {
            const int t = tj[i];
            const float key = make_key(z[i], a.sample, a.tau, a.rng, (uint32_t)r, 1u, (uint32_t)t);
            bc = pack_cand(key, (uint32_t)t);
            const size_t o = ((size_t)r * a.p + lo) * a.b + j;
            if (a.logits_out) a.logits_out[o] = z[i];
            if (a.tokens_out) a.tokens_out[o] = t;
          }
        }
        bc = wave_max_u64(bc);
        if (lane == 0) atomicMax((unsigned long long*)&a.best[r], (unsigned long long)bc);
      }
    }
  }
}

__global__ void k_finalize(const uint64_t* best, int32_t* token, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) token[i] = (int32_t)cand_id(best[i]);
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
#pragma unroll
    for (int i = 0; i < kRPI; ++i) {
      const int t = t0 + i;
      if (lane == i && t < a.V) {
        const float key = make_key(z[i], a.sample, a.tau, a.rng, (uint32_t)r, 1u, (uint32_t)t);
        const uint64_t cnd = pack_cand(key, (uint32_t)t);
        bc = cnd > bc ? cnd : bc;
        if (a.logits) a.logits[(size_t)r * a.V + t] = z[i];
      }
    }
  }
  bc = wave_max_u64(bc);
  if (lane == 0) wmax[wave] = bc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = wmax[0];
    for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
    atomicMax((unsigned long long*)&a.best[r], (unsigned long long)m);
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

__global__ void k_check_counts(const uint32_t* counts, int V, uint32_t* bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V && counts[i] != 1u) atomicOr(bad, 2u);
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
  off = up(off + (size_t)B * c * sizeof(float));
  w.mask = nullptr;
  if (B > 1) {
    w.mask = (uint64_t*)(b ? b + off : nullptr);
    off = up(off + (size_t)c * w.W * sizeof(uint64_t));
  }
  w.best = (uint64_t*)(b ? b + off : nullptr);
  off = up(off + (size_t)B * sizeof(uint64_t));
  w.probes = (int32_t*)(b ? b + off : nullptr);
  off = up(off + (size_t)B * p * sizeof(int32_t));
  w.bytes = off;
  return w;
}

size_t dense_workspace_bytes(int B) { return (((size_t)B * sizeof(uint64_t)) + 255) & ~(size_t)255; }

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
  if (use_mfma(s, s.c_fmt)) {
    MfmaParams p{};
    p.H = (const uint16_t*)h;
    p.M = (const uint16_t*)C;
    p.B = s.B; p.rows = s.c; p.d = s.d;
    p.sample = smp.sample; p.tau = smp.tau; p.rng = rng;
    p.keys = ws.keys; p.keys_out = keys_out; p.mask = ws.mask; p.W = ws.W;
    return launch_mfma<EPI_KEYS>(p, 1 << 30, st);
  }
  ScoreParams a{h, (const char*)C, s.h_bf16, s.B, s.c, s.d, smp.sample, smp.tau, rng,
                ws.keys, keys_out, ws.mask, ws.W};
  const int groups = (s.c + kRPI - 1) / kRPI;
  int wgs = (groups + 3) / 4;
  if (wgs > 4096) wgs = 4096;
  dim3 grid(wgs, s.B);
  const int ch = chunk_slots(s.c_fmt, s.d);
  if (s.c_fmt == RF_F32) {
    FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_scores_gemv<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a));
  } else {
    FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_scores_gemv<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a));
  }
  return hipGetLastError();
}

hipError_t launch_select(const HeadShape& s, int p, const Workspace& ws, int32_t* probe_out, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(s.B), dim3(kSelThreads), 0, st, (const float*)ws.keys, s.c, p,
                     ws.probes, probe_out, ws.mask, ws.W, ws.best);
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
  const int ch = chunk_slots(s.e_fmt, s.d);
  const bool b1 = s.B == 1;
  const dim3 grid(b1 ? p : s.c);
  if (s.e_fmt == RF_F32) {
    if (b1) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_probe<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a)); }
    else    { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_F32, kCH>), grid, dim3(kThreads), 0, st, a)); }
  } else if (s.e_fmt == RF_BF16) {
    if (b1) { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_probe<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a)); }
    else    { FH_DISPATCH_CH(ch, hipLaunchKernelGGL((k_tiles_mask<RF_BF16, kCH>), grid, dim3(kThreads), 0, st, a)); }
  } else {
    if (b1) { FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_tiles_probe<RF_INT4, kCH>), grid, dim3(kThreads), 0, st, a)); }
    else    { FH_DISPATCH_CH_INT4(ch, hipLaunchKernelGGL((k_tiles_mask<RF_INT4, kCH>), grid, dim3(kThreads), 0, st, a)); }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_finalize, dim3((s.B + 255) / 256), dim3(256), 0, st, (const uint64_t*)ws.best, token, s.B);
  return hipGetLastError();
}

hipError_t launch_dense(const HeadShape& s, int V, const void* h, const void* E, const Sampling& smp,
                        uint64_t* best, int32_t* token, float* logits, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_u64, dim3((s.B + 255) / 256), dim3(256), 0, st, best, s.B, (uint64_t)0);
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
  hipLaunchKernelGGL(k_finalize, dim3((s.B + 255) / 256), dim3(256), 0, st, (const uint64_t*)best, token, s.B);
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
