// Row-streaming helpers shared by the head kernels: 16-byte row chunks spread over the
// 64 lanes of a wave, streamed with non-temporal loads, dotted with h held in registers.
#pragma once

#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRPI = 4;          // rows per wave per row-dot step
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

}  // namespace fh
