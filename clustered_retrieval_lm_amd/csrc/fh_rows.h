// Row-streaming helpers shared by the head kernels: 16-byte row chunks spread over the
// 64 lanes of a wave, streamed with non-temporal loads, dotted with h held in registers.
#pragma once

#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

// rows_dot with h read from memory (L2) piece by piece instead of held in registers, for kernels
// that dot the same rows with many hidden states.  fp32 and int4 rows, and bf16 rows with fp32 h:
// the same fused multiply-adds in the same order per row as rows_dot with load_h (bitwise the
// same results).  bf16 rows with bf16 h: the raw words go straight into v_dot2c_f32_bf16 (two
// exact bf16 products and the running sum per instruction, four per 16-byte chunk), with no
// bf16 -> fp32 unpacking of either operand; measured on random operands over 2^+-14 magnitudes,
// with cancelling products and with zero, tiny and huge running sums, one instruction's error
// stays below 2.8 u (|p0| + |p1| + |acc|), u = 2^-24, so a lane's chain of 4 CH instructions
// counts as at most 16 CH roundings.  HB: h is bf16 (compile time, so the chunk loop has no
// branch).
template <int RF, int CH, int NR, bool HB = false>
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
      if (HB) {                                  // h is bf16 (HB): packed bf16 dots on the raw words
        const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        const uint32_t hw[4] = {x.x & m, x.y & m, x.z & m, x.w & m};
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const uint32_t ww[4] = {g.w[r][i].x, g.w[r][i].y, g.w[r][i].z, g.w[r][i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ww[q]),
                                                     __builtin_bit_cast(bf16x2_t, hw[q]), acc[r], false);
        }
      } else {
        float hv[8];
        h_piece8(hv, src, h_bf16, ok);
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = chunk_dot<RF_BF16>(g.w[r][i], hv, acc[r], 0.f);
      }
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
          half2_t q[4];
          nib_pairs(wj, q);
#pragma unroll
          for (int k = 0; k < 8; ++k) s[r] = fmaf(nib_of(q, k), hv[k], s[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = fmaf(__uint_as_float(g.sc[r][i] << 16), s[r], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) out[r] = wave_sum(acc[r]);
}

}  // namespace fh
