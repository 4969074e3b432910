// Device helpers of the FlashHead kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fh {

constexpr int kWave = 64;

// Row formats of the streamed matrices (centroids, tiles, dense E).
enum RowFmt : int { RF_F32 = 0, RF_BF16 = 1, RF_INT4 = 2 };

// Values held by one 16-byte chunk of a row.
template <int RF> struct Fmt;
template <> struct Fmt<RF_F32>  { static constexpr int EPC = 4;  };
template <> struct Fmt<RF_BF16> { static constexpr int EPC = 8;  };
template <> struct Fmt<RF_INT4> { static constexpr int EPC = 32; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Monotone map of float keys onto uint32: a > b (as floats, not NaN) implies ord(a) > ord(b).
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t b = __float_as_uint(f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// Candidate of a max-reduction: larger key first, then the smaller id.
__device__ __forceinline__ uint64_t pack_cand(float key, uint32_t id) {
  return ((uint64_t)ord_key(key) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t cand_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
__device__ __forceinline__ uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t a0 = 0xD2511F53u * x.x, h0 = __umulhi(0xD2511F53u, x.x);
    const uint32_t a1 = 0xCD9E8D57u * x.z, h1 = __umulhi(0xCD9E8D57u, x.z);
    x = make_uint4(h1 ^ x.y ^ k0, a1, h0 ^ x.w ^ k1, a0);
  }
  return x;
}

struct Rng {
  uint32_t k0, k1, step_lo, step_hi4;   // step_hi4 = (step >> 32) << 2
};

__host__ __device__ inline Rng make_rng(uint64_t seed, uint64_t step) {
  return Rng{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)step, (uint32_t)((step >> 32) << 2)};
}

// The word for element n of (row, stream).
__device__ __forceinline__ uint32_t rng_word(const Rng& g, uint32_t row, uint32_t stream, uint32_t n) {
  uint4 ctr = make_uint4(n >> 2, row, g.step_lo, g.step_hi4 | stream);
  uint4 o = philox4x32_10(ctr, g.k0, g.k1);
  const uint32_t s = n & 3u;
  return s == 0 ? o.x : s == 1 ? o.y : s == 2 ? o.z : o.w;
}

// Odd multiples of 2^-24 in (0, 1): exact in fp32.
__device__ __forceinline__ float word_to_uniform(uint32_t w) {
  return (float)(2u * (w >> 9) + 1u) * 0x1p-24f;
}

__device__ __forceinline__ float gumbel(float u) { return -logf(-logf(u)); }

// Probe or token key: the logit itself (greedy) or logit / tau + Gumbel noise (sampling).
__device__ __forceinline__ float make_key(float z, int sample, float tau, const Rng& g, uint32_t row,
                                          uint32_t stream, uint32_t n) {
  if (!sample) return z;
  return z / tau + gumbel(word_to_uniform(rng_word(g, row, stream, n)));
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// ---------------------------------------------------------------- row dot products
// A wave computes dot(h, row) for rows of a row-major matrix whose rows are split into
// 16-byte chunks; lane l owns chunk slots q = l + 64 i (i < CH).  h is held in registers
// as fp32 in the same chunk layout.

template <int RF, int CH>
struct HRegs {
  float v[CH][Fmt<RF>::EPC];
};

// Load h (fp32 or bf16 storage, d values) into the chunk layout of row format RF.
template <int RF, int CH>
__device__ __forceinline__ void load_h(HRegs<RF, CH>& hr, const void* h, int h_bf16, int d, int lane) {
  constexpr int EPC = Fmt<RF>::EPC;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int e0 = (lane + kWave * i) * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int idx = e0 + e;
      float x = 0.f;
      if (idx < d) x = h_bf16 ? bf16_to_f32(((const uint16_t*)h)[idx]) : ((const float*)h)[idx];
      hr.v[i][e] = x;
    }
  }
}

// Partial dot of one 16-byte chunk with h (scale applies to int4 only).
template <int RF>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float* hv, float acc, float scale);

template <>
__device__ __forceinline__ float chunk_dot<RF_F32>(const uint4 w, const float* hv, float acc, float) {
  acc = fmaf(__uint_as_float(w.x), hv[0], acc);
  acc = fmaf(__uint_as_float(w.y), hv[1], acc);
  acc = fmaf(__uint_as_float(w.z), hv[2], acc);
  acc = fmaf(__uint_as_float(w.w), hv[3], acc);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<RF_BF16>(const uint4 w, const float* hv, float acc, float) {
  acc = fmaf(bf16_lo(w.x), hv[0], acc);
  acc = fmaf(bf16_hi(w.x), hv[1], acc);
  acc = fmaf(bf16_lo(w.y), hv[2], acc);
  acc = fmaf(bf16_hi(w.y), hv[3], acc);
  acc = fmaf(bf16_lo(w.z), hv[4], acc);
  acc = fmaf(bf16_hi(w.z), hv[5], acc);
  acc = fmaf(bf16_lo(w.w), hv[6], acc);
  acc = fmaf(bf16_hi(w.w), hv[7], acc);
  return acc;
}

// int4: 32 two's-complement nibbles, element 2i in the low nibble of byte i.  The 32
// products q h are summed first (each is exact in fp32), then scaled by the group's s.
__device__ __forceinline__ float nib(uint32_t w, int k) {
  return (float)((int32_t)(w << (28 - 4 * k)) >> 28);
}

template <>
__device__ __forceinline__ float chunk_dot<RF_INT4>(const uint4 w, const float* hv, float acc, float scale) {
  float s = 0.f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s = fmaf(nib(ws[j], k), hv[8 * j + k], s);
  }
  return fmaf(scale, s, acc);
}

}  // namespace fh
