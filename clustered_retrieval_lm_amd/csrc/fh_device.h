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
__host__ __device__ __forceinline__ uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * b) >> 32);
}

__host__ __device__ __forceinline__ uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t a0 = 0xD2511F53u * x.x, h0 = mulhi32(0xD2511F53u, x.x);
    const uint32_t a1 = 0xCD9E8D57u * x.z, h1 = mulhi32(0xCD9E8D57u, x.z);
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

// The four words of block n4 of (row, stream): the words of elements 4 n4 .. 4 n4 + 3.
__host__ __device__ __forceinline__ uint4 rng_block(const Rng& g, uint32_t row, uint32_t stream, uint32_t n4) {
  return philox4x32_10(make_uint4(n4, row, g.step_lo, g.step_hi4 | stream), g.k0, g.k1);
}

// The word for element n of (row, stream).
__host__ __device__ __forceinline__ uint32_t rng_word(const Rng& g, uint32_t row, uint32_t stream, uint32_t n) {
  const uint4 o = rng_block(g, row, stream, n >> 2);
  const uint32_t s = n & 3u;
  return s == 0 ? o.x : s == 1 ? o.y : s == 2 ? o.z : o.w;
}

// Odd multiples of 2^-24 in (0, 1): exact in fp32.
__host__ __device__ __forceinline__ float word_to_uniform(uint32_t w) {
  return (float)(2u * (w >> 9) + 1u) * 0x1p-24f;
}

__device__ __forceinline__ float gumbel(float u) { return -logf(-logf(u)); }

// Probe or token key: the logit itself (greedy) or logit / tau + Gumbel noise (sampling).
// Adding +0 turns a -0 key into +0 (round to nearest), so keys compare the same as floats
// and as ord_key values.
__device__ __forceinline__ float gumbel_key(float z_over_tau, uint32_t word) {
  return z_over_tau + gumbel(word_to_uniform(word)) + 0.0f;
}

__device__ __forceinline__ float sample_key(float z, float tau, uint32_t word) {
  return gumbel_key(z / tau, word);
}

__device__ __forceinline__ float make_key(float z, int sample, float tau, const Rng& g, uint32_t row,
                                          uint32_t stream, uint32_t n) {
  if (!sample) return z + 0.0f;
  return sample_key(z, tau, rng_word(g, row, stream, n));
}

// ---------------------------------------------------------------- wave reductions
// Sum over the 64 lanes with DPP moves (no LDS traffic): quad swaps, half-row and row
// mirrors, then row broadcasts 15 and 31 carry the row sums up to lane 63, which is read
// back as a wave-uniform value.  A fixed 6-level tree: the rounding order never varies.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);    // quad_perm(1,0,3,2)
  v = dpp_add<0x4E, 0xF>(v);    // quad_perm(2,3,0,1)
  v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);   // row_mirror
  v = dpp_add<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, BOUND);
}

// Inclusive prefix sum over the 64 lanes (row shifts, then row broadcasts 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xF, true>(0, v);   // row_shr:1
  v += dpp_i<0x112, 0xF, true>(0, v);   // row_shr:2
  v += dpp_i<0x114, 0xF, true>(0, v);   // row_shr:4
  v += dpp_i<0x118, 0xF, true>(0, v);   // row_shr:8
  v += dpp_i<0x142, 0xA, false>(0, v);  // row_bcast:15 into rows 1, 3
  v += dpp_i<0x143, 0xC, false>(0, v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Max / min of uint32 over the 64 lanes, returned wave-uniform.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  const int id = MAX ? 0 : -1;
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, (uint32_t)dpp_i<0xB1, 0xF, false>(id, (int)v));
  v = op(v, (uint32_t)dpp_i<0x4E, 0xF, false>(id, (int)v));
  v = op(v, (uint32_t)dpp_i<0x141, 0xF, false>(id, (int)v));
  v = op(v, (uint32_t)dpp_i<0x140, 0xF, false>(id, (int)v));
  v = op(v, (uint32_t)dpp_i<0x142, 0xA, false>(id, (int)v));
  v = op(v, (uint32_t)dpp_i<0x143, 0xC, false>(id, (int)v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Max / min of floats over the 64 lanes (NaN-free inputs), returned wave-uniform.
template <bool MAX>
__device__ __forceinline__ float wave_minmax_f32(float v) {
  const int id = (int)(MAX ? 0xFF800000u : 0x7F800000u);    // -inf / +inf
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  v = op(v, __int_as_float(dpp_i<0xB1, 0xF, false>(id, __float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<0x4E, 0xF, false>(id, __float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<0x141, 0xF, false>(id, __float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<0x140, 0xF, false>(id, __float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<0x142, 0xA, false>(id, __float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<0x143, 0xC, false>(id, __float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// v[lane] for lanes < N (v wave-uniform), v[0] elsewhere: lets lane i handle element i with one
// evaluation of what follows instead of N evaluations with one lane active each.  The empty asm
// keeps the selects as selects: rewritten as an indexed load from v, the array would be moved to
// LDS (4 KB per workgroup, and the work-item ids set up to address it).
// Lane L of v takes the wave-uniform value x (v_writelane: one instruction, where a select
// per lane costs a compare, a move and a select).  The lane is an immediate: a second
// SGPR operand would break the one-SGPR operand limit.  x is often a ballot still in VCC,
// just written by a VALU compare; a VALU that reads VCC as a constant operand must follow
// such a write by at least one wait state, and the compiler inserts none inside inline
// assembly, hence the s_nop.
template <int L>
__device__ __forceinline__ void put_lane_i(uint32_t& v, uint32_t x) {
  asm volatile("s_nop 1\n\tv_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(x), "i"(L));
}

// put_lane_i for a lane that is a constant once the caller's loop is unrolled (0 <= lane < 32).
__device__ __forceinline__ void put_lane(uint32_t& v, uint32_t x, int lane) {
  switch (lane) {
#define FH_PUT_LANE(L) case L: put_lane_i<L>(v, x); break;
    FH_PUT_LANE(0) FH_PUT_LANE(1) FH_PUT_LANE(2) FH_PUT_LANE(3) FH_PUT_LANE(4) FH_PUT_LANE(5) FH_PUT_LANE(6)
    FH_PUT_LANE(7) FH_PUT_LANE(8) FH_PUT_LANE(9) FH_PUT_LANE(10) FH_PUT_LANE(11) FH_PUT_LANE(12) FH_PUT_LANE(13)
    FH_PUT_LANE(14) FH_PUT_LANE(15) FH_PUT_LANE(16) FH_PUT_LANE(17) FH_PUT_LANE(18) FH_PUT_LANE(19) FH_PUT_LANE(20)
    FH_PUT_LANE(21) FH_PUT_LANE(22) FH_PUT_LANE(23) FH_PUT_LANE(24) FH_PUT_LANE(25) FH_PUT_LANE(26) FH_PUT_LANE(27)
    FH_PUT_LANE(28) FH_PUT_LANE(29) FH_PUT_LANE(30) FH_PUT_LANE(31)
#undef FH_PUT_LANE
    default: break;
  }
}

template <int N, typename T>
__device__ __forceinline__ T lane_pick(const T (&v)[N], int lane) {
  T x = v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) {
    x = lane == i ? v[i] : x;
    asm volatile("" : "+v"(x));
  }
  return x;
}

__device__ __forceinline__ int lane_prefix(uint64_t bal) {   // set bits of bal below this lane
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
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

// h as loaded, before the conversion to fp32: the 16-byte words of each chunk slot (fp32
// storage fills all W of them, bf16 storage the first half).  Lets a kernel issue the loads
// of h early and convert after other loads are in flight.
template <int RF, int CH>
struct HRaw {
  static constexpr int W = Fmt<RF>::EPC / 4;
  uint4 r[CH][W];
  uint32_t ok;              // bit i: chunk slot i lies inside h (else it converts to zeros)
};

template <int RF, int CH>
__device__ __forceinline__ void load_h_raw(HRaw<RF, CH>& raw, const void* h, int h_bf16, int d, int lane) {
  constexpr int EPC = Fmt<RF>::EPC, W = HRaw<RF, CH>::W;
  const int esz = h_bf16 ? 2 : 4;
  // 16-byte words per chunk: all W for fp32 h, W / 2 for bf16 h (a half word when W == 1).
  // Slots past d read chunk 0 (always inside h) and are zeroed by unpack_h.
  const int nfull = h_bf16 ? W / 2 : W;
  raw.ok = 0u;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int e0 = (lane + kWave * i) * EPC;
    const bool ok = e0 < d;
    raw.ok |= ok ? (1u << i) : 0u;
    const char* src = (const char*)h + (ok ? (size_t)e0 * esz : 0);
#pragma unroll
    for (int v = 0; v < W; ++v)
      if (v < nfull) raw.r[i][v] = reinterpret_cast<const uint4*>(src)[v];
    if (W == 1 && h_bf16) {
      const uint2 w = *reinterpret_cast<const uint2*>(src);
      raw.r[i][0] = make_uint4(w.x, w.y, 0u, 0u);
    }
  }
}

template <int RF, int CH>
__device__ __forceinline__ void unpack_h(HRegs<RF, CH>& hr, const HRaw<RF, CH>& raw, int h_bf16) {
  constexpr int EPC = Fmt<RF>::EPC, W = HRaw<RF, CH>::W;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (!((raw.ok >> i) & 1u)) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) hr.v[i][e] = 0.f;
      continue;
    }
    if (h_bf16) {
      constexpr int NV = EPC >= 8 ? EPC / 8 : 1, NJ = EPC >= 8 ? 4 : 2;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t ws[4] = {raw.r[i][v].x, raw.r[i][v].y, raw.r[i][v].z, raw.r[i][v].w};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          hr.v[i][8 * v + 2 * j] = bf16_lo(ws[j]);
          hr.v[i][8 * v + 2 * j + 1] = bf16_hi(ws[j]);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < W; ++v) {
        hr.v[i][4 * v + 0] = __uint_as_float(raw.r[i][v].x);
        hr.v[i][4 * v + 1] = __uint_as_float(raw.r[i][v].y);
        hr.v[i][4 * v + 2] = __uint_as_float(raw.r[i][v].z);
        hr.v[i][4 * v + 3] = __uint_as_float(raw.r[i][v].w);
      }
    }
  }
}

// Load h (fp32 or bf16 storage, d values) into the chunk layout of row format RF: every
// 16-byte load is issued before any conversion.
template <int RF, int CH>
__device__ __forceinline__ void load_h(HRegs<RF, CH>& hr, const void* h, int h_bf16, int d, int lane) {
  HRaw<RF, CH> raw;
  load_h_raw<RF, CH>(raw, h, h_bf16, d, lane);
  unpack_h<RF, CH>(hr, raw, h_bf16);
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

// int4: 32 two's-complement nibbles, element 2i in the low nibble of byte i, so element 8j + k
// of a chunk is nibble k of its word j.  The 32 products q h are summed first (each is exact in
// fp32), then scaled by the group's s.
//
// The nibbles are decoded in pairs (k, k + 4) straight into fp16, with no integer-to-float
// conversion.  In the word (shifted right by 8 bits for k = 2, 3) nibble k sits in bits 0..3
// (k = 0, 2) or 4..7 (k = 1, 3) of the low half and nibble k + 4 at the same place in the high
// half; keeping those bits, flipping each nibble's top bit (q + 8 instead of two's complement)
// and setting the exponent field of 1024 makes each half 1024 + (q + 8), or 1024 + 16 (q + 8)
// for odd k, which is exact; one packed fp16 add (or multiply-add by 1/16) leaves q exactly.  Each half feeds one mixed-precision fused multiply-add (v_fma_mix_f32),
// which widens it exactly, so the chain of fused multiply-adds is the one of a float decode:
// 17 instructions per 8 elements instead of 24.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void nib_pairs(uint32_t w, half2_t (&q)[4]) {
  const uint32_t y = w >> 8;                          // nibbles 2, 3, 6, 7 where 0, 1, 4, 5 were
  const half2_t a = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) ^ 0x64086408u);   // 0 and 4
  const half2_t b = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) ^ 0x64806480u);   // 1 and 5
  const half2_t c = __builtin_bit_cast(half2_t, (y & 0x000F000Fu) ^ 0x64086408u);   // 2 and 6
  const half2_t e = __builtin_bit_cast(half2_t, (y & 0x00F000F0u) ^ 0x64806480u);   // 3 and 7
  const half2_t off = {(_Float16)-1032.f, (_Float16)-1032.f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off16 = {(_Float16)-72.f, (_Float16)-72.f};
  q[0] = a + off;
  q[1] = b * sixteenth + off16;
  q[2] = c + off;
  q[3] = e * sixteenth + off16;
}

// Element k (0..7) of a word decoded by nib_pairs.
__device__ __forceinline__ float nib_of(const half2_t (&q)[4], int k) {
  return (float)(k < 4 ? q[k].x : q[k - 4].y);
}

template <>
__device__ __forceinline__ float chunk_dot<RF_INT4>(const uint4 w, const float* hv, float acc, float scale) {
  float s = 0.f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    half2_t q[4];
    nib_pairs(ws[j], q);
#pragma unroll
    for (int k = 0; k < 8; ++k) s = fmaf(nib_of(q, k), hv[8 * j + k], s);
  }
  return fmaf(scale, s, acc);
}

}  // namespace fh
