// device_common.h -- device-side helpers of the speculation-cycle kernels (gfx950).
//
// Counter hash: SplitMix64 (Steele, Lea & Flood 2014; public-domain splitmix64.c), written here
// from its published definition for the GPU.  Row keys chain first outputs over
// (seed, global request id, position, stream); index i of a row draws 32 bits from the
// (i/2 + 1)-th output of a generator started at the row key (high half for even i, low half
// for odd i).  Uniform U = (bits + 1/2) 2^-32, Gumbel noise G = -log(-log1p(-U)).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

constexpr uint64_t SM_GAMMA = 0x9E3779B97F4A7C15ull;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr int CHUNK = 64;

// noise streams
constexpr uint64_t ST_DRAFT = 1, ST_ACCEPT = 2, ST_RESIDUAL = 3, ST_BONUS = 4;
constexpr uint64_t ST_DRAFT_C = 5, ST_RESIDUAL_C = 7, ST_BONUS_C = 8;

__device__ __forceinline__ uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t sm_first(uint64_t x) { return sm_mix(x + SM_GAMMA); }

__device__ __forceinline__ uint64_t row_key(uint64_t seed, uint64_t request, uint64_t pos, uint64_t stream) {
  uint64_t k = sm_first(seed);
  k = sm_first(k ^ request);
  k = sm_first(k ^ pos);
  return sm_first(k ^ stream);
}

// the 64-bit word that carries indices 2p and 2p+1 of a row
__device__ __forceinline__ uint64_t pair_word(uint64_t key, uint32_t p) {
  return sm_mix(key + (uint64_t)(p + 1u) * SM_GAMMA);
}

__device__ __forceinline__ uint32_t bits_at(uint64_t key, uint32_t i) {
  uint64_t w = pair_word(key, i >> 1);
  return (i & 1u) ? (uint32_t)w : (uint32_t)(w >> 32);
}

// hardware transcendentals: v_exp_f32 / v_log_f32 (base 2).  Inputs of ex2 here are <= 0 or
// small; lg2 arguments are positive normal numbers.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Gumbel noise from 32 random bits, fp32: G = -log(E), E = -log(1 - U).  E is taken from
// whichever side keeps its relative precision: the series u + u^2/2 + ... + u^5/5 for u < 1/64
// (truncation error below u^6/6), -log(1 - u) for 1/64 <= u < 1/2 (log2 magnitude >= 0.0227, so
// its absolute error stays a small relative error), and 32 ln2 - log(complement) with the exact
// complement (2^32 - bits - 1/2) 2^-32 for u >= 1/2.  Absolute error of G ~ 1e-6.
__device__ __forceinline__ float gumbel_bits(uint32_t b) {
  float e;
  if (b < 0x80000000u) {
    const float u = ((float)b + 0.5f) * 0x1p-32f;
    if (u < 0.015625f) {
      e = u * fmaf(u, fmaf(u, fmaf(u, fmaf(u, 0.2f, 0.25f), 0.33333334f), 0.5f), 1.0f);
    } else {
      e = -lg2(1.0f - u) * LN2;
    }
  } else {
    const float c = (float)(~b) + 0.5f;
    e = (32.0f - lg2(c)) * LN2;
  }
  return -lg2(e) * LN2;
}

// rigorous upper bound of gumbel_bits(b): U >= 2^(31-clz) 2^-32 and -log1p(-U) >= U
__device__ __forceinline__ float gumbel_bound(uint32_t b) {
  return (float)(__clz((int)b) + 1) * LN2;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// log(exp(a) + exp(b)) in natural units, -inf aware
__device__ __forceinline__ float lse2(float a, float b) {
  float m = fmaxf(a, b);
  if (m == -INFINITY) return a + b;   // both empty: -inf; fmaxf drops a NaN, the sum keeps it
  return m + lg2(ex2((a - m) * LOG2E) + ex2((b - m) * LOG2E)) * LN2;
}

// lane permutes on the VALU (DPP), no LDS round trip.  Within each group of 8 lanes:
// quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror (i <-> 7 - i).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max / sum over the 8 lanes of an aligned group; every lane gets the result
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  return fmaxf(x, dpp<0x141>(x));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  return x + dpp<0x141>(x);
}

// value of lane (l ^ 32) with one v_permlane32_swap
__device__ __forceinline__ float xor32f(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)((threadIdx.x & 32) ? r[0] : r[1]));
}
__device__ __forceinline__ int xor32i(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (int)((threadIdx.x & 32) ? r[0] : r[1]);
}

// argmax merge: larger score wins, equal scores go to the smaller index
__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && (unsigned)i1 < (unsigned)i2);
}

}  // namespace spec
