// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef uint16_t bf16_t;

// ---------------------------------------------------------------- bf16

MOE_DEV float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest, ties to even (inputs are finite).
MOE_DEV bf16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- order keys

// Map a float to a uint32 whose unsigned order is the float order; -0 and
// +0 map to the same key (they compare equal as floats).
MOE_DEV uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Composite key: larger float first, then lower index first.
MOE_DEV uint64_t rank_key(float x, uint32_t idx) {
  return ((uint64_t)order_key(x) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
MOE_DEV uint32_t rank_key_index(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull); }

// ---------------------------------------------------------------- specified exp
// Cody & Waite argument reduction with a two-part ln 2 and a degree-7 Taylor
// polynomial of e^r in Horner form; every step is one IEEE fp32 operation
// (this whole library is built with -ffp-contract=off, and the pragma keeps
// the property if a file is ever built without it).  x < -86 gives 0 (so a
// non-zero result is never subnormal), x > 88 gives +inf.
#define MOE_LN2_D 0.693147180559945309417232121458
MOE_DEV float spec_exp(float x) {
#pragma clang fp contract(off)
  const float kLog2e = (float)(1.0 / MOE_LN2_D);
  // ln 2 rounded to fp32 with its 9 lowest mantissa bits cleared, so that
  // k * kLn2Hi is exact for |k| < 512.
  const float kLn2Hi = __uint_as_float(0x3F317218u & 0xFFFFFE00u);
  const float kLn2Lo = (float)(MOE_LN2_D - (double)__uint_as_float(0x3F317218u & 0xFFFFFE00u));
  if (x < -86.0f) return 0.0f;
  if (x > 88.0f) return __uint_as_float(0x7F800000u);
  const float kf = __builtin_rintf(x * kLog2e);
  const float r = (x - kf * kLn2Hi) - kf * kLn2Lo;
  float p = (float)(1.0 / 5040.0);
  p = p * r + (float)(1.0 / 720.0);
  p = p * r + (float)(1.0 / 120.0);
  p = p * r + (float)(1.0 / 24.0);
  p = p * r + (float)(1.0 / 6.0);
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const int k = (int)kf;
  const float two_k = __uint_as_float((uint32_t)(k + 127) << 23);
  return p * two_k;
}

MOE_DEV float spec_sigmoid(float z) {
#pragma clang fp contract(off)
  return 1.0f / (1.0f + spec_exp(-z));
}

// ---------------------------------------------------------------- specified sqrtsoftplus
// log1p(u) for 0 <= u <= 1 as 2 atanh(s), s = u / (2 + u):
// 2 s (1 + s^2/3 + ... + s^14/15) in Horner form over s^2 (s <= 1/3, so the
// first omitted term is below 2^-30 relative); softplus(z) = max(z, 0) +
// log1p(e^-|z|); the score is its correctly rounded square root.
MOE_DEV float spec_log1p01(float u) {
#pragma clang fp contract(off)
  const float s = u / (2.0f + u);
  const float s2 = s * s;
  float p = (float)(1.0 / 15.0);
  p = p * s2 + (float)(1.0 / 13.0);
  p = p * s2 + (float)(1.0 / 11.0);
  p = p * s2 + (float)(1.0 / 9.0);
  p = p * s2 + (float)(1.0 / 7.0);
  p = p * s2 + (float)(1.0 / 5.0);
  p = p * s2 + (float)(1.0 / 3.0);
  p = p * s2 + 1.0f;
  return (s + s) * p;
}

MOE_DEV float spec_sqrtsoftplus(float z) {
#pragma clang fp contract(off)
  const float sp = fmaxf(z, 0.0f) + spec_log1p01(spec_exp(-fabsf(z)));
  // __builtin_sqrtf lowers to the correctly rounded sequence (v_sqrt_f32,
  // then a one-ulp neighbour test with exact residuals); __fsqrt_rn lowers
  // to the bare v_sqrt_f32 on gfx950, which is not correctly rounded
  return __builtin_sqrtf(sp);
}

// Per-expert score of the bias-balanced recipes: 1 = sigmoid, 2 = sqrtsoftplus.
MOE_DEV float spec_expert_score(float z, int score) {
  return score == 2 ? spec_sqrtsoftplus(z) : spec_sigmoid(z);
}

// ---------------------------------------------------------------- wave64 helpers

// One step of the maximum through the DPP lane network: each lane takes
// the value of the lane kCtrl names (0 where there is none, or in rows
// outside kRowMask), so no LDS round trip as with a shuffle.
template <int kCtrl, int kRowMask>
MOE_DEV uint64_t dpp_max_step_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, kRowMask, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, kRowMask, 0xf, false);
  const uint64_t w = ((uint64_t)hi << 32) | lo;
  return w > v ? w : v;
}

// Maximum over the 64 lanes of a wave (all lanes active; 0 is the identity:
// every key this serves is an unsigned composite).  Lanes shifted right by
// 1, 2, 4, 8 within each 16-lane row give lane 15 of a row the row's
// maximum; broadcasts of lane 15 into rows 1 and 3 and of lane 31 into rows
// 2 and 3 bring the whole wave's into lane 63, which every lane reads.  The
// maximum does not depend on the order of comparisons.
MOE_DEV uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step_u64<0x111, 0xf>(v);   // row_shr:1
  v = dpp_max_step_u64<0x112, 0xf>(v);   // row_shr:2
  v = dpp_max_step_u64<0x114, 0xf>(v);   // row_shr:4
  v = dpp_max_step_u64<0x118, 0xf>(v);   // row_shr:8
  v = dpp_max_step_u64<0x142, 0xa>(v);   // row_bcast:15 into rows 1, 3
  v = dpp_max_step_u64<0x143, 0xc>(v);   // row_bcast:31 into rows 2, 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

MOE_DEV float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Halving-stride tree sum over 64 lanes holding elements 0..63 of a
// zero-padded power-of-two vector of length P <= 64: pass s adds element
// i+s to element i.  The result is valid in lane 0 only.
MOE_DEV float wave_tree_sum(float v, int P) {
#pragma clang fp contract(off)
  for (int s = P >> 1; s >= 1; s >>= 1) v = v + __shfl_down(v, s, 64);
  return v;
}

MOE_DEV int wave_inclusive_scan_i32(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int w = __shfl_up(v, o, 64);
    if (lane >= o) v += w;
  }
  return v;
}

MOE_DEV int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Exclusive scan over a workgroup of NT threads (NT a multiple of 64, at most
// 4096).  `scratch` holds NT/64 ints of LDS.  Returns the exclusive prefix;
// *total receives the workgroup sum in every thread.  Contains barriers:
// every thread of the workgroup must call it.
template <int NT>
MOE_DEV int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan_i32(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wsum = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    const int s = scratch[w];
    if (w < wave) wsum += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wsum + incl - v;
}
