// Device helpers shared by the gfx950 kernels of this library: bf16 bit
// handling, DPP lane exchanges inside 8-lane groups and 64-bit row addressing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint16_t bf16_t;  // bf16 stored as its bit pattern

// Sentinel "minus infinity" for running maxima: finite, so that
// exp2(m_old - m_new) never becomes inf - inf when a lane has seen no key yet.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the hardware v_exp_f32 (inputs here are <= 0; -inf gives 0 and
// results below the fp32 normal range may flush to 0, which is harmless for
// softmax weights).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Dot product of 8 bf16 pairs held in two uint4 (16 bf16 each side), fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// ---- DPP exchanges inside a row of 16 lanes (no LDS traffic) ----
// quad_perm [1,0,3,2] : lane ^ 1
// quad_perm [2,3,0,1] : lane ^ 2
// row_half_mirror     : lane i of each 8-lane half row <-> lane 7 - i
// row_ror 8           : lane i <-> lane i ^ 8 inside a 16-lane row
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRor8 = 0x128;

// Max / sum over the 8 lanes of an aligned 8-lane group, result in every lane.
__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  return x;
}
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

// Reduce-scatter of 8 values across the 8 lanes of a group: on return lane s
// (s = lane & 7) holds the group-wide sum of element s. Partner lanes are
// s ^ 7 (half mirror), then s ^ 2, then s ^ 1; every exchange pairs lanes that
// differ in the bit being resolved, so the kept halves line up.
__device__ __forceinline__ float group8_reduce_scatter(const float (&v)[8], int s) {
  const bool b2 = s & 4, b1 = s & 2, b0 = s & 1;
  float a[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float send = b2 ? v[m] : v[m + 4];
    const float keep = b2 ? v[m + 4] : v[m];
    a[m] = keep + dpp<kDppHalfMirror>(send);
  }
  float c[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float send = b1 ? a[m] : a[m + 2];
    const float keep = b1 ? a[m + 2] : a[m];
    c[m] = keep + dpp<kDppXor2>(send);
  }
  const float send = b0 ? c[0] : c[1];
  const float keep = b0 ? c[1] : c[0];
  return keep + dpp<kDppXor1>(send);
}

__device__ __forceinline__ uint4 load16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load/store with the nontemporal hint, for data touched once per
// call (KV rows streamed by decode, rows copied by the store): it keeps them
// from displacing reused lines and measured ~12% more streaming-read
// bandwidth than plain loads on MI355X.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store16_nt(void* p, const uint4& v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace pa
