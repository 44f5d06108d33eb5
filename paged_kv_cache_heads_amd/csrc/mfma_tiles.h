// MFMA operand helpers shared by the prefill and decode kernels (gfx950):
// the 16x16x32 bf16 matrix instruction, the XOR swizzles of the 256-byte K/V
// rows staged in LDS, the wave's vector-memory wait and the cross-row
// maxima of the 16x16 output layout.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef int v2i_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Byte offset of 16-byte chunk c of row r in a swizzled 64 x 256 B tile.
// K: chunk c ^ (r % 16) -- conflict-free for 16 rows reading one chunk.
// V: chunk c ^ 2 (r % 8) -- conflict-free for the transposed 8-byte reads.
__device__ __forceinline__ uint32_t k_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ uint32_t v_off(int r, int c) { return r * 256 + ((c ^ ((r & 7) << 1)) << 4); }

// Wait until at most N vector-memory instructions of this wave are
// outstanding (s_waitcnt vmcnt(N); expcnt and lgkmcnt left alone). Issued
// through the builtin so that the compiler's own wait bookkeeping sees it.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Maximum of x over lanes l and l ^ 16 (l ^ 32): the row-swap permutes put
// each lane's partner value in one of the two results.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes that hold
// one column of a 16x16 MFMA output).
__device__ __forceinline__ float sum_xor16_32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace pa
