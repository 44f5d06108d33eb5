// Gumbel-max sampler: token_b = argmax_i softmax(l_b / T_b)_i / E_i with
// exponential noise E_i (page "nano-vLLM 最小化vLLM重新实现", "辅助层": the
// sampler uses the Gumbel-max trick, exponential noise and an argmax; "关键设计
// 选择": temperatures above 1e-10, no greedy sampling).
//
// The noise is generated in the kernel (reading a [B, V] noise tensor would
// double the HBM traffic) with Philox4x64-10 (Salmon et al., "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): element i of row b takes a 21-bit
// field of word (i / 3) % 4 of the block at counter (i / 12, b, offset, 0),
// key (seed, 0) -- bits 63..43, 42..22 or 21..1 for i % 3 = 0, 1, 2 -- and
// u = (field + 1/2) / 2^21 (exact in fp32). Three fields per word: the
// generator's 64-bit multiplies, not the HBM stream, set this kernel's time,
// and 12 elements per block instead of 8 took a 256 x 151936 batch from
// about 56 to 48 us. In log2 units the decision is
//   argmax_i  l_i log2(e) / T - log2(-log2(u_i))
// (the row's softmax normaliser and a constant drop out), two v_log_f32 per
// element.
//
// Pass 1: a workgroup scans 12288 consecutive logits of one row (each thread
// one Philox block = 12 elements per round, three 16-byte loads where the
// row is 16-byte aligned, else single loads; 4 rounds),
// reduces (score, index) across the workgroup and writes one partial. Pass 2:
// one wave per row combines the row's partials. Ties go to the lowest index.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pa {

constexpr int kSmpThreads = 256;
constexpr int kSmpRounds = 4;
constexpr int kSmpPerBlock = 12;  // elements per Philox block: 3 fields of each 64-bit word
constexpr uint64_t kPhM0 = 0xD2E7470EE14C6C93ull, kPhM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhW0 = 0x9E3779B97F4A7C15ull, kPhW1 = 0xBB67AE8584CAA73Bull;

// Full 128-bit product of the constant M and x from four 32 x 32 + 64 multiply-
// adds (v_mad_u64_u32) whose partial products both halves share; no step can
// overflow 64 bits: (2^32-1)^2 + 2 (2^32-1) = 2^64 - 1.
template <uint64_t M>
__device__ __forceinline__ void mul128(uint64_t x, uint64_t& hi, uint64_t& lo) {
  constexpr uint32_t ml = (uint32_t)M, mh = (uint32_t)(M >> 32);
  const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
  const uint64_t p00 = (uint64_t)ml * xl;
  const uint64_t t = (uint64_t)ml * xh + (p00 >> 32);
  const uint64_t u = (uint64_t)mh * xl + (uint32_t)t;
  lo = (uint32_t)p00 | (u << 32);
  hi = (uint64_t)mh * xh + ((t >> 32) + (u >> 32));
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&x)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mul128<kPhM0>(x[0], hi0, lo0);
    mul128<kPhM1>(x[2], hi1, lo1);
    const uint64_t y0 = hi1 ^ x[1] ^ k0, y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0, x[1] = lo1, x[2] = y2, x[3] = lo0;
    k0 += kPhW0, k1 += kPhW1;
  }
}

// (score, index) order: higher score first, then the lower index.
__device__ __forceinline__ bool better(float s, int i, float bs, int bi) { return s > bs || (s == bs && i < bi); }

__device__ __forceinline__ void wave_argmax(float& s, int& i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float os = __shfl_xor(s, m);
    const int oi = __shfl_xor(i, m);
    if (better(os, oi, s, i)) s = os, i = oi;
  }
}

__global__ __launch_bounds__(kSmpThreads) void sample_partial_kernel(SampleArgs a) {
  const int row = blockIdx.y;
  const int chunk = blockIdx.x;
  const float t = fmaxf(a.temperatures[row], 1e-10f);
  const float c = 1.4426950408889634f / t;
  const float* lrow = a.logits + (int64_t)row * a.row_stride;
  const bool vec_rows = (reinterpret_cast<uintptr_t>(lrow) & 15) == 0;  // 16-byte loads possible
  float best = -INFINITY;
  int bidx = 0x7FFFFFFF;
#pragma unroll
  for (int r = 0; r < kSmpRounds; ++r) {
    const int64_t g = ((int64_t)chunk * kSmpRounds + r) * kSmpThreads + threadIdx.x;  // Philox block
    const int64_t e0 = g * kSmpPerBlock;
    if (e0 >= a.vocab) break;
    float l[kSmpPerBlock];
    if (vec_rows && e0 + kSmpPerBlock <= a.vocab) {
      typedef float f32x4_nt __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int h = 0; h < kSmpPerBlock / 4; ++h) {
        const f32x4_nt p = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(lrow + e0 + 4 * h));
        l[4 * h] = p.x, l[4 * h + 1] = p.y, l[4 * h + 2] = p.z, l[4 * h + 3] = p.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kSmpPerBlock; ++k) l[k] = e0 + k < a.vocab ? lrow[e0 + k] : -INFINITY;
    }
    uint64_t x[4] = {(uint64_t)g, (uint64_t)row, a.offset, 0};
    philox4x64_10(x, a.seed, 0);
#pragma unroll
    for (int k = 0; k < kSmpPerBlock; ++k) {
      const uint32_t field = (uint32_t)((x[k / 3] >> (43 - 21 * (k % 3))) & 0x1FFFFF);
      const float u = ((float)field + 0.5f) * 0x1p-21f;
      const float s = l[k] * c - __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
      const int i = (int)(e0 + k);
      if (i < a.vocab && s > best) best = s, bidx = i;  // elements come in increasing index
    }
  }
  wave_argmax(best, bidx);
  __shared__ float ss[kSmpThreads / 64];
  __shared__ int si[kSmpThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) ss[wave] = best, si[wave] = bidx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kSmpThreads / 64; ++w)
      if (better(ss[w], si[w], best, bidx)) best = ss[w], bidx = si[w];
    a.ws_score[(int64_t)row * a.chunks + chunk] = best;
    a.ws_index[(int64_t)row * a.chunks + chunk] = bidx;
  }
}

__global__ __launch_bounds__(64) void sample_final_kernel(SampleArgs a) {
  const int row = blockIdx.x;
  float best = -INFINITY;
  int bidx = 0x7FFFFFFF;
  for (int k = threadIdx.x; k < a.chunks; k += 64) {
    const float s = a.ws_score[(int64_t)row * a.chunks + k];
    const int i = a.ws_index[(int64_t)row * a.chunks + k];
    if (better(s, i, best, bidx)) best = s, bidx = i;
  }
  wave_argmax(best, bidx);
  // no candidate (e.g. NaN logits everywhere): token 0
  if (threadIdx.x == 0) a.tokens[row] = (bidx >= 0 && bidx < a.vocab) ? bidx : 0;
}

int32_t sample_chunks(int32_t vocab) {
  const int64_t per = (int64_t)kSmpThreads * kSmpRounds * kSmpPerBlock;
  return (int32_t)((vocab + per - 1) / per);
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  sample_partial_kernel<<<dim3((unsigned)a.chunks, (unsigned)a.num_rows), dim3(kSmpThreads), 0, stream>>>(a);
  sample_final_kernel<<<dim3((unsigned)a.num_rows), dim3(64), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
