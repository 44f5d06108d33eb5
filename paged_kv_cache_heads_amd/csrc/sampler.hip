// Gumbel-max sampler: token_b = argmax_i softmax(l_b / T_b)_i / E_i with
// exponential noise E_i (page "nano-vLLM 最小化vLLM重新实现", "辅助层": the
// sampler uses the Gumbel-max trick, exponential noise and an argmax; "关键设计
// 选择": temperatures above 1e-10, no greedy sampling).
//
// The noise is generated in the kernel (reading a [B, V] noise tensor would
// double the HBM traffic) with Philox4x32-10 (Salmon et al., "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): element i of row b takes field i % 6
// of the block at counter (i / 6, b, offset lo, offset hi), key (seed lo,
// seed hi). The block's words w0..w3 form X0 = w1:w0 and X1 = w3:w2, and
// fields 0..2 (3..5) are bits 63..43, 42..22, 21..1 of X0 (X1); u = (field +
// 1/2) / 2^21 (exact in fp32). In log2 units the decision is
//   argmax_i  l_i log2(e) / T - log2(-log2(u_i))
// (the row's softmax normaliser and a constant drop out), two v_log_f32 per
// element.
//
// Cost: the kernel is bound by vector ALU work, not by HBM: per element it
// spends 1/6 of a Philox block (10 rounds of two 32 x 32 -> 64-bit multiplies
// and two three-input XORs, v_bitop3_b32), two v_log_f32 (quarter rate) and a
// handful of ordinary ops, about 16 VALU instructions against 4 bytes of
// logits. Loads are therefore issued all up front and coalesced, and the
// per-element work is trimmed: fields come out of the 32-bit words with one or
// two ops each, and the argmax takes one max3 and one compare per three
// elements.
//
// Pass 1: a workgroup scans 12288 consecutive logits of one row in 4 rounds;
// in a round each wave covers 768 consecutive logits and each lane scores 12
// consecutive elements (Philox blocks 2g and 2g + 1). Where the wave's 768
// logits are in range and the row is 16-byte aligned, the wave reads them as
// three fully coalesced 16-byte loads per lane and hands each lane its 12 through
// a wave-private 3 KiB LDS buffer; elsewhere (the row's ragged end) lanes read
// single elements with bounds checks. The workgroup reduces (score, index) and
// writes one partial; pass 2 (one wave per row) combines the row's partials.
// Ties go to the lowest index.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pa {

constexpr int kSmpThreads = 256;
constexpr int kSmpRounds = 4;
constexpr int kSmpPerThread = 12;                            // elements per lane per round: two Philox blocks
constexpr int kSmpWaveSpan = 64 * kSmpPerThread;             // 768 logits per wave per round
constexpr uint32_t kPhM0 = 0xD2511F53u, kPhM1 = 0xCD9E8D57u;
constexpr uint32_t kPhW0 = 0x9E3779B9u, kPhW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox4x32_10(uint32_t (&x)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kPhM0 * x[0];  // v_mad_u64_u32
    const uint64_t p1 = (uint64_t)kPhM1 * x[2];
    // a ^ b ^ c in one v_bitop3_b32 (truth table 0x96)
    const uint32_t y0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x[1], k0, 0x96);
    const uint32_t y2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x[3], k1, 0x96);
    x[0] = y0, x[1] = (uint32_t)p1, x[2] = y2, x[3] = (uint32_t)p0;
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

// Score of one field: l log2(e) / T - log2(-log2(u)), u = (field + 1/2) / 2^21.
__device__ __forceinline__ float field_score(float l, float c, uint32_t field) {
  const float u = __builtin_fmaf((float)field, 0x1p-21f, 0x1p-22f);  // exact: 22 significant bits
  return l * c - __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

// Scores s[0..11] of the 12 consecutive elements 12 g .. 12 g + 11 of a row
// (the fields of Philox blocks 2 g and 2 g + 1) with logits l[0..11].
__device__ __forceinline__ void score12(const SampleArgs& a, int row, uint32_t g, const float (&l)[kSmpPerThread],
                                        float c, float (&s)[kSmpPerThread]) {
  const uint32_t o0 = (uint32_t)a.offset, o1 = (uint32_t)(a.offset >> 32);
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  uint32_t x[2][4] = {{2 * g, (uint32_t)row, o0, o1}, {2 * g + 1, (uint32_t)row, o0, o1}};
  philox4x32_10(x[0], k0, k1);
  philox4x32_10(x[1], k0, k1);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // 64-bit value hi:lo = w(2h+1):w(2h); fields are its bits 63..43, 42..22, 21..1
      const uint32_t lo = x[b][2 * h], hi = x[b][2 * h + 1];
      const int k = 6 * b + 3 * h;
      s[k] = field_score(l[k], c, hi >> 11);
      s[k + 1] = field_score(l[k + 1], c, __builtin_amdgcn_alignbit(hi, lo, 22) & 0x1FFFFFu);
      s[k + 2] = field_score(l[k + 2], c, (lo >> 1) & 0x1FFFFFu);
    }
}

// Folds elements e, e + 1, e + 2 (scores s0..s2, in index order) into the
// running (best, bidx) under the strict "higher score, else lower index" rule:
// one max3 and one compare per three elements.
__device__ __forceinline__ void fold3(float s0, float s1, float s2, int e, float& best, int& bidx) {
  const float m = fmaxf(fmaxf(s0, s1), s2);
  if (m > best) best = m, bidx = e + (s0 == m ? 0 : (s1 == m ? 1 : 2));
}

__global__ __launch_bounds__(kSmpThreads) void sample_partial_kernel(SampleArgs a) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ f32x4 xpose[kSmpThreads / 64][kSmpWaveSpan / 4];  // one 3 KiB buffer per wave
  __shared__ float ss[kSmpThreads / 64];
  __shared__ int si[kSmpThreads / 64];
  const int row = blockIdx.y;
  const int chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float t = fmaxf(a.temperatures[row], 1e-10f);
  const float c = 1.4426950408889634f / t;
  const float* lrow = a.logits + (int64_t)row * a.row_stride;
  const bool vec_row = (reinterpret_cast<uintptr_t>(lrow) & 15) == 0;
  // lane group (12 elements) of round r: g0 + r * kSmpThreads; the wave's span starts at 12 (g0 - lane)
  const int64_t g0 = (int64_t)chunk * kSmpRounds * kSmpThreads + wave * 64 + lane;
  auto span_start = [&](int r) -> int64_t { return (g0 - lane + (int64_t)r * kSmpThreads) * kSmpPerThread; };
  // all coalesced loads first (wave-uniform conditions)
  f32x4 p[kSmpRounds][3];
#pragma unroll
  for (int r = 0; r < kSmpRounds; ++r) {
    const int64_t s0 = span_start(r);
    if (vec_row && s0 + kSmpWaveSpan <= a.vocab) {
#pragma unroll
      for (int h = 0; h < 3; ++h)
        p[r][h] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lrow + s0 + 4 * (64 * h + lane)));
    }
  }
  float best = -INFINITY;
  int bidx = 0x7FFFFFFF;
#pragma unroll
  for (int r = 0; r < kSmpRounds; ++r) {
    const int64_t s0 = span_start(r);
    if (s0 >= a.vocab) break;  // wave-uniform: this and later rounds are past the row's end
    const int64_t e0 = s0 + kSmpPerThread * lane;  // this lane's first element
    float l[kSmpPerThread];
    if (vec_row && s0 + kSmpWaveSpan <= a.vocab) {
      // lane j holds logits s0 + 4 (64 h + j) .. + 3; lane j needs s0 + 12 j .. + 11
#pragma unroll
      for (int h = 0; h < 3; ++h) xpose[wave][64 * h + lane] = p[r][h];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const f32x4 q = xpose[wave][3 * lane + h];
        l[4 * h] = q.x, l[4 * h + 1] = q.y, l[4 * h + 2] = q.z, l[4 * h + 3] = q.w;
      }
      // the next round's writes must not pass this round's reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      // ragged end (or a row that is not 16-byte aligned): out-of-range logits are -inf,
      // whose score never beats the running best
#pragma unroll
      for (int k = 0; k < kSmpPerThread; ++k) l[k] = e0 + k < a.vocab ? lrow[e0 + k] : -INFINITY;
    }
    float sc[kSmpPerThread];
    score12(a, row, (uint32_t)(g0 + r * kSmpThreads), l, c, sc);
#pragma unroll
    for (int k = 0; k < kSmpPerThread; k += 3) fold3(sc[k], sc[k + 1], sc[k + 2], (int)(e0 + k), best, bidx);
  }
  wave_argmax(best, bidx);
  if (lane == 0) ss[wave] = best, si[wave] = bidx;
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
  const int64_t per = (int64_t)kSmpThreads * kSmpRounds * kSmpPerThread;
  return (int32_t)((vocab + per - 1) / per);
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  sample_partial_kernel<<<dim3((unsigned)a.chunks, (unsigned)a.num_rows), dim3(kSmpThreads), 0, stream>>>(a);
  sample_final_kernel<<<dim3((unsigned)a.num_rows), dim3(64), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
