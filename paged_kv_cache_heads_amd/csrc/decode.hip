// Paged GQA decode attention with a split-K (partition-and-reduce) pass.
//
// What it computes: for each sequence b and query head h, the softmax over the
// sequence's cached keys of scale * q.k, applied to the cached values
// (page at bxzpzcl.cn/news/2159246, section 2.2.2 "两级注意力加速", manual
// attention softmax(q kᵀ / sqrt(d)) v), where the keys and values of
// positions 0 .. context_len-1 are read through the sequence's block table
// from the paged cache [num_blocks, block_size, num_kv_heads, head_dim]
// (page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制": decode attention
// over the paged KV cache; section 3 "块管理器": fixed-size blocks).
//
// Design for gfx950 (HBM-bound, no MFMA):
// * One workgroup (4 waves) per (partition of `partition` tokens, kv head,
//   sequence). All G query heads of the kv head share each K/V row read.
// * A wave takes 64 tokens at a time. Lane (r = lane / 8, s = lane % 8) loads
//   16 bytes at d = 8s and 16 bytes at d = 64 + 8s of tokens i*8 + r
//   (i = 0..7), so each load instruction reads eight whole 128-byte lines.
// * q.k uses v_dot2_f32_bf16 on the raw bf16 pairs (fp32 accumulate); the
//   8 partial dots per token are combined with a DPP reduce-scatter, after
//   which lane (r, s) holds the score of token s*8 + r.
// * Online softmax state (max, sum) is kept per 8-lane group, so the only
//   per-chunk exchange is a 3-step DPP max; the group's p values are
//   broadcast with ds_bpermute for the p.v update.
// * Masked positions (past the context) are *selected* to -inf and their rows
//   are read from a clamped, valid address, so stale bits in the tail of the
//   last block can never reach the output.
// * A sequence that fits in one partition is normalised and written directly;
//   longer ones write fp32 partials (o, max, sum) that decode_reduce_kernel
//   combines: M = max_p m_p, o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pa {

constexpr int kD = 128;
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = 4;
constexpr int kChunk = 64;

template <int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(DecodeArgs a) {
  __shared__ float red_o[kDecodeWaves][G][kD];
  __shared__ float red_m[G][kDecodeWaves * 8];
  __shared__ float red_l[G][kDecodeWaves * 8];

  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = a.context_lens[b];
  const int start = part * a.partition;
  const int tid = threadIdx.x;
  if (start >= L) {
    if (L <= 0 && part == 0) {
      // Empty context: the output rows are zero.
      uint32_t* o = reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * a.num_q_heads + kvh * G) * kD);
      for (int i = tid; i < G * kD / 2; i += kDecodeThreads) o[i] = 0u;
    }
    return;
  }
  const int end = min(start + a.partition, L);
  const int wave = tid >> 6, lane = tid & 63, r = lane >> 3, s = lane & 7;
  const int64_t row = (int64_t)a.num_kv_heads * kD;
  const int bs = a.block_size;

  uint4 qlo[G], qhi[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const bf16_t* qp = a.q + (int64_t)b * a.q_seq_stride + (int64_t)(kvh * G + j) * kD;
    qlo[j] = load16(qp + 8 * s);
    qhi[j] = load16(qp + 64 + 8 * s);
  }

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegBig;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  }

  const float c = a.scale_log2e;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks_per_seq;

  for (int cb = start + wave * kChunk; cb < end; cb += kDecodeWaves * kChunk) {
    const int nvalid = end - cb;  // >= 1
    // block_size is a multiple of 64 and cb a multiple of 64: one block per chunk
    const int blk = table[cb / bs];
    const int64_t base = ((int64_t)blk * bs + (cb % bs)) * row + kvh * kD;
    const bf16_t* kb = a.k_cache + base;
    const bf16_t* vb = a.v_cache + base;
    uint4 kl[8], kh[8], vl[8], vh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(i * 8 + r, nvalid - 1);
      const int64_t off = (int64_t)t * row;
      kl[i] = load16(kb + off + 8 * s);
      kh[i] = load16(kb + off + 64 + 8 * s);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(i * 8 + r, nvalid - 1);
      const int64_t off = (int64_t)t * row;
      vl[i] = load16(vb + off + 8 * s);
      vh[i] = load16(vb + off + 64 + 8 * s);
    }

    const bool valid = (s * 8 + r) < nvalid;
    float pb[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float sc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float d = 0.f;
        d = dot2_bf16(qlo[j].x, kl[i].x, d);
        d = dot2_bf16(qlo[j].y, kl[i].y, d);
        d = dot2_bf16(qlo[j].z, kl[i].z, d);
        d = dot2_bf16(qlo[j].w, kl[i].w, d);
        d = dot2_bf16(qhi[j].x, kh[i].x, d);
        d = dot2_bf16(qhi[j].y, kh[i].y, d);
        d = dot2_bf16(qhi[j].z, kh[i].z, d);
        d = dot2_bf16(qhi[j].w, kh[i].w, d);
        sc[i] = d;
      }
      float x = group8_reduce_scatter(sc, s);  // score of token s*8 + r
      x = valid ? x * c : -INFINITY;
      const float mnew = fmaxf(m[j], group8_max(x));
      const float alpha = exp2f(m[j] - mnew);
      const float p = exp2f(x - mnew);
      l[j] = l[j] * alpha + p;
      m[j] = mnew;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[j][i] = __shfl(p, (lane & ~7) | i);
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float vv[16];
      vv[0] = bf16_lo(vl[i].x); vv[1] = bf16_hi(vl[i].x);
      vv[2] = bf16_lo(vl[i].y); vv[3] = bf16_hi(vl[i].y);
      vv[4] = bf16_lo(vl[i].z); vv[5] = bf16_hi(vl[i].z);
      vv[6] = bf16_lo(vl[i].w); vv[7] = bf16_hi(vl[i].w);
      vv[8] = bf16_lo(vh[i].x); vv[9] = bf16_hi(vh[i].x);
      vv[10] = bf16_lo(vh[i].y); vv[11] = bf16_hi(vh[i].y);
      vv[12] = bf16_lo(vh[i].z); vv[13] = bf16_hi(vh[i].z);
      vv[14] = bf16_lo(vh[i].w); vv[15] = bf16_hi(vh[i].w);
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = fmaf(pb[j][i], vv[e], acc[j][e]);
    }
  }

  // ---- merge the 32 groups (8 per wave x 4 waves) of this workgroup ----
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float lg = group8_sum(l[j]);
    if (s == 0) {
      red_m[j][wave * 8 + r] = m[j];
      red_l[j][wave * 8 + r] = lg;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < kDecodeWaves * 8; ++k) M = fmaxf(M, red_m[j][k]);
    const float f = exp2f(m[j] - M);
    float v16[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v16[e] = acc[j][e] * f;
    // reduce-scatter over r (lane bits 3, 4, 5)
    const bool h3 = lane & 8, h4 = lane & 16, h5 = lane & 32;
    float v8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float send = h3 ? v16[e] : v16[e + 8];
      const float keep = h3 ? v16[e + 8] : v16[e];
      v8[e] = keep + __shfl_xor(send, 8);
    }
    float v4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float send = h4 ? v8[e] : v8[e + 4];
      const float keep = h4 ? v8[e + 4] : v8[e];
      v4[e] = keep + __shfl_xor(send, 16);
    }
    float v2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float send = h5 ? v4[e] : v4[e + 2];
      const float keep = h5 ? v4[e + 2] : v4[e];
      v2[e] = keep + __shfl_xor(send, 32);
    }
    const int e0 = (h3 ? 8 : 0) + (h4 ? 4 : 0) + (h5 ? 2 : 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = e0 + k;
      const int d = e < 8 ? 8 * s + e : 64 + 8 * s + (e - 8);
      red_o[wave][j][d] = v2[k];
    }
  }
  __syncthreads();

  const int nparts = (L + a.partition - 1) / a.partition;
  for (int idx = tid; idx < G * kD / 2; idx += kDecodeThreads) {
    const int j = idx / (kD / 2);
    const int d = (idx % (kD / 2)) * 2;
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < kDecodeWaves * 8; ++k) M = fmaxf(M, red_m[j][k]);
    float Ls = 0.f;
#pragma unroll
    for (int k = 0; k < kDecodeWaves * 8; ++k) Ls += red_l[j][k] * exp2f(red_m[j][k] - M);
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      o0 += red_o[w][j][d];
      o1 += red_o[w][j][d + 1];
    }
    const int h = kvh * G + j;
    if (nparts == 1) {
      const float inv = 1.f / Ls;
      reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * a.num_q_heads + h) * kD)[d / 2] =
          pack_bf16x2(o0 * inv, o1 * inv);
    } else {
      const int64_t slot = ((int64_t)b * a.num_q_heads + h) * a.num_partitions + part;
      reinterpret_cast<float2*>(a.ws_o + slot * kD)[d / 2] = make_float2(o0, o1);
      if (d == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(M, Ls);
    }
  }
}

// One wave per (sequence, query head) with more than one partition.
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave;
  const int b = blockIdx.y;
  if (h >= a.num_q_heads) return;
  const int L = a.context_lens[b];
  const int np = (L + a.partition - 1) / a.partition;
  if (np <= 1) return;
  const int64_t slot0 = ((int64_t)b * a.num_q_heads + h) * a.num_partitions;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + slot0;
  const float* o = a.ws_o + slot0 * kD;
  float M = kNegBig;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[p].x);
  float Ls = 0.f, o0 = 0.f, o1 = 0.f;
  for (int p = 0; p < np; ++p) {
    const float2 st = ml[p];
    const float w = exp2f(st.x - M);
    Ls += w * st.y;
    const float2 ov = reinterpret_cast<const float2*>(o + (int64_t)p * kD)[lane];
    o0 += w * ov.x;
    o1 += w * ov.y;
  }
  const float inv = 1.f / Ls;
  reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * a.num_q_heads + h) * kD)[lane] = pack_bf16x2(o0 * inv, o1 * inv);
}

template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL(decode_partition_kernel<G>, grid, dim3(kDecodeThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions <= 1) return e;
  dim3 rgrid((a.num_q_heads + 3) / 4, a.num_seqs);
  hipLaunchKernelGGL(decode_reduce_kernel, rgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (group) {
    case 1: return launch_decode_g<1>(a, stream);
    case 2: return launch_decode_g<2>(a, stream);
    case 4: return launch_decode_g<4>(a, stream);
    case 8: return launch_decode_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
