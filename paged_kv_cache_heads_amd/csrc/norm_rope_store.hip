// Fused step before attention: RMSNorm of every query and key head (QK-norm),
// rotary embedding of q and k from a precomputed cos/sin table, and the KV
// store of the rotated K and the untouched V into the paged cache (page
// "nano-vLLM 最小化vLLM重新实现", section 6 "模型" and "辅助层" for QK-norm and
// RotaryEmbedding with its precomputed cos/sin cache; section 5 "注意力机制"
// for the store by slot_mapping).
//
// For head vector x (128 dims) of token t with weight w (q or k):
//   n = x / sqrt(mean(x^2) + eps) * w
//   y[i]      = n[i] cos[p, i] - n[i + 64] sin[p, i]        (i < 64)
//   y[i + 64] = n[i + 64] cos[p, i] + n[i] sin[p, i]
// with p = positions[t]; q heads go to q_out, k heads and the V heads (copied
// bit for bit) to slot slot_mapping[t] of the caches.
//
// The operation reads each head vector once and writes it once: HBM-bound.
// A 16-lane DPP row owns one head vector, 8 dims (16 bytes) per lane, so the
// sum of squares is a 4-step DPP reduction inside the row and the rotation
// partner of lane s (dims 8s ..) is lane s ^ 8 (row_ror:8): no LDS. Each lane
// keeps kItems head vectors' loads in flight before its first store; the 16
// rows of a workgroup take 16 consecutive head vectors per round, so a
// workgroup reads 4 KiB contiguous runs of the fused projection output.
#include "common.h"
#include "launch.h"

namespace pa {

constexpr int kNrThreads = 256;
constexpr int kNrRows = kNrThreads / 16;  // head vectors per round
constexpr int kNrItems = 4;               // rounds per workgroup

// Sum over the 16 lanes of a DPP row, result in every lane.
__device__ __forceinline__ float row16_sum(float x) {
  x = group8_sum(x);
  return x + dpp<kDppRor8>(x);
}

__global__ __launch_bounds__(kNrThreads) void norm_rope_store_kernel(NormRopeArgs a) {
  const int lane16 = threadIdx.x & 15;
  const int row = threadIdx.x >> 4;
  const uint32_t first = blockIdx.x * (uint32_t)(kNrRows * kNrItems) + row;

  // (token, head vector) of each round: one division, then steps of kNrRows
  int32_t tok[kNrItems], hvec[kNrItems];
  bool live[kNrItems];
  {
    uint32_t t = first / (uint32_t)a.num_heads;
    int32_t hv = (int32_t)(first - t * (uint32_t)a.num_heads);
#pragma unroll
    for (int r = 0; r < kNrItems; ++r) {
      tok[r] = (int32_t)t, hvec[r] = hv;
      live[r] = first + (uint32_t)(r * kNrRows) < a.num_items;
      hv += kNrRows;
      while (hv >= a.num_heads) hv -= a.num_heads, ++t;
    }
  }

  // ---- all loads of this lane's head vectors first ----
  uint4 x[kNrItems];
#pragma unroll
  for (int r = 0; r < kNrItems; ++r)
    if (live[r]) x[r] = load16_nt(a.qkv + (int64_t)tok[r] * a.qkv_token_stride + hvec[r] * 128 + lane16 * 8);

#pragma unroll
  for (int r = 0; r < kNrItems; ++r) {
    if (!live[r]) continue;
    const int64_t t = tok[r];
    const int hv = hvec[r];
    const int slot = a.slot_mapping[t];
    const bool store = slot >= 0 && slot < a.capacity;
    const int kv_row_elems = a.num_kv_heads * 128;
    if (hv >= a.num_q_heads + a.num_kv_heads) {  // V head: copy
      if (store)
        store16_nt(a.v_cache + (int64_t)slot * kv_row_elems + (hv - a.num_q_heads - a.num_kv_heads) * 128 +
                       lane16 * 8,
                   x[r]);
      continue;
    }
    const bool is_q = hv < a.num_q_heads;
    if (!is_q && !store) continue;

    float v[8];
    v[0] = bf16_lo(x[r].x), v[1] = bf16_hi(x[r].x), v[2] = bf16_lo(x[r].y), v[3] = bf16_hi(x[r].y);
    v[4] = bf16_lo(x[r].z), v[5] = bf16_hi(x[r].z), v[6] = bf16_lo(x[r].w), v[7] = bf16_hi(x[r].w);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    ss = row16_sum(ss);
    const float inv = rsqrtf(ss * (1.f / 128.f) + a.eps);

    const uint4 w = load16((is_q ? a.q_weight : a.k_weight) + lane16 * 8);
    float n[8];
    n[0] = v[0] * inv * bf16_lo(w.x), n[1] = v[1] * inv * bf16_hi(w.x);
    n[2] = v[2] * inv * bf16_lo(w.y), n[3] = v[3] * inv * bf16_hi(w.y);
    n[4] = v[4] * inv * bf16_lo(w.z), n[5] = v[5] * inv * bf16_hi(w.z);
    n[6] = v[6] * inv * bf16_lo(w.w), n[7] = v[7] * inv * bf16_hi(w.w);

    // rotation: lanes 0..7 hold the first half (dims 8s ..), lanes 8..15 the
    // second; both use angles 8 (s % 8) .. of the position's table row
    const int p = min(max(a.positions[t], 0), a.max_position - 1);
    const float* cs = a.cos_sin + (int64_t)p * 128 + (lane16 & 7) * 8;
    const float4 c0 = *reinterpret_cast<const float4*>(cs), c1 = *reinterpret_cast<const float4*>(cs + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(cs + 64), s1 = *reinterpret_cast<const float4*>(cs + 68);
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const float sign = lane16 < 8 ? -1.f : 1.f;  // y = n cos -/+ partner sin
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float partner = dpp<kDppRor8>(n[i]);
      y[i] = fmaf(n[i], cv[i], sign * partner * sv[i]);
    }
    uint4 o;
    o.x = pack_bf16x2(y[0], y[1]);
    o.y = pack_bf16x2(y[2], y[3]);
    o.z = pack_bf16x2(y[4], y[5]);
    o.w = pack_bf16x2(y[6], y[7]);
    if (is_q)
      *reinterpret_cast<uint4*>(a.q_out + t * a.q_out_token_stride + (int64_t)hv * 128 + lane16 * 8) = o;
    else
      store16_nt(a.k_cache + (int64_t)slot * kv_row_elems + (hv - a.num_q_heads) * 128 + lane16 * 8, o);
  }
}

hipError_t launch_norm_rope_store(const NormRopeArgs& a, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  const int64_t per_block = kNrRows * kNrItems;
  const int64_t blocks = (a.num_items + per_block - 1) / per_block;
  norm_rope_store_kernel<<<dim3((unsigned)blocks), dim3(kNrThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
