// Varlen causal prefill attention with bf16 MFMA, over packed K/V or over the
// paged cache through a block table (prefix caching).
//
// What it computes: for sequence i with nq queries and nk keys (split by
// cu_seqlens_q / cu_seqlens_k), query j of head h attends with softmax weights
// scale * q.k to keys 0 .. nk - nq + j of kv head h / G (causal, queries
// aligned with the last keys), or to all nk keys (non-causal)
// (page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制": varlen prefill
// driven by cu_seqlens with an optional block_table for the prefix cache;
// page at bxzpzcl.cn/news/2159246, section 2.2.2: softmax(q kᵀ / sqrt(d)) v;
// page at hotelren.com/news/2273631, section 4.4: a cached prefix's KV is
// reused and only the remainder is computed).
//
// Design for gfx950:
// * One workgroup (4 waves) per (tile of 128/G query positions, kv head,
//   sequence): it covers all G query heads of the kv head, so every K/V tile
//   staged in LDS serves 128 query rows. Query tiles are issued longest first.
// * Each wave owns two 16-row subtiles (one head, 16 positions each).
// * Scores are computed transposed, Sᵀ = K Qᵀ, with v_mfma_f32_16x16x32_bf16:
//   K (row-major in LDS) is the A operand, Q (registers) the B operand. The
//   result leaves each lane with 4 keys of one query, so the row max/sum
//   need only a 2-step exchange across the 4 lanes of a query, and
//   exp2(s - m) lands in registers already in the layout of the B operand of
//   Oᵀ = Vᵀ Pᵀ (the key order inside a 32-key step is permuted consistently
//   on both operands). Vᵀ is written to LDS transposed, two keys per dword.
// * The next K/V tile is loaded into registers while the current one is
//   computed. Tiles that straddle the causal diagonal or the sequence end are
//   masked by selection (never by multiplication), so stale cache bits
//   cannot leak into the output; fully visible tiles skip the mask.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPD = 128;          // head_dim
constexpr int kBN = 64;           // keys per tile
constexpr int kPThreads = 256;
constexpr int kKStride = kPD + 8;  // bf16 elements per K row in LDS (pad: 16 B)
constexpr int kVStride = kBN + 8;  // bf16 elements per Vᵀ row in LDS (pad: 16 B)

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Address of key row t (already clamped to [0, nk)) of kv head kvh.
__device__ __forceinline__ const bf16_t* key_row(const bf16_t* base, int64_t token_stride, const PrefillArgs& a,
                                                 int seq, int k_beg, int t, int kvh) {
  if (a.block_table == nullptr) return base + (int64_t)(k_beg + t) * token_stride + kvh * kPD;
  const int blk = a.block_table[(int64_t)seq * a.max_blocks_per_seq + t / a.block_size];
  return base + ((int64_t)blk * a.block_size + t % a.block_size) * ((int64_t)a.num_kv_heads * kPD) + kvh * kPD;
}

template <int G>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[kBN * kKStride];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[kPD * kVStride];

  constexpr int QP = 128 / G;   // query positions per workgroup
  constexpr int PB = QP / 16;   // 16-position subtiles per head
  const int qtile = a.num_q_tiles - 1 - (int)blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int q_beg = a.cu_seqlens_q[seq];
  const int nq = a.cu_seqlens_q[seq + 1] - q_beg;
  const int k_beg = a.cu_seqlens_k[seq];
  const int nk = a.cu_seqlens_k[seq + 1] - k_beg;
  const int q0 = qtile * QP;
  if (q0 >= nq) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int shift = nk - nq;  // causal: query j sees keys <= shift + j

  // ---- this lane's two query rows ----
  int head[2], qpos[2], lim[2];
  uint4 qop[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int st = wave * 2 + u;
    head[u] = kvh * G + st / PB;
    qpos[u] = q0 + (st % PB) * 16 + col;
    lim[u] = a.causal ? shift + qpos[u] : nk - 1;
    const int qc = min(qpos[u], nq - 1);
    const bf16_t* qr = a.q + (int64_t)(q_beg + qc) * a.q_token_stride + (int64_t)head[u] * kPD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qop[u][ks] = load16(qr + ks * 32 + 8 * g);
  }

  // keys this workgroup needs, and the first key any of its queries cannot see
  const int q_last = min(q0 + QP, nq) - 1;
  const int k_end = a.causal ? min(nk, shift + q_last + 1) : nk;
  const int full_below = a.causal ? min(nk, shift + q0 + 1) : nk;  // keys < this are visible to every row
  const int ntiles = (k_end + kBN - 1) / kBN;

  f32x4_t oacc[2][8];
  float m[2], l[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    m[u] = kNegBig;
    l[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[u][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // staging assignments: K -> 4 x 16 B per thread; V -> key pair x 16 dims
  const int kv_key = tid >> 4, kv_c = tid & 15;  // K: keys kv_key + 16*u, chunk kv_c
  const int v_pair = tid & 31, v_dr = tid >> 5;   // V: keys 2*v_pair, 2*v_pair+1; dims 16*v_dr ..
  uint4 kreg[4], vreg[4];

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = min(t0 + kv_key + 16 * u, nk - 1);
      kreg[u] = load16(key_row(a.k, a.k_token_stride, a, seq, k_beg, t, kvh) + kv_c * 8);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = min(t0 + 2 * v_pair + u, nk - 1);
      const bf16_t* vr = key_row(a.v, a.v_token_stride, a, seq, k_beg, t, kvh) + v_dr * 16;
      vreg[2 * u] = load16(vr);
      vreg[2 * u + 1] = load16(vr + 8);
    }
  };

  const float c = a.scale_log2e;
  if (ntiles > 0) load_tile(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int t0 = tile * kBN;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(&sK[(kv_key + 16 * u) * kKStride + kv_c * 8]) = kreg[u];
    {
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);  // key 2p, dims 16*v_dr .. +16
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[2]);  // key 2p+1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(v1[e], v0[e], 0x05040100u);  // (v0.lo, v1.lo)
        const uint32_t hi = __builtin_amdgcn_perm(v1[e], v0[e], 0x07060302u);  // (v0.hi, v1.hi)
        *reinterpret_cast<uint32_t*>(&sVt[(v_dr * 16 + 2 * e) * kVStride + 2 * v_pair]) = lo;
        *reinterpret_cast<uint32_t*>(&sVt[(v_dr * 16 + 2 * e + 1) * kVStride + 2 * v_pair]) = hi;
      }
    }
    __syncthreads();
    if (tile + 1 < ntiles) load_tile(t0 + kBN);

    // ---- Sᵀ = K Qᵀ for both subtiles ----
    f32x4_t sacc[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[u][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 kop = *reinterpret_cast<const uint4*>(&sK[(kt * 16 + col) * kKStride + ks * 32 + 8 * g]);
        sacc[0][kt] = mfma16x16x32(kop, qop[0][ks], sacc[0][kt]);
        sacc[1][kt] = mfma16x16x32(kop, qop[1][ks], sacc[1][kt]);
      }
    }

    // ---- online softmax (each lane: one query, keys kt*16 + 4g + i) ----
    const bool need_mask = (t0 + kBN > full_below);
    uint4 pop[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float x[4][4];
      float mx = kNegBig;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[u][kt][i] * c;
          if (need_mask) {
            const int t = t0 + kt * 16 + 4 * g + i;
            v = (t <= lim[u] && t < nk) ? v : -INFINITY;
          }
          x[kt][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[u], mx);
      const float alpha = exp2f(m[u] - mnew);
      m[u] = mnew;
      float ps = 0.f;
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kt][i] = exp2f(x[kt][i] - mnew);
          ps += p[kt][i];
        }
      l[u] = l[u] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[u][dt] *= alpha;
      // B operand of Oᵀ = Vᵀ Pᵀ for 32-key step kk: slots 0..3 <- tile 2kk, slots 4..7 <- tile 2kk+1
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        pop[u][kk].x = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
        pop[u][kk].y = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
        pop[u][kk].z = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
        pop[u][kk].w = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
      }
    }

    // ---- Oᵀ += Vᵀ Pᵀ ----
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16_t* vrow = &sVt[(dt * 16 + col) * kVStride + kk * 32 + 4 * g];
        uint4 vop;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        vop.x = lo.x; vop.y = lo.y; vop.z = hi.x; vop.w = hi.y;
        oacc[0][dt] = mfma16x16x32(vop, pop[0][kk], oacc[0][dt]);
        oacc[1][dt] = mfma16x16x32(vop, pop[1][kk], oacc[1][dt]);
      }
    }
  }

  // ---- epilogue: normalise and write the rows that exist ----
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float ls = l[u];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (qpos[u] >= nq) continue;
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    bf16_t* orow = a.out + ((int64_t)(q_beg + qpos[u]) * a.num_q_heads + head[u]) * kPD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(oacc[u][dt][0] * inv, oacc[u][dt][1] * inv);
      w.y = pack_bf16x2(oacc[u][dt][2] * inv, oacc[u][dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * g) = w;
    }
  }
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t stream) {
  dim3 grid(a.num_q_tiles, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL(prefill_kernel<G>, grid, dim3(kPThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream) {
  if (a.num_seqs == 0 || a.num_q_tiles == 0) return hipSuccess;
  switch (group) {
    case 1: return launch_prefill_g<1>(a, stream);
    case 2: return launch_prefill_g<2>(a, stream);
    case 4: return launch_prefill_g<4>(a, stream);
    case 8: return launch_prefill_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
