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
// Design for gfx950 (HBM-bound; vector arithmetic for 1 and 2 query heads per
// kv head, the matrix cores from 4 on, see decode_mfma_kernel):
// * Work is split stream-K style. The (sequence, kv head) pairs are laid end
//   to end as runs of chunks of 8*TPL tokens, and each of `num_waves`
//   one-wave workgroups takes an equal share of that chunk sequence, so all
//   waves finish together whatever the mix of context lengths. Every wave
//   derives its share from context_lens itself (a wave-wide scan); nothing is
//   read back to the host.
// * All G query heads of a kv head share each K/V row read. Lane
//   (r = lane / 8, s = lane % 8) loads 16 bytes at d = 8s and 16 bytes at
//   d = 64 + 8s of tokens i*8 + r (i < TPL): each load instruction reads eight
//   whole 128-byte lines. The next chunk (possibly of the next pair) is loaded
//   into a second register set while the current one is computed.
// * q.k uses v_dot2_f32_bf16 on the raw bf16 pairs (fp32 accumulate); the
//   per-lane partial dots are combined with a DPP reduce-scatter inside each
//   8-lane group.
// * Online-softmax state (max, sum) lives per 8-lane group, so the only
//   per-chunk exchange is a 3-step DPP max; p values reach the lanes that
//   hold the matching V rows with ds_bpermute. The accumulator rescale is
//   skipped when no group's maximum moved.
// * Masked positions (past the context) are *selected* to -inf and their rows
//   are read from a clamped, valid address, so stale bits in the tail of the
//   last block can never reach the output.
// * When a wave finishes a pair it merges its 8 groups with shuffles. A pair
//   that lies wholly inside one wave's share is normalised and written
//   directly. A pair cut by a share boundary leaves fp32 partials (o, max,
//   sum) in the wave's two workspace slots (slot 0: a piece that continues a
//   pair begun by an earlier wave; slot 1: a piece that starts a pair and
//   is continued by later waves); decode_finalize_kernel combines them:
//   M = max m_i, o = sum 2^(m_i - M) o_i / sum 2^(m_i - M) l_i.
#include <math.h>

#include <mutex>

#include "../../include/pa.h"
#include "common.h"
#include "launch.h"
#include "mfma_tiles.h"

namespace pa {

// Decode scratch for callers that cannot allocate (pa_store_decode_noalloc):
// room for the fp32 partials of the default split (2048 waves x 2 slots) at the
// largest group (8 query heads per kv head), 128 output values + (max, sum)
// per slot and head. Nothing in it has to start at zero: the finalize pass
// reads only the pieces this call's split kernel wrote. Each GPU the library
// runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

int decode_scratch(void** ptr) {
  // The array's name is a host-side stand-in; its device address is looked up
  // once per device, with that device current, and kept.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress of the decode scratch: %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return PA_OK;
}

constexpr int kD = 128;
// Sum of TPL values (tokens i*8 + r, i < TPL) over the 8 lanes of group r.
// On return every lane holds the group sum for token index s / (8 / TPL);
// the 8 / TPL lanes sharing that index hold the same value.
template <int TPL>
__device__ __forceinline__ float group8_reduce(const float (&v)[TPL], int s) {
  if constexpr (TPL == 4) {
    const bool b2 = s & 4, b1 = s & 2;
    float a[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float send = b2 ? v[m] : v[m + 2];
      const float keep = b2 ? v[m + 2] : v[m];
      a[m] = keep + dpp<kDppHalfMirror>(send);
    }
    float c = (b1 ? a[1] : a[0]) + dpp<kDppXor2>(b1 ? a[0] : a[1]);
    return c + dpp<kDppXor1>(c);
  } else {
    static_assert(TPL == 2, "2 or 4 tokens per lane");
    const bool b2 = s & 4;
    float c = (b2 ? v[1] : v[0]) + dpp<kDppHalfMirror>(b2 ? v[0] : v[1]);
    c += dpp<kDppXor2>(c);
    return c + dpp<kDppXor1>(c);
  }
}

template <int TPL>
struct ChunkRegs {
  uint4 k[TPL][2];
  uint4 v[TPL][2];
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Lengths of sequences i0 .. i0 + 3, clamped to n - 1 so every load is valid:
// the four loads are issued together and then pinned by an opaque use, so the
// compiler can neither sink each into its own branch nor wait for each alone.
__device__ __forceinline__ void load4_lens(const int32_t* lens, int i0, int n, int (&out)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) out[u] = lens[min(i0 + u, n - 1)];
  asm volatile("" : "+v"(out[0]), "+v"(out[1]), "+v"(out[2]), "+v"(out[3]));
}

struct Pos {
  int b, g, k;  // sequence, kv head, chunk within the pair (wave-uniform)
  int len, nc;  // context length and chunk count of sequence b
};

// Load the K and V rows of chunk p. Lane (r, s) reads tokens i*8 + r at byte
// lane_off = r * row_bytes + 16 * s from the chunk's first row (uniform
// base), so addresses are a scalar base plus a 32-bit lane offset. Only a
// chunk running past the context end clamps its rows (to the last token).
template <int TPL>
__device__ __forceinline__ void load_chunk(ChunkRegs<TPL>& c, const DecodeArgs& a, const Pos& p, uint32_t row_bytes,
                                           uint32_t lane_off, int r, int s) {
  constexpr int CH = 8 * TPL;
  const int bs = a.block_size;
  const int tok0 = p.k * CH;
  // block_size is a multiple of 64 and tok0 a multiple of the chunk: one block per chunk
  const int blk = a.block_tables[(int64_t)p.b * a.max_blocks_per_seq + tok0 / bs];
  const int64_t base = ((int64_t)blk * bs + tok0 % bs) * a.num_kv_heads * kD + p.g * kD;
  const char* kb = reinterpret_cast<const char*>(a.k_cache + base);
  const char* vb = reinterpret_cast<const char*>(a.v_cache + base);
  const int nvalid = p.len - tok0;
  if (a.k_new && p.k == p.nc - 1) {
    // Fused store (pa_store_decode): the sequence's new token, position L - 1,
    // is read from k_new / v_new row b (kv head g) instead of the cache, which
    // the finalize pass writes it to once this kernel is done. This chunk is
    // the only reader of that position, so no work waits on the store.
    const char* kn = reinterpret_cast<const char*>(a.k_new + p.b * a.k_new_stride + p.g * kD) + 16 * s;
    const char* vn = reinterpret_cast<const char*>(a.v_new + p.b * a.v_new_stride + p.g * kD) + 16 * s;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int tok = min(i * 8 + r, nvalid - 1);
      const uint32_t off = (uint32_t)tok * row_bytes + 16 * s;
      const char* kp = tok == nvalid - 1 ? kn : kb + off;
      c.k[i][0] = load16_nt(kp);
      c.k[i][1] = load16_nt(kp + 128);
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int tok = min(i * 8 + r, nvalid - 1);
      const uint32_t off = (uint32_t)tok * row_bytes + 16 * s;
      const char* vp = tok == nvalid - 1 ? vn : vb + off;
      c.v[i][0] = load16_nt(vp);
      c.v[i][1] = load16_nt(vp + 128);
    }
  } else if (nvalid >= CH) {
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t off = lane_off + i * 8 * row_bytes;
      c.k[i][0] = load16_nt(kb + off);
      c.k[i][1] = load16_nt(kb + off + 128);
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t off = lane_off + i * 8 * row_bytes;
      c.v[i][0] = load16_nt(vb + off);
      c.v[i][1] = load16_nt(vb + off + 128);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t off = (uint32_t)min(i * 8 + r, nvalid - 1) * row_bytes + 16 * s;
      c.k[i][0] = load16_nt(kb + off);
      c.k[i][1] = load16_nt(kb + off + 128);
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t off = (uint32_t)min(i * 8 + r, nvalid - 1) * row_bytes + 16 * s;
      c.v[i][0] = load16_nt(vb + off);
      c.v[i][1] = load16_nt(vb + off + 128);
    }
  }
}

template <int G>
struct DecodeState {
  float m[G], l[G], acc[G][16];
};

// The pair's query, dims 8s..8s+7 (lo) and 64+8s..64+8s+7 (hi) of each of the
// G heads for the lane's s.
template <int G>
struct QRegs {
  uint4 lo[G], hi[G];
  __device__ __forceinline__ uint4 get_lo(int j) const { return lo[j]; }
  __device__ __forceinline__ uint4 get_hi(int j) const { return hi[j]; }
};

template <int G, int TPL>
__device__ __forceinline__ void compute_chunk(DecodeState<G>& st, const QRegs<G>& q, const ChunkRegs<TPL>& c,
                                              int nvalid, float scale_log2e, int lane, int r, int s) {
  constexpr int kDup = 8 / TPL;  // lanes holding each token's score
  const bool valid = ((s / kDup) * 8 + r) < nvalid;
  float pb[G][TPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float sc[TPL];
    const uint4 qlo = q.get_lo(j), qhi = q.get_hi(j);
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      float d = 0.f;
      d = dot2_bf16(qlo.x, c.k[i][0].x, d);
      d = dot2_bf16(qlo.y, c.k[i][0].y, d);
      d = dot2_bf16(qlo.z, c.k[i][0].z, d);
      d = dot2_bf16(qlo.w, c.k[i][0].w, d);
      d = dot2_bf16(qhi.x, c.k[i][1].x, d);
      d = dot2_bf16(qhi.y, c.k[i][1].y, d);
      d = dot2_bf16(qhi.z, c.k[i][1].z, d);
      d = dot2_bf16(qhi.w, c.k[i][1].w, d);
      sc[i] = d;
    }
    float x = group8_reduce<TPL>(sc, s);  // score of token (s / kDup) * 8 + r
    x = valid ? x * scale_log2e : -INFINITY;
    const float mnew = fmaxf(st.m[j], group8_max(x));
    const float p = fast_exp2(x - mnew);
    if (__ballot(mnew != st.m[j])) {
      const float alpha = fast_exp2(st.m[j] - mnew);
      st.l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[j][e] *= alpha;
    }
    st.m[j] = mnew;
    st.l[j] += (s % kDup) ? 0.f : p;  // count each token once
#pragma unroll
    for (int i = 0; i < TPL; ++i) pb[j][i] = __shfl(p, (lane & ~7) | (kDup * i));
  }
#pragma unroll
  for (int i = 0; i < TPL; ++i) {
    float vv[16];
    vv[0] = bf16_lo(c.v[i][0].x); vv[1] = bf16_hi(c.v[i][0].x);
    vv[2] = bf16_lo(c.v[i][0].y); vv[3] = bf16_hi(c.v[i][0].y);
    vv[4] = bf16_lo(c.v[i][0].z); vv[5] = bf16_hi(c.v[i][0].z);
    vv[6] = bf16_lo(c.v[i][0].w); vv[7] = bf16_hi(c.v[i][0].w);
    vv[8] = bf16_lo(c.v[i][1].x); vv[9] = bf16_hi(c.v[i][1].x);
    vv[10] = bf16_lo(c.v[i][1].y); vv[11] = bf16_hi(c.v[i][1].y);
    vv[12] = bf16_lo(c.v[i][1].z); vv[13] = bf16_hi(c.v[i][1].z);
    vv[14] = bf16_lo(c.v[i][1].w); vv[15] = bf16_hi(c.v[i][1].w);
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[j][e] = fmaf(pb[j][i], vv[e], st.acc[j][e]);
  }
}

// Sequences the call covers: num_seqs, or fewer when a device count is given
// (a graph captured at a padded batch size, replayed for a smaller batch:
// sequences at or past the count are empty contexts and their rows are never
// read, except for their lengths, which are masked).
__device__ __forceinline__ int live_seqs(const DecodeArgs& a) {
  return a.live_seqs ? max(0, min(a.num_seqs, *a.live_seqs)) : a.num_seqs;
}

// ---- wave-wide helpers for the work split ----
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan_i32(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int chunks_of(int len, int ch) { return len > 0 ? (len + ch - 1) / ch : 0; }

// First chunk index of wave w's share: floor(w * C / NW).
__device__ __forceinline__ int64_t share_begin(int64_t w, int64_t total, int64_t nw) { return w * total / nw; }

// The wave whose share holds chunk c: the largest w with share_begin(w) <= c.
__device__ __forceinline__ int64_t wave_of_chunk(int64_t c, int64_t total, int64_t nw) {
  return ((c + 1) * nw + total - 1) / total - 1;
}

template <int G>
__device__ __forceinline__ void load_q(QRegs<G>& q, const DecodeArgs& a, int b, int g, int s) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const bf16_t* qp = a.q + (int64_t)b * a.q_seq_stride + (int64_t)(g * G + j) * kD;
    q.lo[j] = load16(qp + 8 * s);
    q.hi[j] = load16(qp + 64 + 8 * s);
  }
}

// Next chunk in (sequence, kv head, chunk) order; skips empty sequences.
__device__ __forceinline__ Pos next_pos(const Pos& p, const DecodeArgs& a, int ch, int ns) {
  if (p.k + 1 < p.nc) return Pos{p.b, p.g, p.k + 1, p.len, p.nc};
  if (p.g + 1 < a.num_kv_heads) return Pos{p.b, p.g + 1, 0, p.len, p.nc};
  Pos n{p.b + 1, 0, 0, 0, 0};
  for (; n.b < ns; ++n.b) {
    n.len = uniform(a.context_lens[n.b]);
    n.nc = chunks_of(n.len, ch);
    if (n.nc > 0) break;
  }
  return n;
}

template <int G>
__device__ __forceinline__ void reset_state(DecodeState<G>& st) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = kNegBig;
    st.l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = 0.f;
  }
}

// Merge the wave's 8 groups for the piece of pair (p.b, p.g) that ends at
// chunk p.k, and write it: final output if the piece is the whole pair, else
// a partial into the wave's slot.
template <int G>
__device__ __forceinline__ void finish_piece(const DecodeState<G>& st, const DecodeArgs& a, const Pos& p, int k0,
                                             int wave, int lane, int s) {
  const bool whole = (k0 == 0) && (p.k == p.nc - 1);
  const int64_t slot = (int64_t)wave * 2 + (k0 > 0 ? 0 : 1);
  const bool h3 = lane & 8, h4 = lane & 16, h5 = lane & 32;
  const int e0 = (h3 ? 8 : 0) + (h4 ? 4 : 0) + (h5 ? 2 : 0);
  const int d = e0 < 8 ? 8 * s + e0 : 64 + 8 * s + (e0 - 8);  // this lane's output pair: d, d + 1
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float M = st.m[j];
    M = fmaxf(M, dpp<kDppRor8>(M));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = fast_exp2(st.m[j] - M);
    float Ls = group8_sum(st.l[j]) * f;
    Ls += dpp<kDppRor8>(Ls);
    Ls += __shfl_xor(Ls, 16);
    Ls += __shfl_xor(Ls, 32);
    float v8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float send = (h3 ? st.acc[j][e] : st.acc[j][e + 8]) * f;
      const float keep = (h3 ? st.acc[j][e + 8] : st.acc[j][e]) * f;
      v8[e] = keep + dpp<kDppRor8>(send);
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
    if (whole) {
      const float inv = 1.f / Ls;
      const int h = p.g * G + j;
      reinterpret_cast<uint32_t*>(a.out + ((int64_t)p.b * a.num_q_heads + h) * kD)[d / 2] =
          pack_bf16x2(v2[0] * inv, v2[1] * inv);
    } else {
      reinterpret_cast<float2*>(a.ws_o + (slot * G + j) * kD)[d / 2] = make_float2(v2[0], v2[1]);
      if (lane == 0) reinterpret_cast<float2*>(a.ws_ml)[slot * G + j] = make_float2(M, Ls);
    }
  }
}

// Wave `wave`'s share [lo, hi) of the chunk sequence (chunks of ch tokens, in
// (sequence, kv head, chunk) order over the ns live sequences) and the
// position of its first chunk. False when the share is empty.
__device__ __forceinline__ bool locate_share(const DecodeArgs& a, int ch, int wave, int lane, int& ns, int64_t& lo,
                                             int64_t& hi, Pos& cur) {
  const int64_t nw = a.num_waves;
  // the first 256 lengths are loaded once and serve both scans below
  int lu0[4];
  load4_lens(a.context_lens, lane * 4, a.num_seqs, lu0);
  ns = live_seqs(a);
  int64_t total = 0;
  for (int base = 0; base < ns; base += 256) {
    int x = 0, lu[4];
    if (base == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) lu[u] = lu0[u];
    } else {
      load4_lens(a.context_lens, base + lane * 4, a.num_seqs, lu);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) x += base + lane * 4 + u < ns ? chunks_of(lu[u], ch) : 0;
    total += uniform(wave_sum_i32(x));
  }
  total *= a.num_kv_heads;
  lo = share_begin(wave, total, nw);
  hi = share_begin(wave + 1, total, nw);
  if (lo >= hi) return false;

  // locate chunk `lo`: the sequence b with kvh*prefix(b) <= lo < kvh*prefix(b+1)
  cur = Pos{0, 0, 0, 0, 0};
  {
    int64_t run = 0;
    for (int base = 0; base < ns; base += 256) {
      int len[4], x[4], sum = 0, lu[4];
      if (base == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) lu[u] = lu0[u];
      } else {
        load4_lens(a.context_lens, base + lane * 4, a.num_seqs, lu);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = base + lane * 4 + u;
        len[u] = b < ns ? lu[u] : 0;
        x[u] = chunks_of(len[u], ch) * a.num_kv_heads;
        sum += x[u];
      }
      const int incl = wave_inclusive_scan_i32(sum, lane);
      const int64_t lane_beg = run + incl - sum;
      const uint64_t hit = __ballot(sum > 0 && lane_beg <= lo && lo < run + incl);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        // walk the 4 sequences of lane src
        int64_t beg = uniform(__shfl((int)(lane_beg - run), src)) + run;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int xu = uniform(__shfl(x[u], src));
          if (xu > 0 && lo < beg + xu && cur.nc == 0) {
            cur.b = base + src * 4 + u;
            cur.len = uniform(__shfl(len[u], src));
            cur.nc = chunks_of(cur.len, ch);
            const int64_t rel = lo - beg;
            cur.g = (int)(rel / cur.nc);
            cur.k = (int)(rel % cur.nc);
          }
          beg += xu;
        }
        break;
      }
      run += uniform(__shfl(incl, 63));
    }
  }

  return true;
}

template <int G, int TPL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_split_kernel(DecodeArgs a) {
  constexpr int CH = 8 * TPL;  // tokens per chunk
  const int wave = blockIdx.x, lane = threadIdx.x;
  const int r = lane >> 3, s = lane & 7;
  int ns;
  int64_t lo, hi;
  Pos cur;
  if (!locate_share(a, CH, wave, lane, ns, lo, hi, cur)) return;

  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * kD * 2;
  const uint32_t lane_off = r * row_bytes + 16 * s;
  ChunkRegs<TPL> c0, c1;
  QRegs<G> q;
  DecodeState<G> st;
  load_chunk(c0, a, cur, row_bytes, lane_off, r, s);
  load_q(q, a, cur.b, cur.g, s);
  reset_state(st);
  int k0 = cur.k;  // first chunk of the current piece
  const float sc = a.scale_log2e;

  // Two stages with the register sets swapped (no copies between them). The
  // query of a new pair is loaded when its first chunk is reached (about once
  // per wave), which keeps the wave within two waves per SIMD of registers.
  for (int64_t c = lo;;) {
    {
      const bool more = c + 1 < hi;
      Pos nxt = cur;
      bool new_pair = false;
      if (more) {
        nxt = next_pos(cur, a, CH, ns);
        new_pair = nxt.b != cur.b || nxt.g != cur.g;
        load_chunk(c1, a, nxt, row_bytes, lane_off, r, s);
      }
      compute_chunk<G, TPL>(st, q, c0, cur.len - cur.k * CH, sc, lane, r, s);
      if (!more || new_pair) {
        finish_piece<G>(st, a, cur, k0, wave, lane, s);
        if (!more) break;
        reset_state(st);
        k0 = 0;
        load_q(q, a, nxt.b, nxt.g, s);
      }
      cur = nxt;
      ++c;
    }
    {
      const bool more = c + 1 < hi;
      Pos nxt = cur;
      bool new_pair = false;
      if (more) {
        nxt = next_pos(cur, a, CH, ns);
        new_pair = nxt.b != cur.b || nxt.g != cur.g;
        load_chunk(c0, a, nxt, row_bytes, lane_off, r, s);
      }
      compute_chunk<G, TPL>(st, q, c1, cur.len - cur.k * CH, sc, lane, r, s);
      if (!more || new_pair) {
        finish_piece<G>(st, a, cur, k0, wave, lane, s);
        if (!more) break;
        reset_state(st);
        k0 = 0;
        load_q(q, a, nxt.b, nxt.g, s);
      }
      cur = nxt;
      ++c;
    }
  }
}

// ---- the split pass on the matrix cores -------------------------------------
//
// With G query heads per kv head the decode is a small dense contraction: G
// query rows against every key of the pair. The kernel above does it with
// vector dot products, whose cost grows with G; from G = 4 on, this kernel
// runs the same stream-K split (32-token chunks) on the MFMA units instead,
// with the G queries as the columns of 16x16x32 bf16 tiles (columns G..15
// are zero and ignored):
// * Each chunk's K and V rows are loaded as whole 128-byte lines (8 rows of
//   a 16-byte piece per lane and instruction) into a register set while the
//   previous chunk is computed; reading K straight into the MFMA operand
//   layout (16 rows x 64 bytes per instruction) measured 10% slower.
// * The chunk is then written to a wave-private LDS tile (swizzled like the
//   prefill's) and read back as operands: K rows for Sᵀ = K Qᵀ (Qᵀ held in
//   registers), V transposed with ds_read_b64_tr_b16 for Oᵀ += Vᵀ Pᵀ.
// * Online softmax in log2 units per query column, rescaled lazily (when a
//   column's maximum grows by more than 2^8), p in fp32; P is split into
//   bf16 high and low parts (p = hi + lo to 2^-16) and both are multiplied,
//   so the weights keep close to fp32 precision; the row sums are the fp32
//   sums of p.
// Pieces go to the same workspace slots, in the same (max, sum, output)
// format, and the same finalize pass combines them.
template <int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int CH = 32;  // tokens per chunk
  static_assert(G <= 16, "the queries of a kv head are the columns of one 16-column tile");
  // the chunk being computed, re-laid out for the operand reads (wave-private)
  __shared__ __attribute__((aligned(1024))) char ksh[CH * 256];
  __shared__ __attribute__((aligned(1024))) char vsh[CH * 256];
  const int wave = blockIdx.x, lane = threadIdx.x;
  const int g = lane >> 4, col = lane & 15;  // MFMA operand lanes
  const int r8 = lane >> 3, s8 = lane & 7;   // load lanes: row r8 + 8 q % 4 of the chunk, 16-byte piece s8
  int ns;
  int64_t lo, hi;
  Pos cur;
  if (!locate_share(a, CH, wave, lane, ns, lo, hi, cur)) return;

  const int64_t row_elems = (int64_t)a.num_kv_heads * kD;  // elements between tokens' rows in the cache
  // K operand reads: lane (g, col) takes key col of a 16-key tile, dims 32 ks + 8 g .. + 7
  uint32_t koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = k_off(col, ks * 4 + g);
  // Vᵀ operand reads: dims 16 dt + col of keys 4 g .. 4 g + 3 (low half) and 16 + 4 g .. (high)
  uint32_t voff[8];
  {
    const int trow = 4 * g + (col >> 2), tq = col & 3;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) voff[dt] = v_off(trow, 2 * dt + (tq >> 1)) + (tq & 1) * 8;
  }

  // Loads of chunk p into registers, whole 128-byte lines per instruction:
  // load q (< 8) takes row r8 + 8 (q % 4), 16-byte piece 8 (q / 4) + s8. Rows
  // past the context end are read from the last token (their scores are
  // masked; their V rows must be finite); the new token (pa_store_decode)
  // comes from k_new / v_new.
  struct ChunkKV {
    uint4 k[8], v[8];
  };
  auto issue = [&](const Pos& p, ChunkKV& c) {
    const int tok0 = p.k * CH;
    const int nvalid = min(CH, p.len - tok0);
    const int blk = a.block_tables[(int64_t)p.b * a.max_blocks_per_seq + tok0 / a.block_size];
    const int64_t base = ((int64_t)blk * a.block_size + tok0 % a.block_size) * row_elems + (int64_t)p.g * kD;
    const bool has_new = a.k_new != nullptr;
    const int new_row = p.len - 1 - tok0;  // row of the new token in this chunk (if < CH)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = min(r8 + 8 * (q & 3), nvalid - 1);
      const int e = 64 * (q >> 2) + 8 * s8;
      const bool is_new = has_new && row == new_row;
      c.k[q] = load16_nt((is_new ? a.k_new + p.b * a.k_new_stride + p.g * kD : a.k_cache + base + row * row_elems) + e);
      c.v[q] = load16_nt((is_new ? a.v_new + p.b * a.v_new_stride + p.g * kD : a.v_cache + base + row * row_elems) + e);
    }
  };

  // Qᵀ operand of the pair: query column col (< G), dims 32 ks + 8 g .. + 7
  uint4 qop[4];
  auto load_qop = [&](const Pos& p) {
    const bf16_t* qr = a.q + (int64_t)p.b * a.q_seq_stride + (int64_t)(p.g * G + min(col, G - 1)) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = load16(qr + 32 * ks + 8 * g);
      qop[ks] = col < G ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  f32x4_t oacc[8];
  float m, lsum;
  bool fresh;
  auto reset = [&]() {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = kNegBig;
    lsum = 0.f;
    fresh = true;
  };
  const float c = a.scale_log2e;
  constexpr float tau = 8.f;  // lazy-rescale threshold, log2 units

  // One chunk: stage it in LDS, scores, softmax, Vᵀ Pᵀ.
  auto compute = [&](const Pos& p, const ChunkKV& kv) {
    const int nvalid = min(CH, p.len - p.k * CH);
    // Every read of the previous chunk precedes these writes in the wave's
    // program order and LDS operations of one wave complete in order; the
    // fences keep the compiler from moving accesses across.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = r8 + 8 * (q & 3), piece = 8 * (q >> 2) + s8;
      *reinterpret_cast<uint4*>(ksh + k_off(row, piece)) = kv.k[q];
      *reinterpret_cast<uint4*>(vsh + v_off(row, piece)) = kv.v[q];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        sacc[t] = mfma16x16x32(*reinterpret_cast<const uint4*>(ksh + t * 16 * 256 + koff[ks]), qop[ks], sacc[t]);
    // lane (g, col): query col, keys 16 t + 4 g + i
    float x[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[t][i] = sacc[t][i] * c;
    if (nvalid < CH) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[t][i] = 16 * t + 4 * g + i < nvalid ? x[t][i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    mx = max_xor32(max_xor16(mx));
    if (__ballot(mx > m + tau)) {
      const float mnew = fmaxf(m, mx);
      if (!fresh) {
        const float alpha = fast_exp2(m - mnew);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
        lsum *= alpha;
      }
      m = mnew;
    }
    fresh = false;
    float pv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[t][i] = fast_exp2(x[t][i] - m);
        lsum += pv[t][i];
      }
    // Pᵀ operand (lane (g, col): query col, keys 4 g .. 4 g + 3 of each 16-key
    // tile), high and low bf16 parts
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const uint32_t h = pack_bf16x2(pv[t][i], pv[t][i + 1]);
        ph[2 * t + i / 2] = h;
        pl[2 * t + i / 2] = pack_bf16x2(pv[t][i] - bf16_lo(h), pv[t][i + 1] - bf16_hi(h));
      }
    const uint4 poph = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    const uint4 popl = make_uint4(pl[0], pl[1], pl[2], pl[3]);
    typedef __attribute__((address_space(3))) const char lds_char_t;
    lds_char_t* vl = (lds_char_t*)vsh;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const s16x4_t l4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vl + voff[dt]));
      const s16x4_t h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vl + 16 * 256 + voff[dt]));
      const v2i_t l2 = __builtin_bit_cast(v2i_t, l4), h2 = __builtin_bit_cast(v2i_t, h4);
      const uint4 vop = make_uint4(l2.x, l2.y, h2.x, h2.y);
      oacc[dt] = mfma16x16x32(vop, poph, oacc[dt]);
      oacc[dt] = mfma16x16x32(vop, popl, oacc[dt]);
    }
  };

  // The pair's piece ends: a whole pair goes to the output, a cut one to its
  // slot (slot 1 of the wave for the piece that starts the pair's cut, slot 0
  // for the piece at the wave's start).
  auto finish = [&](const Pos& p, int k0) {
    const float ls = sum_xor16_32(lsum);
    const bool whole = (k0 == 0) && (p.k == p.nc - 1);
    const int64_t slot = (int64_t)wave * 2 + (k0 > 0 ? 0 : 1);
    if (col < G) {
      if (whole) {
        const float inv = 1.f / ls;
        uint16_t* o = a.out + ((int64_t)p.b * a.num_q_heads + p.g * G + col) * kD + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<uint2*>(o + 16 * dt) =
              make_uint2(pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv), pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv));
      } else {
        float* o = a.ws_o + (slot * G + col) * kD + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<float4*>(o + 16 * dt) = make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
        if (g == 0) reinterpret_cast<float2*>(a.ws_ml)[slot * G + col] = make_float2(m, ls);
      }
    }
  };

  ChunkKV cA, cB;
  issue(cur, cA);
  load_qop(cur);
  reset();
  int k0 = cur.k;  // first chunk of the current piece
  // two stages with the register sets swapped: the next chunk's loads are in
  // flight while the current one is computed
  for (int64_t ci = lo;;) {
    {
      const bool more = ci + 1 < hi;
      Pos nxt = cur;
      bool new_pair = false;
      if (more) {
        nxt = next_pos(cur, a, CH, ns);
        new_pair = nxt.b != cur.b || nxt.g != cur.g;
        issue(nxt, cB);
      }
      compute(cur, cA);
      if (!more || new_pair) {
        finish(cur, k0);
        if (!more) break;
        reset();
        k0 = 0;
        load_qop(nxt);
      }
      cur = nxt;
      ++ci;
    }
    {
      const bool more = ci + 1 < hi;
      Pos nxt = cur;
      bool new_pair = false;
      if (more) {
        nxt = next_pos(cur, a, CH, ns);
        new_pair = nxt.b != cur.b || nxt.g != cur.g;
        issue(nxt, cA);
      }
      compute(cur, cB);
      if (!more || new_pair) {
        finish(cur, k0);
        if (!more) break;
        reset();
        k0 = 0;
        load_qop(nxt);
      }
      cur = nxt;
      ++ci;
    }
  }
}

// Adds pieces i0 .. i0 + P - 1 (those below n) of the current batch to the
// running output: lane l of the batch holds piece l's slot and weights f.
// Piece indexes past n are clamped to n - 1 (a valid slot) and get weight 0.
template <int G, int P>
__device__ __forceinline__ void add_pieces(const DecodeArgs& a, int64_t slot, const float (&f)[G], int i0, int n,
                                           int lane, float (&o0)[G], float (&o1)[G]) {
  float2 ov[P][G];
  float fq[P][G];
#pragma unroll
  for (int q = 0; q < P; ++q) {
    const int i = min(i0 + q, n - 1);
    const int64_t si = __shfl(slot, i);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      fq[q][j] = i0 + q < n ? __shfl(f[j], i) : 0.f;
      ov[q][j] = reinterpret_cast<const float2*>(a.ws_o + (si * G + j) * kD)[lane];
    }
  }
#pragma unroll
  for (int q = 0; q < P; ++q)
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (fq[q][j] != 0.f) {
        o0[j] += fq[q][j] * ov[q][j].x;
        o1[j] += fq[q][j] * ov[q][j].y;
      }
    }
}

// One wave per (sequence, kv head): zero rows for an empty context, and for
// a pair cut by share boundaries, combine the pieces its waves left in their
// slots (slot 1 of the first wave, slot 0 of every later non-empty wave).
template <int G, int TPL>
__global__ __launch_bounds__(64) void decode_finalize_kernel(DecodeArgs a) {
  constexpr int CH = 8 * TPL;
  const int b = blockIdx.x / a.num_kv_heads, g = blockIdx.x % a.num_kv_heads, lane = threadIdx.x;
  // One pass over the lengths (one round of loads): the chunks of sequence b,
  // of the sequences before it, and of all sequences, per kv head.
  int64_t before = 0, all = 0;
  int nc = 0;
  const int ns = live_seqs(a);  // rows at or past it are empty: zero output, nothing stored
  for (int base = 0; base < ns; base += 256) {
    int xb = 0, xa = 0, xm = 0, lu[4];
    load4_lens(a.context_lens, base + lane * 4, a.num_seqs, lu);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sq = base + lane * 4 + u;  // lanes past the end count 0
      const int c = sq < ns ? chunks_of(lu[u], CH) : 0;
      xa += c;
      xb += sq < b ? c : 0;
      xm += sq == b ? c : 0;
    }
    all += uniform(wave_sum_i32(xa));
    before += uniform(wave_sum_i32(xb));
    nc += uniform(wave_sum_i32(xm));
  }
  if (nc == 0) {
    uint32_t* o = reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * a.num_q_heads + g * G) * kD);
    for (int i = lane; i < G * kD / 2; i += 64) o[i] = 0u;
    return;
  }
  if (a.k_new && lane < 32) {
    // fused store (pa_store_decode): the new token's K and V rows of kv head g go
    // to position L - 1 (the split kernel read them from k_new / v_new); lanes
    // 0-15 move 16 B of the K row each, lanes 16-31 of the V row
    const int len = a.context_lens[b];
    const int pos = len - 1;
    const int blk = a.block_tables[(int64_t)b * a.max_blocks_per_seq + pos / a.block_size];
    const int64_t row = ((int64_t)blk * a.block_size + pos % a.block_size) * a.num_kv_heads * kD + g * kD;
    const bool is_v = lane >= 16;
    const int d = (lane & 15) * 8;
    const uint16_t* src = (is_v ? a.v_new + b * a.v_new_stride : a.k_new + b * a.k_new_stride) + g * kD + d;
    uint16_t* dst = const_cast<uint16_t*>(is_v ? a.v_cache : a.k_cache) + row + d;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  const int64_t nw = a.num_waves;
  const int64_t total = all * a.num_kv_heads;
  const int64_t first = before * a.num_kv_heads + (int64_t)g * nc;
  const int64_t w1 = wave_of_chunk(first, total, nw), w2 = wave_of_chunk(first + nc - 1, total, nw);
  if (w1 == w2) return;  // written whole by its wave
  float M[G], Ls[G], o0[G], o1[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    M[j] = kNegBig;
    Ls[j] = 0.f;
    o0[j] = o1[j] = 0.f;
  }
  // pieces in batches of 64, one lane per piece; online rescale across batches
  for (int64_t wb = w1; wb <= w2; wb += 64) {
    const int64_t w = wb + lane;
    const bool live = w <= w2 && (w == w1 || share_begin(w, total, nw) < share_begin(w + 1, total, nw));
    const int64_t slot = w * 2 + (w == w1 ? 1 : 0);
    const int n = (int)min<int64_t>(64, w2 - wb + 1);
    float2 ml[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
      ml[j] = live ? reinterpret_cast<const float2*>(a.ws_ml)[slot * G + j] : make_float2(kNegBig, 0.f);
    float f[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mb = ml[j].x;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
      const float mnew = fmaxf(M[j], mb);
      const float alpha = fast_exp2(M[j] - mnew);
      f[j] = live ? fast_exp2(ml[j].x - mnew) : 0.f;
      float lf = f[j] * ml[j].y;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) lf += __shfl_xor(lf, off);
      Ls[j] = Ls[j] * alpha + lf;
      o0[j] *= alpha;
      o1[j] *= alpha;
      M[j] = mnew;
    }
    // the pieces' rows, added in wave order (a piece with weight 0 is skipped;
    // its slot may hold stale bits): PR pieces' loads in flight at a time (64
    // registers of loads whatever G) while that many remain, then 4 at a time
    constexpr int PR = G <= 2 ? 16 : 32 / G;
    int i0 = 0;
    for (; i0 + PR <= n; i0 += PR) add_pieces<G, PR>(a, slot, f, i0, n, lane, o0, o1);
    for (; i0 < n; i0 += 4) add_pieces<G, 4>(a, slot, f, i0, n, lane, o0, o1);
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float inv = 1.f / Ls[j];
    reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * a.num_q_heads + g * G + j) * kD)[lane] =
        pack_bf16x2(o0[j] * inv, o1[j] * inv);
  }
}

// G >= 4 take the split pass on the matrix cores. Same-box timings (us) of
// the vector pass against the matrix pass: config-2 lengths at Hkv = 8, G = 4
// 207.9 / 196.3 and G = 8 370 / 198.5 (the vector pass at G = 8 spilled and
// ran one wave per SIMD); 512 long contexts at G = 4 2322.9 / 2268.8; G = 2
// 196.9 / 196.8, so G <= 2 keep the vector pass.
constexpr int kMfmaMinGroup = 4;

// Vector split pass: 4 tokens per lane per chunk (32-token chunks). Matrix
// split pass: 32-token chunks.
template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t stream) {
  constexpr bool kMfma = G >= kMfmaMinGroup;
  constexpr int TPL = 4;  // the finalize pass's chunk: 8 TPL tokens
  if constexpr (kMfma) decode_mfma_kernel<G><<<dim3(a.num_waves), dim3(64), 0, stream>>>(a);
  else decode_split_kernel<G, TPL><<<dim3(a.num_waves), dim3(64), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_finalize_kernel<G, TPL><<<dim3(a.num_seqs * a.num_kv_heads), dim3(64), 0, stream>>>(a);
  return hipGetLastError();
}

int decode_chunk_tokens(int) { return 32; }

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
