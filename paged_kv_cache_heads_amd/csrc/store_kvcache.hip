// KV store: copy each new token's K and V rows into the paged cache at the
// slot that slot_mapping names (page "nano-vLLM 最小化vLLM重新实现", section 5
// "注意力机制": the store kernel writes K/V into the paged cache by slot;
// cache layout [num_blocks, block_size, num_kv_heads, head_dim] per layer,
// section 4 "模型运行器").
//
// The work is a pure gather-scatter of 16-byte vectors, bound by HBM. A row
// of num_kv_heads * head_dim bf16 is contiguous both in the (possibly strided)
// source and in the cache, so consecutive lanes move consecutive 16-byte
// pieces of one row: every wave reads and writes whole 64-byte-or-larger runs.
//
// Two layouts of the same copy. When a token's K and V rows together hold a
// power-of-two number of vectors that divides the workgroup (num_kv_heads a
// power of two up to 8 at head_dim 128), each workgroup takes whole tokens
// and each lane one vector, the token and the vector taken from the thread
// id by a shift and a mask. Otherwise the (token, vector) space is flat and
// each lane moves kStoreUnroll vectors, located by a division. Same-box
// timings of the two on the 16k-token varlen batch (caches flushed before
// each call / not flushed): 27.9 / 23.5 us for whole tokens against
// 29.4 / 26.9 us flat, and a plain device copy of the same bytes 26.3 /
// 24.2 us.
#include "common.h"
#include "launch.h"

namespace pa {

constexpr int kStoreThreads = 256;
constexpr int kStoreUnroll = 4;

// Locate the 16-byte vector idx of the flattened (token, K row | V row) space.
// Returns false for vectors past the end and for tokens whose slot is negative
// (padding) or past the cache.
__device__ __forceinline__ bool store_vector(const StoreArgs& a, uint32_t idx, uint32_t total, const uint4*& src,
                                             uint4*& dst) {
  if (idx >= total) return false;
  const uint32_t per_token = 2u * (uint32_t)a.row_vecs;  // K row then V row
  const uint32_t t = idx / per_token;
  uint32_t c = idx - t * per_token;
  const int32_t slot = a.slot_mapping[t];
  if ((uint32_t)slot >= (uint32_t)a.capacity) return false;  // padded token or no such slot: nothing to store
  const bool is_v = c >= (uint32_t)a.row_vecs;
  if (is_v) c -= a.row_vecs;
  const uint16_t* row = is_v ? a.v + (int64_t)t * a.v_token_stride : a.k + (int64_t)t * a.k_token_stride;
  uint16_t* cache = is_v ? a.v_cache : a.k_cache;
  src = reinterpret_cast<const uint4*>(row) + c;
  dst = reinterpret_cast<uint4*>(cache + (int64_t)slot * (a.row_vecs * 8)) + c;
  return true;
}

__global__ __launch_bounds__(kStoreThreads) void store_kvcache_kernel(StoreArgs a) {
  static_assert(kStoreUnroll == 4, "the body below is unrolled by hand");
  const uint32_t total = (uint32_t)a.num_tokens * 2u * (uint32_t)a.row_vecs;
  const uint32_t base = blockIdx.x * (kStoreThreads * kStoreUnroll) + threadIdx.x;
  const uint4 *s0, *s1, *s2, *s3;
  uint4 *d0, *d1, *d2, *d3;
  const bool p0 = store_vector(a, base, total, s0, d0);
  const bool p1 = store_vector(a, base + kStoreThreads, total, s1, d1);
  const bool p2 = store_vector(a, base + 2 * kStoreThreads, total, s2, d2);
  const bool p3 = store_vector(a, base + 3 * kStoreThreads, total, s3, d3);
  // all loads are issued before the first store
  uint4 v0, v1, v2, v3;
  if (p0) v0 = load16_nt(s0);
  if (p1) v1 = load16_nt(s1);
  if (p2) v2 = load16_nt(s2);
  if (p3) v3 = load16_nt(s3);
  if (p0) store16_nt(d0, v0);
  if (p1) store16_nt(d1, v1);
  if (p2) store16_nt(d2, v2);
  if (p3) store16_nt(d3, v3);
}

// Whole tokens per workgroup: 2^vec_shift vectors per token (K row, then V
// row), 2^(8 - vec_shift) tokens per workgroup of kStoreThreads lanes.
__global__ __launch_bounds__(kStoreThreads) void store_tokens_kernel(StoreArgs a, int vec_shift) {
  const int tid = threadIdx.x;
  const int t = (int)(blockIdx.x << (8 - vec_shift)) + (tid >> vec_shift);
  if (t >= a.num_tokens) return;
  const int32_t slot = a.slot_mapping[t];
  if ((uint32_t)slot >= (uint32_t)a.capacity) return;  // padded token or no such slot: nothing to store
  int c = tid & ((1 << vec_shift) - 1);
  const bool is_v = c >= a.row_vecs;
  if (is_v) c -= a.row_vecs;
  const uint16_t* row = is_v ? a.v + (int64_t)t * a.v_token_stride : a.k + (int64_t)t * a.k_token_stride;
  uint16_t* cache = is_v ? a.v_cache : a.k_cache;
  store16_nt(reinterpret_cast<uint4*>(cache + (int64_t)slot * (a.row_vecs * 8)) + c,
             load16_nt(reinterpret_cast<const uint4*>(row) + c));
}

hipError_t launch_store_kvcache(const StoreArgs& a, hipStream_t stream) {
  static_assert(kStoreThreads == 256, "store_tokens_kernel assumes 2^8 lanes");
  if (a.num_tokens == 0) return hipSuccess;
  const int per_token = 2 * a.row_vecs;
  if (per_token <= kStoreThreads && (per_token & (per_token - 1)) == 0) {
    const int vec_shift = __builtin_ctz((unsigned)per_token);
    const int tokens_per_block = kStoreThreads >> vec_shift;
    const uint32_t blocks = (uint32_t)(((int64_t)a.num_tokens + tokens_per_block - 1) / tokens_per_block);
    hipLaunchKernelGGL(store_tokens_kernel, dim3(blocks), dim3(kStoreThreads), 0, stream, a, vec_shift);
    return hipGetLastError();
  }
  const uint64_t total = (uint64_t)a.num_tokens * 2u * (uint64_t)a.row_vecs;
  const uint64_t per_block = kStoreThreads * kStoreUnroll;
  const uint32_t blocks = (uint32_t)((total + per_block - 1) / per_block);
  hipLaunchKernelGGL(store_kvcache_kernel, dim3(blocks), dim3(kStoreThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
