// Host side of the C ABI declared in include/pa.h: argument checks, launch
// geometry (decode partition length, prefill tile count) and error mapping.
// Nothing here reads device memory, so every entry point is graph-capturable.
#include "../../include/pa.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#include "launch.h"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace pa {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Checks shared by the attention entry points.
int check_heads(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads (%d) and num_kv_heads (%d) must be positive", num_q_heads,
                num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", num_q_heads,
                num_kv_heads);
  if (head_dim != kHeadDim) return fail(PA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", head_dim);
  if (!supported_group(num_q_heads / num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "GQA group %d unsupported (1, 2, 4 or 8)", num_q_heads / num_kv_heads);
  return PA_OK;
}

int check_block_size(int32_t block_size) {
  if (block_size <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "block_size %d must be positive", block_size);
  if (block_size % 64 != 0) return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a multiple of 64", block_size);
  return PA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Waves the decode work is split over: enough to keep every CU of an MI355X
// (256 CUs, 8 resident decode waves each) busy, but no more than there are
// chunks of work.
constexpr int32_t kDecodeWaves = 2048;
constexpr int64_t kMinChunksPerWave = 4;

struct DecodeGeometry {
  int32_t num_waves;
  size_t ws_o_bytes;
  size_t ws_bytes;
};

bool decode_geometry(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                     int32_t split_waves, DecodeGeometry* g) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 || split_waves < 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  const int group = num_q_heads / num_kv_heads;
  const int ch = pa::decode_chunk_tokens(group);
  const int64_t max_chunks = (int64_t)num_seqs * num_kv_heads * ((max_context_len + ch - 1) / ch);
  // Default: 2048 waves (8 per CU), but no fewer than kMinChunksPerWave chunks
  // per wave by the length bound: a small batch spread over many more waves
  // leaves every (sequence, kv head) pair in many short pieces, and merging
  // them costs more than the split saves.
  int64_t nw = split_waves > 0 ? split_waves
                               : std::min<int64_t>(kDecodeWaves, (max_chunks + kMinChunksPerWave - 1) / kMinChunksPerWave);
  if (nw > max_chunks) nw = max_chunks;
  if (nw < 1) nw = 1;
  g->num_waves = (int32_t)nw;
  const size_t slots = (size_t)nw * 2 * group;
  g->ws_o_bytes = slots * kHeadDim * sizeof(float);
  g->ws_bytes = g->ws_o_bytes + slots * 2 * sizeof(float);
  return true;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "null pointer";
    case PA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "not enough free cache blocks";
    case PA_ERR_NOT_FOUND: return "unknown sequence";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error; }

int pa_version(void) { return 100; }

int pa_store_kvcache(const void* k, int64_t k_token_stride, const void* v, int64_t v_token_stride, void* k_cache,
                     void* v_cache, const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                     int32_t head_dim, int64_t num_blocks, int32_t block_size, void* stream) {
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens %d is negative", num_tokens);
  if (num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_kv_heads (%d) and head_dim (%d) must be positive", num_kv_heads,
                head_dim);
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks (%lld) and block_size (%d) must be positive",
                (long long)num_blocks, block_size);
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row % 8 != 0) return fail(PA_ERR_ALIGNMENT, "a token row (%lld elements) is not a multiple of 16 bytes",
                                (long long)row);
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_blocks * block_size exceeds the int32 slot range");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_NULL_POINTER, "k, v, k_cache, v_cache and slot_mapping are required");
  if (k_token_stride < row || v_token_stride < row)
    return fail(PA_ERR_INVALID_ARGUMENT, "token strides (%lld, %lld) are below a row (%lld)",
                (long long)k_token_stride, (long long)v_token_stride, (long long)row);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) || k_token_stride % 8 ||
      v_token_stride % 8)
    return fail(PA_ERR_ALIGNMENT, "k, v, caches and token strides must be 16-byte aligned");
  if ((uint64_t)num_tokens * 2u * (uint64_t)(row / 8) > 0xFFFFFFFFull)
    return fail(PA_ERR_UNSUPPORTED, "too many tokens for one call");
  pa::StoreArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_token_stride = k_token_stride;
  a.v_token_stride = v_token_stride;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.row_vecs = (int32_t)(row / 8);
  a.capacity = (int32_t)(num_blocks * block_size);
  return hip_status(pa::launch_store_kvcache(a, static_cast<hipStream_t>(stream)), "store_kvcache launch");
}

int pa_qk_norm_rope_store(void* q_out, int64_t q_out_token_stride, const void* qkv, int64_t qkv_token_stride,
                          const void* q_norm_weight, const void* k_norm_weight, float eps, const float* cos_sin,
                          int32_t max_position, const int32_t* positions, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_blocks, int32_t block_size, void* stream) {
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens %d is negative", num_tokens);
  int st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st) return st;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks (%lld) and block_size (%d) must be positive",
                (long long)num_blocks, block_size);
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_blocks * block_size exceeds the int32 slot range");
  if (!(eps >= 0.f) || isinf(eps)) return fail(PA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (max_position <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "max_position %d must be positive", max_position);
  const int64_t heads = (int64_t)num_q_heads + 2 * (int64_t)num_kv_heads;
  if (qkv_token_stride < heads * head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "qkv_token_stride %lld is below (num_q_heads + 2 num_kv_heads) * head_dim",
                (long long)qkv_token_stride);
  if (q_out_token_stride < (int64_t)num_q_heads * head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_out_token_stride %lld is below num_q_heads * head_dim",
                (long long)q_out_token_stride);
  if ((int64_t)num_tokens * heads >= ((int64_t)1 << 31) - 64)
    return fail(PA_ERR_UNSUPPORTED, "num_tokens * (num_q_heads + 2 num_kv_heads) must stay below 2^31");
  if (num_tokens == 0) return ok();
  if (!q_out || !qkv || !q_norm_weight || !k_norm_weight || !cos_sin || !positions || !k_cache || !v_cache ||
      !slot_mapping)
    return fail(PA_ERR_NULL_POINTER, "every pointer argument is required");
  if (!aligned16(q_out) || !aligned16(qkv) || !aligned16(q_norm_weight) || !aligned16(k_norm_weight) ||
      !aligned16(cos_sin) || !aligned16(k_cache) || !aligned16(v_cache) || q_out_token_stride % 8 ||
      qkv_token_stride % 8)
    return fail(PA_ERR_ALIGNMENT, "pointers and token strides must be 16-byte aligned");
  pa::NormRopeArgs a;
  a.q_out = static_cast<uint16_t*>(q_out);
  a.q_out_token_stride = q_out_token_stride;
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.qkv_token_stride = qkv_token_stride;
  a.q_weight = static_cast<const uint16_t*>(q_norm_weight);
  a.k_weight = static_cast<const uint16_t*>(k_norm_weight);
  a.cos_sin = cos_sin;
  a.positions = positions;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.num_items = (uint32_t)(num_tokens * heads);
  a.num_heads = (int32_t)heads;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_position = max_position;
  a.capacity = (int32_t)(num_blocks * block_size);
  a.eps = eps;
  return hip_status(pa::launch_norm_rope_store(a, static_cast<hipStream_t>(stream)), "qk_norm_rope_store launch");
}

size_t pa_sample_workspace_size(int32_t num_rows, int32_t vocab_size) {
  if (num_rows < 0 || vocab_size <= 0) return 0;
  return (size_t)num_rows * (size_t)pa::sample_chunks(vocab_size) * (sizeof(float) + sizeof(int32_t));
}

int pa_sample_gumbel(int32_t* tokens, const float* logits, int64_t logits_row_stride, const float* temperatures,
                     int32_t num_rows, int32_t vocab_size, uint64_t seed, uint64_t offset, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (num_rows < 0 || vocab_size <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_rows (%d) must be >= 0 and vocab_size (%d) positive", num_rows,
                vocab_size);
  if (num_rows > 65535) return fail(PA_ERR_UNSUPPORTED, "num_rows %d exceeds 65535", num_rows);
  if (logits_row_stride < vocab_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "logits_row_stride %lld is below vocab_size %d",
                (long long)logits_row_stride, vocab_size);
  if (num_rows == 0) return ok();
  if (!tokens || !logits || !temperatures || !workspace)
    return fail(PA_ERR_NULL_POINTER, "tokens, logits, temperatures and workspace are required");
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || !aligned16(workspace))
    return fail(PA_ERR_ALIGNMENT, "logits must be 4-byte and the workspace 16-byte aligned");
  const size_t need = pa_sample_workspace_size(num_rows, vocab_size);
  if (workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, need);
  pa::SampleArgs a;
  a.tokens = tokens;
  a.logits = logits;
  a.row_stride = logits_row_stride;
  a.temperatures = temperatures;
  a.chunks = pa::sample_chunks(vocab_size);
  a.ws_score = static_cast<float*>(workspace);
  a.ws_index = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                          (size_t)num_rows * a.chunks * sizeof(float));
  a.seed = seed;
  a.offset = offset;
  a.num_rows = num_rows;
  a.vocab = vocab_size;
  return hip_status(pa::launch_sample(a, static_cast<hipStream_t>(stream)), "sample launch");
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t split_waves) {
  if (head_dim != kHeadDim) return 0;
  DecodeGeometry g;
  if (!decode_geometry(num_seqs, num_q_heads, num_kv_heads, max_context_len, split_waves, &g)) return 0;
  return g.ws_bytes;
}

int32_t pa_decode_split_waves(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                              int32_t split_waves) {
  DecodeGeometry g;
  if (!decode_geometry(num_seqs, num_q_heads, num_kv_heads, max_context_len, split_waves, &g)) return 0;
  return g.num_waves;
}

}  // extern "C"

static int decode_impl(void* out, const void* q, int64_t q_seq_stride, const void* k_new, int64_t k_new_stride,
                       const void* v_new, int64_t v_new_stride, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_context_len, float scale, int32_t split_waves, void* workspace,
                       size_t workspace_bytes, void* stream, bool static_scratch = false,
                       const int32_t* live_seqs = nullptr) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d is negative", num_seqs);
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs %d exceeds 65535", num_seqs);
  int st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st) return st;
  if (max_context_len > (1 << 24))
    return fail(PA_ERR_UNSUPPORTED, "max_context_len %d exceeds 2^24", max_context_len);
  st = check_block_size(block_size);
  if (st) return st;
  if (max_context_len < 0) return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len %d is negative", max_context_len);
  if (max_blocks_per_seq < 0 || (int64_t)max_blocks_per_seq * block_size < max_context_len)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq (%d) x block_size (%d) < max_context_len (%d)",
                max_blocks_per_seq, block_size, max_context_len);
  if (split_waves < 0) return fail(PA_ERR_INVALID_ARGUMENT, "split_waves %d is negative", split_waves);
  if (!(scale == scale) || isinf(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL_POINTER, "out, q, caches, block_tables and context_lens are required");
  if (q_seq_stride < (int64_t)num_q_heads * head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_seq_stride %lld is below num_q_heads * head_dim",
                (long long)q_seq_stride);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || q_seq_stride % 8)
    return fail(PA_ERR_ALIGNMENT, "out, q, caches and q_seq_stride must be 16-byte aligned");
  if (k_new || v_new) {
    if (!k_new || !v_new) return fail(PA_ERR_NULL_POINTER, "k_new and v_new are required");
    if (k_new_stride < (int64_t)num_kv_heads * head_dim || v_new_stride < (int64_t)num_kv_heads * head_dim)
      return fail(PA_ERR_INVALID_ARGUMENT, "k_new / v_new strides (%lld, %lld) are below num_kv_heads * head_dim",
                  (long long)k_new_stride, (long long)v_new_stride);
    if (!aligned16(k_new) || !aligned16(v_new) || k_new_stride % 8 || v_new_stride % 8)
      return fail(PA_ERR_ALIGNMENT, "k_new, v_new and their strides must be 16-byte aligned");
  }
  DecodeGeometry g;
  decode_geometry(num_seqs, num_q_heads, num_kv_heads, max_context_len, split_waves, &g);
  if (static_scratch) {
    // pa_store_decode_noalloc: the library's static scratch is the workspace
    if (g.ws_bytes > pa::kDecodeScratchBytes)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                  "this split needs %zu bytes of decode scratch; the static scratch holds %zu (at most 2048 "
                  "waves x 8 query heads per kv head)", g.ws_bytes, pa::kDecodeScratchBytes);
    const int sst = pa::decode_scratch(&workspace);
    if (sst) return sst;
    workspace_bytes = pa::kDecodeScratchBytes;
  }
  if (!workspace) return fail(PA_ERR_NULL_POINTER, "workspace of %zu bytes is required", g.ws_bytes);
  if (workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, g.ws_bytes);
  if (!aligned16(workspace)) return fail(PA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  pa::DecodeArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.q_seq_stride = q_seq_stride;
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_new_stride = k_new_stride;
  a.v_new_stride = v_new_stride;
  a.live_seqs = live_seqs;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + g.ws_o_bytes);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.num_waves = g.num_waves;
  a.scale_log2e = scale * kLog2e;
  return hip_status(pa::launch_decode(a, num_q_heads / num_kv_heads, static_cast<hipStream_t>(stream)),
                    "decode launch");
}

namespace pa {

int store_decode_live(const pa_decode_step& s, int32_t num_seqs, hipStream_t stream) {
  return decode_impl(s.out, s.q, s.q_seq_stride, s.k_new, s.k_token_stride, s.v_new, s.v_token_stride, s.k_cache,
                     s.v_cache, s.block_tables, s.max_blocks_per_seq, s.context_lens, num_seqs, s.num_q_heads,
                     s.num_kv_heads, s.head_dim, s.block_size, s.max_context_len, s.scale, s.split_waves,
                     s.workspace, s.workspace_bytes, stream, false, s.live_batch);
}

}  // namespace pa

extern "C" {

int pa_decode(void* out, const void* q, int64_t q_seq_stride, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_context_len, float scale, int32_t split_waves, void* workspace,
              size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, q_seq_stride, nullptr, 0, nullptr, 0, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_context_len, scale, split_waves, workspace, workspace_bytes, stream);
}

int pa_store_decode(void* out, const void* q, int64_t q_seq_stride, const void* k_new, int64_t k_new_stride,
                    const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_context_len, float scale, int32_t split_waves, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_NULL_POINTER, "k_new and v_new are required");
  return decode_impl(out, q, q_seq_stride, k_new, k_new_stride, v_new, v_new_stride, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_context_len, scale, split_waves, workspace, workspace_bytes, stream);
}

int pa_store_decode_noalloc(void* out, const void* q, int64_t q_seq_stride, const void* k_new, int64_t k_new_stride,
                            const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_context_len, float scale, int32_t split_waves,
                            void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_NULL_POINTER, "k_new and v_new are required");
  return decode_impl(out, q, q_seq_stride, k_new, k_new_stride, v_new, v_new_stride, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_context_len, scale, split_waves, nullptr, 0, stream, /*static_scratch=*/true);
}

}  // extern "C"

// Argument checks and launch of the prefill kernel; st (optional) asks for the
// fused store of pa_store_prefill_varlen.
struct PrefillStore {
  const void* k_new;
  const void* v_new;
  int64_t k_new_stride, v_new_stride;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int64_t num_blocks;
  int32_t block_size_for_capacity;
};

static int prefill_impl(void* out, const void* q, int64_t q_token_stride, const void* k, const void* v,
                        int64_t k_token_stride, int64_t v_token_stride, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
                        const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size, void* stream,
                        const PrefillStore* st_args = nullptr) {
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs (%d), max_seqlen_q (%d) and max_seqlen_k (%d) must be >= 0",
                num_seqs, max_seqlen_q, max_seqlen_k);
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs %d exceeds 65535", num_seqs);
  int st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st) return st;
  if (!(scale == scale) || isinf(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be finite");
  const int64_t kv_row = (int64_t)num_kv_heads * head_dim;
  if (kv_row > (int64_t)1 << 23)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * head_dim above 2^23 is not supported");
  if (block_table) {
    st = check_block_size(block_size);
    if (st) return st;
    if (max_blocks_per_seq <= 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq %d must be positive with a block table",
                  max_blocks_per_seq);
    // a table row names at most max_blocks_per_seq blocks: longer key ranges cannot be addressed
    if ((int64_t)max_blocks_per_seq * block_size < max_seqlen_k)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "max_seqlen_k %d exceeds what a block table row covers (%d blocks of %d tokens)", max_seqlen_k,
                  max_blocks_per_seq, block_size);
  } else {
    if (k_token_stride < kv_row || v_token_stride < kv_row)
      return fail(PA_ERR_INVALID_ARGUMENT, "k/v token strides (%lld, %lld) are below a row (%lld)",
                  (long long)k_token_stride, (long long)v_token_stride, (long long)kv_row);
    if (k_token_stride % 8 || v_token_stride % 8)
      return fail(PA_ERR_ALIGNMENT, "k/v token strides must be 16-byte aligned");
    // a 64-token tile must span less than 2 GiB (32-bit offsets inside a tile)
    if (k_token_stride > (int64_t)1 << 23 || v_token_stride > (int64_t)1 << 23)
      return fail(PA_ERR_UNSUPPORTED, "k/v token strides above 2^23 elements are not supported");
  }
  if (num_seqs == 0 || max_seqlen_q == 0) return ok();
  if (!out || !q || !k || !v || !cu_seqlens_q || !cu_seqlens_k)
    return fail(PA_ERR_NULL_POINTER, "out, q, k, v, cu_seqlens_q and cu_seqlens_k are required");
  if (q_token_stride < (int64_t)num_q_heads * head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_token_stride %lld is below num_q_heads * head_dim",
                (long long)q_token_stride);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v) || q_token_stride % 8)
    return fail(PA_ERR_ALIGNMENT, "out, q, k, v and q_token_stride must be 16-byte aligned");
  const int group = num_q_heads / num_kv_heads;
  const int qp = pa::prefill_tile_positions(group);
  pa::PrefillArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.q_token_stride = q_token_stride;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_token_stride = block_table ? kv_row : k_token_stride;
  a.v_token_stride = block_table ? kv_row : v_token_stride;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.block_table = block_table;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_table ? block_size : 0;
  a.num_seqs = num_seqs;
  a.num_q_tiles = (max_seqlen_q + qp - 1) / qp;
  a.items_per_xcd = ((int64_t)num_kv_heads * num_seqs * a.num_q_tiles + 7) / 8;
  if (a.items_per_xcd > (int64_t)INT32_MAX / 8)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * num_seqs * query tiles exceeds the grid range");
  a.max_seqlen_k = max_seqlen_k;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.causal = causal ? 1 : 0;
  a.scale_log2e = scale * kLog2e;
  a.k_new = a.v_new = nullptr;
  a.k_new_stride = a.v_new_stride = 0;
  a.slot_mapping = nullptr;
  a.k_cache_out = a.v_cache_out = nullptr;
  a.store_capacity = 0;
  if (st_args) {
    a.k_new = static_cast<const uint16_t*>(st_args->k_new);
    a.v_new = static_cast<const uint16_t*>(st_args->v_new);
    a.k_new_stride = st_args->k_new_stride;
    a.v_new_stride = st_args->v_new_stride;
    a.slot_mapping = st_args->slot_mapping;
    a.k_cache_out = static_cast<uint16_t*>(st_args->k_cache);
    a.v_cache_out = static_cast<uint16_t*>(st_args->v_cache);
    a.store_capacity = st_args->num_blocks * (int64_t)st_args->block_size_for_capacity;
  }
  return hip_status(pa::launch_prefill(a, group, static_cast<hipStream_t>(stream)), "prefill launch");
}

extern "C" {

int pa_prefill_varlen(void* out, const void* q, int64_t q_token_stride, const void* k, const void* v,
                      int64_t k_token_stride, int64_t v_token_stride, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
                      const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size, void* stream) {
  return prefill_impl(out, q, q_token_stride, k, v, k_token_stride, v_token_stride, cu_seqlens_q, cu_seqlens_k,
                      num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim, scale, causal,
                      block_table, max_blocks_per_seq, block_size, stream);
}

int pa_store_prefill_varlen(void* out, const void* q, int64_t q_token_stride, const void* k_new,
                            int64_t k_new_stride, const void* v_new, int64_t v_new_stride, void* k_cache,
                            void* v_cache, const int32_t* slot_mapping, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            float scale, int32_t causal, const int32_t* block_table, int32_t max_blocks_per_seq,
                            int32_t block_size, int64_t num_blocks, void* stream) {
  const int64_t kv_row = (int64_t)num_kv_heads * head_dim;
  int st = check_block_size(block_size);
  if (st) return st;
  if (num_blocks <= 0 || num_blocks > ((int64_t)1 << 31) / block_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks %lld must be positive with num_blocks * block_size < 2^31",
                (long long)num_blocks);
  if (num_seqs > 0 && max_seqlen_q > 0) {
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
      return fail(PA_ERR_NULL_POINTER, "k_new, v_new, k_cache, v_cache and slot_mapping are required");
    if (k_new_stride < kv_row || v_new_stride < kv_row)
      return fail(PA_ERR_INVALID_ARGUMENT, "k_new / v_new strides (%lld, %lld) are below a row (%lld)",
                  (long long)k_new_stride, (long long)v_new_stride, (long long)kv_row);
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) || k_new_stride % 8 ||
        v_new_stride % 8)
      return fail(PA_ERR_ALIGNMENT, "k_new, v_new, the caches and the strides must be 16-byte aligned");
  }
  PrefillStore sa{k_new, v_new, k_new_stride, v_new_stride, k_cache, v_cache, slot_mapping, num_blocks, block_size};
  // without a block table the keys are the new tokens themselves (packed like the queries)
  const void* k = block_table ? static_cast<const void*>(k_cache) : k_new;
  const void* v = block_table ? static_cast<const void*>(v_cache) : v_new;
  return prefill_impl(out, q, q_token_stride, k, v, k_new_stride, v_new_stride, cu_seqlens_q, cu_seqlens_k, num_seqs,
                      max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim, scale, causal, block_table,
                      max_blocks_per_seq, block_size, stream, &sa);
}

}  // extern "C"
