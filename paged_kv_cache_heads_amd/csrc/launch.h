// Host-side launchers of the kernels (internal to the library). The public
// C ABI in include/pa.h validates arguments, then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct pa_decode_step;

namespace pa {

// Record the message of a failing call (pa_last_error) and return its status;
// ok() clears it and returns PA_OK. Defined in pa_api.cpp.
int fail(int status, const char* fmt, ...);
int ok();

struct StoreArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_token_stride;  // elements
  int64_t v_token_stride;  // elements
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t row_vecs;  // 16-byte vectors per token row (num_kv_heads * head_dim / 8)
  int32_t capacity;  // num_blocks * block_size: slots at or above it are skipped, like negative ones
};

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  int64_t q_seq_stride;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const uint16_t* k_new;  // fused store (pa_store_decode): the new token's K row per sequence, else null
  const uint16_t* v_new;
  int64_t k_new_stride;   // elements between sequences' rows
  int64_t v_new_stride;
  float* ws_o;   // [num_waves * 2 slots, G, head_dim] partial outputs
  float* ws_ml;  // [num_waves * 2 slots, G, 2] (max, sum) of each partial
  const int32_t* live_seqs;  // optional device count: sequences at or past it are empty (graph replays)
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t num_waves;  // waves the chunk sequence is split over
  float scale_log2e;
};

struct PrefillArgs {
  uint16_t* out;
  const uint16_t* q;
  int64_t q_token_stride;
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_token_stride;
  int64_t v_token_stride;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* block_table;  // null: packed k/v
  int32_t max_blocks_per_seq;
  int32_t block_size;
  int32_t num_seqs;
  int32_t num_q_tiles;
  int64_t items_per_xcd;  // ceil(num_kv_heads * num_seqs * num_q_tiles / 8)
  int32_t max_seqlen_k;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t causal;
  float scale_log2e;
  // fused store (pa_store_prefill_varlen), else null: new token j of sequence
  // i is row cu_seqlens_q[i] + j of k_new / v_new (the key at position
  // nk - nq + j), stored at slot_mapping of that row unless the slot is
  // negative or at least store_capacity
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t k_new_stride;  // elements
  int64_t v_new_stride;
  const int32_t* slot_mapping;
  uint16_t* k_cache_out;
  uint16_t* v_cache_out;
  int64_t store_capacity;  // num_blocks * block_size
};

struct NormRopeArgs {
  uint16_t* q_out;
  int64_t q_out_token_stride;   // elements
  const uint16_t* qkv;
  int64_t qkv_token_stride;     // elements
  const uint16_t* q_weight;     // [128]
  const uint16_t* k_weight;     // [128]
  const float* cos_sin;         // [max_position, 128]: 64 cosines, then 64 sines
  const int32_t* positions;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* slot_mapping;
  uint32_t num_items;           // num_tokens * (num_q_heads + 2 * num_kv_heads), below 2^31
  int32_t num_heads;            // num_q_heads + 2 * num_kv_heads
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_position;
  int32_t capacity;             // num_blocks * block_size (slots at or past it are skipped)
  float eps;
};

struct SampleArgs {
  int32_t* tokens;             // [num_rows]
  const float* logits;         // [num_rows, row_stride]
  int64_t row_stride;          // elements
  const float* temperatures;   // [num_rows]
  float* ws_score;             // [num_rows, chunks] per-chunk best score
  int32_t* ws_index;           // [num_rows, chunks] and its index
  uint64_t seed;
  uint64_t offset;
  int32_t num_rows;
  int32_t vocab;
  int32_t chunks;              // sample_chunks(vocab)
};

// Vocabulary chunks (one workgroup each) per row of the sampler.
int32_t sample_chunks(int32_t vocab);
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);

hipError_t launch_store_kvcache(const StoreArgs& a, hipStream_t stream);
hipError_t launch_norm_rope_store(const NormRopeArgs& a, hipStream_t stream);
// group = num_q_heads / num_kv_heads (1, 2, 4 or 8); head_dim is 128.
hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t stream);
// pa_store_decode over the step's buffers at num_seqs rows, with the step's
// device count of live sequences (rows at or past it are empty contexts); the
// call graph-captured decode steps hold. Defined in pa_api.cpp.
int store_decode_live(const struct pa_decode_step& s, int32_t num_seqs, hipStream_t stream);
// Tokens per decode work chunk for a GQA group size.
int decode_chunk_tokens(int group);
// The library's static decode scratch: 2048 waves x 2 slots x 8 heads x
// (128 + 2) fp32 values. decode_scratch() gives its device address on the
// current device (looked up once per device); PA_OK or a pa_status.
constexpr size_t kDecodeScratchBytes = (size_t)2048 * 2 * 8 * (128 + 2) * sizeof(float);
int decode_scratch(void** ptr);
hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream);

// Query positions covered by one prefill workgroup for a GQA group size.
inline int prefill_tile_positions(int group) { return 128 / group; }
// Keys per prefill tile: 32 while sequences are short (at most 1024 keys),
// else 64.
inline int prefill_key_tile(int max_seqlen_k) { return max_seqlen_k <= 1024 ? 32 : 64; }

}  // namespace pa
