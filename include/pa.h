/*
 * pa.h — C ABI of the paged-KV-cache attention library for AMD MI355X (gfx950).
 *
 * Three operations make up the path, as the nano-vLLM pages describe it:
 *   pa_store_kvcache   write new tokens' K/V rows into the paged cache by slot;
 *   pa_decode          one query per sequence against its paged K/V;
 *   pa_prefill_varlen  causal attention over packed variable-length sequences,
 *                      K/V packed or read through a block table (prefix cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *_host are host memory; every other pointer is device
 *   memory on the current HIP device. bf16 tensors are passed as raw 16-bit
 *   storage. Strides are in elements.
 * - A per-layer cache is [num_blocks, block_size, num_kv_heads, head_dim],
 *   contiguous (page "nano-vLLM 最小化vLLM重新实现", section 4 "模型运行器": one
 *   KV tensor [2, num_layers, num_blocks, block_size, num_kv_heads, head_dim],
 *   a layer's K cache and V cache being two of its slices). A flat slot s
 *   names row s % block_size of block s / block_size.
 * - Grouped-query attention: query head h reads kv head h / G with
 *   G = num_q_heads / num_kv_heads (the pages fix only the head counts; this
 *   contiguous grouping is the library's reading).
 * - Supported shapes: head_dim == 128; G in {1, 2, 4, 8}; block_size a
 *   positive multiple of 64 (the pages' default is 256 and they require a
 *   multiple of 256: page "nano-vLLM 最小化vLLM重新实现", "关键设计选择").
 *   All pointers and row strides must be 16-byte aligned.
 * - Ownership: the caller owns every buffer. The compute entry points
 *   allocate nothing and keep no pointer after return. The exceptions are
 *   named where they are declared: the host objects made by
 *   pa_decode_graphs_create and the block manager (pa_blocks.h), which hold
 *   what they are given until destroyed, and the static device scratch of
 *   pa_store_decode_noalloc. Work is enqueued on `stream` (a hipStream_t;
 *   NULL = the null stream) and the call returns without synchronising;
 *   buffers must stay alive until the stream has run the work. No entry point
 *   reads device memory from the host, so all of them may be recorded into a
 *   HIP graph.
 * - Errors: arguments are checked on the host before anything is launched; a
 *   failed check returns a non-zero pa_status and launches nothing. A launch
 *   failure returns PA_ERR_HIP. pa_last_error() gives a message for the most
 *   recent failing call on the calling thread. Device-side preconditions
 *   (block-table entries in range, lengths within the stated maxima) are the
 *   caller's and are not checked on the device. Slots are: every store skips
 *   a token whose slot is negative or past the cache.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  PA_ERR_INVALID_ARGUMENT = 2,    /* negative size, head counts that do not divide, stride too small ... */
  PA_ERR_UNSUPPORTED = 3,         /* valid but not implemented: head_dim, group size, block_size */
  PA_ERR_ALIGNMENT = 4,           /* pointer or stride not 16-byte aligned */
  PA_ERR_WORKSPACE_TOO_SMALL = 5, /* decode workspace smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = 6,                 /* the HIP runtime reported an error at launch */
  PA_ERR_NO_BLOCKS = 7,           /* block manager (pa_blocks.h): too few free blocks; nothing changed */
  PA_ERR_NOT_FOUND = 8            /* block manager: unknown sequence id */
} pa_status;

/* Static description of a status code; never NULL. */
const char* pa_status_string(int status);

/* Message describing the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int pa_version(void);

/*
 * pa_store_kvcache — scatter new tokens' K and V rows into the paged cache.
 *
 * Page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制": the store kernel
 * writes K/V into the paged cache at the slots given by slot_mapping. For each
 * token t with slot_mapping[t] = s >= 0:
 *   k_cache[s / block_size, s % block_size, :, :] = k[t, :, :]
 *   v_cache[s / block_size, s % block_size, :, :] = v[t, :, :]
 * Tokens with a negative slot are skipped (padding), and so are tokens whose
 * slot is num_blocks * block_size or more (no such slot in the cache).
 *
 * k, v          [num_tokens, num_kv_heads, head_dim] bf16; heads x dims
 *               contiguous, token rows k_token_stride / v_token_stride
 *               elements apart (>= num_kv_heads * head_dim; K and V may be
 *               column slices of a fused qkv projection output).
 * k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim] bf16.
 * slot_mapping  [num_tokens] int32. The slots stored to must be pairwise
 *               distinct (with a repeated slot the result is unspecified).
 * Bytes copied are exact (bit-for-bit), NaN patterns included.
 */
int pa_store_kvcache(const void* k, int64_t k_token_stride, const void* v, int64_t v_token_stride, void* k_cache,
                     void* v_cache, const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                     int32_t head_dim, int64_t num_blocks, int32_t block_size, void* stream);

/*
 * pa_qk_norm_rope_store — QK-RMSNorm and rotary embedding of the fused q/k/v
 * projection output, then the KV store, in one pass.
 *
 * Page "nano-vLLM 最小化vLLM重新实现", section 6 "模型" and "辅助层" (RMSNorm
 * of the q and k heads, RotaryEmbedding from a precomputed cos/sin cache) and
 * section 5 "注意力机制" (store by slot_mapping). For token t at position
 * p = positions[t] and each query or key head x (head_dim = 128) with weight w
 * (q_norm_weight for query heads, k_norm_weight for key heads):
 *   n = x / sqrt(mean(x^2) + eps) * w
 *   y[i]      = n[i] cos_sin[p, i] - n[i + 64] cos_sin[p, 64 + i]   (i < 64)
 *   y[i + 64] = n[i + 64] cos_sin[p, i] + n[i] cos_sin[p, 64 + i]
 * Query heads are written to q_out; with s = slot_mapping[t] in
 * [0, num_blocks * block_size), key heads are written to k_cache[s] and the
 * value heads copied bit for bit to v_cache[s]. Computed in fp32 from the bf16
 * inputs, rounded once to bf16 (round to nearest even).
 *
 * q_out         [num_tokens, num_q_heads, head_dim] bf16, rows
 *               q_out_token_stride elements apart. It may be the q columns of
 *               qkv itself (in place); any other overlap with qkv is undefined.
 * qkv           [num_tokens, (num_q_heads + 2 num_kv_heads) * head_dim] bf16:
 *               query heads, then key heads, then value heads; rows
 *               qkv_token_stride elements apart.
 * q_norm_weight, k_norm_weight  [head_dim] bf16.
 * eps           finite, >= 0.
 * cos_sin       [max_position, head_dim] fp32: row p holds the 64 cosines,
 *               then the 64 sines, of position p's angles.
 * positions     [num_tokens] int32; values outside [0, max_position) are
 *               clamped into it.
 * k_cache, v_cache, slot_mapping, num_blocks, block_size: as pa_store_kvcache;
 *               tokens whose slot is negative or >= num_blocks * block_size
 *               store nothing (their q is still written).
 * All pointers and strides 16-byte aligned; head_dim 128; num_q_heads a
 * multiple of num_kv_heads with group 1, 2, 4 or 8.
 */
int pa_qk_norm_rope_store(void* q_out, int64_t q_out_token_stride, const void* qkv, int64_t qkv_token_stride,
                          const void* q_norm_weight, const void* k_norm_weight, float eps, const float* cos_sin,
                          int32_t max_position, const int32_t* positions, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_blocks, int32_t block_size, void* stream);

/*
 * pa_decode_workspace_size — bytes of device workspace pa_decode needs.
 *
 * Host-only and pure. split_waves is the number of waves the decode work is
 * split over (0 = the library's choice, 2048, sized for the 256 CUs of an
 * MI355X; fewer when there is less work). The same arguments must be passed
 * to pa_decode. Returns 0 for invalid arguments.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t split_waves);

/* Number of waves pa_decode splits the work over for these arguments (0 if invalid). */
int32_t pa_decode_split_waves(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                              int32_t split_waves);

/*
 * pa_decode — paged GQA decode attention.
 *
 * Page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制" (decode attention
 * reading the paged KV cache) and page at bxzpzcl.cn/news/2159246, section
 * 2.2.2 (attention = softmax(q kᵀ * scale) v). For sequence b with
 * L = context_lens[b] and query head h:
 *   out[b, h, :] = sum_t w_t v_t,  w = softmax_t(scale * q[b, h] . k_t),
 * over positions t = 0 .. L-1, k_t / v_t being row t % block_size of block
 * block_tables[b, t / block_size], kv head h / G. L counts the token just
 * stored, so a new token attends to itself. L == 0 gives a zero row.
 * Arithmetic: bf16 inputs, fp32 accumulation and softmax, bf16 output
 * (round to nearest even). From G >= 4 the two products run on the matrix
 * cores, the softmax weights entering the second as two bf16 parts (about 16
 * significant bits).
 *
 * Work split: the (sequence, kv head) pairs are cut into chunks of 32 tokens
 * and the chunk sequence is shared equally among
 * split_waves waves; a pair cut by a share boundary is finished by a second,
 * small kernel from fp32 partials (max, sum, unnormalised output) in the
 * workspace (the split-K partition-and-reduce).
 *
 * out           [num_seqs, num_q_heads, head_dim] bf16, contiguous.
 * q             [num_seqs, num_q_heads, head_dim] bf16; heads x dims
 *               contiguous, rows q_seq_stride elements apart.
 * k_cache, v_cache  as in pa_store_kvcache.
 * block_tables  [num_seqs, max_blocks_per_seq] int32; entries past
 *               ceil(L / block_size) are never read.
 * context_lens  [num_seqs] int32, each in [0, max_context_len];
 *               max_context_len <= 2^24.
 * scale         softmax scale (1/sqrt(head_dim) for the pages' models).
 * workspace     device buffer of at least pa_decode_workspace_size(...) bytes,
 *               16-byte aligned; contents undefined after the call; must not
 *               be shared by work running concurrently.
 */
int pa_decode(void* out, const void* q, int64_t q_seq_stride, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_context_len, float scale, int32_t split_waves, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * pa_store_decode — the decode step's store and pa_decode in one call.
 *
 * Same result as pa_store_kvcache of each sequence's new token followed by
 * pa_decode (page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制": the
 * new token's K/V are written to the paged cache, then decode attends over
 * the cache): for every sequence b with L = context_lens[b] >= 1, row b of
 * k_new / v_new (kv heads x dims) is written to position L - 1 of the
 * sequence, i.e. row (L - 1) % block_size of block
 * block_tables[b, (L - 1) / block_size], and out is pa_decode's output over
 * positions 0 .. L - 1, the new token included. Sequences with L == 0 store
 * nothing and give zero rows. The new token's position comes from the block
 * table (no slot_mapping). Two kernels run: the split kernel takes position
 * L - 1's K/V from k_new / v_new instead of the cache (in the one chunk
 * that covers it), and the finalize kernel, which runs after it, writes the
 * row into the cache, so nothing in the call reads the cache row before it
 * is written.
 *
 * k_new, v_new  [num_seqs, num_kv_heads, head_dim] bf16, heads x dims
 *               contiguous, rows k_new_stride / v_new_stride elements apart
 *               (16-byte aligned, at least num_kv_heads * head_dim).
 * k_cache, v_cache  written (the new rows) and read.
 * Every other argument, the workspace and the errors as in pa_decode.
 */
int pa_store_decode(void* out, const void* q, int64_t q_seq_stride, const void* k_new, int64_t k_new_stride,
                    const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_context_len, float scale, int32_t split_waves, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pa_store_decode_noalloc — pa_store_decode without a caller workspace.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments, checks, kernels and results as pa_store_decode (bit for bit),
 * with the workspace taken from a static device array inside the library
 * (16.25 MiB per GPU, held until the process ends; its address is looked up
 * once per device on the first call there). Nothing is allocated: no
 * hipMalloc, no hipFree.
 *
 * Limit: the split must fit the static scratch, i.e. split_waves (or the
 * library's default of 2048) times 2 slots times G query heads per kv head
 * times 520 bytes at most 17,039,360 bytes; the default split fits every
 * supported group. Larger splits return PA_ERR_WORKSPACE_TOO_SMALL and launch
 * nothing.
 *
 * Every call on one GPU shares that GPU's scratch, and nothing in it has to
 * start at zero (each call's finalize pass reads only what its split kernel
 * wrote). Calls that overlap on one GPU (concurrent streams, or threads)
 * race on it and give undefined results; calls ordered on one stream are
 * safe.
 */
int pa_store_decode_noalloc(void* out, const void* q, int64_t q_seq_stride, const void* k_new, int64_t k_new_stride,
                            const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_context_len, float scale, int32_t split_waves,
                            void* stream);

/*
 * pa_prefill_varlen — attention over packed variable-length sequences.
 *
 * Page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制": prefill over
 * variable-length sequences split by cu_seqlens, with an optional block table
 * so that prefix-cached blocks are reused (page at hotelren.com/news/2273631,
 * section 4.4: only the part after the cached prefix is computed).
 * Sequence i has nq = cu_seqlens_q[i+1] - cu_seqlens_q[i] queries and
 * nk = cu_seqlens_k[i+1] - cu_seqlens_k[i] keys, nk >= nq. With causal != 0,
 * query j sits at position nk - nq + j and sees keys 0 .. nk - nq + j (the
 * queries are the last nq positions); with causal == 0 it sees all nk keys.
 *   out[q_i + j, h, :] = softmax_t(scale * q[q_i + j, h] . k_t) . v_t
 * with kv head h / G. Arithmetic: bf16 inputs, bf16 MFMA with fp32
 * accumulation for q.k and p.v, fp32 softmax, p rounded to bf16 for the p.v
 * product, bf16 output.
 *
 * out           [total_q, num_q_heads, head_dim] bf16, contiguous.
 * q             [total_q, num_q_heads, head_dim] bf16, rows q_token_stride apart.
 * k, v          block_table == NULL: packed [total_k, num_kv_heads, head_dim]
 *               bf16, rows k_token_stride / v_token_stride apart, sequence i's
 *               keys at rows cu_seqlens_k[i] ..;
 *               block_table != NULL: the caches [num_blocks, block_size,
 *               num_kv_heads, head_dim] (the strides are then ignored), key
 *               t of sequence i at row t % block_size of block
 *               block_table[i, t / block_size]. Token strides and
 *               num_kv_heads * head_dim above 2^23 elements return
 *               PA_ERR_UNSUPPORTED.
 * cu_seqlens_q, cu_seqlens_k  [num_seqs + 1] int32, non-decreasing from 0.
 * max_seqlen_q  upper bound of every nq (sizes the launch grid).
 * max_seqlen_k  the longest key range the caller expects; selects the key
 *               tile (32 keys up to 1024, else 64). Results do not depend on
 *               it. With a block table, a value above max_blocks_per_seq *
 *               block_size returns PA_ERR_INVALID_ARGUMENT (the table cannot
 *               address that many keys).
 * block_table   optional [num_seqs, max_blocks_per_seq] int32; row i must
 *               name a block for every one of sequence i's keys
 *               (max_blocks_per_seq * block_size >= nk, a precondition the
 *               device does not check); entries past max_blocks_per_seq are
 *               never read.
 */
int pa_prefill_varlen(void* out, const void* q, int64_t q_token_stride, const void* k, const void* v,
                      int64_t k_token_stride, int64_t v_token_stride, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
                      const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size, void* stream);

/*
 * pa_sample_gumbel — one token per row by the Gumbel-max trick.
 *
 * Page "nano-vLLM 最小化vLLM重新实现", "辅助层" (the sampler: exponential
 * noise, then an argmax) and "关键设计选择" (temperature > 1e-10, no greedy
 * sampling). For row b with logits l (vocab_size of them) and temperature
 * T = max(temperatures[b], 1e-10):
 *   tokens[b] = argmax_i softmax(l / T)_i / E_i,  E_i = -ln(u_i),
 * which draws token i with probability softmax(l / T)_i. u_i comes from
 * Philox4x32-10 (Salmon et al., SC 2011) under key (seed mod 2^32, seed div
 * 2^32): element i takes field i % 6 of the block at counter (i / 6, b,
 * offset mod 2^32, offset div 2^32). The block's 32-bit words w0..w3 form
 * X0 = w1:w0 and X1 = w3:w2; fields 0, 1, 2 are bits 63..43, 42..22, 21..1 of
 * X0 and fields 3, 4, 5 the same bits of X1; a field w gives u = (w + 1/2) /
 * 2^21. Pass a new offset (e.g. the step number) for new noise. The decision
 * is taken in fp32 (l log2(e) / T - log2(-log2(u))); ties go to the lowest
 * index; -inf logits are never drawn unless a whole row is -inf (then token 0
 * by the tie rule); NaN logits give an unspecified token in [0, vocab_size).
 *
 * tokens        [num_rows] int32 (device).
 * logits        [num_rows, vocab_size] fp32, rows logits_row_stride elements
 *               apart (>= vocab_size; rows starting 16-byte aligned are read
 *               with 16-byte loads).
 * temperatures  [num_rows] fp32.
 * workspace     >= pa_sample_workspace_size(num_rows, vocab_size) bytes,
 *               16-byte aligned, owned by the caller.
 */
size_t pa_sample_workspace_size(int32_t num_rows, int32_t vocab_size);
int pa_sample_gumbel(int32_t* tokens, const float* logits, int64_t logits_row_stride, const float* temperatures,
                     int32_t num_rows, int32_t vocab_size, uint64_t seed, uint64_t offset, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_store_prefill_varlen — the prefill step's store and pa_prefill_varlen in
 * one call.
 *
 * Same results as pa_store_kvcache of the new tokens followed by
 * pa_prefill_varlen (page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制":
 * the new tokens' K/V are written to the paged cache by slot_mapping, then
 * varlen prefill attends over them, through the block table when a prefix is
 * cached; page at hotelren.com/news/2273631, section 4.4). The new tokens are
 * one per query: new token j of sequence i is row cu_seqlens_q[i] + j of
 * k_new / v_new and is the key at position nk - nq + j; it is stored at
 * slot_mapping[cu_seqlens_q[i] + j] (skipped when that slot is negative or at
 * least num_blocks * block_size).
 *
 * block_table == NULL: every key is a new token, so each sequence must have
 *   nk == nq (cu_seqlens_k equal to cu_seqlens_q); keys come from k_new /
 *   v_new.
 * block_table != NULL: keys 0 .. nk - nq - 1 come from the cache through the
 *   table, keys nk - nq .. nk - 1 from k_new / v_new (they are not read back
 *   from the cache). The result equals the unfused pair when every new
 *   token's slot is its position through the table (slot = block_table[i,
 *   p / block_size] * block_size + p % block_size), as a block manager makes
 *   them; that is a precondition.
 *
 * The query tile of each work item stores its own tokens (each row is written
 * once), after its attention, from the rows its last tiles just read. Cache
 * bytes are bit-exact copies. Outputs are bit-identical to the unfused pair's
 * at the same key tile; with a block table the fused call always runs 64-key
 * tiles (pa_prefill_varlen picks 32-key tiles up to max_seqlen_k 1024), so
 * there the two may differ by rounding only.
 *
 * k_new, v_new  [total_q, num_kv_heads, head_dim] bf16, heads x dims
 *               contiguous, rows k_new_stride / v_new_stride elements apart.
 * k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim]: written
 *               at the new tokens' slots; read through block_table if given.
 * slot_mapping  [total_q] int32.
 * num_blocks    positive, num_blocks * block_size < 2^31.
 * Every other argument, and the errors, as in pa_prefill_varlen.
 */
int pa_store_prefill_varlen(void* out, const void* q, int64_t q_token_stride, const void* k_new,
                            int64_t k_new_stride, const void* v_new, int64_t v_new_stride, void* k_cache,
                            void* v_cache, const int32_t* slot_mapping, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            float scale, int32_t causal, const int32_t* block_table, int32_t max_blocks_per_seq,
                            int32_t block_size, int64_t num_blocks, void* stream);

/*
 * Graph-captured decode steps (pa_store_decode: the new tokens' store and the
 * paged decode, two kernels), one HIP graph per padded batch size, each step
 * replayed with a single graph launch (page "nano-vLLM 最小化vLLM重新实现",
 * section 4 "模型运行器": decode graphs are captured ahead of time at batch
 * sizes 1, 2, 4, 8, 16, 32, ..., 512 and replayed; page at
 * bxzpzcl.cn/news/2159246, section 3.1: graphs remove the per-step launch
 * overhead).
 *
 * pa_decode_step names the device buffers every captured graph reads and
 * writes, sized for the largest batch size: row i of q, k_new, v_new,
 * block_tables, context_lens and out belongs to sequence i of the step.
 * Before each launch the caller fills rows 0 .. batch - 1 and writes batch to
 * *live_batch (a device int32), together with the step's other inputs. The
 * graph of padded size P treats rows batch .. P - 1 as empty contexts:
 * nothing is stored for them, their output rows are zeros, and nothing else of
 * theirs is read (their context_lens entries are read and ignored), so they
 * need not be written. Results of rows 0 .. batch - 1 equal pa_store_decode at
 * batch rows, bit for bit. max_context_len bounds every context length of
 * every launch; workspace must hold pa_decode_workspace_size() for the
 * largest batch size. The buffers must stay allocated, and the struct's values
 * fixed, while the graphs exist.
 */
typedef struct pa_decode_step {
  const void* q;              /* [max_batch, num_q_heads, head_dim] bf16 */
  int64_t q_seq_stride;
  const void* k_new;          /* [max_batch, num_kv_heads, head_dim] bf16 */
  int64_t k_token_stride;
  const void* v_new;
  int64_t v_token_stride;
  const int32_t* live_batch;  /* one device int32: the batch of the next launch */
  const int32_t* block_tables; /* [max_batch, max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
  const int32_t* context_lens; /* [max_batch] */
  void* out;                  /* [max_batch, num_q_heads, head_dim] bf16 */
  void* workspace;
  size_t workspace_bytes;
  void* k_cache;
  void* v_cache;
  int32_t block_size;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float scale;
  int32_t max_context_len;
  int32_t split_waves;
} pa_decode_step;

typedef struct pa_decode_graphs pa_decode_graphs;

/*
 * Capture one graph per entry of batch_sizes (positive, strictly increasing,
 * at most 32 of them) on stream, which must not be the legacy default stream.
 * Each graph is pa_store_decode at that batch size with the step's arguments
 * and its live count; capturing launches nothing. Errors of the captured
 * calls are returned as they are (and nothing is kept); a failed capture
 * returns PA_ERR_HIP.
 */
int pa_decode_graphs_create(const pa_decode_step* step, const int32_t* batch_sizes, int32_t count, void* stream,
                            pa_decode_graphs** out);

/*
 * One decode step of batch sequences (1 <= batch <= the largest captured
 * size): one launch of the graph of the smallest captured size padded >=
 * batch on stream. *live_batch must already hold batch on the device (written
 * by the caller before this call, in stream order). *padded (optional)
 * receives the padded size.
 */
int pa_decode_graphs_launch(pa_decode_graphs* graphs, int32_t batch, void* stream, int32_t* padded);

void pa_decode_graphs_destroy(pa_decode_graphs* graphs);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
