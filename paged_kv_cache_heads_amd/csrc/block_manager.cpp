// Host-side KV block manager (include/pa_blocks.h): the block pool, per-
// sequence block tables and prefix reuse by chained token-block hashes (page
// "nano-vLLM 最小化vLLM重新实现", section 3 "块管理器"; page at
// hotelren.com/news/2273631, sections 2.2 and 4.4).
//
// Data structures: the free list is an intrusive doubly linked list over the
// block array (O(1) take-from-front, release-to-back and removal of a cached
// block that a prompt hits while it is free); the prefix cache maps a block
// hash to the block holding that content; each hashed block keeps its parent
// hash and token ids so a hit is confirmed by comparison, not by the hash
// alone. Metadata for the kernels is written straight into caller arrays.
#include "../../include/pa_blocks.h"

#include <string.h>

#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "launch.h"

namespace {

// ---- XXH64, the published 64-bit xxHash ----
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t kP3 = 0x165667B19E3779F9ull;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ull;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t read64(const unsigned char* p) {
  uint64_t v;
  memcpy(&v, p, 8);  // little-endian host
  return v;
}
inline uint32_t read32(const unsigned char* p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}
inline uint64_t xxh_round(uint64_t acc, uint64_t lane) {
  acc += lane * kP2;
  acc = rotl(acc, 31);
  return acc * kP1;
}
inline uint64_t xxh_merge(uint64_t h, uint64_t acc) {
  h ^= xxh_round(0, acc);
  return h * kP1 + kP4;
}

uint64_t xxh64(const void* data, size_t len, uint64_t seed) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  const unsigned char* end = p + len;
  uint64_t h;
  if (len >= 32) {
    uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
    const unsigned char* limit = end - 32;
    do {
      v1 = xxh_round(v1, read64(p));
      v2 = xxh_round(v2, read64(p + 8));
      v3 = xxh_round(v3, read64(p + 16));
      v4 = xxh_round(v4, read64(p + 24));
      p += 32;
    } while (p <= limit);
    h = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
    h = xxh_merge(h, v1);
    h = xxh_merge(h, v2);
    h = xxh_merge(h, v3);
    h = xxh_merge(h, v4);
  } else {
    h = seed + kP5;
  }
  h += (uint64_t)len;
  for (; p + 8 <= end; p += 8) {
    h ^= xxh_round(0, read64(p));
    h = rotl(h, 27) * kP1 + kP4;
  }
  if (p + 4 <= end) {
    h ^= (uint64_t)read32(p) * kP1;
    h = rotl(h, 23) * kP2 + kP3;
    p += 4;
  }
  for (; p < end; ++p) {
    h ^= (uint64_t)(*p) * kP5;
    h = rotl(h, 11) * kP1;
  }
  h ^= h >> 33;
  h *= kP2;
  h ^= h >> 29;
  h *= kP3;
  h ^= h >> 32;
  return h;
}

// Hash of one block of token ids (int32, little-endian), chained through seed.
inline uint64_t block_hash(const int32_t* tokens, int32_t n, uint64_t seed) {
  return xxh64(tokens, (size_t)n * sizeof(int32_t), seed);
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;
  uint64_t hash = 0, parent = 0;
  std::vector<int32_t> tokens;  // content of a hashed (full) block
  int32_t prev = -1, next = -1;  // free-list links
  bool free = false;
};

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
  uint64_t last_hash = 0;          // hash of the last full block (0 if none)
  std::vector<int32_t> partial;    // tokens of the last, not yet full block
};

}  // namespace

struct pa_block_manager {
  int32_t block_size = 0;
  std::vector<Block> blocks;
  int32_t head = -1, tail = -1, num_free = 0;
  std::unordered_map<uint64_t, int32_t> cache;
  std::unordered_map<int64_t, Seq> seqs;

  void push_back(int32_t b) {
    Block& x = blocks[b];
    x.prev = tail, x.next = -1, x.free = true;
    if (tail >= 0) blocks[tail].next = b;
    else head = b;
    tail = b;
    ++num_free;
  }
  void unlink(int32_t b) {
    Block& x = blocks[b];
    if (x.prev >= 0) blocks[x.prev].next = x.next;
    else head = x.next;
    if (x.next >= 0) blocks[x.next].prev = x.prev;
    else tail = x.prev;
    x.prev = x.next = -1, x.free = false;
    --num_free;
  }
  // Take the front block for new content: it leaves the cache if it was there.
  int32_t take() {
    const int32_t b = head;
    unlink(b);
    Block& x = blocks[b];
    if (x.hashed) {
      auto it = cache.find(x.hash);
      if (it != cache.end() && it->second == b) cache.erase(it);
    }
    x.hashed = false;
    x.tokens.clear();
    x.ref = 1;
    return b;
  }
  void register_block(int32_t b, uint64_t h, uint64_t parent, const int32_t* toks) {
    Block& x = blocks[b];
    x.hashed = true, x.hash = h, x.parent = parent;
    x.tokens.assign(toks, toks + block_size);
    cache.emplace(h, b);  // kept if the hash is already registered
  }
  // The cached block holding these tokens after this parent, or -1.
  int32_t lookup(uint64_t h, uint64_t parent, const int32_t* toks) const {
    auto it = cache.find(h);
    if (it == cache.end()) return -1;
    const Block& x = blocks[it->second];
    if (x.parent != parent || memcmp(x.tokens.data(), toks, (size_t)block_size * sizeof(int32_t)) != 0) return -1;
    return it->second;
  }
};

using pa::fail;
using pa::ok;

extern "C" {

uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed) { return xxh64(data, len, seed); }

int pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* order, pa_block_manager** out) {
  if (!out) return fail(PA_ERR_NULL_POINTER, "out is required");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks (%d) and block_size (%d) must be positive", num_blocks,
                block_size);
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_blocks * block_size exceeds the int32 slot range");
  pa_block_manager* bm = new pa_block_manager();
  bm->block_size = block_size;
  bm->blocks.resize(num_blocks);
  if (order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return fail(PA_ERR_INVALID_ARGUMENT, "order is not a permutation of 0 .. %d", num_blocks - 1);
      }
      seen[b] = 1;
      bm->push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->push_back(b);
  }
  *out = bm;
  return ok();
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                   int32_t* num_cached) {
  if (!bm) return fail(PA_ERR_NULL_POINTER, "manager is required");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens %d is negative", num_tokens);
  if (num_tokens > 0 && !tokens) return fail(PA_ERR_NULL_POINTER, "tokens is required");
  if (bm->seqs.count(seq_id)) return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is already live", (long long)seq_id);
  const int32_t bs = bm->block_size;
  const int64_t n = num_tokens;
  const int64_t nblocks = (n + bs - 1) / bs;
  // longest cached prefix of full blocks (leaving at least one token to compute)
  std::vector<int32_t> hits;
  uint64_t h = 0;
  const int64_t cacheable = n > 0 ? (n - 1) / bs : 0;
  for (int64_t i = 0; i < cacheable; ++i) {
    const int32_t* blk = tokens + i * bs;
    const uint64_t hi = block_hash(blk, bs, h);
    const int32_t b = bm->lookup(hi, h, blk);
    if (b < 0) break;
    hits.push_back(b);
    h = hi;
  }
  int64_t from_free = 0;
  for (int32_t b : hits) from_free += bm->blocks[b].ref == 0;
  if (nblocks - (int64_t)hits.size() + from_free > bm->num_free)
    return fail(PA_ERR_NO_BLOCKS, "prompt of %d tokens needs %lld blocks, %d free", num_tokens,
                (long long)(nblocks - (int64_t)hits.size() + from_free), bm->num_free);
  Seq s;
  s.table.reserve(nblocks);
  for (int32_t b : hits) {
    if (bm->blocks[b].ref == 0) bm->unlink(b);
    ++bm->blocks[b].ref;
    s.table.push_back(b);
  }
  for (int64_t i = (int64_t)hits.size(); i < nblocks; ++i) {
    const int32_t b = bm->take();
    s.table.push_back(b);
    if ((i + 1) * bs <= n) {
      const int32_t* blk = tokens + i * bs;
      const uint64_t hi = block_hash(blk, bs, h);
      bm->register_block(b, hi, h, blk);
      h = hi;
    }
  }
  const int64_t full = n / bs;
  s.len = n;
  s.last_hash = full ? h : 0;
  s.partial.assign(tokens + full * bs, tokens + n);
  bm->seqs.emplace(seq_id, std::move(s));
  if (num_cached) *num_cached = (int32_t)(hits.size() * bs);
  return ok();
}

int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t token) {
  if (!bm) return fail(PA_ERR_NULL_POINTER, "manager is required");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "sequence %lld is not live", (long long)seq_id);
  Seq& s = it->second;
  const int32_t bs = bm->block_size;
  if (s.len % bs == 0) {
    if (bm->num_free == 0) return fail(PA_ERR_NO_BLOCKS, "no free block for sequence %lld", (long long)seq_id);
    s.table.push_back(bm->take());
  }
  s.partial.push_back(token);
  ++s.len;
  if (s.len % bs == 0) {
    const uint64_t hi = block_hash(s.partial.data(), bs, s.last_hash);
    bm->register_block(s.table.back(), hi, s.last_hash, s.partial.data());
    s.last_hash = hi;
    s.partial.clear();
  }
  return ok();
}

int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t count,
                       int32_t* num_done) {
  if (num_done) *num_done = 0;
  if (!bm) return fail(PA_ERR_NULL_POINTER, "manager is required");
  if (count < 0) return fail(PA_ERR_INVALID_ARGUMENT, "count %d is negative", count);
  if (count > 0 && (!seq_ids || !tokens)) return fail(PA_ERR_NULL_POINTER, "seq_ids and tokens are required");
  for (int32_t i = 0; i < count; ++i) {
    const int st = pa_bm_append(bm, seq_ids[i], tokens[i]);
    if (st != PA_OK) return st;
    if (num_done) *num_done = i + 1;
  }
  return ok();
}

int pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return fail(PA_ERR_NULL_POINTER, "manager is required");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "sequence %lld is not live", (long long)seq_id);
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b)
    if (--bm->blocks[*b].ref == 0) bm->push_back(*b);
  bm->seqs.erase(it);
  return ok();
}

int32_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->num_free : -1; }

int32_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : (int32_t)it->second.len;
}

int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity,
                      int32_t* num_blocks) {
  if (!bm || !num_blocks) return fail(PA_ERR_NULL_POINTER, "manager and num_blocks are required");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "sequence %lld is not live", (long long)seq_id);
  const std::vector<int32_t>& t = it->second.table;
  *num_blocks = (int32_t)t.size();
  if ((int64_t)t.size() > capacity || (!out && !t.empty()))
    return fail(PA_ERR_INVALID_ARGUMENT, "table of %zu blocks does not fit %d", t.size(), capacity);
  if (!t.empty()) memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return ok();
}

int pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int32_t capacity, int32_t* count) {
  if (!bm || !count) return fail(PA_ERR_NULL_POINTER, "manager and count are required");
  *count = bm->num_free;
  if (bm->num_free > capacity || (!out && bm->num_free))
    return fail(PA_ERR_INVALID_ARGUMENT, "free list of %d blocks does not fit %d", bm->num_free, capacity);
  int32_t i = 0;
  for (int32_t b = bm->head; b >= 0; b = bm->blocks[b].next) out[i++] = b;
  return ok();
}

int32_t pa_bm_block_ref(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= (int32_t)bm->blocks.size()) return -1;
  return bm->blocks[block].ref;
}

int pa_bm_decode_metadata(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs, int32_t width,
                          int32_t* block_tables, int32_t* context_lens, int32_t* slot_mapping) {
  if (!bm) return fail(PA_ERR_NULL_POINTER, "manager is required");
  if (num_seqs < 0 || width <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d / width %d", num_seqs, width);
  if (num_seqs == 0) return ok();
  if (!seq_ids || !block_tables || !context_lens || !slot_mapping)
    return fail(PA_ERR_NULL_POINTER, "seq_ids and the output arrays are required");
  const int32_t bs = bm->block_size;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "sequence %lld is not live", (long long)seq_ids[i]);
    if ((int64_t)it->second.table.size() > width)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld needs %zu table entries > width %d",
                  (long long)seq_ids[i], it->second.table.size(), width);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * width;
    const int32_t nb = (int32_t)s.table.size();
    for (int32_t j = 0; j < width; ++j) row[j] = j < nb ? s.table[j] : -1;
    context_lens[i] = (int32_t)s.len;
    slot_mapping[i] = s.len > 0 ? s.table[(s.len - 1) / bs] * bs + (int32_t)((s.len - 1) % bs) : -1;
  }
  return ok();
}

int pa_bm_prefill_metadata(const pa_block_manager* bm, const int64_t* seq_ids, const int32_t* num_cached,
                           int32_t num_seqs, int32_t width, int32_t* block_tables, int32_t* cu_seqlens_q,
                           int32_t* cu_seqlens_k, int32_t* slot_mapping, int64_t slot_capacity) {
  if (!bm) return fail(PA_ERR_NULL_POINTER, "manager is required");
  if (num_seqs < 0 || width <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d / width %d", num_seqs, width);
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(PA_ERR_NULL_POINTER, "cu_seqlens_q and cu_seqlens_k are required");
  cu_seqlens_q[0] = cu_seqlens_k[0] = 0;
  if (num_seqs == 0) return ok();
  if (!seq_ids || !num_cached || !block_tables) return fail(PA_ERR_NULL_POINTER, "inputs and block_tables are required");
  int64_t total_q = 0, total_k = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "sequence %lld is not live", (long long)seq_ids[i]);
    const Seq& s = it->second;
    if (num_cached[i] < 0 || num_cached[i] > s.len)
      return fail(PA_ERR_INVALID_ARGUMENT, "num_cached[%d] = %d outside 0 .. %lld", i, num_cached[i], (long long)s.len);
    if ((int64_t)s.table.size() > width)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld needs %zu table entries > width %d",
                  (long long)seq_ids[i], s.table.size(), width);
    total_q += s.len - num_cached[i];
    total_k += s.len;
  }
  if (total_k > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "more than 2^31 - 1 keys in one batch");
  if (total_q > slot_capacity || (total_q > 0 && !slot_mapping))
    return fail(PA_ERR_INVALID_ARGUMENT, "%lld query tokens do not fit slot_capacity %lld", (long long)total_q,
                (long long)slot_capacity);
  const int32_t bs = bm->block_size;
  int64_t q = 0, k = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * width;
    const int32_t nb = (int32_t)s.table.size();
    for (int32_t j = 0; j < width; ++j) row[j] = j < nb ? s.table[j] : -1;
    for (int64_t p = num_cached[i]; p < s.len; ++p) slot_mapping[q++] = s.table[p / bs] * bs + (int32_t)(p % bs);
    k += s.len;
    cu_seqlens_q[i + 1] = (int32_t)q;
    cu_seqlens_k[i + 1] = (int32_t)k;
  }
  return ok();
}

}  // extern "C"
