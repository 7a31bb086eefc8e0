// Host-side KV block manager with prefix caching: the allocator that produces the
// block tables and slot mappings the decode kernels consume.
//
// The pages describe the paged KV cache as managed in fixed-size blocks with
// prefix caching (miniVLLM docs, "What is miniVLLM?") and the engine's block
// manager / block allocation (hysenlabs MinivLLM review, "The structure
// block ..." and "What main.py actually does"); the review lists xxhash among
// the dependencies, i.e. blocks are identified by a hash of their tokens. This
// file is written from that description:
//
//  * A block is "full" when all block_size of its token slots are known. A full
//    block's key is a 64-bit chained hash of (key of the previous block of the
//    sequence, its block_size token ids), so equal keys mean equal prefixes.
//    Keys index a table of cached blocks; a match is confirmed by comparing the
//    stored token ids and the stored key of the previous block, so aliasing two
//    different prefixes would need a collision of the 64-bit chained keys.
//  * Blocks are reference counted. A sequence whose leading full blocks match
//    cached ones reuses them (count + 1); its tokens there need no recompute.
//  * A freed block whose count drops to zero stays cached (evictable, least
//    recently freed first) if it is full, and returns to the free list if not.
//    Allocation takes free blocks first, then evicts the oldest cached block.
//  * fork() shares every block of a sequence with a new one (parallel sampling).
//    Appending to a shared, partially filled last block copies it first
//    (copy-on-write): the manager picks the destination and reports the copy
//    the caller must perform on the device.
//
// The hash mixes 64-bit words with the splitmix64 finalizer (Steele, Lea and
// Flood, "Fast splittable pseudorandom number generators", 2014).

#include "pagedattn.h"

#include <stdarg.h>
#include <stdio.h>

#include <cstdint>
#include <list>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

thread_local std::string t_bm_error;

int bm_fail(int code, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_bm_error = buf;
  return code;
}

uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t block_key(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = mix64(parent ^ 0x6A09E667F3BCC908ull);
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h;
}

constexpr uint64_t kRootKey = 0x3C6EF372FE94F82Bull;

struct Block {
  int32_t ref = 0;
  bool hashed = false;           // full and registered in the cache table
  uint64_t key = 0;
  uint64_t parent_key = 0;       // key of the previous block of the sequence that filled it
  std::vector<int32_t> tokens;   // token ids of a full block (for collision checks)
  std::list<int32_t>::iterator lru;  // position in the evictable list when ref == 0 && hashed
  bool in_lru = false;
};

struct Sequence {
  std::vector<int32_t> blocks;
  std::vector<int32_t> tokens;
  uint64_t last_full_key = 0;  // chained key of the sequence's last full block (root key if none)
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<Block> blocks;
  std::vector<int32_t> free_list;        // never-hashed free blocks (stack)
  std::list<int32_t> evictable;          // cached blocks with ref 0, oldest first
  std::unordered_map<uint64_t, int32_t> cache;  // key -> block
  std::unordered_map<int64_t, Sequence> seqs;
  std::mutex mu;
  int64_t hits = 0, misses = 0, evictions = 0;

  int32_t available() const { return (int32_t)(free_list.size() + evictable.size()); }

  void unlink_lru(int32_t b) {
    Block& blk = blocks[b];
    if (blk.in_lru) {
      evictable.erase(blk.lru);
      blk.in_lru = false;
    }
  }

  void unregister(int32_t b) {
    Block& blk = blocks[b];
    if (blk.hashed) {
      auto it = cache.find(blk.key);
      if (it != cache.end() && it->second == b) cache.erase(it);
      blk.hashed = false;
      blk.tokens.clear();
    }
  }

  // A block with ref 1 and no cache entry; -1 if none is left.
  int32_t take() {
    int32_t b = -1;
    if (!free_list.empty()) {
      b = free_list.back();
      free_list.pop_back();
    } else if (!evictable.empty()) {
      b = evictable.front();
      evictable.pop_front();
      blocks[b].in_lru = false;
      unregister(b);
      ++evictions;
    } else {
      return -1;
    }
    blocks[b].ref = 1;
    return b;
  }

  void release(int32_t b) {
    Block& blk = blocks[b];
    if (--blk.ref > 0) return;
    if (blk.hashed) {
      evictable.push_back(b);
      blk.lru = std::prev(evictable.end());
      blk.in_lru = true;
    } else {
      free_list.push_back(b);
    }
  }

  // Registers block b (full, holding `tokens`) under `key` unless the key is already cached.
  void register_full(int32_t b, uint64_t key, uint64_t parent_key, const int32_t* tokens) {
    Block& blk = blocks[b];
    if (blk.hashed || cache.count(key)) return;
    blk.hashed = true;
    blk.key = key;
    blk.parent_key = parent_key;
    blk.tokens.assign(tokens, tokens + block_size);
    cache.emplace(key, b);
  }

};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) {
    bm_fail(PA_ERR_SHAPE, "num_blocks %d and block_size %d must be positive", num_blocks, block_size);
    return nullptr;
  }
  pa_block_manager* m = new pa_block_manager();
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->blocks.resize(num_blocks);
  m->free_list.reserve(num_blocks);
  for (int32_t b = num_blocks - 1; b >= 0; --b) m->free_list.push_back(b);  // hand out 0, 1, 2, ... first
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                       int32_t* num_cached_tokens) {
  if (!m) return bm_fail(PA_ERR_NULL, "manager is NULL");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) return bm_fail(PA_ERR_SHAPE, "bad token list");
  std::lock_guard<std::mutex> lock(m->mu);
  if (m->seqs.count(seq_id)) return bm_fail(PA_ERR_SHAPE, "sequence %lld already exists", (long long)seq_id);
  const int bs = m->block_size;
  const int nfull = num_tokens / bs;
  const int nblk = (num_tokens + bs - 1) / bs;
  // Leading full blocks already cached: walk keys until the first miss.
  std::vector<int32_t> hit_blocks;
  uint64_t key = kRootKey;
  std::vector<uint64_t> keys(nfull);
  for (int j = 0; j < nfull; ++j) {
    key = block_key(key, tokens + (size_t)j * bs, bs);
    keys[j] = key;
  }
  for (int j = 0; j < nfull; ++j) {
    auto it = m->cache.find(keys[j]);
    if (it == m->cache.end()) break;
    const Block& blk = m->blocks[it->second];
    bool same = blk.parent_key == (j > 0 ? keys[j - 1] : kRootKey);
    for (int i = 0; i < bs && same; ++i) same = blk.tokens[i] == tokens[(size_t)j * bs + i];
    if (!same) break;
    hit_blocks.push_back(it->second);
  }
  // Capacity: hits that are evictable leave the pool when reused; new blocks come from the rest.
  int32_t hits_from_lru = 0;
  for (int32_t b : hit_blocks) hits_from_lru += m->blocks[b].ref == 0 ? 1 : 0;
  const int32_t need = nblk - (int32_t)hit_blocks.size();
  if (m->available() - hits_from_lru < need)
    return bm_fail(PA_ERR_CAPACITY, "need %d free blocks, %d available", need, m->available() - hits_from_lru);
  Sequence s;
  s.tokens.assign(tokens, tokens + num_tokens);
  s.last_full_key = nfull > 0 ? keys[nfull - 1] : kRootKey;
  for (int32_t b : hit_blocks) {
    Block& blk = m->blocks[b];
    if (blk.ref == 0) m->unlink_lru(b);
    ++blk.ref;
    s.blocks.push_back(b);
  }
  m->hits += (int64_t)hit_blocks.size();
  for (int j = (int)hit_blocks.size(); j < nblk; ++j) {
    const int32_t b = m->take();
    s.blocks.push_back(b);
    ++m->misses;
    if (j < nfull) m->register_full(b, keys[j], j > 0 ? keys[j - 1] : kRootKey, tokens + (size_t)j * bs);
  }
  if (num_cached_tokens) *num_cached_tokens = (int32_t)hit_blocks.size() * bs;
  m->seqs.emplace(seq_id, std::move(s));
  t_bm_error.clear();
  return PA_OK;
}

int pa_bm_append_token(pa_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot, int32_t* copy_src,
                       int32_t* copy_dst) {
  if (!m || !slot) return bm_fail(PA_ERR_NULL, "manager or slot is NULL");
  std::lock_guard<std::mutex> lock(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PA_ERR_SHAPE, "unknown sequence %lld", (long long)seq_id);
  Sequence& s = it->second;
  const int bs = m->block_size;
  const int64_t pos = (int64_t)s.tokens.size();
  const int off = (int)(pos % bs);
  if (copy_src) *copy_src = -1;
  if (copy_dst) *copy_dst = -1;
  if (off == 0) {
    const int32_t b = m->take();
    if (b < 0) return bm_fail(PA_ERR_CAPACITY, "no free block for sequence %lld", (long long)seq_id);
    s.blocks.push_back(b);
  } else {
    const int32_t last = s.blocks.back();
    if (m->blocks[last].ref > 1) {
      // Shared partial block: the new token must not become visible to the other owners.
      const int32_t b = m->take();
      if (b < 0) return bm_fail(PA_ERR_CAPACITY, "no free block for copy-on-write");
      m->release(last);
      s.blocks.back() = b;
      if (copy_src) *copy_src = last;
      if (copy_dst) *copy_dst = b;
    }
  }
  s.tokens.push_back(token);
  const int32_t b = s.blocks.back();
  *slot = b * bs + off;
  if (off == bs - 1) {
    const uint64_t parent = s.last_full_key;
    s.last_full_key = block_key(parent, s.tokens.data() + (pos - off), bs);
    m->register_full(b, s.last_full_key, parent, s.tokens.data() + (pos - off));
  }
  t_bm_error.clear();
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id) {
  if (!m) return bm_fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lock(m->mu);
  auto it = m->seqs.find(parent_id);
  if (it == m->seqs.end()) return bm_fail(PA_ERR_SHAPE, "unknown sequence %lld", (long long)parent_id);
  if (m->seqs.count(child_id)) return bm_fail(PA_ERR_SHAPE, "sequence %lld already exists", (long long)child_id);
  Sequence child = it->second;
  for (int32_t b : child.blocks) ++m->blocks[b].ref;
  m->seqs.emplace(child_id, std::move(child));
  t_bm_error.clear();
  return PA_OK;
}

int pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id) {
  if (!m) return bm_fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lock(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PA_ERR_SHAPE, "unknown sequence %lld", (long long)seq_id);
  // Release from the last block backwards so a prefix's leading blocks are evicted last.
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) m->release(*b);
  m->seqs.erase(it);
  t_bm_error.clear();
  return PA_OK;
}

int pa_bm_block_table(pa_block_manager* m, int64_t seq_id, int32_t* out, int32_t max_blocks, int32_t* num_blocks,
                      int32_t* num_tokens) {
  if (!m) return bm_fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lock(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PA_ERR_SHAPE, "unknown sequence %lld", (long long)seq_id);
  const Sequence& s = it->second;
  if (num_blocks) *num_blocks = (int32_t)s.blocks.size();
  if (num_tokens) *num_tokens = (int32_t)s.tokens.size();
  if (out) {
    if ((int32_t)s.blocks.size() > max_blocks)
      return bm_fail(PA_ERR_SHAPE, "sequence has %zu blocks, row holds %d", s.blocks.size(), max_blocks);
    for (size_t j = 0; j < s.blocks.size(); ++j) out[j] = s.blocks[j];
  }
  t_bm_error.clear();
  return PA_OK;
}

int pa_bm_slots(pa_block_manager* m, int64_t seq_id, int32_t first_token, int32_t count, int32_t* slots) {
  if (!m || !slots) return bm_fail(PA_ERR_NULL, "manager or slots is NULL");
  std::lock_guard<std::mutex> lock(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PA_ERR_SHAPE, "unknown sequence %lld", (long long)seq_id);
  const Sequence& s = it->second;
  if (first_token < 0 || count < 0 || (int64_t)first_token + count > (int64_t)s.tokens.size())
    return bm_fail(PA_ERR_SHAPE, "token range [%d, %d) outside the sequence", first_token, first_token + count);
  const int bs = m->block_size;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t t = first_token + i;
    slots[i] = s.blocks[t / bs] * bs + t % bs;
  }
  t_bm_error.clear();
  return PA_OK;
}

int pa_bm_stats(pa_block_manager* m, int32_t* free_blocks, int32_t* cached_blocks, int64_t* hits, int64_t* misses,
                int64_t* evictions) {
  if (!m) return bm_fail(PA_ERR_NULL, "manager is NULL");
  std::lock_guard<std::mutex> lock(m->mu);
  if (free_blocks) *free_blocks = m->available();
  if (cached_blocks) *cached_blocks = (int32_t)m->cache.size();
  if (hits) *hits = m->hits;
  if (misses) *misses = m->misses;
  if (evictions) *evictions = m->evictions;
  return PA_OK;
}

int32_t pa_bm_block_ref(pa_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  std::lock_guard<std::mutex> lock(m->mu);
  return m->blocks[block].ref;
}

const char* pa_bm_last_error(void) { return t_bm_error.c_str(); }

}  // extern "C"
