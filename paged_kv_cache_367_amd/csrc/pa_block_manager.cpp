// pa_block_manager.cpp - host-side KV block manager: free list, reference counts,
// append-on-full, copy-on-write, prefix-cache key chain and LRU eviction of released
// cached blocks. The policy and its sources are stated in include/pa_block_manager.h.
//
// State: per physical block a reference count, a "cached" flag (its key is in the map)
// and, when cached, its key and token ids; a FIFO free list; the evictable queue as an
// intrusive doubly linked list over block ids (O(1) removal on a cache hit); a hash map
// key -> block; per sequence its blocks, token ids, full-block keys and salt.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <unordered_map>
#include <vector>

#include "../../include/paged_attention.h"
#include "../../include/pa_block_manager.h"

namespace {

// FNV-1a, 64-bit: offset basis 14695981039346656037, prime 1099511628211
constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

inline uint64_t fnv_bytes(uint64_t h, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; ++i) {
    h ^= (v >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

uint64_t block_key(uint64_t prev, uint64_t salt, const int32_t* tok, int n) {
  uint64_t h = kFnvOffset;
  h = fnv_bytes(h, prev, 8);
  h = fnv_bytes(h, salt, 8);
  for (int i = 0; i < n; ++i) h = fnv_bytes(h, (uint32_t)tok[i], 4);
  return h;
}

struct Seq {
  std::vector<int32_t> blocks;   // device blocks, or host blocks while swapped out
  std::vector<int32_t> tokens;
  std::vector<uint64_t> keys;    // one per full block
  uint64_t salt = 0;
  bool swapped = false;
};

}  // namespace

struct pa_block_manager {
  int32_t N, bs;
  bool prefix;
  std::vector<int32_t> ref;
  std::vector<uint8_t> cached;
  std::vector<uint64_t> key;
  std::vector<int32_t> btok;         // [N * bs] token ids of cached blocks
  std::deque<int32_t> free_list;
  std::vector<int32_t> prev, next;   // evictable queue links (-1 = none)
  std::vector<uint8_t> in_q;
  int32_t q_head = -1, q_tail = -1, q_len = 0;
  std::unordered_map<uint64_t, int32_t> map;
  std::unordered_map<int64_t, Seq> seqs;
  int32_t host_blocks = 0;
  std::deque<int32_t> host_free;

  pa_block_manager(int32_t n, int32_t b, bool p)
      : N(n), bs(b), prefix(p), ref(n, 0), cached(n, 0), key(n, 0), btok((size_t)n * b, 0),
        prev(n, -1), next(n, -1), in_q(n, 0) {
    for (int32_t i = 0; i < n; ++i) free_list.push_back(i);
  }

  void q_push(int32_t blk) {
    prev[blk] = q_tail;
    next[blk] = -1;
    if (q_tail >= 0) next[q_tail] = blk;
    else q_head = blk;
    q_tail = blk;
    in_q[blk] = 1;
    ++q_len;
  }
  void q_remove(int32_t blk) {
    if (prev[blk] >= 0) next[prev[blk]] = next[blk];
    else q_head = next[blk];
    if (next[blk] >= 0) prev[next[blk]] = prev[blk];
    else q_tail = prev[blk];
    prev[blk] = next[blk] = -1;
    in_q[blk] = 0;
    --q_len;
  }
  int32_t available() const { return (int32_t)free_list.size() + q_len; }

  // a block for new contents: free list head, else evict the queue head
  int32_t allocate() {
    int32_t blk;
    if (!free_list.empty()) {
      blk = free_list.front();
      free_list.pop_front();
    } else {
      blk = q_head;
      q_remove(blk);
      map.erase(key[blk]);
      cached[blk] = 0;
    }
    ref[blk] = 1;
    return blk;
  }
  void release(int32_t blk) {
    if (--ref[blk] > 0) return;
    if (cached[blk]) q_push(blk);
    else free_list.push_back(blk);
  }
  // register a full block under its key unless the key is taken
  void register_full(int32_t blk, uint64_t k, const int32_t* tok) {
    if (!prefix || cached[blk] || map.count(k)) return;
    map.emplace(k, blk);
    cached[blk] = 1;
    key[blk] = k;
    memcpy(&btok[(size_t)blk * bs], tok, sizeof(int32_t) * bs);
  }
  // cached block holding exactly these tokens under key k, or -1
  int32_t lookup(uint64_t k, const int32_t* tok) const {
    if (!prefix) return -1;
    auto it = map.find(k);
    if (it == map.end()) return -1;
    if (memcmp(&btok[(size_t)it->second * bs], tok, sizeof(int32_t) * bs) != 0) return -1;
    return it->second;
  }
};

extern "C" {

pa_block_manager_t* pa_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t enable_prefix_cache) {
  if (num_blocks < 1 || num_blocks > (1 << 30) || block_size < 1 || block_size > 1024)
    return nullptr;
  try {
    return new pa_block_manager(num_blocks, block_size, enable_prefix_cache != 0);
  } catch (...) {                     // the per-block arrays did not fit in host memory
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager_t* bm) { delete bm; }

int32_t pa_bm_add(pa_block_manager_t* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                  uint64_t salt, int32_t* num_cached) {
  try {
    if (!bm) return PA_ERR_NULL;
    if (n < 0) return PA_ERR_SHAPE;
    if (n > 0 && !tokens) return PA_ERR_NULL;
    if (bm->seqs.count(seq_id)) return PA_ERR_UNKNOWN_SEQ;
    const int32_t bs = bm->bs;
    const int32_t nfull = n / bs, nb = (n + bs - 1) / bs;
    // keys of the full prompt blocks, and the leading run of cache hits
    std::vector<uint64_t> keys(nfull);
    uint64_t prev = 0;
    for (int32_t j = 0; j < nfull; ++j) prev = keys[j] = block_key(prev, salt, tokens + j * bs, bs);
    std::vector<int32_t> hits;
    for (int32_t j = 0; j < nfull; ++j) {
      const int32_t blk = bm->lookup(keys[j], tokens + j * bs);
      if (blk < 0) break;
      hits.push_back(blk);
    }
    int32_t hits_in_q = 0;
    for (int32_t blk : hits) hits_in_q += bm->in_q[blk];
    if (nb - (int32_t)hits.size() > bm->available() - hits_in_q) return PA_ERR_NO_BLOCKS;
  
    Seq s;
    s.salt = salt;
    s.tokens.assign(tokens, tokens + n);
    s.keys = keys;
    for (int32_t blk : hits) {
      if (bm->in_q[blk]) bm->q_remove(blk);
      ++bm->ref[blk];
      s.blocks.push_back(blk);
    }
    for (int32_t j = (int32_t)hits.size(); j < nb; ++j) {
      const int32_t blk = bm->allocate();
      s.blocks.push_back(blk);
      if (j < nfull) bm->register_full(blk, keys[j], tokens + j * bs);
    }
    if (num_cached) *num_cached = (int32_t)hits.size() * bs;
    bm->seqs.emplace(seq_id, std::move(s));
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_append(pa_block_manager_t* bm, int64_t seq_id, int32_t token, int64_t* slot,
                     int64_t* cow_src, int64_t* cow_dst) {
  try {
    if (!bm) return PA_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    Seq& s = it->second;
    if (s.swapped) return PA_ERR_UNSUPPORTED;
    const int32_t bs = bm->bs;
    const int32_t len = (int32_t)s.tokens.size(), off = len % bs;
    int64_t src = -1, dst = -1;
    if (off == 0) {                                      // last block full (or none): append
      if (bm->available() < 1) return PA_ERR_NO_BLOCKS;
      s.blocks.push_back(bm->allocate());
    } else if (bm->ref[s.blocks.back()] > 1) {           // shared partial block: copy first
      if (bm->available() < 1) return PA_ERR_NO_BLOCKS;
      const int32_t old = s.blocks.back();
      const int32_t blk = bm->allocate();
      --bm->ref[old];                                    // still > 0: another sequence holds it
      s.blocks.back() = blk;
      src = old;
      dst = blk;
    }
    s.tokens.push_back(token);
    const int32_t last = s.blocks.back();
    if (slot) *slot = (int64_t)last * bs + off;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
    if (off == bs - 1) {                                 // the block is full now
      const uint64_t prev = s.keys.empty() ? 0 : s.keys.back();
      const int32_t* tok = s.tokens.data() + (size_t)(len + 1 - bs);
      const uint64_t k = block_key(prev, s.salt, tok, bs);
      s.keys.push_back(k);
      bm->register_full(last, k, tok);
    }
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_append_batch(pa_block_manager_t* bm, const int64_t* seq_ids,
                           const int32_t* tokens, int32_t n, int64_t* slots, int64_t* cow_pairs,
                           int32_t* num_cow, int32_t* done) {
  try {
    if (!bm || !done) return PA_ERR_NULL;
    *done = 0;
    if (num_cow) *num_cow = 0;
    if (n < 0) return PA_ERR_SHAPE;
    if (n > 0 && (!seq_ids || !tokens || !slots || !cow_pairs || !num_cow)) return PA_ERR_NULL;
    int32_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
      int64_t src, dst;
      const int32_t st = pa_bm_append(bm, seq_ids[i], tokens[i], &slots[i], &src, &dst);
      if (st != PA_OK) return st;
      if (src >= 0) {
        cow_pairs[2 * k] = src;
        cow_pairs[2 * k + 1] = dst;
        ++k;
        *num_cow = k;
      }
      *done = i + 1;
    }
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_fork(pa_block_manager_t* bm, int64_t parent_id, int64_t child_id) {
  try {
    if (!bm) return PA_ERR_NULL;
    auto it = bm->seqs.find(parent_id);
    if (it == bm->seqs.end() || bm->seqs.count(child_id)) return PA_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PA_ERR_UNSUPPORTED;
    Seq child = it->second;                 // copies and inserts first: if either runs out
    auto ins = bm->seqs.emplace(child_id, std::move(child));   // of memory, no count moved
    for (int32_t blk : ins.first->second.blocks) ++bm->ref[blk];
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_free(pa_block_manager_t* bm, int64_t seq_id) {
  try {
    if (!bm) return PA_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    const std::vector<int32_t>& b = it->second.blocks;
    if (it->second.swapped) {
      for (int32_t h : b) bm->host_free.push_back(h);
    } else {
      for (size_t i = b.size(); i-- > 0;) bm->release(b[i]);   // tail first
    }
    bm->seqs.erase(it);
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_slots(const pa_block_manager_t* bm, int64_t seq_id, int32_t first,
                    int32_t count, int64_t* slots) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const Seq& s = it->second;
  if (s.swapped) return PA_ERR_UNSUPPORTED;
  if (first < 0 || count < 0 || (int64_t)first + count > (int64_t)s.tokens.size())
    return PA_ERR_SHAPE;
  if (count > 0 && !slots) return PA_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t p = first + i;
    slots[i] = (int64_t)s.blocks[p / bm->bs] * bm->bs + p % bm->bs;
  }
  return PA_OK;
}

int32_t pa_bm_block_table(const pa_block_manager_t* bm, int64_t seq_id, int32_t* row,
                          int32_t width) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  if (it->second.swapped) return PA_ERR_UNSUPPORTED;
  const std::vector<int32_t>& b = it->second.blocks;
  if (width < (int32_t)b.size()) return PA_ERR_SHAPE;
  if (width > 0 && !row) return PA_ERR_NULL;
  for (int32_t j = 0; j < width; ++j) row[j] = j < (int32_t)b.size() ? b[j] : -1;
  return (int32_t)b.size();
}

int32_t pa_bm_tables(const pa_block_manager_t* bm, const int64_t* seq_ids, int32_t n,
                     int32_t* tables, int32_t width, int32_t* context_lens) {
  try {
    if (!bm) return PA_ERR_NULL;
    if (n < 0 || width < 0) return PA_ERR_SHAPE;
    if (n > 0 && (!seq_ids || !tables || !context_lens)) return PA_ERR_NULL;
    std::vector<const Seq*> seqs(n);
    for (int32_t i = 0; i < n; ++i) {          // check everything before writing anything
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
      if (it->second.swapped) return PA_ERR_UNSUPPORTED;
      if ((int32_t)it->second.blocks.size() > width) return PA_ERR_SHAPE;
      seqs[i] = &it->second;
    }
    for (int32_t i = 0; i < n; ++i) {
      const std::vector<int32_t>& b = seqs[i]->blocks;
      int32_t* row = tables + (size_t)i * width;
      if (!b.empty()) memcpy(row, b.data(), sizeof(int32_t) * b.size());
      std::fill(row + b.size(), row + width, -1);
      context_lens[i] = (int32_t)seqs[i]->tokens.size();
    }
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_seq_len(const pa_block_manager_t* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? PA_ERR_UNKNOWN_SEQ : (int32_t)it->second.tokens.size();
}

int32_t pa_bm_refcount(const pa_block_manager_t* bm, int32_t block) {
  if (!bm) return PA_ERR_NULL;
  if (block < 0 || block >= bm->N) return PA_ERR_SHAPE;
  return bm->ref[block];
}

int32_t pa_bm_block_key(const pa_block_manager_t* bm, int64_t seq_id, int32_t j,
                        uint64_t* key) {
  if (!bm || !key) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  if (j < 0 || j >= (int32_t)it->second.keys.size()) return PA_ERR_SHAPE;
  *key = it->second.keys[j];
  return PA_OK;
}

int32_t pa_bm_stats(const pa_block_manager_t* bm, int32_t* num_free, int32_t* num_evictable,
                    int32_t* num_cached) {
  if (!bm) return PA_ERR_NULL;
  if (num_free) *num_free = (int32_t)bm->free_list.size();
  if (num_evictable) *num_evictable = bm->q_len;
  if (num_cached) *num_cached = (int32_t)bm->map.size();
  return PA_OK;
}

int32_t pa_bm_evictable(const pa_block_manager_t* bm, int32_t* out, int32_t cap) {
  if (!bm) return PA_ERR_NULL;
  if (cap < 0) return PA_ERR_SHAPE;
  if (cap > 0 && !out) return PA_ERR_NULL;
  int32_t n = 0;
  for (int32_t b = bm->q_head; b >= 0 && n < cap; b = bm->next[b]) out[n++] = b;
  return n;
}

int32_t pa_bm_set_host_blocks(pa_block_manager_t* bm, int32_t host_blocks) {
  try {
    if (!bm) return PA_ERR_NULL;
    if (host_blocks < 1 || host_blocks > (1 << 30) || bm->host_blocks > 0) return PA_ERR_SHAPE;
    bm->host_blocks = host_blocks;
    for (int32_t i = 0; i < host_blocks; ++i) bm->host_free.push_back(i);
    return PA_OK;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_swap_out(pa_block_manager_t* bm, int64_t seq_id, int64_t* pairs, int32_t cap) {
  try {
    if (!bm) return PA_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    Seq& s = it->second;
    const int32_t nb = (int32_t)s.blocks.size();
    if (s.swapped) return PA_ERR_UNSUPPORTED;
    for (int32_t blk : s.blocks)
      if (bm->ref[blk] > 1) return PA_ERR_UNSUPPORTED;
    if (cap < nb) return PA_ERR_SHAPE;
    if (nb > 0 && !pairs) return PA_ERR_NULL;
    if ((int32_t)bm->host_free.size() < nb) return PA_ERR_NO_BLOCKS;
    std::vector<int32_t> host(nb);
    for (int32_t j = 0; j < nb; ++j) {
      host[j] = bm->host_free.front();
      bm->host_free.pop_front();
      pairs[2 * j] = s.blocks[j];
      pairs[2 * j + 1] = host[j];
    }
    for (int32_t j = nb; j-- > 0;) bm->release(s.blocks[j]);    // tail first, as pa_bm_free
    s.blocks = std::move(host);
    s.swapped = true;
    return nb;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_swap_in(pa_block_manager_t* bm, int64_t seq_id, int64_t* pairs, int32_t cap) {
  try {
    if (!bm) return PA_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    Seq& s = it->second;
    const int32_t nb = (int32_t)s.blocks.size();
    if (!s.swapped) return PA_ERR_UNSUPPORTED;
    if (cap < nb) return PA_ERR_SHAPE;
    if (nb > 0 && !pairs) return PA_ERR_NULL;
    if (bm->available() < nb) return PA_ERR_NO_BLOCKS;
    std::vector<int32_t> dev(nb);
    for (int32_t j = 0; j < nb; ++j) {
      dev[j] = bm->allocate();
      pairs[2 * j] = s.blocks[j];
      pairs[2 * j + 1] = dev[j];
      if (j < (int32_t)s.keys.size())
        bm->register_full(dev[j], s.keys[j], s.tokens.data() + (size_t)j * bm->bs);
    }
    for (int32_t h : s.blocks) bm->host_free.push_back(h);
    s.blocks = std::move(dev);
    s.swapped = false;
    return nb;
  } catch (...) {                 // allocation failure inside the C++ containers
    return PA_ERR_NO_MEMORY;
  }
}

int32_t pa_bm_host_free(const pa_block_manager_t* bm) {
  if (!bm) return PA_ERR_NULL;
  return (int32_t)bm->host_free.size();
}

}  // extern "C"
