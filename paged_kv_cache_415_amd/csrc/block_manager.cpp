// Host-side block manager with a prefix cache (C ABI in include/pa_blocks.h).
//
// What it keeps (datawhalechina page "17. vLLM PagedAttention", Step 4 and
// its reference solution: a free list, ceil(len / block_size) blocks per
// prompt, one more block when a sequence crosses a block boundary, OOM when
// the free list runs short; ybb.press page "vLLM 与 LLM 推理部署实战" §2.2:
// reference counts, copy-on-write of a shared block, and reuse of cached
// blocks whose prefix hash matches; bogosort page §16 Prefix Caching: the
// cache key is a hash, tenants must be isolated, blocks are reference
// counted):
//  - a FIFO free list (blocks handed out from the front, returned to the
//    back) in a caller-given initial order;
//  - a reference count per block;
//  - the prefix cache: every full block of a prompt is keyed by a 64-bit
//    FNV-1a hash of (parent key, namespace, the block's token ids), the
//    parent key of block 0 being 0; a hit must also match the stored
//    namespace, parent key and tokens, so a hash collision never shares a
//    block and two namespaces never share one;
//  - cached blocks whose count drops to zero stay cached on an LRU list and
//    are evicted (front first) only when the free list is empty.
// Everything is deterministic, so a plain re-implementation of the same
// rules yields the same block ids.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_blocks.h"

namespace pa {
pa_status report(pa_status code, const char* message);   // pa_api.cpp
}

namespace {

constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// Little-endian bytes of the key material, hashed in order.
uint64_t block_key(uint64_t parent, uint64_t ns, const int32_t* tokens, int bs) {
  unsigned char buf[16];
  for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)(parent >> (8 * i));
  for (int i = 0; i < 8; ++i) buf[8 + i] = (unsigned char)(ns >> (8 * i));
  uint64_t h = fnv1a(kFnvOffset, buf, 16);
  for (int t = 0; t < bs; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    unsigned char b[4] = {(unsigned char)v, (unsigned char)(v >> 8), (unsigned char)(v >> 16),
                          (unsigned char)(v >> 24)};
    h = fnv1a(h, b, 4);
  }
  return h;
}

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;
  std::deque<int32_t> free_list;
  // prefix cache
  std::unordered_map<uint64_t, int32_t> by_key;
  std::vector<uint8_t> cached;
  std::vector<uint64_t> key, parent, ns;
  std::vector<int32_t> tokens;          // [num_blocks][block_size]
  // LRU of cached blocks with ref == 0 (intrusive doubly linked list)
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_lru;
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;

  void lru_push_back(int32_t b) {
    prev[b] = lru_tail;
    next[b] = -1;
    if (lru_tail >= 0) next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    in_lru[b] = 1;
    ++lru_size;
  }
  void lru_remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else lru_head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else lru_tail = prev[b];
    prev[b] = next[b] = -1;
    in_lru[b] = 0;
    --lru_size;
  }
  void uncache(int32_t b) {
    by_key.erase(key[b]);
    cached[b] = 0;
  }
  // A block for new contents: the free list's front, else the least recently
  // released cached block (evicted from the cache).  The caller has checked
  // that one exists.
  int32_t take() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else {
      b = lru_head;
      lru_remove(b);
      uncache(b);
    }
    ref[b] = 1;
    return b;
  }
  int32_t available() const { return (int32_t)free_list.size() + lru_size; }
  void drop(int32_t b) {
    if (--ref[b] == 0) {
      if (cached[b]) lru_push_back(b); else free_list.push_back(b);
    }
  }
};

namespace {

pa_status bad(const char* msg) { return pa::report(PA_ERR_INVALID_ARG, msg); }
pa_status oom() { return pa::report(PA_ERR_OUT_OF_BLOCKS, "not enough free blocks"); }
pa_status done() { return pa::report(PA_OK, ""); }

// Every block of the table is in use at least as often as it appears there.
bool tables_blocks_in_use(const pa_block_manager* m, const int32_t* table, int32_t n) {
  std::unordered_map<int32_t, int32_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = table[i];
    if (b < 0 || b >= m->num_blocks) return false;
    if (++seen[b] > m->ref[b]) return false;
  }
  return true;
}

bool valid_block(const pa_block_manager* m, int32_t b) { return b >= 0 && b < m->num_blocks; }

}  // namespace

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                       pa_block_manager** out) {
  if (!out) return bad("null out");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || block_size > 4096) return bad("sizes");
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return bad("out of host memory");
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  try {
    m->ref.assign(num_blocks, 0);
    m->cached.assign(num_blocks, 0);
    m->key.assign(num_blocks, 0);
    m->parent.assign(num_blocks, 0);
    m->ns.assign(num_blocks, 0);
    m->tokens.assign((size_t)num_blocks * block_size, 0);
    m->prev.assign(num_blocks, -1);
    m->next.assign(num_blocks, -1);
    m->in_lru.assign(num_blocks, 0);
  } catch (...) {
    delete m;
    return bad("out of host memory");
  }
  if (order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete m;
        return bad("order is not a permutation");
      }
      seen[b] = 1;
      m->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  }
  *out = m;
  return done();
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_num_free(const pa_block_manager* m) { return m ? (int32_t)m->free_list.size() : -1; }
int32_t pa_bm_num_evictable(const pa_block_manager* m) { return m ? m->lru_size : -1; }
int32_t pa_bm_num_cached(const pa_block_manager* m) { return m ? (int32_t)m->by_key.size() : -1; }
int32_t pa_bm_ref_count(const pa_block_manager* m, int32_t block) {
  return (m && valid_block(m, block)) ? m->ref[block] : -1;
}

pa_status pa_bm_allocate_prompt(pa_block_manager* m, uint64_t namespace_id, const int32_t* tokens,
                                int32_t num_tokens, int32_t* blocks_out, int32_t capacity,
                                int32_t* num_blocks_out, int32_t* num_cached_blocks_out) {
  if (!m || !num_blocks_out || num_tokens < 0 || (num_tokens > 0 && (!tokens || !blocks_out)))
    return bad("arguments");
  const int32_t bs = m->block_size;
  const int32_t nb = (num_tokens + bs - 1) / bs;
  const int32_t full = num_tokens / bs;
  if (nb > capacity) return bad("capacity");
  // hits: the longest chain of full blocks already cached
  std::vector<uint64_t> keys(full);
  int32_t hits = 0;
  uint64_t par = 0;
  for (int32_t i = 0; i < full; ++i) {
    keys[i] = block_key(par, namespace_id, tokens + (size_t)i * bs, bs);
    if (hits == i) {
      auto it = m->by_key.find(keys[i]);
      if (it != m->by_key.end()) {
        const int32_t b = it->second;
        if (m->ns[b] == namespace_id && m->parent[b] == par &&
            std::memcmp(&m->tokens[(size_t)b * bs], tokens + (size_t)i * bs, sizeof(int32_t) * bs) == 0)
          ++hits;
      }
    }
    par = keys[i];
  }
  // all or nothing: fresh blocks must exist once the hit blocks leave the LRU
  int32_t hits_in_lru = 0;
  for (int32_t i = 0; i < hits; ++i) hits_in_lru += m->in_lru[m->by_key.at(keys[i])];
  if (nb - hits > m->available() - hits_in_lru) return oom();
  for (int32_t i = 0; i < hits; ++i) {
    const int32_t b = m->by_key.at(keys[i]);
    if (m->in_lru[b]) m->lru_remove(b);
    ++m->ref[b];
    blocks_out[i] = b;
  }
  par = hits > 0 ? keys[hits - 1] : 0;
  for (int32_t i = hits; i < nb; ++i) {
    const int32_t b = m->take();
    blocks_out[i] = b;
    // a fresh full block becomes cached unless its key is already taken
    if (i < full && m->by_key.find(keys[i]) == m->by_key.end()) {
      m->by_key[keys[i]] = b;
      m->cached[b] = 1;
      m->key[b] = keys[i];
      m->parent[b] = par;
      m->ns[b] = namespace_id;
      std::memcpy(&m->tokens[(size_t)b * bs], tokens + (size_t)i * bs, sizeof(int32_t) * bs);
    }
    if (i < full) par = keys[i];
  }
  *num_blocks_out = nb;
  if (num_cached_blocks_out) *num_cached_blocks_out = hits;
  return done();
}

pa_status pa_bm_register_blocks(pa_block_manager* m, uint64_t namespace_id, const int32_t* tokens,
                                int32_t num_tokens, const int32_t* table, int32_t num_blocks,
                                int32_t* num_registered_out) {
  if (!m || num_tokens < 0 || num_blocks < 0 || (num_tokens > 0 && !tokens) || (num_blocks > 0 && !table))
    return bad("arguments");
  const int32_t bs = m->block_size;
  const int32_t full = num_tokens / bs;
  if (full > num_blocks) return bad("the table is shorter than the full blocks of the tokens");
  for (int32_t i = 0; i < full; ++i)
    if (!valid_block(m, table[i]) || m->ref[table[i]] <= 0) return bad("block not in use");
  int32_t added = 0;
  uint64_t par = 0;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* tk = tokens + (size_t)i * bs;
    const uint64_t k = block_key(par, namespace_id, tk, bs);
    const int32_t b = table[i];
    if (!m->cached[b] && m->by_key.find(k) == m->by_key.end()) {
      m->by_key[k] = b;
      m->cached[b] = 1;
      m->key[b] = k;
      m->parent[b] = par;
      m->ns[b] = namespace_id;
      std::memcpy(&m->tokens[(size_t)b * bs], tk, sizeof(int32_t) * bs);
      ++added;
    }
    par = k;
  }
  if (num_registered_out) *num_registered_out = added;
  return done();
}

pa_status pa_bm_append(pa_block_manager* m, int32_t* table, int32_t num_blocks, int32_t capacity,
                       int32_t new_len, int32_t* num_blocks_out) {
  if (!m || !num_blocks_out || num_blocks < 0 || new_len < 0 || (num_blocks > 0 && !table))
    return bad("arguments");
  const int32_t need = (new_len + m->block_size - 1) / m->block_size;
  if (need > capacity) return bad("capacity");
  if (need - num_blocks > m->available()) return oom();
  int32_t n = num_blocks;
  while (n < need) table[n++] = m->take();
  *num_blocks_out = n;
  return done();
}

pa_status pa_bm_fork(pa_block_manager* m, const int32_t* table, int32_t num_blocks) {
  if (!m || num_blocks < 0 || (num_blocks > 0 && !table)) return bad("arguments");
  for (int32_t i = 0; i < num_blocks; ++i)
    if (!valid_block(m, table[i]) || m->ref[table[i]] <= 0) return bad("block not in use");
  for (int32_t i = 0; i < num_blocks; ++i) ++m->ref[table[i]];
  return done();
}

pa_status pa_bm_copy_on_write(pa_block_manager* m, int32_t* table, int32_t num_blocks,
                              int32_t logical, int64_t* pair_out) {
  if (!m || !table || !pair_out || logical < 0 || logical >= num_blocks) return bad("arguments");
  const int32_t b = table[logical];
  if (!valid_block(m, b) || m->ref[b] <= 0) return bad("block not in use");
  pair_out[0] = pair_out[1] = -1;
  if (m->ref[b] <= 1) return done();
  if (m->available() < 1) return oom();
  const int32_t dst = m->take();
  --m->ref[b];
  table[logical] = dst;
  pair_out[0] = b;
  pair_out[1] = dst;
  return done();
}

pa_status pa_bm_release(pa_block_manager* m, const int32_t* table, int32_t num_blocks) {
  if (!m || num_blocks < 0 || (num_blocks > 0 && !table)) return bad("arguments");
  if (!tables_blocks_in_use(m, table, num_blocks)) return bad("block not in use");
  // last block first, so that a prompt's tail is evicted before its head
  for (int32_t i = num_blocks - 1; i >= 0; --i) m->drop(table[i]);
  return done();
}

}  // extern "C"
