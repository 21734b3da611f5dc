// Host-side manager of the KV block pool: free block queue, allocate_slots,
// reference counts, hash-chained prefix caching, and the per-step inputs of
// pa_step. The semantics and the passages they follow are stated in
// pa_kv_manager.h; this file holds only the mechanics.
//
// Data structures:
//  - blocks: per block its reference count, its cached hash (if any) and
//    its links in the free queue, an intrusive doubly linked list, so that a
//    prefix hit on a free block leaves the queue in O(1);
//  - cache: hash -> (block, parent hash, tokens) of every cached block; the
//    stored parent hash and tokens make a lookup exact;
//  - reqs: per request its tokens, salt, computed count, blocks and the
//    hashes of its full blocks, in order.
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"
#include "pa_kv_manager.h"

namespace {

// 64-bit mixing step (the finaliser of Steele, Lea and Flood's SplitMix64).
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// Hash of a block from its parent's hash and its tokens.
uint64_t block_hash(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = mix64(parent + 0x9e3779b97f4a7c15ull);
  for (int i = 0; i < n; ++i) {
    const uint64_t t = static_cast<uint32_t>(tokens[i]);
    h = mix64(h ^ (t + 0x632be59bd9b4e019ull * static_cast<uint64_t>(i + 1)));
  }
  return h;
}

// The parent hash of a request's first block: depends on the cache salt only.
uint64_t root_hash(uint64_t salt) { return mix64(salt ^ 0x5851f42d4c957f2dull); }

constexpr int32_t kNone = -1;

struct Block {
  int32_t ref = 0;
  bool cached = false;
  uint64_t hash = 0;
  int32_t prev = kNone, next = kNone;
  bool in_free = false;
};

struct CacheEntry {
  int32_t block;
  uint64_t parent;
  std::vector<int32_t> tokens;
};

struct Request {
  std::vector<int32_t> tokens;
  uint64_t salt = 0;
  int64_t computed = 0;
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;  // of blocks [0, hashes.size()), all full
};

}  // namespace

struct pa_kv_manager {
  int32_t nb = 0, bs = 0;
  bool caching = false;
  std::vector<Block> blocks;
  int32_t head = kNone, tail = kNone, n_free = 0;
  std::unordered_map<uint64_t, CacheEntry> cache;
  std::unordered_map<int64_t, Request> reqs;

  void push_back(int32_t b) {
    Block& x = blocks[b];
    x.prev = tail;
    x.next = kNone;
    x.in_free = true;
    if (tail != kNone) blocks[tail].next = b; else head = b;
    tail = b;
    ++n_free;
  }
  void unlink(int32_t b) {
    Block& x = blocks[b];
    if (x.prev != kNone) blocks[x.prev].next = x.next; else head = x.next;
    if (x.next != kNone) blocks[x.next].prev = x.prev; else tail = x.prev;
    x.prev = x.next = kNone;
    x.in_free = false;
    --n_free;
  }
  // Take the front of the free queue; a recycled block loses its cached hash.
  int32_t pop_front() {
    const int32_t b = head;
    unlink(b);
    Block& x = blocks[b];
    if (x.cached) {
      auto it = cache.find(x.hash);
      if (it != cache.end() && it->second.block == b) cache.erase(it);
      x.cached = false;
    }
    x.ref = 1;
    return b;
  }
  // The cached block holding exactly these tokens after this parent, or kNone.
  int32_t lookup(uint64_t h, uint64_t parent, const int32_t* tokens) const {
    auto it = cache.find(h);
    if (it == cache.end()) return kNone;
    const CacheEntry& e = it->second;
    if (e.parent != parent || std::memcmp(e.tokens.data(), tokens, sizeof(int32_t) * bs) != 0) return kNone;
    return e.block;
  }
  uint64_t parent_of(const Request& r, size_t i) const { return i == 0 ? root_hash(r.salt) : r.hashes[i - 1]; }
};

namespace {

pa_status bad_request(int64_t id, const char* what) {
  return pa::report(PA_ERR_REQUEST, "request %lld: %s", static_cast<long long>(id), what);
}

}  // namespace

extern "C" {

pa_status pa_kv_manager_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_caching,
                               pa_kv_manager** out) {
  if (!out) return pa::report(PA_ERR_NULL, "pa_kv_manager_create: out is NULL");
  if (num_blocks < 1 || block_size < 1)
    return pa::report(PA_ERR_SHAPE, "pa_kv_manager_create: %d blocks of %d slots", num_blocks, block_size);
  pa_kv_manager* m = new pa_kv_manager;
  m->nb = num_blocks;
  m->bs = block_size;
  m->caching = enable_prefix_caching != 0;
  m->blocks.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) m->push_back(b);
  *out = m;
  return pa::report_ok();
}

void pa_kv_manager_destroy(pa_kv_manager* m) { delete m; }

int32_t pa_kv_manager_num_free_blocks(const pa_kv_manager* m) { return m ? m->n_free : -1; }

pa_status pa_kv_manager_add_request(pa_kv_manager* m, int64_t req_id, const int32_t* prompt, int64_t n_prompt,
                                    uint64_t salt, int64_t* num_cached_tokens) {
  if (!m || !num_cached_tokens) return pa::report(PA_ERR_NULL, "pa_kv_manager_add_request: NULL argument");
  if (n_prompt < 1) return bad_request(req_id, "empty prompt");
  if (!prompt) return pa::report(PA_ERR_NULL, "pa_kv_manager_add_request: prompt is NULL");
  if (m->reqs.count(req_id)) return bad_request(req_id, "id already in use");
  Request r;
  // room for generated tokens, so the first ones do not copy the prompt
  r.tokens.reserve(static_cast<size_t>(n_prompt) + 256);
  r.tokens.assign(prompt, prompt + n_prompt);
  r.salt = salt;
  if (m->caching) {
    // hits stop one block short of the whole prompt: its last token is computed
    const int64_t max_hits = (n_prompt - 1) / m->bs;
    for (int64_t i = 0; i < max_hits; ++i) {
      const uint64_t parent = m->parent_of(r, static_cast<size_t>(i));
      const int32_t* tok = r.tokens.data() + i * m->bs;
      const uint64_t h = block_hash(parent, tok, m->bs);
      const int32_t b = m->lookup(h, parent, tok);
      if (b == kNone) break;
      r.blocks.push_back(b);
      r.hashes.push_back(h);
    }
    for (int32_t b : r.blocks) {
      if (m->blocks[b].in_free) m->unlink(b);
      ++m->blocks[b].ref;
    }
    r.computed = static_cast<int64_t>(r.blocks.size()) * m->bs;
  }
  *num_cached_tokens = r.computed;
  m->reqs.emplace(req_id, std::move(r));
  return pa::report_ok();
}

pa_status pa_kv_manager_append_tokens(pa_kv_manager* m, int64_t req_id, const int32_t* tokens, int64_t n) {
  if (!m || (n > 0 && !tokens)) return pa::report(PA_ERR_NULL, "pa_kv_manager_append_tokens: NULL argument");
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return bad_request(req_id, "unknown");
  if (n < 0) return bad_request(req_id, "negative token count");
  it->second.tokens.insert(it->second.tokens.end(), tokens, tokens + n);
  return pa::report_ok();
}

pa_status pa_kv_manager_allocate_slots(pa_kv_manager* m, int64_t req_id, int64_t num_new_tokens) {
  if (!m) return pa::report(PA_ERR_NULL, "pa_kv_manager_allocate_slots: NULL manager");
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return bad_request(req_id, "unknown");
  Request& r = it->second;
  if (num_new_tokens < 0 || r.computed + num_new_tokens > static_cast<int64_t>(r.tokens.size()))
    return bad_request(req_id, "scheduling more tokens than it holds");
  const int64_t need_total = (r.computed + num_new_tokens + m->bs - 1) / m->bs;
  const int64_t missing = need_total - static_cast<int64_t>(r.blocks.size());
  if (missing <= 0) return pa::report_ok();
  if (missing > m->n_free)
    return pa::report(PA_ERR_NO_BLOCKS, "request %lld needs %lld more blocks, %d free", static_cast<long long>(req_id),
                      static_cast<long long>(missing), m->n_free);
  for (int64_t i = 0; i < missing; ++i) r.blocks.push_back(m->pop_front());
  return pa::report_ok();
}

pa_status pa_kv_manager_commit(pa_kv_manager* m, int64_t req_id, int64_t num_new_tokens) {
  if (!m) return pa::report(PA_ERR_NULL, "pa_kv_manager_commit: NULL manager");
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return bad_request(req_id, "unknown");
  Request& r = it->second;
  const int64_t upto = r.computed + num_new_tokens;
  if (num_new_tokens < 0 || upto > static_cast<int64_t>(r.tokens.size()) ||
      upto > static_cast<int64_t>(r.blocks.size()) * m->bs)
    return bad_request(req_id, "committing positions without tokens or slots");
  r.computed = upto;
  if (!m->caching) return pa::report_ok();
  while (static_cast<int64_t>(r.hashes.size() + 1) * m->bs <= r.computed) {
    const size_t i = r.hashes.size();
    const uint64_t parent = m->parent_of(r, i);
    const int32_t* tok = r.tokens.data() + i * m->bs;
    const uint64_t h = block_hash(parent, tok, m->bs);
    r.hashes.push_back(h);
    const int32_t b = r.blocks[i];
    Block& x = m->blocks[b];
    if (x.cached) continue;  // a hit block, cached already
    if (m->cache.count(h)) continue;  // the same contents are cached in another block (or a colliding hash)
    m->cache.emplace(h, CacheEntry{b, parent, std::vector<int32_t>(tok, tok + m->bs)});
    x.cached = true;
    x.hash = h;
  }
  return pa::report_ok();
}

pa_status pa_kv_manager_free(pa_kv_manager* m, int64_t req_id) {
  if (!m) return pa::report(PA_ERR_NULL, "pa_kv_manager_free: NULL manager");
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return bad_request(req_id, "unknown");
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b)
    if (--m->blocks[*b].ref == 0) m->push_back(*b);
  m->reqs.erase(it);
  return pa::report_ok();
}

pa_status pa_kv_manager_build_step(const pa_kv_manager* m, int64_t num_reqs, const int64_t* req_ids,
                                   const int64_t* num_new, int64_t max_blocks, int32_t* query_start_loc,
                                   int32_t* seq_lens, int32_t* context_lens, int32_t* block_tables,
                                   int64_t* slot_mapping) {
  if (!m || !query_start_loc) return pa::report(PA_ERR_NULL, "pa_kv_manager_build_step: NULL argument");
  if (num_reqs < 0 || max_blocks < 0) return pa::report(PA_ERR_SHAPE, "pa_kv_manager_build_step: negative size");
  if (num_reqs > 0 && (!req_ids || !num_new || !seq_lens || !context_lens || (max_blocks > 0 && !block_tables)))
    return pa::report(PA_ERR_NULL, "pa_kv_manager_build_step: NULL argument");
  // validate everything before writing anything
  std::vector<const Request*> rs(static_cast<size_t>(num_reqs));
  std::unordered_map<int64_t, int> seen;
  int64_t T = 0;
  for (int64_t i = 0; i < num_reqs; ++i) {
    auto it = m->reqs.find(req_ids[i]);
    if (it == m->reqs.end()) return bad_request(req_ids[i], "unknown");
    if (!seen.emplace(req_ids[i], 1).second) return bad_request(req_ids[i], "listed twice in one step");
    const Request& r = it->second;
    const int64_t L = r.computed + num_new[i];
    if (num_new[i] < 1 || L > static_cast<int64_t>(r.blocks.size()) * m->bs ||
        L > static_cast<int64_t>(r.tokens.size()))
      return bad_request(req_ids[i], "new tokens without tokens or slots");
    if (static_cast<int64_t>(r.blocks.size()) > max_blocks)
      return pa::report(PA_ERR_SHAPE, "request %lld holds %zu blocks, table width %lld",
                        static_cast<long long>(req_ids[i]), r.blocks.size(), static_cast<long long>(max_blocks));
    if (L > INT32_MAX || T + num_new[i] > INT32_MAX)
      return pa::report(PA_ERR_SHAPE, "pa_kv_manager_build_step: positions exceed 32 bits");
    rs[static_cast<size_t>(i)] = &r;
    T += num_new[i];
  }
  if (T > 0 && !slot_mapping) return pa::report(PA_ERR_NULL, "pa_kv_manager_build_step: slot_mapping is NULL");
  int64_t t = 0;
  query_start_loc[0] = 0;
  for (int64_t i = 0; i < num_reqs; ++i) {
    const Request& r = *rs[static_cast<size_t>(i)];
    const int64_t C = r.computed, L = C + num_new[i];
    seq_lens[i] = static_cast<int32_t>(L);
    context_lens[i] = static_cast<int32_t>(C);
    int32_t* row = block_tables + i * max_blocks;
    std::copy(r.blocks.begin(), r.blocks.end(), row);
    std::fill(row + r.blocks.size(), row + max_blocks, 0);
    for (int64_t p = C; p < L; ++p)
      slot_mapping[t++] = static_cast<int64_t>(r.blocks[static_cast<size_t>(p / m->bs)]) * m->bs + p % m->bs;
    query_start_loc[i + 1] = static_cast<int32_t>(t);
  }
  return pa::report_ok();
}

pa_status pa_kv_manager_request_blocks(const pa_kv_manager* m, int64_t req_id, int32_t* out, int64_t cap,
                                       int64_t* n_blocks, int64_t* num_computed) {
  if (!m || (cap > 0 && !out)) return pa::report(PA_ERR_NULL, "pa_kv_manager_request_blocks: NULL argument");
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return bad_request(req_id, "unknown");
  const Request& r = it->second;
  const int64_t n = static_cast<int64_t>(r.blocks.size());
  for (int64_t i = 0; i < std::min(n, cap); ++i) out[i] = r.blocks[static_cast<size_t>(i)];
  if (n_blocks) *n_blocks = n;
  if (num_computed) *num_computed = r.computed;
  return pa::report_ok();
}

int32_t pa_kv_manager_ref_count(const pa_kv_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->nb) return -1;
  return m->blocks[block].ref;
}

int32_t pa_kv_manager_is_cached(const pa_kv_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->nb) return -1;
  return m->blocks[block].cached ? 1 : 0;
}

}  // extern "C"
