// pages_host.cpp -- host control plane of the paged KV cache (declared in
// include/pagedkv_host.h): page allocator with reference counts, generations
// and dirty flags; sequences as ordered page lists; the step-metadata
// builder; and a page-trie prefix index.
//
// Page "[Draft] kv paged kernels" (ROCm/maxtext #93): the commit adding the
// host page allocator (pages rather than token indices, double release and
// stale handles diagnosed, recycled pages dirty until confirmed) and the
// commit adding the prefix index (one page per trie node, keys chained from
// a namespace digest, counter-based recency, matches one page short of a
// fully cached prompt).  Written from those descriptions; no GPU code here.
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <functional>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "pagedkv_host.h"

namespace {

constexpr int64_t kIdMask = 0xFFFFFFFFll;

// A handle is (generation << 32 | id) with the generation's low 31 bits, so
// handles stay non-negative; a generation is compared the same way.
constexpr uint32_t kGenMask = 0x7FFFFFFFu;
int64_t make_handle(uint32_t gen, int64_t id) { return (int64_t)((uint64_t)(gen & kGenMask) << 32) | id; }
uint32_t handle_gen(int64_t handle) { return (uint32_t)(handle >> 32) & kGenMask; }

// 64-bit mixing step (splitmix64 finaliser constants, a published integer
// hash) for the trie's chained keys
uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  return x;
}

struct Seq {
  uint32_t epoch = 0;
  bool live = false;
  int64_t len = 0;
  std::vector<int64_t> pages;  // page ids, in order
};

struct Node {
  uint64_t key = 0;
  int64_t parent = -1;  // node index, -1 = a root (namespace) child
  int64_t page = -1;
  int64_t children = 0;
  uint64_t last_use = 0;
  bool live = false;
  std::vector<int32_t> tokens;  // the block's token ids (compared exactly)
};

}  // namespace

struct pkv_page_pool {
  int64_t num_pages = 0;
  int32_t page_size = 0;
  std::vector<int32_t> ref;     // per page: references (0 = free)
  std::vector<uint32_t> gen;    // per page: generation
  std::vector<uint8_t> dirty;   // per page: holds a previous owner's rows
  std::vector<int64_t> free_list;  // stack: the most recently freed on top
  std::vector<Seq> seqs;
  std::vector<int64_t> free_seq_slots;
  std::vector<Node> nodes;
  std::vector<int64_t> free_nodes;
  std::unordered_multimap<uint64_t, int64_t> by_key;
  uint64_t clock = 0;
  int64_t index_pages = 0;

  // sequence slot of a live handle, or -1
  int64_t seq_slot(int64_t handle) const {
    const int64_t slot = handle & kIdMask;
    if (handle < 0 || slot >= (int64_t)seqs.size()) return -1;
    const Seq& s = seqs[(size_t)slot];
    if (!s.live || (s.epoch & kGenMask) != handle_gen(handle)) return -1;
    return slot;
  }

  void unref(int64_t page) {
    if (--ref[(size_t)page] == 0) {
      ++gen[(size_t)page];
      dirty[(size_t)page] = 1;
      free_list.push_back(page);
    }
  }

  bool take_pages(int64_t n, std::vector<int64_t>& out) {
    if ((int64_t)free_list.size() < n) return false;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t pg = free_list.back();
      free_list.pop_back();
      ref[(size_t)pg] = 1;
      out.push_back(pg);
    }
    return true;
  }

  int64_t new_seq() {
    int64_t slot;
    if (!free_seq_slots.empty()) {
      slot = free_seq_slots.back();
      free_seq_slots.pop_back();
    } else {
      slot = (int64_t)seqs.size();
      seqs.emplace_back();
    }
    Seq& s = seqs[(size_t)slot];
    s.live = true;
    s.len = 0;
    s.pages.clear();
    return make_handle(s.epoch, slot);
  }

  static uint64_t block_key(uint64_t parent_key, const int32_t* tok, int32_t n) {
    uint64_t h = mix64(parent_key ^ 0x9E3779B97F4A7C15ull);
    for (int32_t i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tok[i]);
    return h;
  }

  // child of `parent` (-1 = root of the namespace) holding this block, or -1
  int64_t find_child(int64_t parent, uint64_t key, const int32_t* tok) const {
    auto range = by_key.equal_range(key);
    for (auto it = range.first; it != range.second; ++it) {
      const Node& nd = nodes[(size_t)it->second];
      if (nd.live && nd.parent == parent && std::memcmp(nd.tokens.data(), tok, sizeof(int32_t) * page_size) == 0)
        return it->second;
    }
    return -1;
  }
};

extern "C" {

pkv_page_pool* pkv_pool_create(int64_t num_pages, int32_t page_size) {
  if (num_pages <= 0 || page_size <= 0 || num_pages > kIdMask) return nullptr;
  pkv_page_pool* p = new (std::nothrow) pkv_page_pool;
  if (!p) return nullptr;
  try {
    p->num_pages = num_pages;
    p->page_size = page_size;
    p->ref.assign((size_t)num_pages, 0);
    p->gen.assign((size_t)num_pages, 0);
    p->dirty.assign((size_t)num_pages, 0);
    p->free_list.reserve((size_t)num_pages);
    for (int64_t i = num_pages - 1; i >= 0; --i) p->free_list.push_back(i);  // page 0 first
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

void pkv_pool_destroy(pkv_page_pool* pool) { delete pool; }

int64_t pkv_pool_free_pages(const pkv_page_pool* pool) { return pool ? (int64_t)pool->free_list.size() : PKV_ERR_NULL; }

int64_t pkv_pool_used_pages(const pkv_page_pool* pool) {
  return pool ? pool->num_pages - (int64_t)pool->free_list.size() : PKV_ERR_NULL;
}

int pkv_page_alloc(pkv_page_pool* pool, int64_t n, int64_t* handles_out) {
  if (!pool || (n > 0 && !handles_out)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  std::vector<int64_t> got;
  if (!pool->take_pages(n, got)) return PKV_ERR_NO_PAGES;
  for (int64_t i = 0; i < n; ++i) handles_out[i] = make_handle(pool->gen[(size_t)got[(size_t)i]], got[(size_t)i]);
  return PKV_OK;
}

int pkv_page_release(pkv_page_pool* pool, const int64_t* handles, int64_t n) {
  if (!pool || (n > 0 && !handles)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  // validate everything first: each handle current, no page released more
  // often than it is held
  std::unordered_map<int64_t, int32_t> count;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t h = handles[i], pg = h & kIdMask;
    if (h < 0 || pg >= pool->num_pages) return PKV_ERR_BAD_HANDLE;
    if (pool->ref[(size_t)pg] == 0 || (pool->gen[(size_t)pg] & kGenMask) != handle_gen(h)) return PKV_ERR_BAD_HANDLE;
    if (++count[pg] > pool->ref[(size_t)pg]) return PKV_ERR_BAD_HANDLE;
  }
  for (int64_t i = 0; i < n; ++i) pool->unref(handles[i] & kIdMask);
  return PKV_OK;
}

int pkv_page_confirm(pkv_page_pool* pool, const int64_t* page_ids, int64_t n) {
  if (!pool || (n > 0 && !page_ids)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int64_t i = 0; i < n; ++i)
    if (page_ids[i] < 0 || page_ids[i] >= pool->num_pages || pool->ref[(size_t)page_ids[i]] == 0)
      return PKV_ERR_BAD_HANDLE;
  for (int64_t i = 0; i < n; ++i) pool->dirty[(size_t)page_ids[i]] = 0;
  return PKV_OK;
}

int32_t pkv_page_refcount(const pkv_page_pool* pool, int64_t page_id) {
  if (!pool || page_id < 0 || page_id >= pool->num_pages) return -1;
  return pool->ref[(size_t)page_id];
}

int32_t pkv_page_dirty(const pkv_page_pool* pool, int64_t page_id) {
  if (!pool || page_id < 0 || page_id >= pool->num_pages) return -1;
  return pool->dirty[(size_t)page_id];
}

int pkv_seq_create(pkv_page_pool* pool, int64_t* seq_out) {
  if (!pool || !seq_out) return PKV_ERR_NULL;
  *seq_out = pool->new_seq();
  return PKV_OK;
}

int pkv_seq_append(pkv_page_pool* pool, int64_t seq, int64_t n, int64_t* slots_out) {
  if (!pool || (n > 0 && !slots_out)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  const int64_t slot = pool->seq_slot(seq);
  if (slot < 0) return PKV_ERR_BAD_HANDLE;
  Seq& s = pool->seqs[(size_t)slot];
  const int64_t ps = pool->page_size;
  const int64_t need = (s.len + n + ps - 1) / ps - (int64_t)s.pages.size();
  std::vector<int64_t> got;
  if (need > 0 && !pool->take_pages(need, got)) return PKV_ERR_NO_PAGES;
  s.pages.insert(s.pages.end(), got.begin(), got.end());
  for (int64_t i = 0; i < n; ++i) {
    const int64_t pos = s.len + i;
    slots_out[i] = s.pages[(size_t)(pos / ps)] * ps + pos % ps;
  }
  s.len += n;
  return PKV_OK;
}

int pkv_seq_append_batch(pkv_page_pool* pool, const int64_t* seqs, int64_t B, const int64_t* n, int64_t* slots_out) {
  if (!pool || (B > 0 && (!seqs || !n))) return PKV_ERR_NULL;
  if (B < 0) return PKV_ERR_SHAPE;
  const int64_t ps = pool->page_size;
  int64_t need = 0, total = 0;
  std::vector<int64_t> slot_of((size_t)B);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t slot = pool->seq_slot(seqs[b]);
    if (slot < 0) return PKV_ERR_BAD_HANDLE;
    if (n[b] < 0) return PKV_ERR_SHAPE;
    slot_of[(size_t)b] = slot;
    const Seq& s = pool->seqs[(size_t)slot];
    need += (s.len + n[b] + ps - 1) / ps - (int64_t)s.pages.size();
    total += n[b];
  }
  std::vector<int64_t> sorted(slot_of);
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return PKV_ERR_BAD_HANDLE;
  if (total > 0 && !slots_out) return PKV_ERR_NULL;
  if (need > (int64_t)pool->free_list.size()) return PKV_ERR_NO_PAGES;
  int64_t k = 0;
  for (int64_t b = 0; b < B; ++b) {
    Seq& s = pool->seqs[(size_t)slot_of[(size_t)b]];
    const int64_t more = (s.len + n[b] + ps - 1) / ps - (int64_t)s.pages.size();
    std::vector<int64_t> got;
    if (more > 0) pool->take_pages(more, got);  // cannot fail: counted above
    s.pages.insert(s.pages.end(), got.begin(), got.end());
    for (int64_t i = 0; i < n[b]; ++i, ++k) {
      const int64_t pos = s.len + i;
      slots_out[k] = s.pages[(size_t)(pos / ps)] * ps + pos % ps;
    }
    s.len += n[b];
  }
  return PKV_OK;
}

int pkv_seq_fork(pkv_page_pool* pool, int64_t parent, int64_t n_tokens, int64_t* child_out, int64_t* copy_out) {
  if (!pool || !child_out || !copy_out) return PKV_ERR_NULL;
  const int64_t ps_slot = pool->seq_slot(parent);
  if (ps_slot < 0) return PKV_ERR_BAD_HANDLE;
  const int64_t parent_len = pool->seqs[(size_t)ps_slot].len;
  if (n_tokens < 0 || n_tokens > parent_len) return PKV_ERR_SHAPE;
  const int64_t ps = pool->page_size;
  const int64_t whole = n_tokens / ps, rows = n_tokens % ps;
  std::vector<int64_t> fresh;
  if (rows > 0 && !pool->take_pages(1, fresh)) return PKV_ERR_NO_PAGES;
  const int64_t child = pool->new_seq();  // (may reallocate seqs: index afresh below)
  Seq& par = pool->seqs[(size_t)ps_slot];
  Seq& c = pool->seqs[(size_t)(child & kIdMask)];
  for (int64_t i = 0; i < whole; ++i) {
    const int64_t pg = par.pages[(size_t)i];
    ++pool->ref[(size_t)pg];
    c.pages.push_back(pg);
  }
  copy_out[0] = copy_out[1] = copy_out[2] = 0;
  if (rows > 0) {
    c.pages.push_back(fresh[0]);
    copy_out[0] = par.pages[(size_t)whole] * ps;
    copy_out[1] = fresh[0] * ps;
    copy_out[2] = rows;
  }
  c.len = n_tokens;
  *child_out = child;
  return PKV_OK;
}

int pkv_seq_release(pkv_page_pool* pool, int64_t seq) {
  if (!pool) return PKV_ERR_NULL;
  const int64_t slot = pool->seq_slot(seq);
  if (slot < 0) return PKV_ERR_BAD_HANDLE;
  Seq& s = pool->seqs[(size_t)slot];
  for (int64_t pg : s.pages) pool->unref(pg);
  s.pages.clear();
  s.len = 0;
  s.live = false;
  ++s.epoch;
  pool->free_seq_slots.push_back(slot);
  return PKV_OK;
}

int64_t pkv_seq_length(const pkv_page_pool* pool, int64_t seq) {
  if (!pool) return PKV_ERR_NULL;
  const int64_t slot = pool->seq_slot(seq);
  return slot < 0 ? PKV_ERR_BAD_HANDLE : pool->seqs[(size_t)slot].len;
}

int64_t pkv_seq_pages(const pkv_page_pool* pool, int64_t seq, int64_t* page_ids_out, int64_t capacity) {
  if (!pool || (capacity > 0 && !page_ids_out)) return PKV_ERR_NULL;
  const int64_t slot = pool->seq_slot(seq);
  if (slot < 0) return PKV_ERR_BAD_HANDLE;
  const std::vector<int64_t>& pg = pool->seqs[(size_t)slot].pages;
  const int64_t n = (int64_t)pg.size();
  for (int64_t i = 0; i < std::min(n, capacity); ++i) page_ids_out[i] = pg[(size_t)i];
  return n;
}

int pkv_build_step(const pkv_page_pool* pool, const int64_t* seqs, int64_t B, const int64_t* n_new,
                   int64_t max_blocks, int64_t pad_page, int64_t* block_table, int64_t* seq_lens,
                   int64_t* query_start_loc) {
  if (!pool || !query_start_loc) return PKV_ERR_NULL;
  if (B < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
  if (B > 0 && (!seqs || !n_new || !seq_lens || (max_blocks > 0 && !block_table))) return PKV_ERR_NULL;
  // validate all rows before writing any output
  for (int64_t b = 0; b < B; ++b) {
    const int64_t slot = pool->seq_slot(seqs[b]);
    if (slot < 0) return PKV_ERR_BAD_HANDLE;
    const Seq& s = pool->seqs[(size_t)slot];
    if ((int64_t)s.pages.size() > max_blocks) return PKV_ERR_SHAPE;
    if (n_new[b] < 0 || n_new[b] > s.len) return PKV_ERR_SHAPE;
    for (int64_t pg : s.pages)
      if (pool->dirty[(size_t)pg]) return PKV_ERR_DIRTY;
  }
  query_start_loc[0] = 0;
  for (int64_t b = 0; b < B; ++b) {
    const Seq& s = pool->seqs[(size_t)pool->seq_slot(seqs[b])];
    int64_t* row = block_table + b * max_blocks;
    const int64_t np = (int64_t)s.pages.size();
    for (int64_t j = 0; j < max_blocks; ++j) row[j] = j < np ? s.pages[(size_t)j] : pad_page;
    seq_lens[b] = s.len;
    query_start_loc[b + 1] = query_start_loc[b] + n_new[b];
  }
  return PKV_OK;
}

int pkv_prefix_insert(pkv_page_pool* pool, uint64_t namespace_digest, int64_t seq, const int32_t* tokens,
                      int64_t n_tokens) {
  if (!pool || (n_tokens > 0 && !tokens)) return PKV_ERR_NULL;
  const int64_t slot = pool->seq_slot(seq);
  if (slot < 0) return PKV_ERR_BAD_HANDLE;
  if (n_tokens < 0 || n_tokens > pool->seqs[(size_t)slot].len) return PKV_ERR_SHAPE;
  const int32_t ps = pool->page_size;
  const int64_t blocks = n_tokens / ps;
  uint64_t key = namespace_digest;
  int64_t parent = -1;
  for (int64_t i = 0; i < blocks; ++i) {
    const int32_t* tok = tokens + i * ps;
    key = pkv_page_pool::block_key(key, tok, ps);
    int64_t nd = pool->find_child(parent, key, tok);
    if (nd < 0) {
      if (!pool->free_nodes.empty()) {
        nd = pool->free_nodes.back();
        pool->free_nodes.pop_back();
      } else {
        nd = (int64_t)pool->nodes.size();
        pool->nodes.emplace_back();
      }
      Node& n = pool->nodes[(size_t)nd];
      n.key = key;
      n.parent = parent;
      n.page = pool->seqs[(size_t)slot].pages[(size_t)i];
      n.children = 0;
      n.live = true;
      n.tokens.assign(tok, tok + ps);
      ++pool->ref[(size_t)n.page];
      ++pool->index_pages;
      if (parent >= 0) ++pool->nodes[(size_t)parent].children;
      pool->by_key.emplace(key, nd);
    }
    pool->nodes[(size_t)nd].last_use = ++pool->clock;
    parent = nd;
  }
  return PKV_OK;
}

int pkv_prefix_match(pkv_page_pool* pool, uint64_t namespace_digest, const int32_t* tokens, int64_t n_tokens,
                     int64_t* seq_out, int64_t* matched_out) {
  if (!pool || !seq_out || !matched_out || (n_tokens > 0 && !tokens)) return PKV_ERR_NULL;
  if (n_tokens < 0) return PKV_ERR_SHAPE;
  const int32_t ps = pool->page_size;
  const int64_t limit = n_tokens > 0 ? (n_tokens - 1) / ps : 0;  // leave a token to run
  std::vector<int64_t> path;
  uint64_t key = namespace_digest;
  int64_t parent = -1;
  for (int64_t i = 0; i < limit; ++i) {
    const int32_t* tok = tokens + i * ps;
    key = pkv_page_pool::block_key(key, tok, ps);
    const int64_t nd = pool->find_child(parent, key, tok);
    if (nd < 0) break;
    path.push_back(nd);
    parent = nd;
  }
  const int64_t seq = pool->new_seq();
  Seq& s = pool->seqs[(size_t)(seq & kIdMask)];
  for (int64_t nd : path) {
    Node& n = pool->nodes[(size_t)nd];
    n.last_use = ++pool->clock;
    ++pool->ref[(size_t)n.page];
    s.pages.push_back(n.page);
  }
  s.len = (int64_t)path.size() * ps;
  *seq_out = seq;
  *matched_out = s.len;
  return PKV_OK;
}

int pkv_prefix_evict(pkv_page_pool* pool, int64_t pages, int64_t* freed_out) {
  if (!pool || !freed_out) return PKV_ERR_NULL;
  if (pages < 0) return PKV_ERR_SHAPE;
  // Evict, one at a time, the least recently used leaf whose page only the
  // index holds.  The candidates sit in a min-heap by recency (the clock
  // values are distinct); evicting a node can only add its parent to them.
  auto evictable = [&](int64_t i) {
    const Node& n = pool->nodes[(size_t)i];
    return n.live && n.children == 0 && pool->ref[(size_t)n.page] == 1;
  };
  using Cand = std::pair<uint64_t, int64_t>;  // (last_use, node)
  std::vector<Cand> heap;
  if (pages > 0)
    for (int64_t i = 0; i < (int64_t)pool->nodes.size(); ++i)
      if (evictable(i)) heap.emplace_back(pool->nodes[(size_t)i].last_use, i);
  std::make_heap(heap.begin(), heap.end(), std::greater<Cand>());
  int64_t freed = 0;
  while (freed < pages && !heap.empty()) {
    std::pop_heap(heap.begin(), heap.end(), std::greater<Cand>());
    const int64_t best = heap.back().second;
    heap.pop_back();
    Node& n = pool->nodes[(size_t)best];
    auto range = pool->by_key.equal_range(n.key);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == best) {
        pool->by_key.erase(it);
        break;
      }
    const int64_t parent = n.parent;
    if (parent >= 0) --pool->nodes[(size_t)parent].children;
    pool->unref(n.page);
    --pool->index_pages;
    n.live = false;
    n.tokens.clear();
    pool->free_nodes.push_back(best);
    ++freed;
    if (parent >= 0 && evictable(parent)) {
      heap.emplace_back(pool->nodes[(size_t)parent].last_use, parent);
      std::push_heap(heap.begin(), heap.end(), std::greater<Cand>());
    }
  }
  *freed_out = freed;
  return PKV_OK;
}

int64_t pkv_prefix_pages(const pkv_page_pool* pool) { return pool ? pool->index_pages : PKV_ERR_NULL; }

}  // extern "C"
