// Host block allocator: block tables, on-demand blocks, shared blocks under a reference count,
// copy-on-write, all-or-nothing appends.
//
// Pages (by title): «第 7 章推理框架：vLLM 与 PagedAttention» 7.1 「三个关键机制」 (16-token blocks,
// per-request block table, a new block once the last is full, shared prefix blocks with a reference
// count, any free block serves any request); «vLLM 与 PagedAttention：把 GPU 显存当操作系统内存管»
// PagedAttention section (share, then copy on write); «GPU 学习日报 Day 28：vLLM 与 PagedAttention：
// GPU Memory 管理的艺术» §三 3.1 (table figure), §四 4.2 (on-demand blocks, uniform pool, CoW),
// §六 items 3-4 (count 2 on shared blocks; a writer gets a new block, copies, count - 1), FAQ Q3
// (running out of blocks is still possible).
//
// Readings where the pages are silent: the free list is a FIFO queue with a caller-given initial
// order; freed blocks join its tail in table order; the slot of position p is
// table[p / b] * b + p % b; an append that cannot get every block it needs changes nothing.
//
// Prefix cache (7.1 again, and its vLLM parameter list: requests with the same system-prompt
// prefix share its physical blocks, only the differing suffixes get blocks of their own; Day 28 §七:
// requests sharing a cached prompt skip its prefill; FAQ Q5: worth it when the prefix is long and
// stable).  Readings: only full blocks are cached, under the key (entry id of the block before, or 0,
// and the block's token ids); entry ids are never reused, so a key names one exact token prefix.  A
// new sequence attaches the longest matching run of cached blocks but leaves at least one prompt
// token to compute.  A cached block whose count falls to zero is kept, and is reclaimed (its entry
// dropped), least recently released first, only when the free list is empty; one release queues
// its cached blocks from the table's end, so chains shrink from their deepest block.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache
  struct Key {
    int64_t parent;
    std::vector<int32_t> tokens;
    bool operator==(const Key& o) const { return parent == o.parent && tokens == o.tokens; }
  };
  struct KeyHash {
    size_t operator()(const Key& k) const {
      uint64_t h = 1469598103934665603ull ^ static_cast<uint64_t>(k.parent);   // FNV-1a over the ids
      for (int32_t t : k.tokens) h = (h ^ static_cast<uint32_t>(t)) * 1099511628211ull;
      return static_cast<size_t>(h);
    }
  };
  struct Entry {
    int32_t block;
    Key key;
  };
  bool caching = false;
  std::unordered_map<Key, int64_t, KeyHash> entries;   // key -> entry id
  std::unordered_map<int64_t, Entry> entry;            // entry id -> block and key
  std::vector<int64_t> block_entry;                    // 0: the block is not cached
  std::list<int32_t> evictable;                        // cached blocks with count 0, oldest first
  std::vector<std::list<int32_t>::iterator> evict_pos;
  int64_t next_entry = 1;
};

namespace {

// A block taken by an append: from the free-list head, or reclaimed from the cache.
struct Take {
  int32_t block;
  bool reclaimed;
  int64_t eid;                      // the dropped cache entry (reclaimed blocks)
  pa_allocator::Key key;
};

// Undo record of one append: enough to restore the state exactly.
struct AppendUndo {
  int64_t seq_id;
  int64_t old_len;
  size_t old_table_size;
  std::vector<Take> taken;                             // in order
  std::vector<std::pair<int32_t, int32_t>> cow;        // (logical index, old block)
};

int64_t available(const pa_allocator* a) {
  return static_cast<int64_t>(a->free_list.size()) + static_cast<int64_t>(a->evictable.size());
}

// The next block for an append: the free-list head, else the least recently released cached block
// nobody points at (its cache entry is dropped).  The caller has checked that one exists.
int32_t take_block(pa_allocator* a, AppendUndo* undo) {
  if (!a->free_list.empty()) {
    const int32_t blk = a->free_list.front();
    a->free_list.pop_front();
    if (undo) undo->taken.push_back(Take{blk, false, 0, {}});
    return blk;
  }
  const int32_t blk = a->evictable.front();
  a->evictable.pop_front();
  const int64_t eid = a->block_entry[blk];
  auto it = a->entry.find(eid);
  if (undo) undo->taken.push_back(Take{blk, true, eid, it->second.key});
  a->entries.erase(it->second.key);
  a->entry.erase(it);
  a->block_entry[blk] = 0;
  return blk;
}

// One reference to each block of a table dropped.  Unreferenced blocks join the free-list tail in
// table order; unreferenced cached blocks are kept, queued (newest at the back) from the table's
// last block to its first, so that a chain loses its deepest blocks first and its head, where every
// lookup starts, stays matchable.
void release_table(pa_allocator* a, const std::vector<int32_t>& table) {
  for (int32_t blk : table)
    if (--a->ref[blk] == 0 && a->block_entry[blk] == 0) a->free_list.push_back(blk);
  for (auto it = table.rbegin(); it != table.rend(); ++it)
    if (a->ref[*it] == 0 && a->block_entry[*it] != 0)
      a->evict_pos[*it] = a->evictable.insert(a->evictable.end(), *it);
}

int32_t blocks_needed(const pa_allocator* a, const pa_allocator::Seq& s, int32_t n) {
  const int64_t b = a->block_size;
  int32_t need = 0;
  if (n > 0 && s.len % b != 0 && a->ref[s.table[s.len / b]] > 1) need += 1;
  const int64_t new_len = s.len + n;
  need += static_cast<int32_t>((new_len + b - 1) / b - static_cast<int64_t>(s.table.size()));
  return need;
}

// Performs an append known to fit.  Writes slots; appends CoW pairs to `cow_out`.
void do_append(pa_allocator* a, int64_t seq_id, pa_allocator::Seq& s, int32_t n, int64_t* slots,
               std::vector<int32_t>& cow_out, AppendUndo* undo) {
  const int64_t b = a->block_size;
  if (undo) {
    undo->seq_id = seq_id;
    undo->old_len = s.len;
    undo->old_table_size = s.table.size();
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t p = s.len;
    const int64_t logical = p / b;
    if (p % b == 0) {
      const int32_t blk = take_block(a, undo);
      a->ref[blk] = 1;
      s.table.push_back(blk);
    } else if (a->ref[s.table[logical]] > 1) {
      const int32_t old = s.table[logical];
      const int32_t fresh = take_block(a, undo);
      a->ref[old] -= 1;
      a->ref[fresh] = 1;
      s.table[logical] = fresh;
      cow_out.push_back(old);
      cow_out.push_back(fresh);
      if (undo) undo->cow.emplace_back(static_cast<int32_t>(logical), old);
    }
    slots[i] = static_cast<int64_t>(s.table[logical]) * b + p % b;
    s.len = p + 1;
  }
}

void undo_append(pa_allocator* a, const AppendUndo& u) {
  pa_allocator::Seq& s = a->seqs[u.seq_id];
  for (auto it = u.cow.rbegin(); it != u.cow.rend(); ++it) {
    const int32_t fresh = s.table[it->first];
    a->ref[fresh] = 0;
    a->ref[it->second] += 1;
    s.table[it->first] = it->second;
  }
  while (s.table.size() > u.old_table_size) {
    a->ref[s.table.back()] = 0;
    s.table.pop_back();
  }
  for (auto it = u.taken.rbegin(); it != u.taken.rend(); ++it) {
    if (!it->reclaimed) {
      a->free_list.push_front(it->block);
      continue;
    }
    a->entries.emplace(it->key, it->eid);
    a->entry.emplace(it->eid, pa_allocator::Entry{it->block, it->key});
    a->block_entry[it->block] = it->eid;
    a->evict_pos[it->block] = a->evictable.insert(a->evictable.begin(), it->block);
  }
  s.len = u.old_len;
}

}  // namespace

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                          pa_allocator** out) {
  if (!out) return pa_fail(PA_ERR_INVALID, "pa_alloc_create: out is null");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa_fail(PA_ERR_INVALID, "pa_alloc_create: num_blocks and block_size must be positive");
  if (order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      if (order[i] < 0 || order[i] >= num_blocks || seen[order[i]])
        return pa_fail(PA_ERR_INVALID, "pa_alloc_create: initial order is not a permutation");
      seen[order[i]] = 1;
    }
  }
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return pa_fail(PA_ERR_OOM, "pa_alloc_create: host allocation failed");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ref.assign(num_blocks, 0);
  a->block_entry.assign(num_blocks, 0);
  a->evict_pos.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) a->free_list.push_back(order ? order[i] : i);
  *out = a;
  return pa_ok();
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

pa_status pa_alloc_add_seq(pa_allocator* a, int64_t id) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  if (a->seqs.count(id)) return pa_fail(PA_ERR_INVALID, "pa_alloc_add_seq: sequence exists");
  a->seqs.emplace(id, pa_allocator::Seq());
  return pa_ok();
}

pa_status pa_alloc_fork(pa_allocator* a, int64_t parent, int64_t child) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "pa_alloc_fork: unknown parent");
  if (a->seqs.count(child)) return pa_fail(PA_ERR_INVALID, "pa_alloc_fork: child exists");
  pa_allocator::Seq c = it->second;
  for (int32_t blk : c.table) a->ref[blk] += 1;
  a->seqs.emplace(child, std::move(c));
  return pa_ok();
}

pa_status pa_alloc_blocks_needed(const pa_allocator* a, int64_t id, int32_t n, int32_t* out) {
  if (!a || !out) return pa_fail(PA_ERR_INVALID, "null argument");
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "unknown sequence");
  if (n < 0) return pa_fail(PA_ERR_INVALID, "negative token count");
  *out = blocks_needed(a, it->second, n);
  return pa_ok();
}

pa_status pa_alloc_append(pa_allocator* a, int64_t id, int32_t n, int64_t* slots, int32_t* cow_pairs,
                          int32_t cow_cap, int32_t* n_cow) {
  if (!a || !n_cow) return pa_fail(PA_ERR_INVALID, "pa_alloc_append: null argument");
  *n_cow = 0;
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "pa_alloc_append: unknown sequence");
  if (n < 0) return pa_fail(PA_ERR_INVALID, "pa_alloc_append: negative token count");
  if (n > 0 && !slots) return pa_fail(PA_ERR_INVALID, "pa_alloc_append: slots_out is null");
  pa_allocator::Seq& s = it->second;
  const int32_t need = blocks_needed(a, s, n);
  if (need > available(a)) return pa_fail(PA_ERR_OOM, "pa_alloc_append: not enough free blocks");
  const int64_t b = a->block_size;
  const bool cow = n > 0 && s.len % b != 0 && a->ref[s.table[s.len / b]] > 1;
  if (cow && (cow_cap < 1 || !cow_pairs))
    return pa_fail(PA_ERR_INVALID, "pa_alloc_append: cow_pairs_out too small for the copy needed");
  std::vector<int32_t> pairs;
  do_append(a, id, s, n, slots, pairs, nullptr);
  for (size_t i = 0; i < pairs.size(); ++i) cow_pairs[i] = pairs[i];
  *n_cow = static_cast<int32_t>(pairs.size() / 2);
  return pa_ok();
}

pa_status pa_alloc_append_batch(pa_allocator* a, const int64_t* ids, const int32_t* ns, int32_t m,
                                int64_t* slots, int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow) {
  if (!a || !n_cow || (m > 0 && (!ids || !ns)))
    return pa_fail(PA_ERR_INVALID, "pa_alloc_append_batch: null argument");
  *n_cow = 0;
  int64_t total = 0;
  for (int32_t i = 0; i < m; ++i) {
    if (!a->seqs.count(ids[i])) return pa_fail(PA_ERR_INVALID, "pa_alloc_append_batch: unknown sequence");
    if (ns[i] < 0) return pa_fail(PA_ERR_INVALID, "pa_alloc_append_batch: negative token count");
    for (int32_t j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return pa_fail(PA_ERR_INVALID, "pa_alloc_append_batch: repeated sequence");
    total += ns[i];
  }
  if (total > 0 && !slots) return pa_fail(PA_ERR_INVALID, "pa_alloc_append_batch: slots_out is null");
  std::vector<AppendUndo> undo;
  undo.reserve(m);
  std::vector<int32_t> pairs;
  int64_t off = 0;
  for (int32_t i = 0; i < m; ++i) {
    pa_allocator::Seq& s = a->seqs[ids[i]];
    const int32_t need = blocks_needed(a, s, ns[i]);
    if (need > available(a)) {
      for (auto it = undo.rbegin(); it != undo.rend(); ++it) undo_append(a, *it);
      return pa_fail(PA_ERR_OOM, "pa_alloc_append_batch: not enough free blocks");
    }
    undo.emplace_back();
    do_append(a, ids[i], s, ns[i], slots + off, pairs, &undo.back());
    off += ns[i];
  }
  const int32_t npairs = static_cast<int32_t>(pairs.size() / 2);
  if (npairs > 0 && (npairs > cow_cap || !cow_pairs)) {
    for (auto it = undo.rbegin(); it != undo.rend(); ++it) undo_append(a, *it);
    return pa_fail(PA_ERR_INVALID, "pa_alloc_append_batch: cow_pairs_out too small");
  }
  for (size_t i = 0; i < pairs.size(); ++i) cow_pairs[i] = pairs[i];
  *n_cow = npairs;
  return pa_ok();
}

pa_status pa_alloc_free_seq(pa_allocator* a, int64_t id) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "pa_alloc_free_seq: unknown sequence");
  release_table(a, it->second.table);
  a->seqs.erase(it);
  return pa_ok();
}

pa_status pa_alloc_enable_prefix_cache(pa_allocator* a) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  a->caching = true;
  return pa_ok();
}

pa_status pa_alloc_add_seq_prefix(pa_allocator* a, int64_t id, const int32_t* tokens, int32_t n_tokens,
                                  int32_t* n_cached) {
  if (!a || !n_cached) return pa_fail(PA_ERR_INVALID, "pa_alloc_add_seq_prefix: null argument");
  *n_cached = 0;
  if (n_tokens < 0 || (n_tokens > 0 && !tokens))
    return pa_fail(PA_ERR_INVALID, "pa_alloc_add_seq_prefix: bad prompt");
  if (a->seqs.count(id)) return pa_fail(PA_ERR_INVALID, "pa_alloc_add_seq_prefix: sequence exists");
  pa_allocator::Seq& s = a->seqs.emplace(id, pa_allocator::Seq()).first->second;
  if (!a->caching) return pa_ok();
  const int64_t b = a->block_size;
  pa_allocator::Key key{0, {}};
  while ((static_cast<int64_t>(s.table.size()) + 1) * b <= static_cast<int64_t>(n_tokens) - 1) {
    const int64_t j = static_cast<int64_t>(s.table.size());
    key.tokens.assign(tokens + j * b, tokens + (j + 1) * b);
    auto it = a->entries.find(key);
    if (it == a->entries.end()) break;
    const int32_t blk = a->entry[it->second].block;
    if (a->ref[blk] == 0) a->evictable.erase(a->evict_pos[blk]);
    a->ref[blk] += 1;
    s.table.push_back(blk);
    key.parent = it->second;
  }
  s.len = static_cast<int64_t>(s.table.size()) * b;
  *n_cached = static_cast<int32_t>(s.len);
  return pa_ok();
}

pa_status pa_alloc_cache_seq(pa_allocator* a, int64_t id, const int32_t* tokens, int64_t n_tokens) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "pa_alloc_cache_seq: unknown sequence");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return pa_fail(PA_ERR_INVALID, "pa_alloc_cache_seq: bad tokens");
  if (n_tokens > it->second.len)
    return pa_fail(PA_ERR_INVALID, "pa_alloc_cache_seq: more tokens than the sequence holds");
  if (!a->caching) return pa_ok();
  const int64_t b = a->block_size;
  const auto& table = it->second.table;
  pa_allocator::Key key{0, {}};
  for (int64_t j = 0; j < n_tokens / b; ++j) {
    key.tokens.assign(tokens + j * b, tokens + (j + 1) * b);
    auto e = a->entries.find(key);
    int64_t eid;
    if (e != a->entries.end()) {
      eid = e->second;
    } else {
      const int32_t blk = table[j];
      if (a->block_entry[blk] != 0)
        return pa_fail(PA_ERR_INVALID, "pa_alloc_cache_seq: a block is cached under other tokens");
      eid = a->next_entry++;
      a->entries.emplace(key, eid);
      a->entry.emplace(eid, pa_allocator::Entry{blk, key});
      a->block_entry[blk] = eid;
    }
    key.parent = eid;
  }
  return pa_ok();
}

pa_status pa_alloc_move_seq(pa_allocator* src, pa_allocator* dst, int64_t id, int32_t* pairs, int32_t cap,
                            int32_t* n_pairs) {
  if (!src || !dst || !n_pairs) return pa_fail(PA_ERR_INVALID, "pa_alloc_move_seq: null argument");
  *n_pairs = 0;
  if (src == dst) return pa_fail(PA_ERR_INVALID, "pa_alloc_move_seq: source and destination are one allocator");
  if (src->block_size != dst->block_size)
    return pa_fail(PA_ERR_INVALID, "pa_alloc_move_seq: the pools have different block sizes");
  auto it = src->seqs.find(id);
  if (it == src->seqs.end()) return pa_fail(PA_ERR_INVALID, "pa_alloc_move_seq: unknown sequence");
  if (dst->seqs.count(id)) return pa_fail(PA_ERR_INVALID, "pa_alloc_move_seq: sequence exists in the destination");
  const std::vector<int32_t>& table = it->second.table;
  const int64_t n = static_cast<int64_t>(table.size());
  if (n > cap || (n > 0 && !pairs)) return pa_fail(PA_ERR_INVALID, "pa_alloc_move_seq: pairs_out too small");
  if (n > available(dst)) return pa_fail(PA_ERR_OOM, "pa_alloc_move_seq: not enough blocks in the destination");
  pa_allocator::Seq moved;
  moved.len = it->second.len;
  moved.table.reserve(table.size());
  for (size_t j = 0; j < table.size(); ++j) {
    const int32_t blk = take_block(dst, nullptr);
    dst->ref[blk] = 1;
    moved.table.push_back(blk);
    pairs[2 * j] = table[j];
    pairs[2 * j + 1] = blk;
  }
  dst->seqs.emplace(id, std::move(moved));
  release_table(src, it->second.table);
  src->seqs.erase(it);
  *n_pairs = static_cast<int32_t>(n);
  return pa_ok();
}

pa_status pa_plan_cache_hint(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t num_seqs,
                             int32_t block_size, int32_t* shared_blocks) {
  if (num_seqs < 0 || max_blocks < 0 || block_size < 1)
    return pa_fail(PA_ERR_INVALID, "pa_plan_cache_hint: negative size or block_size < 1");
  if (num_seqs == 0) return pa_ok();
  if (!tables || !lens || !shared_blocks) return pa_fail(PA_ERR_INVALID, "pa_plan_cache_hint: null argument");
  // used entries of every row, then how many times each physical block is named
  std::unordered_map<int32_t, int32_t> uses;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (lens[s] < 0) return pa_fail(PA_ERR_INVALID, "pa_plan_cache_hint: negative length");
    const int64_t nb = (static_cast<int64_t>(lens[s]) + block_size - 1) / block_size;
    if (nb > max_blocks) return pa_fail(PA_ERR_INVALID, "pa_plan_cache_hint: a length needs more than max_blocks entries");
    const int32_t* row = tables + static_cast<int64_t>(s) * max_blocks;
    for (int64_t j = 0; j < nb; ++j) ++uses[row[j]];
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t nb = (static_cast<int64_t>(lens[s]) + block_size - 1) / block_size;
    const int32_t* row = tables + static_cast<int64_t>(s) * max_blocks;
    int64_t k = 0;
    while (k < nb && uses[row[k]] > 1) ++k;
    shared_blocks[s] = static_cast<int32_t>(k);
  }
  return pa_ok();
}

pa_status pa_plan_shared_blocks(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t num_seqs,
                                int32_t block_size, int32_t width, int32_t* shared_blocks) {
  if (!shared_blocks || (num_seqs > 0 && (!tables || !lens)))
    return pa_fail(PA_ERR_INVALID, "pa_plan_shared_blocks: null argument");
  if (width < 1 || block_size < 1 || max_blocks < 0 || num_seqs < 0 || num_seqs % width != 0)
    return pa_fail(PA_ERR_INVALID, "pa_plan_shared_blocks: num_seqs must be a multiple of width >= 1");
  for (int32_t g = 0; g < num_seqs / width; ++g) {
    const int32_t* t0 = tables + static_cast<int64_t>(g) * width * max_blocks;
    int64_t k = max_blocks;
    for (int32_t w = 0; w < width; ++w) {
      const int32_t s = g * width + w;
      if (lens[s] < 0) return pa_fail(PA_ERR_INVALID, "pa_plan_shared_blocks: negative length");
      k = std::min<int64_t>(k, lens[s] / block_size);   // whole blocks inside every member's context
      const int32_t* t = tables + static_cast<int64_t>(s) * max_blocks;
      int64_t c = 0;
      while (c < k && t[c] == t0[c]) ++c;
      k = c;
    }
    shared_blocks[g] = static_cast<int32_t>(k);
  }
  return pa_ok();
}

pa_status pa_plan_beam_tails(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t num_seqs,
                             int32_t block_size, int32_t width, const int32_t* shared_blocks, int32_t* tail_tables,
                             int32_t tail_max_blocks, int32_t* tail_lens, int32_t* needed_max_blocks) {
  if (!shared_blocks || !tail_lens || (num_seqs > 0 && (!tables || !lens)))
    return pa_fail(PA_ERR_INVALID, "pa_plan_beam_tails: null argument");
  if (width < 1 || block_size < 1 || max_blocks < 0 || num_seqs < 0 || num_seqs % width != 0 || tail_max_blocks < 0)
    return pa_fail(PA_ERR_INVALID, "pa_plan_beam_tails: num_seqs must be a multiple of width >= 1");
  int64_t need = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t k = shared_blocks[s / width];
    const int64_t tail = static_cast<int64_t>(lens[s]) - k * block_size;
    if (k < 0 || tail < 0) return pa_fail(PA_ERR_INVALID, "pa_plan_beam_tails: shared blocks beyond a length");
    const int64_t nb = (tail + block_size - 1) / block_size;
    if (k + nb > max_blocks) return pa_fail(PA_ERR_INVALID, "pa_plan_beam_tails: table row shorter than the length");
    need = std::max(need, nb);
    tail_lens[s] = static_cast<int32_t>(tail);
  }
  if (needed_max_blocks) *needed_max_blocks = static_cast<int32_t>(need);
  if (!tail_tables) return pa_ok();
  if (need > tail_max_blocks)
    return pa_fail(PA_ERR_INVALID, "pa_plan_beam_tails: tail_max_blocks is smaller than the longest tail");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t k = shared_blocks[s / width];
    const int64_t nb = (static_cast<int64_t>(tail_lens[s]) + block_size - 1) / block_size;
    const int32_t* row = tables + static_cast<int64_t>(s) * max_blocks + k;
    int32_t* out = tail_tables + static_cast<int64_t>(s) * tail_max_blocks;
    for (int64_t j = 0; j < tail_max_blocks; ++j) out[j] = j < nb ? row[j] : 0;
  }
  return pa_ok();
}

pa_status pa_alloc_cache_stats(const pa_allocator* a, int32_t* num_cached, int32_t* num_evictable) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  if (num_cached) *num_cached = static_cast<int32_t>(a->entries.size());
  if (num_evictable) *num_evictable = static_cast<int32_t>(a->evictable.size());
  return pa_ok();
}

pa_status pa_alloc_evictable_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!a || !n_out) return pa_fail(PA_ERR_INVALID, "null argument");
  *n_out = static_cast<int32_t>(a->evictable.size());
  if (*n_out > cap) return pa_fail(PA_ERR_INVALID, "evictable list longer than cap");
  if (*n_out > 0 && !out) return pa_fail(PA_ERR_INVALID, "out is null");
  int32_t i = 0;
  for (int32_t blk : a->evictable) out[i++] = blk;
  return pa_ok();
}

pa_status pa_alloc_seq_len(const pa_allocator* a, int64_t id, int64_t* len) {
  if (!a || !len) return pa_fail(PA_ERR_INVALID, "null argument");
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "unknown sequence");
  *len = it->second.len;
  return pa_ok();
}

pa_status pa_alloc_block_table(const pa_allocator* a, int64_t id, int32_t* out, int32_t cap,
                               int32_t* n_out) {
  if (!a || !n_out) return pa_fail(PA_ERR_INVALID, "null argument");
  auto it = a->seqs.find(id);
  if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "unknown sequence");
  const auto& t = it->second.table;
  *n_out = static_cast<int32_t>(t.size());
  if (static_cast<int64_t>(t.size()) > cap) return pa_fail(PA_ERR_INVALID, "table longer than cap");
  if (!t.empty()) {
    if (!out) return pa_fail(PA_ERR_INVALID, "out is null");
    std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  }
  return pa_ok();
}

pa_status pa_alloc_fill_tables(const pa_allocator* a, const int64_t* ids, int32_t m, int32_t* out,
                               int32_t max_blocks, int32_t pad) {
  if (!a || (m > 0 && (!ids || !out)) || max_blocks < 0)
    return pa_fail(PA_ERR_INVALID, "pa_alloc_fill_tables: bad argument");
  for (int32_t i = 0; i < m; ++i) {
    auto it = a->seqs.find(ids[i]);
    if (it == a->seqs.end()) return pa_fail(PA_ERR_INVALID, "pa_alloc_fill_tables: unknown sequence");
    const auto& t = it->second.table;
    if (static_cast<int64_t>(t.size()) > max_blocks)
      return pa_fail(PA_ERR_INVALID, "pa_alloc_fill_tables: a table is longer than max_blocks");
    int32_t* row = out + static_cast<int64_t>(i) * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < static_cast<int32_t>(t.size()) ? t[j] : pad;
  }
  return pa_ok();
}

pa_status pa_alloc_refcount(const pa_allocator* a, int32_t block, int32_t* out) {
  if (!a || !out) return pa_fail(PA_ERR_INVALID, "null argument");
  if (block < 0 || block >= a->num_blocks) return pa_fail(PA_ERR_INVALID, "block out of range");
  *out = a->ref[block];
  return pa_ok();
}

pa_status pa_alloc_stats(const pa_allocator* a, int32_t* num_free, int32_t* num_used, int64_t* refs) {
  if (!a) return pa_fail(PA_ERR_INVALID, "allocator is null");
  int32_t used = 0;
  int64_t total = 0;
  for (int32_t r : a->ref) {
    used += r > 0;
    total += r;
  }
  if (num_free) *num_free = static_cast<int32_t>(a->free_list.size());
  if (num_used) *num_used = used;
  if (refs) *refs = total;
  return pa_ok();
}

pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!a || !n_out) return pa_fail(PA_ERR_INVALID, "null argument");
  *n_out = static_cast<int32_t>(a->free_list.size());
  if (*n_out > cap) return pa_fail(PA_ERR_INVALID, "free list longer than cap");
  if (*n_out > 0 && !out) return pa_fail(PA_ERR_INVALID, "out is null");
  int32_t i = 0;
  for (int32_t blk : a->free_list) out[i++] = blk;
  return pa_ok();
}

}  // extern "C"
