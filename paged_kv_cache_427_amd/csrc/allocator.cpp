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
#include <cstdint>
#include <cstring>
#include <deque>
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
};

namespace {

// Undo record of one append: enough to restore the state exactly.
struct AppendUndo {
  int64_t seq_id;
  int64_t old_len;
  size_t old_table_size;
  std::vector<int32_t> popped;                         // blocks taken from the free-list head, in order
  std::vector<std::pair<int32_t, int32_t>> cow;        // (logical index, old block)
};

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
      const int32_t blk = a->free_list.front();
      a->free_list.pop_front();
      a->ref[blk] = 1;
      s.table.push_back(blk);
      if (undo) undo->popped.push_back(blk);
    } else if (a->ref[s.table[logical]] > 1) {
      const int32_t old = s.table[logical];
      const int32_t fresh = a->free_list.front();
      a->free_list.pop_front();
      a->ref[old] -= 1;
      a->ref[fresh] = 1;
      s.table[logical] = fresh;
      cow_out.push_back(old);
      cow_out.push_back(fresh);
      if (undo) {
        undo->popped.push_back(fresh);
        undo->cow.emplace_back(static_cast<int32_t>(logical), old);
      }
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
  for (auto it = u.popped.rbegin(); it != u.popped.rend(); ++it) a->free_list.push_front(*it);
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
  if (need > static_cast<int32_t>(a->free_list.size()))
    return pa_fail(PA_ERR_OOM, "pa_alloc_append: not enough free blocks");
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
    if (need > static_cast<int32_t>(a->free_list.size())) {
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
  for (int32_t blk : it->second.table) {
    a->ref[blk] -= 1;
    if (a->ref[blk] == 0) a->free_list.push_back(blk);
  }
  a->seqs.erase(it);
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
