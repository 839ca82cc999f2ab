// Host-side checks of the device-resident inputs of the attention, cache-write and block-copy
// calls (host only, no HIP).  The kernels trust these values (out of range they read the wrong
// blocks); a caller that builds them by other means than pa_alloc_* can check them here before
// copying them to the device.  The table indirection checked here is the method's own: logical
// block j of a sequence lives in physical block table[j] of the pool («GPU 学习日报 Day 28：vLLM 与
// PagedAttention：GPU Memory 管理的艺术» §三 3.1), and a slot is block * block_size + offset.
#include <cinttypes>
#include <cstdarg>
#include <cstdio>
#include <unordered_set>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local char msg[320];

pa_status bad(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
pa_status bad(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  return pa_fail(PA_ERR_INVALID, msg);
}

bool pool_ok(const pa_pool_desc* p) { return p && p->num_blocks > 0 && p->block_size > 0; }

// The table entries a sequence of `len` tokens uses: 0 .. ceil(len / b) - 1, each in the pool.
pa_status check_row(const char* who, const pa_pool_desc* pool, const int32_t* row, int32_t max_blocks,
                    int64_t len, int32_t s) {
  const int64_t used = (len + pool->block_size - 1) / pool->block_size;
  if (used > max_blocks)
    return bad("%s: sequence %d needs %" PRId64 " table entries, more than max_blocks_per_seq %d", who, s, used,
               max_blocks);
  for (int64_t j = 0; j < used; ++j)
    if (row[j] < 0 || row[j] >= pool->num_blocks)
      return bad("%s: sequence %d, table entry %" PRId64 " = %d is outside the pool of %d blocks", who, s, j, row[j],
                 pool->num_blocks);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_validate_decode(const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                             const int32_t* lens, int32_t num_seqs, int32_t max_context_len) {
  const char* who = "pa_validate_decode";
  if (!pool_ok(pool)) return bad("%s: bad pool descriptor", who);
  if (num_seqs < 0 || max_blocks < 0 || max_context_len < 0) return bad("%s: negative size", who);
  if (num_seqs == 0) return pa_ok();
  if (!tables || !lens) return bad("%s: null pointer", who);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (lens[s] < 0 || lens[s] > max_context_len)
      return bad("%s: sequence %d has context length %d, outside [0, max_context_len %d]", who, s, lens[s],
                 max_context_len);
    const pa_status st = check_row(who, pool, tables + static_cast<int64_t>(s) * max_blocks, max_blocks, lens[s], s);
    if (st != PA_OK) return st;
  }
  return pa_ok();
}

pa_status pa_validate_prefill(const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                              const int32_t* qsl, const int32_t* prior, int32_t num_seqs, int32_t max_chunk_len,
                              int64_t total_q) {
  const char* who = "pa_validate_prefill";
  if (!pool_ok(pool)) return bad("%s: bad pool descriptor", who);
  if (num_seqs < 0 || max_blocks < 0 || max_chunk_len < 0 || total_q < 0) return bad("%s: negative size", who);
  if (num_seqs == 0) return pa_ok();
  if (!tables || !qsl || !prior) return bad("%s: null pointer", who);
  if (qsl[0] < 0) return bad("%s: query_start_loc[0] = %d is negative", who, qsl[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t chunk = static_cast<int64_t>(qsl[s + 1]) - qsl[s];
    if (chunk < 0) return bad("%s: query_start_loc decreases at sequence %d", who, s);
    if (chunk > max_chunk_len)
      return bad("%s: sequence %d has a chunk of %" PRId64 " queries, more than max_chunk_len %d", who, s, chunk,
                 max_chunk_len);
    if (prior[s] < 0) return bad("%s: sequence %d has a negative prior context length", who, s);
    const pa_status st = check_row(who, pool, tables + static_cast<int64_t>(s) * max_blocks, max_blocks,
                                   static_cast<int64_t>(prior[s]) + chunk, s);
    if (st != PA_OK) return st;
  }
  if (qsl[num_seqs] > total_q)
    return bad("%s: query_start_loc[%d] = %d exceeds the %" PRId64 " query rows", who, num_seqs, qsl[num_seqs],
               total_q);
  return pa_ok();
}

pa_status pa_validate_slots(const pa_pool_desc* pool, const int64_t* slots, int64_t num_tokens) {
  const char* who = "pa_validate_slots";
  if (!pool_ok(pool)) return bad("%s: bad pool descriptor", who);
  if (num_tokens < 0) return bad("%s: negative num_tokens", who);
  if (num_tokens == 0) return pa_ok();
  if (!slots) return bad("%s: null pointer", who);
  const int64_t cap = static_cast<int64_t>(pool->num_blocks) * pool->block_size;
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(num_tokens));
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;   // skipped token
    if (slots[t] >= cap)
      return bad("%s: token %" PRId64 " has slot %" PRId64 ", outside the pool's %" PRId64 " slots", who, t, slots[t],
                 cap);
    if (!seen.insert(slots[t]).second)
      return bad("%s: slot %" PRId64 " is written by two tokens (token %" PRId64 ")", who, slots[t], t);
  }
  return pa_ok();
}

pa_status pa_validate_pairs(const pa_pool_desc* src_pool, const pa_pool_desc* dst_pool, const int32_t* pairs,
                            int32_t num_pairs, int32_t in_place) {
  const char* who = "pa_validate_pairs";
  if (!pool_ok(src_pool) || !pool_ok(dst_pool)) return bad("%s: bad pool descriptor", who);
  if (num_pairs < 0) return bad("%s: negative num_pairs", who);
  if (num_pairs == 0) return pa_ok();
  if (!pairs) return bad("%s: null pointer", who);
  std::unordered_set<int32_t> dsts, srcs;
  for (int32_t k = 0; k < num_pairs; ++k) {
    const int32_t src = pairs[2 * k], dst = pairs[2 * k + 1];
    if (src < 0 || src >= src_pool->num_blocks)
      return bad("%s: pair %d has source block %d, outside the pool of %d blocks", who, k, src, src_pool->num_blocks);
    if (dst < 0 || dst >= dst_pool->num_blocks)
      return bad("%s: pair %d has destination block %d, outside the pool of %d blocks", who, k, dst,
                 dst_pool->num_blocks);
    if (!dsts.insert(dst).second) return bad("%s: destination block %d appears twice", who, dst);
    srcs.insert(src);
  }
  if (in_place)
    for (int32_t k = 0; k < num_pairs; ++k)
      if (srcs.count(pairs[2 * k + 1]))
        return bad("%s: block %d is both a source and a destination of one call", who, pairs[2 * k + 1]);
  return pa_ok();
}

}  // extern "C"
