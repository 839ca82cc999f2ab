// C-ABI layer of libpa: argument validation, derived launch parameters, dispatch to the kernels.
// Every entry point returns a pa_status; failures leave a message in a thread-local buffer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxGridYZ = 65535;

pa_status hip_fail(int e, const char* where) {
  char msg[512];
  std::snprintf(msg, sizeof msg, "%s: %s", where, hipGetErrorString(static_cast<hipError_t>(e)));
  return pa_fail(PA_ERR_HIP, msg);
}

pa_status launch_status(int rc, const char* where) {
  if (rc == 0) return pa_ok();
  if (rc < 0) return pa_fail(PA_ERR_UNSUPPORTED, where);
  return hip_fail(rc, where);
}

bool is_pow2_block(int b) { return b == 8 || b == 16 || b == 32; }

pa_status check_pool(const pa_pool_desc* p, const char* who) {
  static thread_local char msg[256];
  if (!p) {
    std::snprintf(msg, sizeof msg, "%s: pool descriptor is null", who);
    return pa_fail(PA_ERR_INVALID, msg);
  }
  if (p->num_blocks <= 0 || p->num_kv_heads <= 0) {
    std::snprintf(msg, sizeof msg, "%s: num_blocks and num_kv_heads must be positive", who);
    return pa_fail(PA_ERR_INVALID, msg);
  }
  if (!is_pow2_block(p->block_size)) {
    std::snprintf(msg, sizeof msg, "%s: block_size must be 8, 16 or 32 (got %d)", who, p->block_size);
    return pa_fail(PA_ERR_INVALID, msg);
  }
  if (p->head_dim != 64 && p->head_dim != 128) {
    std::snprintf(msg, sizeof msg, "%s: head_dim must be 64 or 128 (got %d)", who, p->head_dim);
    return pa_fail(PA_ERR_INVALID, msg);
  }
  if (p->dtype != PA_F32 && p->dtype != PA_BF16 && p->dtype != PA_FP8_E4M3) {
    std::snprintf(msg, sizeof msg, "%s: unknown pool dtype %d", who, p->dtype);
    return pa_fail(PA_ERR_INVALID, msg);
  }
  if (p->dtype == PA_FP8_E4M3 && !(std::isfinite(p->k_scale) && p->k_scale > 0.f &&
                                   std::isfinite(p->v_scale) && p->v_scale > 0.f)) {
    std::snprintf(msg, sizeof msg, "%s: fp8 pool scales must be finite and positive", who);
    return pa_fail(PA_ERR_INVALID, msg);
  }
  return PA_OK;
}

int elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : 1; }

// Tokens per decode partition: the caller's size, or (0) one partition spanning every sequence.
int32_t decode_partition(int32_t max_ctx, int32_t partition_size) {
  if (partition_size > 0) return partition_size;
  return max_ctx > 0 ? (max_ctx + 31) / 32 * 32 : 32;   // a multiple of the 32-key decode unit
}

int64_t decode_max_parts(int32_t max_ctx, int32_t part) {
  if (max_ctx <= 0) return 1;
  return (static_cast<int64_t>(max_ctx) + part - 1) / part;
}

}  // namespace

extern "C" {

pa_status pa_cache_write(const void* k, const void* v, int32_t in_dtype, int64_t num_tokens,
                         const int64_t* slots, void* k_pool, void* v_pool, const pa_pool_desc* pool,
                         pa_stream stream) {
  pa_status st = check_pool(pool, "pa_cache_write");
  if (st != PA_OK) return st;
  if (num_tokens < 0) return pa_fail(PA_ERR_INVALID, "pa_cache_write: negative num_tokens");
  if (in_dtype != PA_F32 && in_dtype != PA_BF16)
    return pa_fail(PA_ERR_INVALID, "pa_cache_write: in_dtype must be PA_F32 or PA_BF16");
  if (pool->dtype != PA_FP8_E4M3 && pool->dtype != in_dtype)
    return pa_fail(PA_ERR_INVALID, "pa_cache_write: an f32/bf16 pool must have the dtype of k and v");
  if (num_tokens == 0) return pa_ok();
  if (!k || !v || !slots || !k_pool || !v_pool) return pa_fail(PA_ERR_INVALID, "pa_cache_write: null pointer");
  if (num_tokens * pool->num_kv_heads * (pool->head_dim / 4) > (int64_t(1) << 31))
    return pa_fail(PA_ERR_INVALID, "pa_cache_write: too many tokens for one launch");
  pa::CacheWriteArgs a{};
  a.k = k;
  a.v = v;
  a.in_dtype = in_dtype;
  a.num_tokens = num_tokens;
  a.slots = slots;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_size = pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.pool_dtype = pool->dtype;
  a.k_inv_scale = pool->dtype == PA_FP8_E4M3 ? 1.0f / pool->k_scale : 1.0f;
  a.v_inv_scale = pool->dtype == PA_FP8_E4M3 ? 1.0f / pool->v_scale : 1.0f;
  a.num_slots = static_cast<int64_t>(pool->num_blocks) * pool->block_size;
  return launch_status(pa::launch_cache_write(a, stream), "pa_cache_write");
}

pa_status pa_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc* pool, const int32_t* pairs,
                         int32_t num_pairs, pa_stream stream) {
  pa_status st = check_pool(pool, "pa_copy_blocks");
  if (st != PA_OK) return st;
  if (num_pairs < 0) return pa_fail(PA_ERR_INVALID, "pa_copy_blocks: negative num_pairs");
  if (num_pairs == 0) return pa_ok();
  if (!k_pool || !v_pool || !pairs) return pa_fail(PA_ERR_INVALID, "pa_copy_blocks: null pointer");
  pa::CopyBlocksArgs a{};
  a.src_k = k_pool;
  a.src_v = v_pool;
  a.dst_k = k_pool;
  a.dst_v = v_pool;
  a.block_bytes = static_cast<int64_t>(pool->num_kv_heads) * pool->block_size * pool->head_dim *
                  elem_bytes(pool->dtype);
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.num_layers = 1;
  a.layer_stride = 0;
  a.src_blocks = a.dst_blocks = pool->num_blocks;
  return launch_status(pa::launch_copy_blocks(a, stream), "pa_copy_blocks");
}

pa_status pa_copy_blocks_layers(void* k_pools, void* v_pools, int64_t layer_stride_bytes, int32_t num_layers,
                                const pa_pool_desc* pool, const int32_t* pairs, int32_t num_pairs,
                                pa_stream stream) {
  pa_status st = check_pool(pool, "pa_copy_blocks_layers");
  if (st != PA_OK) return st;
  if (num_pairs < 0) return pa_fail(PA_ERR_INVALID, "pa_copy_blocks_layers: negative num_pairs");
  if (num_layers < 1 || num_layers > 32767)
    return pa_fail(PA_ERR_INVALID, "pa_copy_blocks_layers: num_layers must be in 1..32767");
  const int64_t block_bytes = static_cast<int64_t>(pool->num_kv_heads) * pool->block_size * pool->head_dim *
                              elem_bytes(pool->dtype);
  if (num_layers > 1 && layer_stride_bytes < block_bytes * pool->num_blocks)
    return pa_fail(PA_ERR_INVALID, "pa_copy_blocks_layers: layer_stride_bytes is smaller than one layer's pool");
  if (layer_stride_bytes % 16 != 0)
    return pa_fail(PA_ERR_INVALID, "pa_copy_blocks_layers: layer_stride_bytes must be a multiple of 16");
  if (num_pairs == 0) return pa_ok();
  if (!k_pools || !v_pools || !pairs) return pa_fail(PA_ERR_INVALID, "pa_copy_blocks_layers: null pointer");
  pa::CopyBlocksArgs a{};
  a.src_k = k_pools;
  a.src_v = v_pools;
  a.dst_k = k_pools;
  a.dst_v = v_pools;
  a.block_bytes = block_bytes;
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.num_layers = num_layers;
  a.layer_stride = layer_stride_bytes;
  a.src_blocks = a.dst_blocks = pool->num_blocks;
  return launch_status(pa::launch_copy_blocks(a, stream), "pa_copy_blocks_layers");
}

namespace {

// The address through which kernels reach a pool: device (or managed) memory as it is; pinned host
// memory through its device mapping.  Pageable host memory and unknown pointers are refused, so
// that a swap never makes the device touch memory it cannot reach.
bool device_reachable(const void* p, const void** out) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();   // not sticky: clear it so the next launch check does not see it
    return false;
  }
  switch (attr.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      *out = p;
      return true;
    case hipMemoryTypeHost:
      if (!attr.devicePointer || !attr.hostPointer) return false;
      *out = static_cast<const char*>(attr.devicePointer) +
             (static_cast<const char*>(p) - static_cast<const char*>(attr.hostPointer));
      return true;
    default:
      return false;
  }
}

bool same_format(const pa_pool_desc* a, const pa_pool_desc* b) {
  return a->block_size == b->block_size && a->num_kv_heads == b->num_kv_heads && a->head_dim == b->head_dim &&
         a->dtype == b->dtype && a->k_scale == b->k_scale && a->v_scale == b->v_scale;
}

}  // namespace

pa_status pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, const pa_pool_desc* dst_pool, const void* src_k_pool,
                         const void* src_v_pool, const pa_pool_desc* src_pool, const int32_t* pairs,
                         int32_t num_pairs, pa_stream stream) {
  pa_status st = check_pool(dst_pool, "pa_swap_blocks");
  if (st != PA_OK) return st;
  st = check_pool(src_pool, "pa_swap_blocks");
  if (st != PA_OK) return st;
  if (!same_format(dst_pool, src_pool))
    return pa_fail(PA_ERR_INVALID, "pa_swap_blocks: the pools differ in block format or scales");
  if (num_pairs < 0) return pa_fail(PA_ERR_INVALID, "pa_swap_blocks: negative num_pairs");
  if (num_pairs == 0) return pa_ok();
  if (!dst_k_pool || !dst_v_pool || !src_k_pool || !src_v_pool || !pairs)
    return pa_fail(PA_ERR_INVALID, "pa_swap_blocks: null pointer");
  pa::CopyBlocksArgs a{};
  const void* dk = nullptr;
  const void* dv = nullptr;
  const void* pp = nullptr;
  if (!device_reachable(src_k_pool, &a.src_k) || !device_reachable(src_v_pool, &a.src_v) ||
      !device_reachable(dst_k_pool, &dk) || !device_reachable(dst_v_pool, &dv) || !device_reachable(pairs, &pp))
    return pa_fail(PA_ERR_INVALID,
                   "pa_swap_blocks: a pool or the pairs are neither device memory nor pinned host memory");
  a.dst_k = const_cast<void*>(dk);
  a.dst_v = const_cast<void*>(dv);
  a.pairs = static_cast<const int32_t*>(pp);
  a.block_bytes = static_cast<int64_t>(src_pool->num_kv_heads) * src_pool->block_size * src_pool->head_dim *
                  elem_bytes(src_pool->dtype);
  a.num_pairs = num_pairs;
  a.num_layers = 1;
  a.layer_stride = 0;
  a.src_blocks = src_pool->num_blocks;
  a.dst_blocks = dst_pool->num_blocks;
  return launch_status(pa::launch_copy_blocks(a, stream), "pa_swap_blocks");
}

pa_status pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_size, size_t* bytes) {
  if (!bytes) return pa_fail(PA_ERR_INVALID, "pa_decode_workspace_size: bytes is null");
  *bytes = 0;
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_size < 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_workspace_size: negative or zero size");
  if (partition_size != 0 && partition_size % 32 != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_workspace_size: partition_size must be a multiple of 32");
  const int32_t part = decode_partition(max_context_len, partition_size);
  const int64_t mp = decode_max_parts(max_context_len, part);
  *bytes = pa::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, mp, pa::decode_max_waves());
  return pa_ok();
}

pa_status pa_decode(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                    const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                    const int32_t* lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                    int32_t partition_size, int32_t max_context_len, void* workspace,
                    size_t workspace_bytes, void* out, int32_t out_dtype, pa_stream stream) {
  return pa_decode_ex(q, q_dtype, nullptr, k_pool, v_pool, pool, tables, max_blocks, lens, num_seqs, num_q_heads,
                      scale, partition_size, max_context_len, workspace, workspace_bytes, out, out_dtype, nullptr,
                      nullptr, nullptr, stream);
}

pa_status pa_decode_ex(const void* q, int32_t q_dtype, const int64_t* q_strides, const void* k_pool,
                       const void* v_pool, const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                       const int32_t* lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                       int32_t partition_size, int32_t max_context_len, void* workspace, size_t workspace_bytes,
                       void* out, int32_t out_dtype, const int64_t* out_strides, float* lse_out,
                       const int32_t* shared_blocks, pa_stream stream) {
  pa_status st = check_pool(pool, "pa_decode");
  if (st != PA_OK) return st;
  if (num_seqs < 0) return pa_fail(PA_ERR_INVALID, "pa_decode: negative num_seqs");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode: num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / pool->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode: group size must be 1, 2, 4 or 8");
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return pa_fail(PA_ERR_INVALID, "pa_decode: bad q_dtype");
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return pa_fail(PA_ERR_INVALID, "pa_decode: bad out_dtype");
  if ((pool->dtype == PA_F32) != (q_dtype == PA_F32))
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode: an f32 pool needs f32 q; bf16/fp8 pools need bf16 q");
  if (!std::isfinite(scale)) return pa_fail(PA_ERR_INVALID, "pa_decode: scale is not finite");
  if (max_context_len < 0) return pa_fail(PA_ERR_INVALID, "pa_decode: negative max_context_len");
  if (partition_size < 0 || (partition_size != 0 && partition_size % 32 != 0))
    return pa_fail(PA_ERR_INVALID, "pa_decode: partition_size must be 0 or a positive multiple of 32");
  const int64_t need_blocks = (static_cast<int64_t>(max_context_len) + pool->block_size - 1) / pool->block_size;
  if (max_blocks < need_blocks)
    return pa_fail(PA_ERR_INVALID, "pa_decode: max_blocks_per_seq < ceil(max_context_len / block_size)");
  if (num_seqs > kMaxGridYZ || pool->num_kv_heads > kMaxGridYZ)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode: more than 65535 sequences or KV heads in one call");
  if (num_seqs == 0) return pa_ok();
  if (!q || !k_pool || !v_pool || !tables || !lens || !out)
    return pa_fail(PA_ERR_INVALID, "pa_decode: null pointer");
  // stream positions (KV heads x 32-key units of all sequences) must fit in 31 bits
  if (static_cast<int64_t>(pool->num_kv_heads) * num_seqs * ((static_cast<int64_t>(max_context_len) + 31) / 32) >=
      (int64_t(1) << 31))
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode: more than 2^31 32-key units of K/V in one call");
  const int32_t part = decode_partition(max_context_len, partition_size);
  const int64_t mp = decode_max_parts(max_context_len, part);
  if (mp > (int64_t(1) << 30)) return pa_fail(PA_ERR_INVALID, "pa_decode: too many partitions");
  size_t need = 0;
  st = pa_decode_workspace_size(num_seqs, num_q_heads, pool->head_dim, max_context_len, partition_size, &need);
  if (st != PA_OK) return st;
  if (!workspace || workspace_bytes < need)
    return pa_fail(PA_ERR_INVALID, "pa_decode: workspace missing or smaller than pa_decode_workspace_size");
  pa::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = tables;
  a.max_blocks = max_blocks;
  a.lens = lens;
  a.shared_blocks = shared_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_blocks = pool->num_blocks;
  const float kscale = pool->dtype == PA_FP8_E4M3 ? pool->k_scale : 1.0f;
  a.qk_scale = static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  a.v_scale = pool->dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
  a.part_tokens = part;
  a.max_parts = static_cast<int32_t>(mp);
  a.max_ctx = max_context_len;
  pa::decode_workspace_carve(a, workspace);
  a.out = out;
  const int64_t D = pool->head_dim;
  const int64_t G = group;
  const int64_t dense[3] = {static_cast<int64_t>(num_q_heads) * D, G * D, D};
  const int64_t* qs = q_strides ? q_strides : dense;
  const int64_t* os = out_strides ? out_strides : dense;
  // q rows are read in 16-byte pieces (4 f32 or 8 bf16 elements); out rows are written 4 elements
  // at a time (16 bytes of f32, 8 of bf16)
  const int64_t q_step = 16 / elem_bytes(q_dtype);
  for (int k = 0; k < 3; ++k) {
    if (qs[k] < 0 || os[k] < 0)
      return pa_fail(PA_ERR_INVALID, "pa_decode_ex: negative stride");
    if (qs[k] % q_step != 0)
      return pa_fail(PA_ERR_INVALID, "pa_decode_ex: q strides must be multiples of 16 bytes (8 bf16 / 4 f32 elements)");
    if (os[k] % 4 != 0)
      return pa_fail(PA_ERR_INVALID, "pa_decode_ex: out strides must be multiples of 4 elements");
    if (lse_out && os[k] % D != 0)
      return pa_fail(PA_ERR_INVALID, "pa_decode_ex: with lse_out, out strides must be multiples of head_dim");
  }
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode: q must start at a 16-byte boundary");
  if (reinterpret_cast<uintptr_t>(out) % (4 * elem_bytes(out_dtype)) != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode: out must start at a boundary of 4 elements");
  a.q_sseq = qs[0];
  a.q_skv = qs[1];
  a.q_sg = qs[2];
  a.o_sseq = os[0];
  a.o_skv = os[1];
  a.o_sg = os[2];
  a.lse = lse_out;
  return launch_status(pa::launch_decode(a, pool->dtype, q_dtype, out_dtype, pool->block_size,
                                         pool->head_dim, stream),
                       "pa_decode: no kernel for this dtype / head_dim / block_size combination");
}

pa_status pa_decode_noalloc(const void* q, int32_t q_dtype, const int64_t* q_strides, const void* k_pool,
                            const void* v_pool, const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                            const int32_t* lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                            int32_t partition_size, int32_t max_context_len, void* out, int32_t out_dtype,
                            const int64_t* out_strides, float* lse_out, const int32_t* shared_blocks,
                            pa_stream stream) {
  pa_status st = check_pool(pool, "pa_decode_noalloc");
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0) return pa_fail(PA_ERR_INVALID, "pa_decode_noalloc: bad num_seqs or num_q_heads");
  size_t need = 0;
  st = pa_decode_workspace_size(num_seqs, num_q_heads, pool->head_dim, max_context_len, partition_size, &need);
  if (st != PA_OK) return st;
  if (need > PA_DECODE_STATIC_WORKSPACE_BYTES) {
    static thread_local char msg[256];
    std::snprintf(msg, sizeof msg,
                  "pa_decode_noalloc: this call needs %zu bytes of workspace, more than the static %zu; "
                  "use fewer sequences or partitions, or pa_decode with a workspace",
                  need, static_cast<size_t>(PA_DECODE_STATIC_WORKSPACE_BYTES));
    return pa_fail(PA_ERR_INVALID, msg);
  }
  if (num_seqs == 0) return pa_ok();
  size_t cap = 0;
  void* ws = nullptr;
  const int rc = pa::decode_static_workspace(&ws, &cap);
  if (rc != 0) return hip_fail(rc, "pa_decode_noalloc: device address of the static workspace");
  return pa_decode_ex(q, q_dtype, q_strides, k_pool, v_pool, pool, tables, max_blocks, lens, num_seqs, num_q_heads,
                      scale, partition_size, max_context_len, ws, cap, out, out_dtype, out_strides, lse_out,
                      shared_blocks, stream);
}

pa_status pa_merge_states(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b, int64_t rows,
                          int32_t head_dim, void* out, int32_t out_dtype, float* lse_out, pa_stream stream) {
  if (rows < 0) return pa_fail(PA_ERR_INVALID, "pa_merge_states: negative rows");
  if (head_dim <= 0 || head_dim % 4 != 0) return pa_fail(PA_ERR_INVALID, "pa_merge_states: head_dim must be a positive multiple of 4");
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return pa_fail(PA_ERR_INVALID, "pa_merge_states: bad out_dtype");
  if (rows == 0) return pa_ok();
  if (!o_a || !lse_a || !o_b || !lse_b || !out) return pa_fail(PA_ERR_INVALID, "pa_merge_states: null pointer");
  pa::MergeStatesArgs a{o_a, lse_a, o_b, lse_b, rows, head_dim, out, lse_out};
  return launch_status(pa::launch_merge_states(a, out_dtype, stream), "pa_merge_states");
}

pa_status pa_decode_tail_merge(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                               const pa_pool_desc* pool, const int32_t* tail_tables, int32_t max_blocks,
                               const int32_t* tail_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                               int32_t max_tail_len, const float* o_prev, const float* lse_prev, void* out,
                               int32_t out_dtype, pa_stream stream) {
  pa_status st = check_pool(pool, "pa_decode_tail_merge");
  if (st != PA_OK) return st;
  if (num_seqs < 0) return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: negative num_seqs");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / pool->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_tail_merge: group size must be 1, 2, 4 or 8");
  if (q_dtype != PA_BF16 || pool->dtype == PA_F32)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_tail_merge: needs bf16 q and a bf16 or fp8 pool");
  if (pool->head_dim != 128) return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_tail_merge: head_dim must be 128");
  if (out_dtype != PA_F32 && out_dtype != PA_BF16)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: bad out_dtype");
  if (!std::isfinite(scale)) return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: scale is not finite");
  if (max_tail_len < 0) return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: negative max_tail_len");
  if (max_tail_len > 32)
    return pa_fail(PA_ERR_UNSUPPORTED,
                   "pa_decode_tail_merge: tails of more than 32 keys (use pa_decode_ex and pa_merge_states)");
  if (max_blocks < (max_tail_len + pool->block_size - 1) / pool->block_size || max_blocks <= 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: max_blocks_per_seq < ceil(max_tail_len / block_size)");
  if (num_seqs == 0) return pa_ok();
  if (!q || !k_pool || !v_pool || !tail_tables || !tail_lens || !o_prev || !lse_prev || !out)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: null pointer");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: q must start at a 16-byte boundary");
  if (reinterpret_cast<uintptr_t>(o_prev) % 8 != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: o_prev must start at an 8-byte boundary");
  if (reinterpret_cast<uintptr_t>(out) % (2 * elem_bytes(out_dtype)) != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_tail_merge: out must start at a boundary of 2 elements");
  pa::TailMergeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = tail_tables;
  a.max_blocks = max_blocks;
  a.lens = tail_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_blocks = pool->num_blocks;
  const float kscale = pool->dtype == PA_FP8_E4M3 ? pool->k_scale : 1.0f;
  a.qk_scale = static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  a.v_scale = pool->dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
  a.max_tail = max_tail_len;
  a.o_prev = o_prev;
  a.lse_prev = lse_prev;
  a.out = out;
  return launch_status(pa::launch_tail_merge(a, pool->dtype, pool->block_size, pool->head_dim, out_dtype, stream),
                       "pa_decode_tail_merge: no kernel for this combination");
}

pa_status pa_decode_beam(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                         const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                         const int32_t* shared_lens, int32_t max_shared_len, const int32_t* tail_tables,
                         int32_t tail_max_blocks, const int32_t* tail_lens, int32_t max_tail_len, int32_t num_seqs,
                         int32_t width, float scale, void* workspace, size_t workspace_bytes, void* out,
                         int32_t out_dtype, int32_t phases, pa_stream stream) {
  pa_status st = check_pool(pool, "pa_decode_beam");
  if (st != PA_OK) return st;
  if (phases != PA_BEAM_SHARED && phases != PA_BEAM_TAILS && phases != (PA_BEAM_SHARED | PA_BEAM_TAILS))
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: phases must be PA_BEAM_SHARED, PA_BEAM_TAILS or both");
  if (width != 2 && width != 4 && width != 8)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_beam: width must be 2, 4 or 8");
  if (num_seqs < 0 || num_seqs % width != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: num_seqs must be a non-negative multiple of width");
  if (q_dtype != PA_BF16 || pool->dtype == PA_F32)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_beam: needs bf16 q and a bf16 or fp8 pool");
  if (pool->head_dim != 128) return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_beam: head_dim must be 128");
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return pa_fail(PA_ERR_INVALID, "pa_decode_beam: bad out_dtype");
  if (!std::isfinite(scale)) return pa_fail(PA_ERR_INVALID, "pa_decode_beam: scale is not finite");
  if (max_shared_len < 0 || max_tail_len < 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: negative max_shared_len or max_tail_len");
  if (max_tail_len > 32)
    return pa_fail(PA_ERR_UNSUPPORTED,
                   "pa_decode_beam: tails of more than 32 keys (use pa_decode_ex and pa_merge_states)");
  const int32_t b = pool->block_size;
  if (max_blocks <= 0 || max_blocks < (static_cast<int64_t>(max_shared_len) + b - 1) / b)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: max_blocks_per_seq < ceil(max_shared_len / block_size)");
  if (static_cast<int64_t>(max_blocks) * width > INT32_MAX)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_beam: max_blocks_per_seq * width exceeds 2^31 - 1");
  if (tail_max_blocks <= 0 || tail_max_blocks < (max_tail_len + b - 1) / b)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: tail_max_blocks < ceil(max_tail_len / block_size)");
  const int32_t groups = num_seqs / width;
  const int32_t heads = pool->num_kv_heads;
  if (groups > kMaxGridYZ || heads > kMaxGridYZ)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_beam: more than 65535 groups or KV heads in one call");
  if (static_cast<int64_t>(heads) * groups * ((static_cast<int64_t>(max_shared_len) + 31) / 32) >= (int64_t(1) << 31))
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_beam: more than 2^31 32-key units of shared K/V in one call");
  size_t need = 0;
  st = pa_decode_workspace_size(groups, width * heads, pool->head_dim, max_shared_len, 0, &need);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return pa_ok();
  if (!workspace || workspace_bytes < need)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: workspace missing or smaller than pa_decode_workspace_size");
  if (!q || !k_pool || !v_pool || !tables || !shared_lens || !tail_tables || !tail_lens || !out)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: null pointer");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: q must start at a 16-byte boundary");
  if (reinterpret_cast<uintptr_t>(out) % (2 * elem_bytes(out_dtype)) != 0)
    return pa_fail(PA_ERR_INVALID, "pa_decode_beam: out must start at a boundary of 2 elements");
  const int64_t D = pool->head_dim;
  const float kscale = pool->dtype == PA_FP8_E4M3 ? pool->k_scale : 1.0f;
  const float qk_scale = static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  const float v_scale = pool->dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
  // The shared part: group g's width branches are the query heads of each KV head, over the table row
  // of its first branch; every piece is left as a partial record in the workspace.
  pa::DecodeArgs r{};
  r.q = q;
  r.k_pool = k_pool;
  r.v_pool = v_pool;
  r.tables = tables;
  r.max_blocks = max_blocks * width;
  r.lens = shared_lens;
  r.num_seqs = groups;
  r.num_q_heads = width * heads;
  r.num_kv_heads = heads;
  r.num_blocks = pool->num_blocks;
  r.qk_scale = qk_scale;
  r.v_scale = v_scale;
  r.part_tokens = decode_partition(max_shared_len, 0);
  r.max_parts = static_cast<int32_t>(decode_max_parts(max_shared_len, r.part_tokens));
  r.max_ctx = max_shared_len;
  r.records_only = 1;
  pa::decode_workspace_carve(r, workspace);
  r.q_sseq = width * heads * D;   // group
  r.q_skv = D;                    // KV head
  r.q_sg = heads * D;             // branch
  pa::decode_launch_shape(r, pool->dtype);
  if (phases & PA_BEAM_SHARED) {
    st = launch_status(pa::launch_decode(r, pool->dtype, q_dtype, out_dtype, b, pool->head_dim, stream),
                       "pa_decode_beam: no decode kernel for this combination");
    if (st != PA_OK) return st;
  }
  if (phases & PA_BEAM_TAILS) {
    pa::TailMergeArgs t{};
    t.q = q;
    t.k_pool = k_pool;
    t.v_pool = v_pool;
    t.tables = tail_tables;
    t.max_blocks = tail_max_blocks;
    t.lens = tail_lens;
    t.num_seqs = num_seqs;
    t.num_q_heads = heads;
    t.num_kv_heads = heads;
    t.num_blocks = pool->num_blocks;
    t.qk_scale = qk_scale;
    t.v_scale = v_scale;
    t.max_tail = max_tail_len;
    t.out = out;
    t.width = width;
    t.shared = r;
    st = launch_status(pa::launch_tail_merge(t, pool->dtype, b, pool->head_dim, out_dtype, stream),
                       "pa_decode_beam: no tail kernel for this combination");
  }
  return st;
}

pa_status pa_prefill_chunk(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                           const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks,
                           const int32_t* qsl, const int32_t* prior, int32_t num_seqs,
                           int32_t num_q_heads, float scale, int32_t max_chunk_len, void* out,
                           int32_t out_dtype, pa_stream stream) {
  pa_status st = check_pool(pool, "pa_prefill_chunk");
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_chunk_len < 0) return pa_fail(PA_ERR_INVALID, "pa_prefill_chunk: negative size");
  if (q_dtype != PA_BF16) return pa_fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: q must be PA_BF16");
  if (out_dtype != PA_F32 && out_dtype != PA_BF16)
    return pa_fail(PA_ERR_INVALID, "pa_prefill_chunk: bad out_dtype");
  if (pool->dtype == PA_F32 || pool->head_dim != 128)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: needs a bf16 or fp8 pool with head_dim 128");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return pa_fail(PA_ERR_INVALID, "pa_prefill_chunk: num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / pool->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: group size must be 1, 2, 4 or 8");
  if (!std::isfinite(scale)) return pa_fail(PA_ERR_INVALID, "pa_prefill_chunk: scale is not finite");
  if (num_seqs > kMaxGridYZ || pool->num_kv_heads > kMaxGridYZ)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: more than 65535 sequences or KV heads");
  if (num_seqs == 0 || max_chunk_len == 0) return pa_ok();
  if (!q || !k_pool || !v_pool || !tables || !qsl || !prior || !out)
    return pa_fail(PA_ERR_INVALID, "pa_prefill_chunk: null pointer");
  if (max_blocks <= 0) return pa_fail(PA_ERR_INVALID, "pa_prefill_chunk: max_blocks_per_seq must be positive");
  pa::PrefillArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = tables;
  a.max_blocks = max_blocks;
  a.qsl = qsl;
  a.prior = prior;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_blocks = pool->num_blocks;
  const float kscale = pool->dtype == PA_FP8_E4M3 ? pool->k_scale : 1.0f;
  a.qk_scale = static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  a.v_scale = pool->dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
  a.max_chunk = max_chunk_len;
  a.out = out;
  return launch_status(pa::launch_prefill(a, pool->dtype, out_dtype, pool->block_size, pool->head_dim, stream),
                       "pa_prefill_chunk: no kernel for this combination");
}

pa_status pa_fp8_decode_table(float* out, pa_stream stream) {
  if (!out) return pa_fail(PA_ERR_INVALID, "pa_fp8_decode_table: out is null");
  return launch_status(pa::launch_fp8_table(out, stream), "pa_fp8_decode_table");
}

pa_status pa_hbm_read_probe(const void* buf, size_t bytes, void* sink, pa_stream stream) {
  if (!buf || !sink) return pa_fail(PA_ERR_INVALID, "pa_hbm_read_probe: null pointer");
  if (bytes == 0 || bytes % 16 != 0) return pa_fail(PA_ERR_INVALID, "pa_hbm_read_probe: bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return pa_fail(PA_ERR_INVALID, "pa_hbm_read_probe: buf is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(sink) % 4 != 0) return pa_fail(PA_ERR_INVALID, "pa_hbm_read_probe: sink is not 4-byte aligned");
  return launch_status(pa::launch_read_probe(buf, static_cast<int64_t>(bytes / 16), static_cast<uint32_t*>(sink), stream),
                       "pa_hbm_read_probe");
}

}  // extern "C"
