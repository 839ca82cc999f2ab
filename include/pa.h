/*
 * pa.h -- C ABI of libpa: paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title):
 *   [ch7]   «第 7 章推理框架：vLLM 与 PagedAttention»
 *   [exp]   «vLLM 与 PagedAttention：把 GPU 显存当操作系统内存管»
 *   [day28] «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术»
 * The KV cache is cut into fixed-size blocks (16 tokens by default) that lie anywhere in a physical
 * pool; each sequence's block table maps its logical blocks to physical ones; blocks of a common
 * prefix are shared under a reference count and copied before a write (copy-on-write); attention
 * reaches a sequence's scattered K/V through its table ([ch7] 7.1; [exp] PagedAttention section;
 * [day28] §三 3.1-3.2, §四 4.2, §六).
 *
 * Conventions for every call:
 *   - Every call returns pa_status; no exception or abort crosses this boundary.  On failure the
 *     text of pa_last_error() (thread-local) says what was wrong.
 *   - Device pointers are caller-owned (typically allocated by PyTorch) and must stay valid until
 *     the work queued on `stream` has finished.  The library never allocates device memory; the
 *     one device array it owns, the static workspace of pa_decode_noalloc, is reserved by the code
 *     object loader on each GPU the library runs on.
 *   - Host arguments are validated (null pointers, dtypes, shapes, sizes, alignment).  Values that
 *     live in device memory (slots, tables, lengths, copy pairs) are checked on the host only by
 *     pa_validate_* (the caller's allocator, pa_alloc_*, produces valid ones).  On the device a block
 *     id outside the pool is clamped into it, and a slot or copy pair outside it is skipped, so a bad
 *     value gives a wrong result but no access outside the pools; lengths are clamped to the
 *     launch's bounds.  Prefill's query_start_loc must stay inside q and out (pa_validate_prefill).
 *   - Launches are asynchronous on `stream` (a hipStream_t; NULL = the default stream), in order,
 *     with no implicit synchronisation.  Calls that overlap on different streams and touch the same
 *     pool blocks race.
 *
 * Pool layout (fixed by this ABI).  K and V live in two separate device arrays of elements of
 * `dtype`, row-major:
 *     K: [num_blocks][num_kv_heads][block_size][head_dim]   (token-major tiles)
 *     V: [num_blocks][num_kv_heads][head_dim][block_size]   (dim-major tiles)
 * One (block, KV head) tile is block_size * head_dim elements contiguous in memory, so the tokens of
 * one block are read with whole-cache-line loads and the only indirection is one table lookup per
 * block ([day28] §三 3.2: contiguous inside a block, a pointer jump between blocks).  Inside a tile,
 * element (row o, dim d) sits at o * head_dim + d in K and at d * block_size + o in V: K rows feed
 * the q.k products dim-contiguous, V columns feed the p.v products key-contiguous.  Token at slot s
 * lies in block s / block_size, row s % block_size.  An fp8 pool stores OCP e4m3 codes;
 * value = decode(code) * scale, with one fp32 scale per pool (k_scale for K, v_scale for V).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* a host argument is out of range or null */
  PA_ERR_OOM = 2,         /* allocator: not enough free blocks (state unchanged) */
  PA_ERR_HIP = 3,         /* the HIP runtime reported an error (launch or device query) */
  PA_ERR_UNSUPPORTED = 4  /* a valid combination the library has no kernel for */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,      /* IEEE binary32 */
  PA_BF16 = 1,     /* bfloat16 */
  PA_FP8_E4M3 = 2  /* OCP 8-bit E4M3 ("FN"): bias 7, no infinities, max 448 (pools only) */
} pa_dtype;

/* A KV pool.  Supported: block_size in {8, 16, 32}; head_dim in {64, 128};
 * dtype PA_F32, PA_BF16 or PA_FP8_E4M3; scales are used only for PA_FP8_E4M3 (must be > 0). */
typedef struct pa_pool_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;   /* pa_dtype */
  float k_scale;
  float v_scale;
} pa_pool_desc;

typedef void* pa_stream; /* hipStream_t */

/* Short name of a status code (static string). */
const char* pa_status_str(int32_t status);
/* Detail of the last failure on this thread (static thread-local buffer; "" after success). */
const char* pa_last_error(void);
/* ABI version: (major << 16) | minor (2.0: pa_decode without the cache hint, pa_decode_noalloc;
 * 2.1: pa_validate_*, pa_plan_beam_tails, device-side clamping of block ids; 2.2:
 * pa_decode_tail_merge; 2.3: pa_decode_beam). */
int32_t pa_version(void);

/* ---------------------------------------------------------------------------------------------
 * pa_cache_write -- scatter new tokens' K and V into their slots.
 * [day28] FAQ Q4: K/V produced by prefill are written into pool blocks just as decode's are;
 * [ch7] 7.1: each generated token's K/V goes into the sequence's current block.
 *
 *   k, v          device [num_tokens][num_kv_heads][head_dim] of in_dtype (PA_F32 or PA_BF16),
 *                 contiguous rows
 *   slot_mapping  device int64 [num_tokens]; token t goes to slot slot_mapping[t]; a negative slot
 *                 skips the token
 *   k_pool/v_pool device pools described by `pool`
 * A PA_F32 / PA_BF16 pool must have dtype == in_dtype and receives the bits unchanged.  A
 * PA_FP8_E4M3 pool receives, per element, e4m3(round_to_nearest_even(clamp(x * inv, -448, 448)))
 * where inv = fp32(1 / scale) is rounded once on the host and the product is an fp32 multiply.
 * Slots must be distinct among non-negative entries (duplicate slots race).
 * num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_cache_write(const void* k, const void* v, int32_t in_dtype, int64_t num_tokens,
                         const int64_t* slot_mapping, void* k_pool, void* v_pool,
                         const pa_pool_desc* pool, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_copy_blocks -- copy-on-write block copies ([day28] §四 4.2, §六 item 4: a sequence about to
 * write a shared block gets a new block holding a copy of it).
 *
 *   pairs  device int32 [num_pairs][2] = (source block, destination block), as returned by
 *          pa_alloc_append.  Whole K and V blocks (all KV heads) are copied.  Destinations must be
 *          distinct and must not appear as a source in the same call (copies run concurrently).
 * num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc* pool, const int32_t* pairs,
                         int32_t num_pairs, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_copy_blocks_layers -- the copy-on-write copies of one step for every layer of a model, in one
 * launch.  A block id names the same block in every layer's pools ([ch7] 7.1: the KV cache holds
 * K and V of every layer; one block table serves them all).
 *
 *   k_pools, v_pools    layer 0's K and V pools; layer l's start l * layer_stride_bytes later
 *                       (a multiple of 16, at least one layer's pool size when num_layers > 1)
 *   num_layers          1 .. 32767
 *   pool, pairs, n      as pa_copy_blocks (pool describes one layer)
 * ------------------------------------------------------------------------------------------- */
pa_status pa_copy_blocks_layers(void* k_pools, void* v_pools, int64_t layer_stride_bytes, int32_t num_layers,
                                const pa_pool_desc* pool, const int32_t* pairs, int32_t num_pairs,
                                pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_swap_blocks -- whole-block copies from one pool to another of the same block format: the
 * data movement of a swap-out (device pool -> pinned host pool) or swap-in (host -> device) of a
 * preempted sequence ([day28] §六 question 4).
 *
 *   dst_*  destination K and V pools and their descriptor
 *   src_*  source K and V pools and their descriptor (num_blocks may differ; block_size,
 *          num_kv_heads, head_dim, dtype and the fp8 scales must be equal: codes move unchanged)
 *   pairs  int32 [num_pairs][2] = (source block, destination block), as pa_alloc_move_seq
 *          returns them, in device or pinned host memory.  Destinations must be distinct.
 * Each pool pointer must be device memory or pinned host memory (hipHostMalloc), which the kernel
 * reaches over the host link; anything else (pageable memory, unknown pointers) is refused with
 * PA_ERR_INVALID before any launch.  Block ids are not checked (out of range is undefined
 * behaviour).  One kernel launch on the stream, asynchronous like every call here: the pools and
 * the pairs must stay allocated, and unchanged, until it completes.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, const pa_pool_desc* dst_pool,
                         const void* src_k_pool, const void* src_v_pool, const pa_pool_desc* src_pool,
                         const int32_t* pairs, int32_t num_pairs, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs for these sizes, on the
 * current device (the size depends on its compute-unit count).
 *   partition_size 0 means the library's choice (the same choice pa_decode makes for 0).
 * The workspace holds the work plan (per-sequence unit counts, the split of the work among the
 * resident waves) and the partial (max, sum, unnormalised output) records of context pieces: one
 * record of head_dim + 4 floats per (query head, sequence, partition) plus a bounded number per
 * resident wave.  pa_decode rewrites all of it on every call.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_size, size_t* bytes);

/* ---------------------------------------------------------------------------------------------
 * pa_decode -- one query token per sequence attends to its cached context through its table.
 * [day28] §三 3.1-3.2: the kernel gathers the scattered K/V by indirection through the block table,
 * dotting the query with every cached key and combining the values.  For sequence s and query head
 * h (KV head g = h / (num_q_heads / num_kv_heads)):
 *     out[s,h,:] = sum_j softmax_j(scale * q[s,h,:] . K_s[j,g,:]) V_s[j,g,:],   0 <= j < L_s
 * with K_s[j] = k_pool[table[s][j / b]][g][j % b] (times k_scale for fp8; V likewise).
 *
 *   q             device [num_seqs][num_q_heads][head_dim] of q_dtype (PA_F32 or PA_BF16)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries past ceil(L_s / b) unused
 *   context_lens  device int32 [num_seqs]; L_s in [0, max_context_len]; L_s == 0 gives zeros
 *   num_q_heads   multiple of pool->num_kv_heads; group size num_q_heads / num_kv_heads in {1,2,4,8}
 *   scale         fp32 softmax scale (e.g. fp32(1/sqrt(head_dim)))
 *   partition_size  tokens per context partition, a positive multiple of 32, or 0 (library choice:
 *                 no partition boundaries).  The context of every (sequence, KV head) is split into
 *                 pieces for load balance; no piece crosses a partition boundary, and a second
 *                 kernel merges the pieces of each output (max, rescaled sums).
 *   max_context_len  an upper bound of every L_s (sizes the launch and the workspace)
 *   workspace     device buffer of at least pa_decode_workspace_size(...) bytes; its content on
 *                 entry does not matter.  Calls that share a workspace must not overlap.
 *   out           device [num_seqs][num_q_heads][head_dim] of out_dtype (PA_F32 or PA_BF16;
 *                 bf16 rounds to nearest-even from the fp32 accumulator)
 * q must start at a 16-byte boundary and out at a boundary of 4 elements (rows are read in 16-byte
 * pieces and written 4 elements at a time).
 * Combinations: pool PA_F32 needs q PA_F32; pools PA_BF16 / PA_FP8_E4M3 need q PA_BF16.
 * Results are deterministic: the pieces and every reduction order depend only on the sizes and
 * lengths.  The cache-policy hint of a shared prefix is an argument of pa_decode_ex.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_decode(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                    const pa_pool_desc* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                    int32_t partition_size, int32_t max_context_len, void* workspace,
                    size_t workspace_bytes, void* out, int32_t out_dtype, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_prefill_chunk -- causal attention of a chunk of new query tokens per sequence over the
 * sequence's paged context plus the chunk itself ([day28] FAQ Q4: prefill K/V are written into
 * pool blocks; chunked prefill slices a long prompt and is scheduled together with decode).
 * The chunk's own K/V must already be in the pool (pa_cache_write first).  Query i of sequence s
 * sits at position P_s + i and attends keys 0 .. P_s + i inclusive, all read through the table.
 *
 *   q                  device [total_q][num_q_heads][head_dim] bf16, chunks back to back
 *   query_start_loc    device int32 [num_seqs + 1]; chunk of s = rows [qsl[s], qsl[s+1])
 *   prior_context_lens device int32 [num_seqs]; P_s tokens held before the chunk
 *   max_chunk_len      upper bound of every chunk length (sizes the launch)
 *   out                device [total_q][num_q_heads][head_dim], PA_BF16 or PA_F32
 * Pools: PA_BF16 or PA_FP8_E4M3, head_dim 128.  The products run on bf16 MFMA with fp32
 * accumulation (fp8 K/V are widened to bf16 exactly; scales are applied in fp32).
 * ------------------------------------------------------------------------------------------- */
pa_status pa_prefill_chunk(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                           const pa_pool_desc* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* query_start_loc,
                           const int32_t* prior_context_lens, int32_t num_seqs, int32_t num_q_heads,
                           float scale, int32_t max_chunk_len, void* out, int32_t out_dtype,
                           pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_decode_ex -- pa_decode with strided q and out and an optional log-sum-exp output.  Beam
 * branches share their prompt's blocks ([day28] §六 question 3); with these, one call can read a
 * shared segment once for the queries of every branch (the branches' queries of one KV head as its
 * query heads), and pa_merge_states combines that result with each branch's private tail.
 *
 *   q_strides, out_strides  NULL (dense [num_seqs][num_q_heads][head_dim]) or host int64 [3]:
 *                 element strides for (sequence, KV head, head within the KV head's group); the
 *                 head_dim elements of a row are contiguous.  q strides are multiples of 16 bytes
 *                 (4 f32 or 8 bf16 elements), out strides multiples of 4 elements; with lse_out, out
 *                 strides are also multiples of head_dim.  Base pointers as for pa_decode.
 *   lse_out       NULL or device float: ln(sum_j exp(scale * q . k_j)) of each (sequence, head) row
 *                 (k_j with k_scale applied), at the row's out offset divided by head_dim; -inf
 *                 for L_s == 0.
 *   shared_blocks NULL or device int32 [num_seqs]: how many leading entries of each sequence's
 *                 table other sequences of the call also read (a shared prefix, [day28] §六 question
 *                 2).  Only the cache policy depends on it, never the results: K/V of those blocks
 *                 are read through the caches so that their repeats hit; every other block is
 *                 streamed with non-temporal loads (read once, kept out of the way of the shared
 *                 ones): its V, and for fp8 pools its K too.  NULL: no block is shared.
 * Everything else as pa_decode; pa_decode is pa_decode_ex with NULL strides, lse_out and
 * shared_blocks.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_decode_ex(const void* q, int32_t q_dtype, const int64_t* q_strides, const void* k_pool,
                       const void* v_pool, const pa_pool_desc* pool, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_q_heads, float scale, int32_t partition_size, int32_t max_context_len,
                       void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                       const int64_t* out_strides, float* lse_out, const int32_t* shared_blocks,
                       pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_decode_noalloc -- pa_decode_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Instead of a caller
 * workspace it uses a static device array that the library holds on each GPU it runs on, of
 * PA_DECODE_STATIC_WORKSPACE_BYTES (64 MiB), until the process ends.  The call itself allocates
 * nothing.
 *   Arguments as pa_decode_ex without workspace and workspace_bytes.  PA_ERR_INVALID (nothing
 *   launched) when pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
 *   partition_size) exceeds PA_DECODE_STATIC_WORKSPACE_BYTES: with partition_size 0 that holds
 *   up to about 40 000 (sequence, query head) rows at head_dim 128.
 * Every call on one GPU shares that GPU's array, and each call rewrites what it uses (nothing in it
 * needs to start at zero), so calls on one GPU must not overlap: two streams, or two threads,
 * that decode at the same time race on it.  Results are bit-identical to pa_decode_ex with a
 * workspace of its own.
 * ------------------------------------------------------------------------------------------- */
#define PA_DECODE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(const void* q, int32_t q_dtype, const int64_t* q_strides, const void* k_pool,
                            const void* v_pool, const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_q_heads, float scale, int32_t partition_size, int32_t max_context_len,
                            void* out, int32_t out_dtype, const int64_t* out_strides, float* lse_out,
                            const int32_t* shared_blocks, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_plan_cache_hint (host) -- the shared_blocks hint of pa_decode_ex for a batch: for each
 * sequence, the length of the leading run of its table entries (within its ceil(lens[s] /
 * block_size) used ones) whose physical block another used entry of the batch also names, i.e.
 * the blocks of a shared prefix that several rows read ([day28] §六 question 3; [exp]
 * 「PagedAttention：向操作系统借思路」 on sharing blocks between sequences).  tables host int32
 * [num_seqs][max_blocks], lens host int32 [num_seqs], shared_blocks host int32 [num_seqs] (out).
 * PA_ERR_INVALID on a negative size or length, or a length needing more than max_blocks entries.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_plan_cache_hint(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t num_seqs,
                             int32_t block_size, int32_t* shared_blocks);

/* ---------------------------------------------------------------------------------------------
 * pa_plan_shared_blocks (host) -- for a decode batch laid out as groups of `width` consecutive
 * sequences (the branches of one request), the number of leading blocks every member of group g
 * shares: shared_blocks[g] = the longest k such that all members have the same first k table
 * entries and k * block_size <= every member's length.  tables host int32 [num_seqs][max_blocks],
 * lens host int32 [num_seqs], shared_blocks host int32 [num_seqs / width].  PA_ERR_INVALID if
 * num_seqs is not a multiple of width.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_plan_shared_blocks(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t num_seqs,
                                int32_t block_size, int32_t width, int32_t* shared_blocks);

/* ---------------------------------------------------------------------------------------------
 * pa_plan_beam_tails (host) -- the private tails of a beam decode batch laid out as in
 * pa_plan_shared_blocks: sequence s of group g = s / width keeps its blocks from shared_blocks[g]
 * on.  tail_lens host int32 [num_seqs] receives lens[s] - shared_blocks[g] * block_size;
 * tail_tables host int32 [num_seqs][tail_max_blocks] receives each tail's table entries, padded
 * with 0; *needed_max_blocks (may be NULL) the longest tail in blocks.  tail_tables may be NULL to
 * get only the lengths and the needed width.  PA_ERR_INVALID if a group's shared blocks exceed a
 * member's length, a row is shorter than its length, or tail_max_blocks is too small.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_plan_beam_tails(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t num_seqs,
                             int32_t block_size, int32_t width, const int32_t* shared_blocks, int32_t* tail_tables,
                             int32_t tail_max_blocks, int32_t* tail_lens, int32_t* needed_max_blocks);

/* ---------------------------------------------------------------------------------------------
 * pa_merge_states -- combine two attention results of the same query rows over disjoint key sets
 * (a shared segment and a private tail), the rescaled combination the split merge uses:
 *     M = max(lse_a, lse_b),  w_x = exp(lse_x - M),
 *     out = (o_a w_a + o_b w_b) / (w_a + w_b),  lse_out = M + ln(w_a + w_b).
 *   o_a, o_b      device float [rows][head_dim];  lse_a, lse_b  device float [rows]
 *   out           device [rows][head_dim] of out_dtype (PA_F32 or PA_BF16); may be o_a or o_b
 *   lse_out       NULL or device float [rows]
 * A row whose two lse are -inf (no keys) gives zeros and -inf.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_merge_states(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                          int64_t rows, int32_t head_dim, void* out, int32_t out_dtype, float* lse_out,
                          pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_decode_tail_merge -- the private tails of a beam decode and the merge with the shared part, in
 * one launch, for tails of at most 32 keys ([day28] §六 question 3: branches read their common
 * prompt blocks once; each branch then has only the few tokens it generated since the fork).  For
 * sequence s and query head h (KV head g = h / (num_q_heads / num_kv_heads)), with the tail's
 * keys T_s[j] = pool[tail_tables[s][j / b]][g][j % b], 0 <= j < tail_lens[s]:
 *     lse_t = ln sum_j exp(scale q[s,h,:] . K_T[j]),  o_t = softmax_j(...) V_T
 *     out[s,h,:] = (o_prev[s,h,:] e^(lse_prev[s,h] - M) + o_t e^(lse_t - M)) / (e^(lse_prev - M) + e^(lse_t - M))
 * with M the larger of the two log-sum-exps: what pa_decode_ex over the tails (with lse_out)
 * followed by pa_merge_states computes.  A row with no tail keys gets o_prev; a row with neither
 * gets zeros.
 *   q            device bf16 [num_seqs][num_q_heads][128], 16-byte aligned; the pool bf16 or fp8
 *                (PA_ERR_UNSUPPORTED otherwise, and for head_dim other than 128)
 *   tail_tables  device int32 [num_seqs][max_blocks_per_seq]; tail_lens device int32 [num_seqs],
 *                each clamped to [0, max_tail_len] on the device
 *   max_tail_len a bound of every tail length, at most 32 (PA_ERR_UNSUPPORTED above: decode such
 *                tails with pa_decode_ex and combine them with pa_merge_states)
 *   o_prev       device float [num_seqs][num_q_heads][128], 8-byte aligned, and lse_prev device
 *                float [num_seqs][num_q_heads] (natural log; -inf for no keys): the other part's
 *                result, as pa_decode_ex writes it with lse_out
 *   out          device [num_seqs][num_q_heads][128] of out_dtype (PA_F32 or PA_BF16), aligned to
 *                two elements; it must not overlap o_prev
 * The tail's P.V products run in fp32 (the probabilities are not rounded to bf16).
 * ------------------------------------------------------------------------------------------- */
pa_status pa_decode_tail_merge(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                               const pa_pool_desc* pool, const int32_t* tail_tables, int32_t max_blocks_per_seq,
                               const int32_t* tail_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                               int32_t max_tail_len, const float* o_prev, const float* lse_prev, void* out,
                               int32_t out_dtype, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_decode_beam -- the whole beam decode in at most two launches ([day28] §六 question 3): the
 * shared blocks of each request read once for all its branches, then every branch's private tail of
 * at most 32 keys, folded into the shared part's partial results as it is read.  The batch is
 * num_seqs sequences in groups of `width` consecutive branches (the members of one request), one
 * query head per KV head (H = num_kv_heads of the pool).  For sequence s of group g = s / width and
 * head h, the keys are those of pa_decode_ex over the shared part followed by those of the tail:
 *     shared  pool[tables[g * width][j / b]][h][j % b], 0 <= j < shared_lens[g]
 *     tail    pool[tail_tables[s][j / b]][h][j % b],    0 <= j < tail_lens[s]
 * and out[s,h,:] = softmax over both key sets of scale q[s,h,:] . K, times V: what pa_decode_ex over
 * the shared part (the branches as query heads) and pa_decode_tail_merge compute, without the
 * shared part's output and log-sum-exp ever being written.  A row with neither shared nor tail keys
 * gets zeros.
 *   q              device bf16 [num_seqs][H][128], 16-byte aligned; the pool bf16 or fp8
 *                  (PA_ERR_UNSUPPORTED otherwise, and for head_dim other than 128)
 *   tables         device int32 [num_seqs][max_blocks_per_seq] (only the rows of each group's first
 *                  member are read, for their shared blocks); shared_lens device int32 [num_seqs /
 *                  width], clamped to [0, max_shared_len] on the device
 *   tail_tables    device int32 [num_seqs][tail_max_blocks]; tail_lens device int32 [num_seqs],
 *                  clamped to [0, max_tail_len]; max_tail_len at most 32 (PA_ERR_UNSUPPORTED above)
 *                  (pa_plan_shared_blocks and pa_plan_beam_tails make these from the batch's tables)
 *   width          2, 4 or 8, dividing num_seqs
 *   workspace      device memory of at least pa_decode_workspace_size(num_seqs / width, width * H,
 *                  128, max_shared_len, 0) bytes: the shared part's plan and partial records
 *   out            device [num_seqs][H][128] of out_dtype (PA_F32 or PA_BF16), two-element aligned
 *   phases         PA_BEAM_SHARED: the shared part only (it leaves its records in the workspace);
 *                  PA_BEAM_TAILS: the tails and the output, reading the records that the last
 *                  PA_BEAM_SHARED call with the same sizes, tables, lengths and workspace left;
 *                  both: the two in order.  The split lets the shared part run before the step's
 *                  cache writes and copy-on-write copies, which never touch a shared block; keep
 *                  the workspace untouched between the two calls.
 * ------------------------------------------------------------------------------------------- */
enum { PA_BEAM_SHARED = 1, PA_BEAM_TAILS = 2 };
pa_status pa_decode_beam(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                         const pa_pool_desc* pool, const int32_t* tables, int32_t max_blocks_per_seq,
                         const int32_t* shared_lens, int32_t max_shared_len, const int32_t* tail_tables,
                         int32_t tail_max_blocks, const int32_t* tail_lens, int32_t max_tail_len, int32_t num_seqs,
                         int32_t width, float scale, void* workspace, size_t workspace_bytes, void* out,
                         int32_t out_dtype, int32_t phases, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * Host checks of device-resident inputs (no GPU).  The kernels use these values as given; out of
 * range they would address the wrong memory, so the kernels also clamp a block id into the pool and
 * skip slots and copy pairs outside it -- a bad value then gives a wrong result for its sequence or
 * token, never an access outside the pools.  These calls check host copies of the values before
 * they are sent to the device, and name the first bad entry in pa_last_error() ([day28] §三 3.1:
 * logical block j of a sequence lives in physical block table[j]; FAQ Q3).
 *   pa_validate_decode   table entries 0 .. ceil(L_s / block_size) - 1 of every sequence inside the
 *                        pool; 0 <= L_s <= max_context_len; ceil(L_s / b) <= max_blocks_per_seq
 *   pa_validate_prefill  query_start_loc non-decreasing from >= 0, every chunk <= max_chunk_len,
 *                        qsl[num_seqs] <= total_q, prior lengths >= 0, table entries of
 *                        prior + chunk tokens inside the pool
 *   pa_validate_slots    every non-negative slot < num_blocks * block_size, and distinct
 *   pa_validate_pairs    sources inside src_pool, destinations inside dst_pool and distinct; with
 *                        in_place != 0 (copy-on-write) no destination is also a source
 * All pointers are host pointers.  PA_OK, or PA_ERR_INVALID.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_validate_decode(const pa_pool_desc* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len);
pa_status pa_validate_prefill(const pa_pool_desc* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* query_start_loc, const int32_t* prior_context_lens, int32_t num_seqs,
                              int32_t max_chunk_len, int64_t total_q);
pa_status pa_validate_slots(const pa_pool_desc* pool, const int64_t* slot_mapping, int64_t num_tokens);
pa_status pa_validate_pairs(const pa_pool_desc* src_pool, const pa_pool_desc* dst_pool, const int32_t* pairs,
                            int32_t num_pairs, int32_t in_place);

/* ---------------------------------------------------------------------------------------------
 * Self-check of the device fp8 decoding: out[c] = value of e4m3 code c (c = 0..255) as decoded by
 * the same conversion the attention kernels use (NaN codes give NaN).  out: device float [256].
 * ------------------------------------------------------------------------------------------- */
pa_status pa_fp8_decode_table(float* out, pa_stream stream);

/* ---------------------------------------------------------------------------------------------
 * pa_hbm_read_probe -- measurement aid: streams `bytes` of device memory at buf once with 16-byte
 * non-temporal loads (32 workgroups per compute unit, four loads in flight per thread), so that
 * its time gives the read bandwidth this device reaches with plain streaming loads: the practical
 * ceiling against which a bandwidth-bound kernel's achieved GB/s is read (the pages expect paged
 * attention to cost little against a contiguous layout: [day28] §七).  buf: device pointer,
 * 16-byte aligned; bytes: a positive multiple of 16.  sink: device pointer to one uint32 that the
 * kernel writes only if the data folds to a value it never takes in practice (it keeps the loads
 * from being removed; its content afterwards is unspecified).  PA_ERR_INVALID on a null pointer,
 * misalignment or a size that is not a positive multiple of 16.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_hbm_read_probe(const void* buf, size_t bytes, void* sink, pa_stream stream);

/* =============================================================================================
 * Host block allocator (no GPU).  [ch7] 7.1 「三个关键机制」; [exp] PagedAttention section;
 * [day28] §三 3.1, §四 4.2, §六, FAQ Q3.
 *   - blocks of block_size token slots; a sequence takes a new block only when its last block is
 *     full; the free list is a FIFO queue whose initial order the caller gives (any free block
 *     serves any sequence); a finished sequence's blocks whose count drops to zero join its tail,
 *     in table order;
 *   - fork: the child shares all of the parent's blocks (each count + 1);
 *   - append: a token landing in a block whose count is > 1 first moves the sequence to a fresh
 *     block (copy-on-write); the (source, destination) pair is reported so the caller can run
 *     pa_copy_blocks before writing the token;
 *   - all-or-nothing: PA_ERR_OOM leaves the state unchanged.
 * A handle is not thread-safe; use one per thread or lock around it.
 * ============================================================================================= */
typedef struct pa_allocator pa_allocator;

/* initial_free_order: host int32 [num_blocks], a permutation of 0..num_blocks-1 (NULL = 0..N-1). */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                          pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);
/* New empty sequence; PA_ERR_INVALID if the id exists. */
pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq_id);
/* child shares every block of parent; PA_ERR_INVALID if parent is unknown or child exists. */
pa_status pa_alloc_fork(pa_allocator* a, int64_t parent_id, int64_t child_id);
/* Slots for n_tokens new tokens of seq_id, written to host int64 slots_out[n_tokens]; the
 * copy-on-write pairs (at most one per call) go to host int32 cow_pairs_out[cow_cap][2] and their
 * count to *n_cow_out.  PA_ERR_OOM (state unchanged) if the free list is too short;
 * PA_ERR_INVALID if cow_cap is too small for the copies needed. */
pa_status pa_alloc_append(pa_allocator* a, int64_t seq_id, int32_t n_tokens, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out);
/* Appends for several distinct sequences in order, all-or-nothing across the batch.  slots_out
 * receives sum(n_tokens) slots, sequence after sequence. */
pa_status pa_alloc_append_batch(pa_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                                int32_t num_seqs, int64_t* slots_out, int32_t* cow_pairs_out,
                                int32_t cow_cap, int32_t* n_cow_out);
/* Free blocks an append of n_tokens would take (new blocks plus a copy-on-write). */
pa_status pa_alloc_blocks_needed(const pa_allocator* a, int64_t seq_id, int32_t n_tokens,
                                 int32_t* out);
/* Drop the sequence; blocks reaching count 0 join the free list. */
pa_status pa_alloc_free_seq(pa_allocator* a, int64_t seq_id);
pa_status pa_alloc_seq_len(const pa_allocator* a, int64_t seq_id, int64_t* len_out);
/* The sequence's table into host int32 out[cap]; *n_out = its length (PA_ERR_INVALID if > cap). */
pa_status pa_alloc_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                               int32_t* n_out);
/* Tables of several sequences as rows of host int32 out[num_seqs][max_blocks], padded with `pad`. */
pa_status pa_alloc_fill_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t* out, int32_t max_blocks, int32_t pad);
pa_status pa_alloc_refcount(const pa_allocator* a, int32_t block, int32_t* out);
pa_status pa_alloc_stats(const pa_allocator* a, int32_t* num_free, int32_t* num_used,
                         int64_t* total_refs);
/* The free list in queue order into host int32 out[cap]; *n_out = its length. */
pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out);

/* ---------------------------------------------------------------------------------------------
 * Prefix cache.  [ch7] 7.1 「三个关键机制」 and its vLLM parameter list (requests with the same
 * system prompt share its physical blocks under a reference count); [day28] §七 (a request whose
 * prompt starts with a cached prefix skips that prefill); [day28] FAQ Q5 (it pays when the prefix
 * is long and stable).  Off until enabled; while off, the calls below change nothing.
 *   - only full blocks are cached, each under the key (the entry id of the block before it, 0 for
 *     the first, and its block_size token ids); entry ids are never reused, so a key names one
 *     exact token prefix;
 *   - a cached block whose count drops to zero is kept ("evictable", least recently released
 *     first) and reclaimed, entry dropped, only once the free list is empty: appends and OOM
 *     checks count free + evictable blocks, and a failed append restores the cache too;
 *   - pa_alloc_free_seq queues a sequence's cached blocks from its table's last block to its
 *     first, so under pressure a cached prompt loses its deepest blocks first and the rest still
 *     matches (a lookup always starts at a prompt's first block).
 * ------------------------------------------------------------------------------------------- */
pa_status pa_alloc_enable_prefix_cache(pa_allocator* a);
/* New sequence with prompt host int32 tokens[n_tokens]: its table starts with the longest run of
 * cached blocks matching the prompt, leaving at least one prompt token uncovered (its K/V are
 * already in the pool); *n_cached_out = the tokens covered (a multiple of block_size, also the
 * sequence length).  The caller appends and computes only tokens[*n_cached_out:].  PA_ERR_INVALID
 * if the id exists or the prompt pointer is null with n_tokens > 0. */
pa_status pa_alloc_add_seq_prefix(pa_allocator* a, int64_t seq_id, const int32_t* tokens,
                                  int32_t n_tokens, int32_t* n_cached_out);
/* Register the full blocks of seq_id holding tokens[0:n_tokens] (host int32), whose K/V the caller
 * has written.  Blocks whose key is cached already keep the existing entry.  PA_ERR_INVALID if the
 * sequence is unknown, n_tokens exceeds its length, or one of its blocks is cached under other
 * tokens (entries registered before the error stay). */
pa_status pa_alloc_cache_seq(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int64_t n_tokens);
/* ---------------------------------------------------------------------------------------------
 * Swap of a preempted sequence between two pools of one block format, each with its own allocator
 * (say the device pool and a pinned host pool).  [day28] §六 question 4 (preemption swaps a
 * request's KV cache to CPU memory; paging makes that a copy of the blocks its table lists) and
 * FAQ Q3 (memory can still run out).  Every block of the sequence's table gets a block from dst's
 * supply (free list, then idle cached blocks), in table order; the sequence keeps its length and
 * id and is then freed in src like a finished one (a block it shared keeps its other references).
 * The (src block, dst block) pairs go to host int32 pairs_out[cap][2], *n_pairs_out = their count
 * (= the table length); run pa_swap_blocks on them before the freed src blocks are reused.
 * PA_ERR_OOM (both states unchanged) if dst cannot supply every block; PA_ERR_INVALID if the id is
 * unknown in src or exists in dst, the block sizes differ, src == dst, or cap is too small.
 * ------------------------------------------------------------------------------------------- */
pa_status pa_alloc_move_seq(pa_allocator* src, pa_allocator* dst, int64_t seq_id, int32_t* pairs_out,
                            int32_t cap, int32_t* n_pairs_out);
/* Number of cache entries and of evictable blocks (either pointer may be NULL). */
pa_status pa_alloc_cache_stats(const pa_allocator* a, int32_t* num_cached, int32_t* num_evictable);
/* The evictable blocks, least recently released first, into host int32 out[cap]; *n_out = count. */
pa_status pa_alloc_evictable_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
