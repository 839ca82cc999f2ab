// Internal declarations shared by the C-ABI layer and the kernel launchers of libpa.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pa.h"

// Records `msg` as this thread's last error and returns `st`.
pa_status pa_fail(pa_status st, const char* msg);
// Clears this thread's last error and returns PA_OK.
pa_status pa_ok();

namespace pa {

// Dtype codes used as template arguments of the kernels.
enum Dt : int { kF32 = PA_F32, kBF16 = PA_BF16, kFP8 = PA_FP8_E4M3 };

struct CacheWriteArgs {
  const void* k;
  const void* v;
  int in_dtype;
  int64_t num_tokens;
  const int64_t* slots;
  void* k_pool;
  void* v_pool;
  int block_size;
  int num_kv_heads;
  int head_dim;
  int pool_dtype;
  float k_inv_scale;  // fp32(1 / k_scale), rounded once on the host
  float v_inv_scale;
  int64_t num_slots;  // num_blocks * block_size: slots at or beyond it are skipped
};

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v); the same pools for copy-on-write,
// different ones (device and pinned host memory) for swaps.
struct CopyBlocksArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  int64_t block_bytes;  // bytes of one block of one pool (all KV heads)
  const int32_t* pairs;
  int32_t num_pairs;
  int32_t num_layers;    // layer l's pools start layer_stride bytes after layer l - 1's
  int64_t layer_stride;
  int32_t src_blocks;    // blocks of the source and destination pools: pairs outside are skipped
  int32_t dst_blocks;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  int32_t max_blocks;
  const int32_t* lens;
  const int32_t* shared_blocks;   // optional: leading table entries per sequence that other rows also read
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;    // pool blocks: a table entry outside [0, num_blocks) is clamped into it
  float qk_scale;        // scale * k_scale * log2(e): logits in base-2 units
  float v_scale;
  int32_t part_tokens;   // tokens per partition (a multiple of 16; no sequence crosses one when it
                         // covers max_ctx)
  int32_t max_parts;     // partitions of the longest sequence
  int32_t max_ctx;       // bound on every context length (lengths are clamped to it on the device)
  int32_t streams;       // unit streams: 8 (one per XCD; KV head h in stream h % 8) or 1
  int32_t stream_waves;  // waves per stream
  int32_t max_shares;    // bound on the shares of one stream
  int32_t self_plan;     // 1: the stream kernel plans the launch itself (no plan kernel)
  int32_t fill_empty;    // 1: no merge launch; the stream kernel writes the zeros of empty sequences
  int32_t records_only;  // 1: every piece, a whole segment too, is left as a partial record (no output,
                         // no merge launch) for a later kernel to fold (the beam decode's tails)
  int64_t stream_slots;  // partial-record slots per stream
  int32_t* ws_pref;      // [num_seqs + 1] units (32 keys) of sequences before s, for one KV head
  int32_t* ws_sched;     // share size, share count
  int32_t* ws_share;     // [max_shares][4] start cursor of each share: head slot, sequence, unit, units
  float* ws_part;        // [streams * stream_slots][G][head_dim + 4]: max, sum, -, -, unnormalised o
  void* out;
  // Element strides of q and out for (sequence, KV head, head within the group); the head_dim
  // elements of one row are contiguous.  Dense [seq][head][dim] is (Hq * D, G * D, D).
  int64_t q_sseq, q_skv, q_sg;
  int64_t o_sseq, o_skv, o_sg;
  float* lse;            // optional: natural log of each row's softmax denominator, at out's row
                         // index divided by head_dim (strides o_s* / D)
};

// Bytes of the decode workspace for a launch of `waves` waves (see pa_decode_workspace_size).
size_t decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_parts,
                              int64_t waves);
// Waves of one decode launch on the current device (an upper bound for any dtype).
int decode_max_waves();
// The launch shape of a decode (streams, waves per stream, share bound, plan mode, record slots),
// set in `a` from its sizes, the pool dtype and the device only, so that a later launch over the
// same sizes finds this launch's records.  Returns the stream kernel's workgroups.
int64_t decode_launch_shape(DecodeArgs& a, int kv_dtype);
// Compute units of the current device (cached per device; 256 when the query fails).
int device_cus();
// Sets the workspace pointers of `a` (num_seqs set) inside a workspace of decode_workspace_bytes().
void decode_workspace_carve(DecodeArgs& a, void* workspace);
// The current device's copy of the library's static decode workspace (PA_DECODE_STATIC_WORKSPACE_BYTES):
// its device address in *ptr and its size in *bytes.  Returns 0, or the hipError_t of the lookup.
int decode_static_workspace(void** ptr, size_t* bytes);

struct PrefillArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  int32_t max_blocks;
  const int32_t* qsl;
  const int32_t* prior;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;    // pool blocks: a table entry outside [0, num_blocks) is clamped into it
  float qk_scale;        // scale * k_scale * log2(e)
  float v_scale;
  int32_t max_chunk;
  void* out;
};

// Launchers return a hipError_t value as int (0 = success).
int launch_cache_write(const CacheWriteArgs& a, void* stream);
int launch_copy_blocks(const CopyBlocksArgs& a, void* stream);

struct MergeStatesArgs {
  const float* o_a;
  const float* lse_a;
  const float* o_b;
  const float* lse_b;
  int64_t rows;
  int32_t head_dim;
  void* out;
  float* lse_out;
};
int launch_merge_states(const MergeStatesArgs& a, int out_dtype, void* stream);
struct TailMergeArgs {
  const void* q;         // bf16 [num_seqs][num_q_heads][128]
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables; // [num_seqs][max_blocks]: the tail's blocks, key j in block j / block_size
  int32_t max_blocks;
  const int32_t* lens;   // [num_seqs] tail keys, clamped to [0, max_tail]
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;    // pool blocks: a table entry outside [0, num_blocks) is clamped into it
  float qk_scale;        // scale * k_scale * log2(e)
  float v_scale;
  int32_t max_tail;      // at most 32
  const float* o_prev;   // [num_seqs][num_q_heads][128] normalised output over the other keys
  const float* lse_prev; // [num_seqs][num_q_heads] their natural log-sum-exp
  void* out;             // [num_seqs][num_q_heads][128] of out dtype
  // Records mode (width > 0, one query head per KV head): the other keys' state is read from the
  // partial records of `shared`, a records_only decode launch over groups of `width` consecutive
  // sequences (row (s, h) is head s % width of segment (s / width, h)); o_prev and lse_prev unused.
  int32_t width;
  DecodeArgs shared;
};
// Returns 0 on success, -1 when no kernel exists for the combination, else a hipError_t.
int launch_tail_merge(const TailMergeArgs& a, int kv_dtype, int block_size, int head_dim, int out_dtype,
                      void* stream);
// Returns 0 on success, -1 when no kernel exists for the combination, else a hipError_t.
int launch_decode(const DecodeArgs& a, int kv_dtype, int q_dtype, int out_dtype, int block_size,
                  int head_dim, void* stream);
int launch_prefill(const PrefillArgs& a, int kv_dtype, int out_dtype, int block_size, int head_dim,
                   void* stream);
int launch_fp8_table(float* out, void* stream);
int launch_read_probe(const void* buf, int64_t n16, uint32_t* sink, void* stream);

}  // namespace pa
