// Pool writes: slot scatter of new tokens' K/V (with fp8 quantisation), copy-on-write block copies.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» FAQ Q4: K/V of prefill and of
// decode are both written into pool blocks; §四 4.2 and §六 item 4: a write into a shared block is
// preceded by a copy of the block.  The slot of a token is table[p / b] * b + p % b (§三 3.1 figure);
// the allocator computes it on the host, these kernels only follow it.
//
// All kernels here are HBM-bound streams.  In the K pool (tiles [row][dim]) a token's row for one head
// is head_dim contiguous elements, written with 16-byte stores; in the V pool (tiles [dim][row]) a
// token's values stride by block_size elements, and consecutive lanes take consecutive tokens so
// that the tokens of one block land side by side in each dim row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// Input elements -> stored codes of one pool element: the bits themselves for an fp32/bf16 pool,
// one rounded fp32 product with the host-rounded reciprocal scale and then the e4m3 rounding for fp8.
template <int IN>
__device__ __forceinline__ void load_in8(const char* src, float (&x)[8]) {
  if constexpr (IN == kBF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(src);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(ws[j]);
      x[2 * j + 1] = bf16_hi(ws[j]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 w = reinterpret_cast<const uint4*>(src)[h];
      x[4 * h] = __uint_as_float(w.x);
      x[4 * h + 1] = __uint_as_float(w.y);
      x[4 * h + 2] = __uint_as_float(w.z);
      x[4 * h + 3] = __uint_as_float(w.w);
    }
  }
}

// K pool (token-major tiles): one thread per 16-byte chunk of one stored (token, KV head) row.
template <int IN, int POOL>
__global__ void __launch_bounds__(kThreads) cache_write_k_kernel(CacheWriteArgs a, int log2_bs,
                                                                 int chunks_per_row) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t total = a.num_tokens * a.num_kv_heads * chunks_per_row;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks_per_row);
  const int64_t row = idx / chunks_per_row;            // token * Hkv + head
  const int head = static_cast<int>(row % a.num_kv_heads);
  const int64_t t = row / a.num_kv_heads;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;   // skipped token, or a slot outside the pool
  const int64_t blk = slot >> log2_bs;
  const int64_t off = slot & ((1 << log2_bs) - 1);
  constexpr int kOutElem = POOL == kF32 ? 4 : POOL == kBF16 ? 2 : 1;
  constexpr int kInElem = IN == kF32 ? 4 : 2;
  constexpr int kElems = 16 / kOutElem;                 // elements per stored chunk
  const int64_t row_bytes = static_cast<int64_t>(a.head_dim) * kOutElem;
  const int64_t dst_off = ((blk * a.num_kv_heads + head) * (1 << log2_bs) + off) * row_bytes + c * 16;
  const char* src = static_cast<const char*>(a.k) + (row * a.head_dim + static_cast<int64_t>(c) * kElems) * kInElem;
  char* dst = static_cast<char*>(a.k_pool) + dst_off;
  if constexpr (POOL == IN) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else {
    static_assert(POOL == kFP8, "only fp8 pools convert");
    uint32_t packed[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x[8];
      load_in8<IN>(src + h * 8 * kInElem, x);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t p = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) p |= f32_to_e4m3(__fmul_rn(x[4 * i + j], a.k_inv_scale)) << (8 * j);
        packed[2 * h + i] = p;
      }
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

// A store, non-temporal when NT.
template <bool NT, typename T>
__device__ __forceinline__ void put(T* p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// V pool (dim-major tiles: element (row o, dim d) of a tile at d * block_size + o).  One thread per
// (token, KV head, group of 8 dims); a wave takes 8 consecutive tokens x 8 consecutive dim groups of
// one head.  Its loads read 128 contiguous bytes of each token's row (bf16), and each of its stores
// puts the 8 tokens of one dim row side by side when they fill consecutive slots.  (64 tokens of one
// dim group per wave would make every load lane touch a different row: slower by 2x on long prompts.)
// A decode step writes one token per sequence, so every V store fills a few bytes of a line that
// nothing else in the call writes; with NT the stores are non-temporal and those lines go out to
// memory during the write, instead of being written back from L2 while the step's decode streams the
// pools (see launch_cache_write for when).
template <int IN, int POOL, bool NT>
__global__ void __launch_bounds__(kThreads) cache_write_v_kernel(CacheWriteArgs a, int log2_bs) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int groups = a.head_dim / 8;                    // a multiple of 8 (head_dim 64 or 128)
  const int ghi = groups / 8;
  const int64_t t_blocks = (a.num_tokens + 7) / 8;
  if (idx >= t_blocks * 64 * a.num_kv_heads * ghi) return;
  const int lane = static_cast<int>(idx & 63);
  int64_t rest = idx >> 6;
  const int dg = static_cast<int>(rest % ghi) * 8 + (lane & 7);
  rest /= ghi;
  const int head = static_cast<int>(rest % a.num_kv_heads);
  const int64_t t = (rest / a.num_kv_heads) * 8 + (lane >> 3);
  if (t >= a.num_tokens) return;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;   // skipped token, or a slot outside the pool
  const int bs = 1 << log2_bs;
  const int64_t blk = slot >> log2_bs;
  const int off = static_cast<int>(slot & (bs - 1));
  constexpr int kOutElem = POOL == kF32 ? 4 : POOL == kBF16 ? 2 : 1;
  constexpr int kInElem = IN == kF32 ? 4 : 2;
  const char* src = static_cast<const char*>(a.v) +
                    ((t * a.num_kv_heads + head) * a.head_dim + 8 * dg) * static_cast<int64_t>(kInElem);
  // element (off, d) of tile (blk, head)
  char* tile = static_cast<char*>(a.v_pool) +
               (blk * a.num_kv_heads + head) * static_cast<int64_t>(bs) * a.head_dim * kOutElem;
  char* dst = tile + (static_cast<int64_t>(8 * dg) * bs + off) * kOutElem;
  const int64_t dstep = static_cast<int64_t>(bs) * kOutElem;
  if constexpr (POOL == IN) {
    if constexpr (IN == kBF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(src);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        put<NT>(reinterpret_cast<uint16_t*>(dst + (2 * j) * dstep), static_cast<uint16_t>(ws[j] & 0xffffu));
        put<NT>(reinterpret_cast<uint16_t*>(dst + (2 * j + 1) * dstep), static_cast<uint16_t>(ws[j] >> 16));
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 w = reinterpret_cast<const uint4*>(src)[h];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) put<NT>(reinterpret_cast<uint32_t*>(dst + (4 * h + j) * dstep), ws[j]);
      }
    }
  } else {
    static_assert(POOL == kFP8, "only fp8 pools convert");
    float x[8];
    load_in8<IN>(src, x);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      put<NT>(reinterpret_cast<uint8_t*>(dst + j * dstep), static_cast<uint8_t>(f32_to_e4m3(__fmul_rn(x[j], a.v_inv_scale))));
  }
}

// grid (num_pairs, 2 pools x layers, splits): each workgroup copies a share of one block of one pool
// of one layer (blockIdx.y = 2 * layer + (0 for K, 1 for V)).
__global__ void __launch_bounds__(kThreads) copy_blocks_kernel(CopyBlocksArgs a) {
  const int pair = blockIdx.x;
  const int32_t src = a.pairs[2 * pair];
  const int32_t dst = a.pairs[2 * pair + 1];
  // a pair naming a block outside its pool is skipped (no memory outside the pools is touched)
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const int64_t layer_off = static_cast<int64_t>(blockIdx.y >> 1) * a.layer_stride;
  const char* sbase = static_cast<const char*>((blockIdx.y & 1) ? a.src_v : a.src_k) + layer_off;
  char* dbase = static_cast<char*>((blockIdx.y & 1) ? a.dst_v : a.dst_k) + layer_off;
  const uint4* s = reinterpret_cast<const uint4*>(sbase + static_cast<int64_t>(src) * a.block_bytes);
  uint4* d = reinterpret_cast<uint4*>(dbase + static_cast<int64_t>(dst) * a.block_bytes);
  const int64_t n16 = a.block_bytes / 16;
  // Non-temporal stores: the copies' lines go out to memory during the copy instead of being written
  // back from L2 while the next launch (the step's decode) streams the pools.  Measured on MI355X
  // inside the step: fork storm (896 copies, 229 MB) copy 75 -> 81 us, decode 616 -> 595 us, step
  // 749 -> 745 us; shared-prefix step (256 copies) decode 1367 -> 1350 us, step 1432 -> 1428 us.
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  for (int64_t i = static_cast<int64_t>(blockIdx.z) * kThreads + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.z) * kThreads)
    __builtin_nontemporal_store(reinterpret_cast<const v4*>(s)[i], reinterpret_cast<v4*>(d) + i);
}

__global__ void fp8_table_kernel(float* out) {
  const uint32_t c = threadIdx.x;
  float a, b;
  fp8x2_to_f32<false>(c, a, b);
  out[c] = a;
}

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

}  // namespace

int launch_cache_write(const CacheWriteArgs& a, void* stream) {
  const int out_elem = a.pool_dtype == kF32 ? 4 : a.pool_dtype == kBF16 ? 2 : 1;
  const int chunks = a.head_dim * out_elem / 16;
  const int64_t total_k = a.num_tokens * a.num_kv_heads * chunks;
  const int64_t total_v = (a.num_tokens + 7) / 8 * 64 * a.num_kv_heads * (a.head_dim / 64);
  const dim3 gk(static_cast<unsigned>((total_k + kThreads - 1) / kThreads));
  const dim3 gv(static_cast<unsigned>((total_v + kThreads - 1) / kThreads));
  const int lb = ilog2(a.block_size);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Non-temporal V stores for small writes (at most kNtRows (token, KV head) rows, a decode step of a
  // small batch): measured inside the step on MI355X, the Llama-7B-shaped decode step (2048 rows)
  // write 14 -> 17 us, decode 208 -> 198 us; at 10 240 rows (the shared-prefix step) the write went
  // 26 -> 68 us for a decode 37 us shorter, and at the mixed step's 67 000 (prefill chunks, whose
  // consecutive tokens fill whole lines in L2) 28 -> 90 us, so larger writes keep ordinary stores.
  constexpr int64_t kNtRows = 4096;
  const bool nt = a.num_tokens * a.num_kv_heads <= kNtRows;
  auto v_kernel = [&](auto in_c, auto pool_c) {
    constexpr int IN = decltype(in_c)::value, POOL = decltype(pool_c)::value;
    if (nt)
      hipLaunchKernelGGL((cache_write_v_kernel<IN, POOL, true>), gv, dim3(kThreads), 0, s, a, lb);
    else
      hipLaunchKernelGGL((cache_write_v_kernel<IN, POOL, false>), gv, dim3(kThreads), 0, s, a, lb);
  };
  using F32 = std::integral_constant<int, kF32>;
  using BF16 = std::integral_constant<int, kBF16>;
  using FP8 = std::integral_constant<int, kFP8>;
  if (a.pool_dtype == kF32) {
    hipLaunchKernelGGL((cache_write_k_kernel<kF32, kF32>), gk, dim3(kThreads), 0, s, a, lb, chunks);
    v_kernel(F32{}, F32{});
  } else if (a.pool_dtype == kBF16) {
    hipLaunchKernelGGL((cache_write_k_kernel<kBF16, kBF16>), gk, dim3(kThreads), 0, s, a, lb, chunks);
    v_kernel(BF16{}, BF16{});
  } else if (a.in_dtype == kBF16) {
    hipLaunchKernelGGL((cache_write_k_kernel<kBF16, kFP8>), gk, dim3(kThreads), 0, s, a, lb, chunks);
    v_kernel(BF16{}, FP8{});
  } else {
    hipLaunchKernelGGL((cache_write_k_kernel<kF32, kFP8>), gk, dim3(kThreads), 0, s, a, lb, chunks);
    v_kernel(F32{}, FP8{});
  }
  return static_cast<int>(hipGetLastError());
}

int launch_copy_blocks(const CopyBlocksArgs& a, void* stream) {
  const int64_t n16 = a.block_bytes / 16;
  int splits = static_cast<int>((n16 + 4 * kThreads - 1) / (4 * kThreads));  // ~4 loads per thread
  if (splits < 1) splits = 1;
  if (splits > 64) splits = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, 2 * a.num_layers, splits), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

namespace {
// Streaming read of n16 16-byte pieces: each thread takes four pieces per round (grid-stride,
// non-temporal loads), XORs them into a register, and stores only if the fold hits a value it
// practically never takes.  Measured on MI355X over 2 GiB: 8 workgroups per CU 5.4 TB/s with
// ordinary loads, 5.8 non-temporal; 32 per CU (four times what fits at once) 6.1-6.3.
__global__ void __launch_bounds__(kThreads) read_probe_kernel(const uint4* p, int64_t n16, uint32_t* sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = __builtin_nontemporal_load(q + i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(q + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}
}  // namespace

int launch_read_probe(const void* buf, int64_t n16, uint32_t* sink, void* stream) {
  const int64_t wgs = std::min<int64_t>(static_cast<int64_t>(device_cus()) * 32, (n16 + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(std::max<int64_t>(wgs, 1))), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), n16, sink);
  return static_cast<int>(hipGetLastError());
}

int launch_fp8_table(float* out, void* stream) {
  hipLaunchKernelGGL(fp8_table_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), out);
  return static_cast<int>(hipGetLastError());
}

}  // namespace pa
