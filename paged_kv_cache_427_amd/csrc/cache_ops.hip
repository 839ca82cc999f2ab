// Pool writes: slot scatter of new tokens' K/V (with fp8 quantisation), copy-on-write block copies.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» FAQ Q4: K/V of prefill and of
// decode are both written into pool blocks; §四 4.2 and §六 item 4: a write into a shared block is
// preceded by a copy of the block.  The slot of a token is table[p / b] * b + p % b (§三 3.1 figure);
// the allocator computes it on the host, these kernels only follow it.
//
// Both kernels are HBM-bound streams of 16-byte vector loads and stores; the pool layout
// [block][kv_head][row][dim] makes one (token, head) row R = head_dim * elem bytes contiguous.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte chunk of one stored (token, KV head) row, for K and for V.
template <int IN, int POOL>
__global__ void __launch_bounds__(kThreads) cache_write_kernel(CacheWriteArgs a, int log2_bs,
                                                               int chunks_per_row) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t total = a.num_tokens * a.num_kv_heads * chunks_per_row;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks_per_row);
  const int64_t row = idx / chunks_per_row;            // token * Hkv + head
  const int head = static_cast<int>(row % a.num_kv_heads);
  const int64_t t = row / a.num_kv_heads;
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t blk = slot >> log2_bs;
  const int64_t off = slot & ((1 << log2_bs) - 1);
  constexpr int kOutElem = POOL == kF32 ? 4 : POOL == kBF16 ? 2 : 1;
  constexpr int kInElem = IN == kF32 ? 4 : 2;
  constexpr int kElems = 16 / kOutElem;                 // elements per stored chunk
  const int64_t row_bytes = static_cast<int64_t>(a.head_dim) * kOutElem;
  const int64_t dst_off = ((blk * a.num_kv_heads + head) * (1 << log2_bs) + off) * row_bytes + c * 16;
  const int64_t src_elem = row * a.head_dim + static_cast<int64_t>(c) * kElems;
  if constexpr (POOL == IN) {
    const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(a.k) + src_elem * kInElem);
    const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(a.v) + src_elem * kInElem);
    *reinterpret_cast<uint4*>(static_cast<char*>(a.k_pool) + dst_off) = *ks;
    *reinterpret_cast<uint4*>(static_cast<char*>(a.v_pool) + dst_off) = *vs;
  } else {
    static_assert(POOL == kFP8, "only fp8 pools convert");
    constexpr int kIn16 = kElems * kInElem / 16;         // 16-byte input loads per output chunk
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const char* src = static_cast<const char*>(which ? a.v : a.k) + src_elem * kInElem;
      const float inv = which ? a.v_inv_scale : a.k_inv_scale;
      float x[kElems];
#pragma unroll
      for (int i = 0; i < kIn16; ++i) {
        const uint4 w = reinterpret_cast<const uint4*>(src)[i];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (IN == kBF16) {
            x[i * 8 + 2 * j] = bf16_lo(ws[j]);
            x[i * 8 + 2 * j + 1] = bf16_hi(ws[j]);
          } else {
            x[i * 4 + j] = __uint_as_float(ws[j]);
          }
        }
      }
      uint32_t packed[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t p = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // one rounded fp32 product, then the e4m3 rounding
          const float y = __fmul_rn(x[4 * i + j], inv);
          p |= f32_to_e4m3(y) << (8 * j);
        }
        packed[i] = p;
      }
      *reinterpret_cast<uint4*>(static_cast<char*>(which ? a.v_pool : a.k_pool) + dst_off) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
  }
}

// grid (num_pairs, 2 pools, splits): each workgroup copies a share of one block of one pool.
__global__ void __launch_bounds__(kThreads) copy_blocks_kernel(CopyBlocksArgs a) {
  const int pair = blockIdx.x;
  const int32_t src = a.pairs[2 * pair];
  const int32_t dst = a.pairs[2 * pair + 1];
  char* base = static_cast<char*>(blockIdx.y ? a.v_pool : a.k_pool);
  const uint4* s = reinterpret_cast<const uint4*>(base + static_cast<int64_t>(src) * a.block_bytes);
  uint4* d = reinterpret_cast<uint4*>(base + static_cast<int64_t>(dst) * a.block_bytes);
  const int64_t n16 = a.block_bytes / 16;
  for (int64_t i = static_cast<int64_t>(blockIdx.z) * kThreads + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.z) * kThreads)
    d[i] = s[i];
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
  const int64_t total = a.num_tokens * a.num_kv_heads * chunks;
  const dim3 grid(static_cast<unsigned>((total + kThreads - 1) / kThreads));
  const int lb = ilog2(a.block_size);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.pool_dtype == kF32)
    hipLaunchKernelGGL((cache_write_kernel<kF32, kF32>), grid, dim3(kThreads), 0, s, a, lb, chunks);
  else if (a.pool_dtype == kBF16)
    hipLaunchKernelGGL((cache_write_kernel<kBF16, kBF16>), grid, dim3(kThreads), 0, s, a, lb, chunks);
  else if (a.in_dtype == kBF16)
    hipLaunchKernelGGL((cache_write_kernel<kBF16, kFP8>), grid, dim3(kThreads), 0, s, a, lb, chunks);
  else
    hipLaunchKernelGGL((cache_write_kernel<kF32, kFP8>), grid, dim3(kThreads), 0, s, a, lb, chunks);
  return static_cast<int>(hipGetLastError());
}

int launch_copy_blocks(const CopyBlocksArgs& a, void* stream) {
  const int64_t n16 = a.block_bytes / 16;
  int splits = static_cast<int>((n16 + 4 * kThreads - 1) / (4 * kThreads));  // ~4 loads per thread
  if (splits < 1) splits = 1;
  if (splits > 64) splits = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, 2, splits), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_fp8_table(float* out, void* stream) {
  hipLaunchKernelGGL(fp8_table_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), out);
  return static_cast<int>(hipGetLastError());
}

}  // namespace pa
