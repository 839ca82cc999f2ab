// Merge of two attention results over disjoint key sets of the same query rows.
//
// Beam branches share their prompt's blocks («GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU
// Memory 管理的艺术», §六 question 3).  A decode can then read the shared blocks once, for the
// queries of every branch (one pa_decode_ex call over the shared part, the branches' queries as the
// query heads of each KV head), read each private tail on its own, and combine the two results of
// every row with their log-sum-exps: the same rescaled combination as the merge of split pieces.
// One thread per 4 dims of a row: an HBM-bound elementwise pass.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) merge_states_kernel(MergeStatesArgs a, int out_bf16) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int q4 = a.head_dim / 4;
  if (idx >= a.rows * q4) return;
  const int64_t r = idx / q4;
  const int d = static_cast<int>(idx % q4) * 4;
  const float la = a.lse_a[r], lb = a.lse_b[r];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f;
  if (m != -INFINITY) {
    wa = __expf(la - m);
    wb = __expf(lb - m);
  }
  const float sum = wa + wb;
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  const float4 x = *reinterpret_cast<const float4*>(a.o_a + r * a.head_dim + d);
  const float4 y = *reinterpret_cast<const float4*>(a.o_b + r * a.head_dim + d);
  const float o0 = (x.x * wa + y.x * wb) * inv, o1 = (x.y * wa + y.y * wb) * inv;
  const float o2 = (x.z * wa + y.z * wb) * inv, o3 = (x.w * wa + y.w * wb) * inv;
  if (out_bf16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + r * a.head_dim + d) =
        make_uint2(f32_to_bf16_bits(o0) | (f32_to_bf16_bits(o1) << 16), f32_to_bf16_bits(o2) | (f32_to_bf16_bits(o3) << 16));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + r * a.head_dim + d) = make_float4(o0, o1, o2, o3);
  }
  if (a.lse_out && d == 0) a.lse_out[r] = m == -INFINITY ? -INFINITY : m + __logf(sum);
}

}  // namespace

int launch_merge_states(const MergeStatesArgs& a, int out_dtype, void* stream) {
  const int64_t total = a.rows * (a.head_dim / 4);
  if (total == 0) return 0;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL(merge_states_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a, out_dtype == kBF16 ? 1 : 0);
  return static_cast<int>(hipGetLastError());
}

}  // namespace pa
