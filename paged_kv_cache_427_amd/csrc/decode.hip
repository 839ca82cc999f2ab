// Paged decode attention for gfx950: one query token per sequence over its block-table-mapped K/V.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» §三 3.1-3.2: the kernel gets
// the sequence's scattered K/V through its block table -- one indirection per block, contiguous
// coalesced reads inside it -- and dots the query with every cached key; §七 notes the indirection
// costs a little.  softmax(scale * q K^T) V is the textbook form of what the pages describe in words.
//
// Design (HBM-bound: at most 8 flop per byte of K/V, far below the MI355X ridge):
//  * grid (partition, kv_head, sequence); a workgroup of 4 wave64s owns one context partition of
//    one KV head and serves all G query heads of that group, so each K/V byte is read once.
//  * waves take the partition's blocks round-robin; the table entry is a wave-uniform scalar load.
//  * each block tile (block_size rows x head_dim) is read with 16-byte loads in which every group
//    of NL lanes covers 16*NL contiguous bytes of one token row (whole 128-byte lines), so a wave
//    instruction touches 64/NL whole rows; the next block's K/V is loaded before the current one
//    is consumed.
//  * logits are reduced over the NL lanes of a row with DPP; every lane keeps its own running max,
//    exp-sum and output partial (base-2 online softmax) for the tokens it saw, so the inner loop has
//    no cross-row traffic; lanes, then waves (through LDS), are merged once per partition.
//  * a sequence with several partitions writes (max, sum, normalised partial) per partition and a
//    second kernel merges them; a single-partition sequence writes its output directly.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int KV>
struct KvChunk;

template <>
struct KvChunk<kF32> {
  static constexpr int kElem = 4, kN = 4;
  __device__ static void cvt(const uint4& c, float* f) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  }
};

template <>
struct KvChunk<kBF16> {
  static constexpr int kElem = 2, kN = 8;
  __device__ static void cvt(const uint4& c, float* f) {
    f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x);
    f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
    f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z);
    f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
  }
};

template <>
struct KvChunk<kFP8> {
  static constexpr int kElem = 1, kN = 16;
  __device__ static void cvt(const uint4& c, float* f) {
    fp8x2_to_f32<false>(c.x, f[0], f[1]);  fp8x2_to_f32<true>(c.x, f[2], f[3]);
    fp8x2_to_f32<false>(c.y, f[4], f[5]);  fp8x2_to_f32<true>(c.y, f[6], f[7]);
    fp8x2_to_f32<false>(c.z, f[8], f[9]);  fp8x2_to_f32<true>(c.z, f[10], f[11]);
    fp8x2_to_f32<false>(c.w, f[12], f[13]); fp8x2_to_f32<true>(c.w, f[14], f[15]);
  }
};

template <typename T>
__device__ __forceinline__ float load_act(const T* p);
template <>
__device__ __forceinline__ float load_act<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

__device__ __forceinline__ void store_out(void* out, int64_t i, float x, bool bf16) {
  if (bf16)
    static_cast<uint16_t*>(out)[i] = static_cast<uint16_t>(f32_to_bf16_bits(x));
  else
    static_cast<float*>(out)[i] = x;
}

// Lane geometry of one (block, KV head) tile.
template <int KV, int D, int BS>
struct Geo {
  static constexpr int kE = KvChunk<KV>::kElem;
  static constexpr int kRow = D * kE;                 // bytes of one token row
  static constexpr int kC = kRow / 16;                // 16-byte chunks per row
  static constexpr int kNL = kC < 8 ? kC : 8;         // lanes sharing one row in a load
  static constexpr int kTPI = 64 / kNL;               // rows per wave load
  static constexpr int kTG = BS / kTPI;               // row groups per block
  static constexpr int kCPL = kC / kNL;               // chunks per lane per row
  static constexpr int kEPC = KvChunk<KV>::kN;        // elements per chunk
  static constexpr int kDL = kCPL * kEPC;             // dims per lane
  static constexpr bool kOk = (BS % kTPI == 0) && kTG >= 1 && (kC % kNL == 0);
};

template <int KV, int D, int BS, int G, typename QT>
__global__ void __launch_bounds__(kThreads) decode_part_kernel(DecodeArgs a, int out_bf16) {
  using Gm = Geo<KV, D, BS>;
  constexpr int NL = Gm::kNL, TPI = Gm::kTPI, TG = Gm::kTG, CPL = Gm::kCPL, EPC = Gm::kEPC,
                DL = Gm::kDL, ROW = Gm::kRow;
  constexpr int TILE = BS * ROW;                      // bytes of one (block, head) tile

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  // a length outside [0, max_ctx] is clamped so that table, workspace and output stay in bounds
  const int L = min(max(a.lens[seq], 0), a.max_ctx);
  const int n_parts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
  if (part >= n_parts) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tokset = lane / NL;
  const int cl = lane % NL;
  const int t0 = part * a.part_tokens;
  const int t1 = min(L, t0 + a.part_tokens);
  const int blk0 = t0 / BS;
  const int blk1 = (t1 + BS - 1) / BS;

  // query slice of this lane, pre-multiplied by scale * k_scale * log2(e)
  float qv[G][DL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const QT* qp = static_cast<const QT*>(a.q) +
                   (static_cast<int64_t>(seq) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int cr = 0; cr < CPL; ++cr)
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        qv[g][cr * EPC + e] = load_act<QT>(qp + (cr * NL + cl) * EPC + e) * a.qk_scale;
  }

  float m[G], l[G], acc[G][DL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[g][i] = 0.f;
  }

  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int32_t* tab = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  const int64_t head_off = static_cast<int64_t>(kvh) * TILE;
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * TILE;
  int lane_off[TG][CPL];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int cr = 0; cr < CPL; ++cr) lane_off[tg][cr] = (tg * TPI + tokset) * ROW + (cr * NL + cl) * 16;

  uint4 kc[TG][CPL], vc[TG][CPL];
  int b = blk0 + wave;
  if (b < blk1) {
    const int64_t base = tab[b] * blk_stride + head_off;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr) {
        kc[tg][cr] = *reinterpret_cast<const uint4*>(kbase + base + lane_off[tg][cr]);
        vc[tg][cr] = *reinterpret_cast<const uint4*>(vbase + base + lane_off[tg][cr]);
      }
  }
  for (; b < blk1; b += kWaves) {
    // issue the next block's loads before consuming this one
    uint4 kn[TG][CPL], vn[TG][CPL];
    const int bn = b + kWaves;
    if (bn < blk1) {
      const int64_t base = tab[bn] * blk_stride + head_off;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int cr = 0; cr < CPL; ++cr) {
          kn[tg][cr] = *reinterpret_cast<const uint4*>(kbase + base + lane_off[tg][cr]);
          vn[tg][cr] = *reinterpret_cast<const uint4*>(vbase + base + lane_off[tg][cr]);
        }
    }
    bool valid[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) valid[tg] = b * BS + tg * TPI + tokset < t1;

    float s[G][TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
      for (int g = 0; g < G; ++g) s[g][tg] = 0.f;
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr) {
        float kf[EPC];
        KvChunk<KV>::cvt(kc[tg][cr], kf);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPC; ++e) s[g][tg] = fmaf(qv[g][cr * EPC + e], kf[e], s[g][tg]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s[g][tg] = group_sum<NL>(s[g][tg]);
        s[g][tg] = valid[tg] ? s[g][tg] : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = s[g][0];
#pragma unroll
      for (int tg = 1; tg < TG; ++tg) mx = fmaxf(mx, s[g][tg]);
      const float mn = fmaxf(m[g], mx);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(m[g] - ms);
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[g][i] *= alpha;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) s[g][tg] = exp2f(s[g][tg] - ms);  // 0 for invalid rows
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
      for (int g = 0; g < G; ++g) l[g] += s[g][tg];
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr) {
        float vf[EPC];
        KvChunk<KV>::cvt(vc[tg][cr], vf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) vf[e] = valid[tg] ? vf[e] : 0.f;  // rows past the end hold poison
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[g][cr * EPC + e] = fmaf(s[g][tg], vf[e], acc[g][cr * EPC + e]);
      }
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr) {
        kc[tg][cr] = kn[tg][cr];
        vc[tg][cr] = vn[tg][cr];
      }
  }

  // merge the lanes of different row sets (same dims) inside the wave
#pragma unroll
  for (int mask = NL; mask < 64; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = shfl_xor(m[g], mask);
      const float lo = shfl_xor(l[g], mask);
      const float mn = fmaxf(m[g], mo);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float a1 = exp2f(m[g] - ms);
      const float a2 = exp2f(mo - ms);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[g][i] = acc[g][i] * a1 + shfl_xor(acc[g][i], mask) * a2;
      m[g] = mn;
    }
  }

  // merge the waves through LDS
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[wave][g] = m[g];
      sm_l[wave][g] = l[g];
    }
  }
  if (tokset == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr)
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm_o[wave][g][(cr * NL + cl) * EPC + e] = acc[g][cr * EPC + e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx % D;
    float mm = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][g]);
    const float ms = mm == -INFINITY ? 0.f : mm;
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(sm_m[w][g] - ms);
      lsum += sm_l[w][g] * f;
      o += sm_o[w][g][d] * f;
    }
    const float res = lsum > 0.f ? o / lsum * a.v_scale : 0.f;
    const int h = kvh * G + g;
    const int64_t sh = static_cast<int64_t>(seq) * a.num_q_heads + h;
    if (n_parts == 1) {
      store_out(a.out, sh * D + d, res, out_bf16 != 0);
    } else {
      const int64_t pi = sh * a.max_parts + part;
      a.ws_o[pi * D + d] = res;
      if (d == 0) {
        a.ws_m[pi] = mm;
        a.ws_l[pi] = lsum;
      }
    }
  }
}

// Merge of partitions: out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max m).
template <int D>
__global__ void __launch_bounds__(D) decode_reduce_kernel(DecodeArgs a, int out_bf16) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int L = min(max(a.lens[seq], 0), a.max_ctx);
  const int n_parts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
  if (n_parts <= 1) return;
  const int d = threadIdx.x;
  const int64_t sh = static_cast<int64_t>(seq) * a.num_q_heads + h;
  const float* mp = a.ws_m + sh * a.max_parts;
  const float* lp = a.ws_l + sh * a.max_parts;
  const float* op = a.ws_o + sh * a.max_parts * D;
  float mm = -INFINITY;
  for (int p = 0; p < n_parts; ++p) mm = fmaxf(mm, mp[p]);
  const float ms = mm == -INFINITY ? 0.f : mm;
  float wsum = 0.f, o = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float w = lp[p] * exp2f(mp[p] - ms);
    wsum += w;
    o += w * op[static_cast<int64_t>(p) * D + d];
  }
  store_out(a.out, sh * D + d, wsum > 0.f ? o / wsum : 0.f, out_bf16 != 0);
}

template <int KV, int D, int BS, int G, typename QT>
int launch_one(const DecodeArgs& a, int out_bf16, hipStream_t s) {
  if constexpr (!Geo<KV, D, BS>::kOk) {
    return -1;
  } else {
    const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_part_kernel<KV, D, BS, G, QT>), grid, dim3(kThreads), 0, s, a, out_bf16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
    if (a.max_parts > 1) {
      hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(a.num_q_heads, a.num_seqs), dim3(D), 0, s, a,
                         out_bf16);
      e = hipGetLastError();
    }
    return static_cast<int>(e);
  }
}

template <int KV, int D, int BS, typename QT>
int pick_group(const DecodeArgs& a, int out_bf16, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_one<KV, D, BS, 1, QT>(a, out_bf16, s);
    case 2: return launch_one<KV, D, BS, 2, QT>(a, out_bf16, s);
    case 4: return launch_one<KV, D, BS, 4, QT>(a, out_bf16, s);
    case 8: return launch_one<KV, D, BS, 8, QT>(a, out_bf16, s);
    default: return -1;
  }
}

template <int KV, int D, typename QT>
int pick_block(const DecodeArgs& a, int bs, int out_bf16, hipStream_t s) {
  switch (bs) {
    case 8: return pick_group<KV, D, 8, QT>(a, out_bf16, s);
    case 16: return pick_group<KV, D, 16, QT>(a, out_bf16, s);
    case 32: return pick_group<KV, D, 32, QT>(a, out_bf16, s);
    default: return -1;
  }
}

template <int KV, typename QT>
int pick_dim(const DecodeArgs& a, int bs, int d, int out_bf16, hipStream_t s) {
  switch (d) {
    case 64: return pick_block<KV, 64, QT>(a, bs, out_bf16, s);
    case 128: return pick_block<KV, 128, QT>(a, bs, out_bf16, s);
    default: return -1;
  }
}

}  // namespace

int launch_decode(const DecodeArgs& a, int kv_dtype, int q_dtype, int out_dtype, int block_size,
                  int head_dim, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ob = out_dtype == kBF16;
  if (kv_dtype == kF32 && q_dtype == kF32) return pick_dim<kF32, float>(a, block_size, head_dim, ob, s);
  if (kv_dtype == kBF16 && q_dtype == kBF16) return pick_dim<kBF16, uint16_t>(a, block_size, head_dim, ob, s);
  if (kv_dtype == kFP8 && q_dtype == kBF16) return pick_dim<kFP8, uint16_t>(a, block_size, head_dim, ob, s);
  return -1;
}

}  // namespace pa
