// Merge of two attention results over disjoint key sets of the same query rows, and the attention of
// short private tails folded into such a merge.
//
// Beam branches share their prompt's blocks («GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU
// Memory 管理的艺术», §六 question 3).  A decode can then read the shared blocks once, for the
// queries of every branch (one pa_decode_ex call over the shared part, the branches' queries as the
// query heads of each KV head), read each private tail on its own, and combine the two results of
// every row with their log-sum-exps: the same rescaled combination as the merge of split pieces.
//  * merge_states_kernel: one thread per 4 dims of a row, an HBM-bound elementwise pass;
//  * tail_merge_kernel: the tail of at most KM (16 or 32) keys and the merge in one pass, one wave
//    per (sequence, KV head).  Lanes j, j + KM, ... dot key j's slices of the dims with the G query
//    heads (packed bf16 dots, fp32 sums); the softmax is a reduction over KM lanes; each lane then adds
//    two output dims over the keys, the probabilities read from their lanes as scalars, in fp32;
//    and the shared part's (output, log-sum-exp) is folded in before the row is written.  In records
//    mode (pa_decode_beam) the shared part is the partial records a records_only decode launch left
//    in its workspace: the wave walks its row's pieces as the decode's merge kernel would and folds
//    them in, so the shared part needs neither an output nor a merge launch.
#include <hip/hip_runtime.h>

#include <cmath>

#include "decode_records.h"
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

constexpr int kTailMax = 32;   // keys of the longest tail this kernel takes

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot_bf16x2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                         false);
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <int KV, int BS, int G, bool REC, int KM>
__global__ void __launch_bounds__(kThreads) tail_merge_kernel(TailMergeArgs a, int out_bf16) {
  constexpr int D = 128;
  constexpr int E = KV == kBF16 ? 2 : 1;
  constexpr int TILE = BS * D * E;                 // bytes of one (block, KV head) tile
  static_assert(KM == 16 || KM == 32, "tails of at most 16 or 32 keys");
  constexpr int LPK = 64 / KM;                     // lanes per key, each with DL of its dims
  constexpr int DL = D / LPK;
  constexpr int NB = (KM + BS - 1) / BS;           // blocks a tail can touch
  constexpr int NP = BS / 8;                       // 8-token pieces of a V^T row of one block
  constexpr int PW = 2 * E;                        // dwords of one piece (bf16 4, fp8 2)
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar reads below
  if (w >= static_cast<int64_t>(a.num_seqs) * a.num_kv_heads) return;
  const int seq = static_cast<int>(w / a.num_kv_heads);
  const int kvh = static_cast<int>(w % a.num_kv_heads);
  // the length and the row's first table entries are read together (the entries before the length
  // is known, inside the row); a length outside [0, max_tail] is clamped, and a block id outside
  // the pool is clamped into it
  // records mode: the plan of this row's shared segment (sequence seq / width, KV head kvh), read
  // first so that its loads are in flight beside the tail's (width and the stream count are powers
  // of two)
  int rec_nj = 0, rec_p0 = 0, rec_s = 1, rec_pu = 1, rec_grp = 0, rec_x = 0, rec_hh = 0;
  int p_lo = 0, p_hi = 0, p_all = 0;
  if constexpr (REC) {
    const DecodeArgs& r = a.shared;
    const int wl2 = __builtin_ctz(static_cast<unsigned>(a.width));
    const int sl2 = __builtin_ctz(static_cast<unsigned>(r.streams));
    rec_grp = seq >> wl2;
    rec_x = kvh & (r.streams - 1);
    rec_hh = kvh >> sl2;
    const ro_i32 pref = ro(r.ws_pref);
    p_lo = pref[rec_grp];
    p_hi = pref[rec_grp + 1];
    p_all = pref[r.num_seqs];
    rec_s = ro(r.ws_sched)[0];
    rec_pu = r.part_tokens / kDecodeUnit;
  }
  const int32_t* tab = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  const int len_raw = a.lens[seq];
  int32_t ent[NB];   // entries past the row's width read its last entry again and are set to 0
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const int32_t e = ro(tab)[min(q, a.max_blocks - 1)];
    ent[q] = q < a.max_blocks ? e : 0;
  }
  if constexpr (REC) {
    // the plan's loads complete with the table entries' (one wait before the K/V loads are issued),
    // instead of being sunk to their first use after those loads
    asm volatile("" ::"s"(p_lo), "s"(p_hi), "s"(p_all), "s"(rec_s), "s"(rec_pu));
    // a plan that the shared launch did not write (a broken call order) gives wrong rows, never a
    // walk outside the records: the counts are clamped to what any plan of these sizes can hold
    rec_s = max(rec_s, 1);
    rec_nj = min(max(p_hi - p_lo, 0), (a.shared.max_ctx + kDecodeUnit - 1) / kDecodeUnit);
    rec_p0 = max(rec_hh * p_all + p_lo, 0);
  }
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * TILE;
  const char* kbase = static_cast<const char*>(a.k_pool) + static_cast<int64_t>(kvh) * TILE;
  const char* vbase = static_cast<const char*>(a.v_pool) + static_cast<int64_t>(kvh) * TILE;
  const int64_t row0 = static_cast<int64_t>(seq) * a.num_q_heads + static_cast<int64_t>(kvh) * G;
  const int j = lane & (KM - 1), part = lane / KM;   // key j, dims DL part .. + DL

  // ---- every load first, so that the wave waits on memory once: q (for one head; a larger group
  // reads each head's q when it dots it, so as not to hold them all) and the prior state, which need
  // no table entry, then K and V ----
  auto q_row = [&](int g) __attribute__((always_inline)) {
    return static_cast<const char*>(a.q) + ((row0 + g) * D + part * DL) * 2;
  };
  uint4 q1[DL / 8];
  if constexpr (G == 1) {
#pragma unroll
    for (int c = 0; c < DL / 8; ++c) q1[c] = *reinterpret_cast<const uint4*>(q_row(0) + 16 * c);
  }
  float2 po[G];
  float lp[G];
  if constexpr (!REC) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      po[g] = *reinterpret_cast<const float2*>(a.o_prev + (row0 + g) * D + 2 * lane);
      lp[g] = a.lse_prev[row0 + g];
    }
  }
  const int L = __builtin_amdgcn_readfirstlane(min(max(len_raw, 0), a.max_tail));
  int64_t phys[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) phys[q] = q * BS < L ? min(max(ent[q], 0), a.num_blocks - 1) : 0;
  // K: key j's dims DL part .. + DL (lanes j, j + KM, ...); zeros past the tail
  uint32_t kraw[DL * E / 4];   // DL dims: DL / 2 dwords of bf16, DL / 4 of fp8
#pragma unroll
  for (int c = 0; c < DL * E / 4; ++c) kraw[c] = 0u;
  if (j < L) {
    const char* krow = kbase + phys[j / BS] * blk_stride + (j % BS) * (D * E) + part * DL * E;
#pragma unroll
    for (int c = 0; c < DL * E / 16; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(krow + 16 * c);
      kraw[4 * c] = v.x; kraw[4 * c + 1] = v.y; kraw[4 * c + 2] = v.z; kraw[4 * c + 3] = v.w;
    }
  }
  // V^T rows of dims 2 lane and 2 lane + 1, the 8-token pieces that hold tail keys
  uint32_t vraw[NB][NP][2][PW];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int c = 0; c < NP; ++c)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int k = 0; k < PW; ++k) vraw[q][c][r][k] = 0u;
        if (q * BS + 8 * c < L) {
          const char* src = vbase + phys[q] * blk_stride + static_cast<int64_t>(2 * lane + r) * BS * E + 8 * E * c;
          if constexpr (E == 2) {
            const uint4 u = *reinterpret_cast<const uint4*>(src);
            vraw[q][c][r][0] = u.x; vraw[q][c][r][1] = u.y; vraw[q][c][r][2] = u.z; vraw[q][c][r][3] = u.w;
          } else {
            const uint2 u = *reinterpret_cast<const uint2*>(src);
            vraw[q][c][r][0] = u.x; vraw[q][c][r][1] = u.y;
          }
        }
      }

  // ---- records mode: fold the shared part's pieces of this row (usually one or two) into a base-2
  // maximum ms, a sum ls and unnormalised dims os, a few pieces' loads in flight at a time ----
  float ms = -INFINITY, ls = 0.f;
  float2 os = make_float2(0.f, 0.f);
  if constexpr (REC) {
    static_assert(G == 1, "records mode serves one query head per KV head");
    const DecodeArgs& r = a.shared;
    if (rec_nj > 0) {
      constexpr int kRec = D + 4;
      constexpr int kB = 4;
      const int gs = seq & (a.width - 1);
      const int64_t rec_slots = static_cast<int64_t>(r.streams) * r.stream_slots;   // slots the records hold
      PieceWalk walk;
      walk.init(segment_slot(r, rec_x, rec_hh, rec_grp), rec_p0, rec_nj, rec_pu, rec_s);
      while (!walk.done()) {
        // up to kB pieces; the loads of every slot are issued unconditionally (slots past cnt read
        // piece 0 again and are then ignored), so no load waits on a branch
        int64_t off[kB];
        int cnt = 0;
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          if (b == 0 || !walk.done()) {
            off[b] = (min(max(walk.next(), int64_t(0)), rec_slots - 1) * a.width + gs) * kRec;
            cnt = b + 1;
          } else {
            off[b] = off[0];
          }
        }
        float mj[kB], lj[kB];
        float2 oj[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const float2 ml = *reinterpret_cast<const float2*>(r.ws_part + off[b]);   // (max, sum)
          oj[b] = *reinterpret_cast<const float2*>(r.ws_part + off[b] + 4 + 2 * lane);
          mj[b] = b < cnt ? ml.x : -INFINITY;
          lj[b] = ml.y;
        }
        float mn = ms;
#pragma unroll
        for (int b = 0; b < kB; ++b) mn = fmaxf(mn, mj[b]);
        const float alpha = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mn);
        ls *= alpha;
        os.x *= alpha;
        os.y *= alpha;
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const float wb = b < cnt && mj[b] != -INFINITY ? __builtin_amdgcn_exp2f(mj[b] - mn) : 0.f;
          ls += lj[b] * wb;
          os.x += oj[b].x * wb;
          os.y += oj[b].y * wb;
        }
        ms = mn;
      }
    }
  }

  // ---- base-2 logits of key j for each head (-inf past the tail) ----
  uint32_t kw[DL / 2];   // bf16 pairs of the DL dims
  if constexpr (E == 2) {
#pragma unroll
    for (int c = 0; c < DL / 2; ++c) kw[c] = kraw[c];
  } else {
#pragma unroll
    for (int c = 0; c < DL / 4; ++c) {
      kw[2 * c] = fp8x2_bf16<false>(kraw[c]);
      kw[2 * c + 1] = fp8x2_bf16<true>(kraw[c]);
    }
  }
  float x[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < DL / 8; ++c) {
      const uint4 qv = G == 1 ? q1[c] : *reinterpret_cast<const uint4*>(q_row(g) + 16 * c);
      acc = dot_bf16x2(kw[4 * c], qv.x, acc);
      acc = dot_bf16x2(kw[4 * c + 1], qv.y, acc);
      acc = dot_bf16x2(kw[4 * c + 2], qv.z, acc);
      acc = dot_bf16x2(kw[4 * c + 3], qv.w, acc);
    }
#pragma unroll
    for (int off = KM; off < 64; off <<= 1) acc += shfl_xor(acc, off);   // the key's other dims
    x[g] = j < L ? acc * a.qk_scale : -INFINITY;
  }
  // ---- softmax statistics over the KM keys (every lane of a key holds the same values) ----
  float p[G], m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = x[g];
#pragma unroll
    for (int off = KM / 2; off > 0; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
    m[g] = mx;
    p[g] = L > 0 ? __builtin_amdgcn_exp2f(x[g] - mx) : 0.f;   // 0 past the tail
    float sm = p[g];
#pragma unroll
    for (int off = KM / 2; off > 0; off >>= 1) sm += shfl_xor(sm, off);
    l[g] = sm;
  }
  // ---- sum over the keys of p v, dims 2 lane and 2 lane + 1; values past the tail (any bits) are
  // skipped, never multiplied ----
  float o[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) o[g][0] = o[g][1] = 0.f;
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      const int t0 = q * BS + 8 * c;
      if (t0 >= L) continue;   // wave-uniform
      float v0[8], v1[8];
#pragma unroll
      for (int k = 0; k < PW; ++k) {
        if constexpr (E == 2) {
          v0[2 * k] = bf16_lo(vraw[q][c][0][k]); v0[2 * k + 1] = bf16_hi(vraw[q][c][0][k]);
          v1[2 * k] = bf16_lo(vraw[q][c][1][k]); v1[2 * k + 1] = bf16_hi(vraw[q][c][1][k]);
        } else {
          fp8x2_to_f32<false>(vraw[q][c][0][k], v0[4 * k], v0[4 * k + 1]);
          fp8x2_to_f32<true>(vraw[q][c][0][k], v0[4 * k + 2], v0[4 * k + 3]);
          fp8x2_to_f32<false>(vraw[q][c][1][k], v1[4 * k], v1[4 * k + 1]);
          fp8x2_to_f32<true>(vraw[q][c][1][k], v1[4 * k + 2], v1[4 * k + 3]);
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t0 + t >= L) continue;   // wave-uniform
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[g]), t0 + t));
          o[g][0] += pj * v0[t];
          o[g][1] += pj * v1[t];
        }
      }
    }
  // ---- fold in the prior (output, natural log-sum-exp; or, in records mode, its maximum, sum and
  // unnormalised dims) and write the row ----
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t r = row0 + g;
    float r0v = 0.f, r1v = 0.f;
    if constexpr (REC) {
      const float M = fmaxf(ms, L > 0 ? m[g] : -INFINITY);
      if (M != -INFINITY) {
        const float wp = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);   // weight of os, ls
        const float wt = L > 0 ? __builtin_amdgcn_exp2f(m[g] - M) : 0.f;           // weight of o, l
        const float den = ls * wp + l[g] * wt;
        const float inv = den > 0.f ? a.v_scale / den : 0.f;
        r0v = (os.x * wp + o[g][0] * wt) * inv;
        r1v = (os.y * wp + o[g][1] * wt) * inv;
      }
    } else {
      const float lpb = lp[g] * kLog2e;                           // base 2
      const float lt = L > 0 ? m[g] + __log2f(l[g]) : -INFINITY;
      const float M = fmaxf(lpb, lt);
      if (M != -INFINITY) {
        const float wp = __builtin_amdgcn_exp2f(lpb - M);         // 0 when the prior is empty
        const float wt = L > 0 ? __builtin_amdgcn_exp2f(m[g] - M) : 0.f;   // weight of the sums o
        const float inv = 1.f / (wp + wt * l[g]);
        r0v = (po[g].x * wp + o[g][0] * wt * a.v_scale) * inv;
        r1v = (po[g].y * wp + o[g][1] * wt * a.v_scale) * inv;
      }
    }
    if (out_bf16) {
      static_cast<uint32_t*>(a.out)[r * (D / 2) + lane] = f32_to_bf16_bits(r0v) | (f32_to_bf16_bits(r1v) << 16);
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + r * D + 2 * lane) = make_float2(r0v, r1v);
    }
  }
}

template <int KV, int BS, int KM>
int launch_tail_g(const TailMergeArgs& a, int ob, hipStream_t s, unsigned blocks) {
  if (a.width > 0) {
    if (a.num_q_heads != a.num_kv_heads) return -1;
    hipLaunchKernelGGL((tail_merge_kernel<KV, BS, 1, true, KM>), dim3(blocks), dim3(kThreads), 0, s, a, ob);
    return static_cast<int>(hipGetLastError());
  }
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: hipLaunchKernelGGL((tail_merge_kernel<KV, BS, 1, false, KM>), dim3(blocks), dim3(kThreads), 0, s, a, ob); break;
    case 2: hipLaunchKernelGGL((tail_merge_kernel<KV, BS, 2, false, KM>), dim3(blocks), dim3(kThreads), 0, s, a, ob); break;
    case 4: hipLaunchKernelGGL((tail_merge_kernel<KV, BS, 4, false, KM>), dim3(blocks), dim3(kThreads), 0, s, a, ob); break;
    case 8: hipLaunchKernelGGL((tail_merge_kernel<KV, BS, 8, false, KM>), dim3(blocks), dim3(kThreads), 0, s, a, ob); break;
    default: return -1;
  }
  return static_cast<int>(hipGetLastError());
}

// Tails of at most 16 keys take the 16-key form: four lanes per key, each with 32 of its dims, and
// one 16-key V block at most, so the wave holds half the K, q and V registers of the 32-key form.
template <int KV, int BS>
int launch_tail_k(const TailMergeArgs& a, int ob, hipStream_t s, unsigned blocks) {
  return a.max_tail <= 16 ? launch_tail_g<KV, BS, 16>(a, ob, s, blocks) : launch_tail_g<KV, BS, 32>(a, ob, s, blocks);
}

template <int KV>
int launch_tail_bs(const TailMergeArgs& a, int block_size, int ob, hipStream_t s, unsigned blocks) {
  switch (block_size) {
    case 8: return launch_tail_k<KV, 8>(a, ob, s, blocks);
    case 16: return launch_tail_k<KV, 16>(a, ob, s, blocks);
    case 32: return launch_tail_k<KV, 32>(a, ob, s, blocks);
    default: return -1;
  }
}

}  // namespace

int launch_tail_merge(const TailMergeArgs& a, int kv_dtype, int block_size, int head_dim, int out_dtype,
                      void* stream) {
  if (head_dim != 128 || a.max_tail > kTailMax) return -1;
  const int64_t waves = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  if (waves == 0) return 0;
  const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7fffffff) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int ob = out_dtype == kBF16 ? 1 : 0;
  if (kv_dtype == kBF16) return launch_tail_bs<kBF16>(a, block_size, ob, s, static_cast<unsigned>(blocks));
  if (kv_dtype == kFP8) return launch_tail_bs<kFP8>(a, block_size, ob, s, static_cast<unsigned>(blocks));
  return -1;
}

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
