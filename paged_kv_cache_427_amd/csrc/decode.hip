// Paged decode attention for gfx950: one query token per sequence over its block-table-mapped K/V.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» §三 3.1-3.2: the kernel gets
// the sequence's scattered K/V through its block table -- one indirection per block, contiguous
// coalesced reads inside it -- and dots the query with every cached key; §七 notes the indirection
// costs a little.  softmax(scale * q K^T) V is the textbook form of what the pages describe in words.
//
// Design (HBM-bound: at most 8 flop per byte of K/V, far below the MI355X ridge, so the goal is to
// keep the vector ALUs out of the way of the loads):
//  * a work item is one context partition of one KV head, for all G query heads of that group, so
//    each K/V byte is read once; a persistent grid of workgroups (4 wave64s each, as many as are
//    resident at once) loops over the items.  Items are numbered so that all work of one KV head
//    lands on one XCD (initial dispatch is round-robin over the 8 XCDs): blocks shared by many
//    sequences (a common prefix) are then re-read from that XCD's L2, not from HBM.
//  * a wave takes 16-key units of the partition round-robin; the unit's table entry is a
//    wave-uniform scalar load.  Both products of a unit run on 16x16 MFMA tiles fed straight from
//    the loads, with no LDS staging:
//      S^T[key][head] = K[key][:] . Q[head][:]     A = K rows (token-major tile), B = Q^T
//      O^T[dim][head] += V^T[dim][key] P^T[key][head]   A = V^T rows (dim-major tile), B = P^T
//    The G query heads occupy columns 0..G-1 of the 16 (the rest are zero).  The S^T accumulator
//    layout -- lane l holds keys 4*(l/16)+r of the unit for head l%16 -- is, after rounding to bf16,
//    exactly the B operand of the 16x16x16 P.V product, so the scores never cross lanes.
//  * bf16 pools use v_mfma_f32_16x16x32_bf16 (S) and v_mfma_f32_16x16x16_bf16 (P.V); fp8 codes
//    widen exactly to bf16 first (v_cvt_scalef32_pk_bf16_fp8, scales kept in fp32); fp32 pools use
//    v_mfma_f32_16x16x4_f32.  The
//    probabilities are rounded to bf16 for the bf16/fp8 products and the running sum uses the same
//    rounded values; the fp32 path keeps fp32 probabilities.
//  * base-2 online softmax with one running max per head.  The max is raised only when a logit
//    exceeds it by more than 2^8 (so every exp stays <= 256); that test is one wave-wide ballot, and
//    only then are the lanes' maxima exchanged and the accumulators rescaled.  Each lane keeps a
//    partial exp-sum of its own keys; lanes, then waves (through LDS), merge once per partition.
//  * a ring of register stages keeps the next units' K/V in flight while one is consumed (2 for
//    bf16, 4 for fp8), within a register budget that leaves 3 workgroups per CU.
//  * a sequence with several partitions writes (max, sum, normalised partial) per partition and a
//    second kernel merges them; a single-partition sequence writes its output directly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = 32;          // keys per unit of one wave (two 16x16 S^T tiles)
constexpr float kSlack = 8.0f;     // log2 of the growth allowed before the accumulators are rescaled

template <int KV>
struct Elem {
  static constexpr int kBytes = KV == kF32 ? 4 : KV == kBF16 ? 2 : 1;
};

// Workgroups per CU that the register budget of a kernel allows.
template <int KV, int D>
struct Pipe {
  static constexpr int kOcc = KV == kF32 ? 2 : 3;
};

// 16x16 MFMA tiles: 32-deep bf16 products (S^T over 32 dims; P.V over 32 keys) or 4-deep fp32 ones.
__device__ __forceinline__ f32x4 mma_s(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_s(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Codes in bytes 0,1 (HI = false) or 2,3 (HI = true) of w -> two bf16 in one dword (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

__device__ __forceinline__ void store_out(void* out, int64_t i, float x, bool bf16) {
  if (bf16)
    static_cast<uint16_t*>(out)[i] = static_cast<uint16_t>(f32_to_bf16_bits(x));
  else
    static_cast<float*>(out)[i] = x;
}

// Raw registers of one 32-key unit, as loaded by one lane (i = lane % 16, kg = lane / 16).
//  k[t][c]: key 16t + i of the unit, 16 bytes at byte 64c + 16kg of its row
//           (bf16: dims 32c+8kg..+8; fp8: dims 64c+16kg..+16; fp32: dims 16c+4kg..+4)
//  v[d][p]: dim 16d + i, keys 16p + 4kg .. +4 of the unit (VW dwords)
template <int KV, int D>
struct UnitRegs {
  static constexpr int E = Elem<KV>::kBytes;
  static constexpr int KL = D * E / 64;   // 16-byte K loads per 16-key tile
  static constexpr int VW = E;            // dwords per 4-key V piece
  uint4 k[2][KL];
  uint32_t v[D / 16][2][VW];
};

template <int VW>
__device__ __forceinline__ void load_piece(uint32_t (&dst)[VW], const char* p) {
  if constexpr (VW == 1) {
    dst[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (VW == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    dst[0] = w.x; dst[1] = w.y;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
  }
}

// One (sequence, KV head) segment as the loads see it.
struct SeqView {
  const char* kbase;       // K pool + this KV head's tile offset
  const char* vbase;
  const int32_t* tab;      // this sequence's block table
  int64_t blk_stride;      // bytes of one block of one pool (all KV heads)
  int nblk;                // valid table entries: ceil(L / BS)
};

// Physical blocks of the unit starting at key U (32 keys: 4, 2 or 1 blocks of 8, 16 or 32 tokens).
// A block past the sequence's last one (only in a unit that ends the sequence) is replaced by the
// last one; its keys are masked afterwards.
template <int BS>
struct UnitBlocks {
  static constexpr int N = kUnit / BS;
  int64_t b[N];
};

template <int BS>
__device__ __forceinline__ UnitBlocks<BS> unit_blocks(const SeqView& sv, int U) {
  const int j0 = U / BS;
  UnitBlocks<BS> ub;
#pragma unroll
  for (int q = 0; q < UnitBlocks<BS>::N; ++q) ub.b[q] = sv.tab[min(j0 + q, sv.nblk - 1)];
  return ub;
}

// Issues the loads of the unit starting at key U (a multiple of 32) from its blocks `ub`.
template <int KV, int D, int BS>
__device__ __forceinline__ void load_unit(UnitRegs<KV, D>& R, const SeqView& sv, const UnitBlocks<BS>& ub, int i,
                                          int kg) {
  using R_t = UnitRegs<KV, D>;
  constexpr int E = R_t::E, KL = R_t::KL, VW = R_t::VW;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const char* krow;                                   // key 16t + i of the unit
    if constexpr (BS == 8) {
      krow = sv.kbase + ((i >> 3) ? ub.b[2 * t + 1] : ub.b[2 * t]) * sv.blk_stride + (i & 7) * (D * E);
    } else if constexpr (BS == 16) {
      krow = sv.kbase + ub.b[t] * sv.blk_stride + i * (D * E);
    } else {
      krow = sv.kbase + ub.b[0] * sv.blk_stride + (16 * t + i) * (D * E);
    }
#pragma unroll
    for (int c = 0; c < KL; ++c) R.k[t][c] = *reinterpret_cast<const uint4*>(krow + 64 * c + 16 * kg);
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const char* vrow;                                   // keys 16p + 4kg .. +4 of the unit
    if constexpr (BS == 8) {
      vrow = sv.vbase + ((kg >> 1) ? ub.b[2 * p + 1] : ub.b[2 * p]) * sv.blk_stride + (4 * (kg & 1)) * E;
    } else if constexpr (BS == 16) {
      vrow = sv.vbase + ub.b[p] * sv.blk_stride + (4 * kg) * E;
    } else {
      vrow = sv.vbase + ub.b[0] * sv.blk_stride + (16 * p + 4 * kg) * E;
    }
#pragma unroll
    for (int d = 0; d < D / 16; ++d) load_piece<VW>(R.v[d][p], vrow + (16 * d + i) * BS * E);
  }
}

template <int KV, int D, int G>
struct DecodeState {
  static constexpr int NQB = KV == kF32 ? D / 4 : D / 32;   // MFMAs per 16-key S^T tile
  typedef typename std::conditional<KV == kF32, float, bf16x8>::type QOp;
  QOp qb[NQB];         // Q^T operand of each S^T MFMA (zero for columns >= G)
  f32x4 o[D / 16];     // O^T: lane holds dims 16t + 4kg + r for head lane % 16
  float m;             // running max (base-2 logits) of head lane % 16; equal across the 4 lane groups
  float l;             // this lane's partial exp-sum

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  __device__ __forceinline__ void consume(UnitRegs<KV, D>& R, int U, int t1, int kg, int col,
                                          float qk_scale) {
    using R_t = UnitRegs<KV, D>;
    constexpr int KL = R_t::KL;
    // ---- S^T of the unit's two 16-key tiles: lane holds keys 16t + 4kg + r for head col ----
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KL; ++c) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 w = R.k[t][c];
        if constexpr (KV == kBF16) {
          s[t] = mma_s(__builtin_bit_cast(bf16x8, w), qb[c], s[t]);
        } else if constexpr (KV == kFP8) {
          s[t] = mma_s(as_bf16x8(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                                 fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y)),
                       qb[2 * c], s[t]);
          s[t] = mma_s(as_bf16x8(fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z),
                                 fp8x2_to_bf16x2<false>(w.w), fp8x2_to_bf16x2<true>(w.w)),
                       qb[2 * c + 1], s[t]);
        } else {
          s[t] = mma_s(__uint_as_float(w.x), qb[4 * c + 0], s[t]);
          s[t] = mma_s(__uint_as_float(w.y), qb[4 * c + 1], s[t]);
          s[t] = mma_s(__uint_as_float(w.z), qb[4 * c + 2], s[t]);
          s[t] = mma_s(__uint_as_float(w.w), qb[4 * c + 3], s[t]);
        }
      }
    }
    // ---- base-2 logits; keys at or past the context end are masked (last unit only) ----
    float x[8];   // x[4t + r]: key 16t + 4kg + r of the unit
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * t + r] = s[t][r] * qk_scale;
    if (U + kUnit > t1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (U + 16 * t + 4 * kg + r >= t1) x[4 * t + r] = -INFINITY;
      // masked keys may hold any bits (even NaN): zero their values so that 0 * v stays 0
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (U + 16 * p + 4 * kg + e < t1) continue;
#pragma unroll
          for (int d = 0; d < D / 16; ++d) {
            if constexpr (KV == kF32) {
              R.v[d][p][e] = 0u;
            } else if constexpr (KV == kBF16) {
              R.v[d][p][e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            } else {
              R.v[d][p][0] &= ~(0xffu << (8 * e));
            }
          }
        }
    }
    // ---- running max: raised only when a logit exceeds it by more than the slack ----
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    const bool grow = col < G && mx > m + kSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));                  // max over the head's 32 keys
      const float mn = mx > m + kSlack ? mx : m;
      const float alpha = mn == m ? 1.f : __builtin_amdgcn_exp2f(m - mn);   // 0 when m was -inf
      m = mn;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D / 16; ++d) o[d] *= alpha;
    }
    const float ms = m == -INFINITY ? 0.f : m;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(x[e] - ms);   // 0 for masked keys
    // ---- O^T += V^T P^T: k-slot e of lane group kg is key 16(e/4) + 4kg + e%4 ----
    if constexpr (KV == kF32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) l += p[e];
#pragma unroll
      for (int d = 0; d < D / 16; ++d)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[d] = mma_s(__uint_as_float(R.v[d][e / 4][e % 4]), p[e], o[d]);
    } else {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[e] = static_cast<__bf16>(p[e]);
        l += static_cast<float>(pb[e]);
      }
#pragma unroll
      for (int d = 0; d < D / 16; ++d) {
        bf16x8 va;
        if constexpr (KV == kBF16) {
          va = as_bf16x8(R.v[d][0][0], R.v[d][0][1], R.v[d][1][0], R.v[d][1][1]);
        } else {
          va = as_bf16x8(fp8x2_to_bf16x2<false>(R.v[d][0][0]), fp8x2_to_bf16x2<true>(R.v[d][0][0]),
                         fp8x2_to_bf16x2<false>(R.v[d][1][0]), fp8x2_to_bf16x2<true>(R.v[d][1][0]));
        }
        o[d] = mma_s(va, pb, o[d]);
      }
    }
  }
};

// A length outside [0, max_ctx] is clamped so that table, workspace and output stay in bounds.
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int seq) { return min(max(a.lens[seq], 0), a.max_ctx); }

// ---- work plan: units (16 keys) of every sequence, as a prefix sum --------------------------------
constexpr int kPlanThreads = 1024;

// One workgroup: pref[s] = sum over sequences s' < s of ceil(L_s' / 16).
__global__ void __launch_bounds__(kPlanThreads) decode_plan_kernel(DecodeArgs a) {
  __shared__ int csum[kPlanThreads];
  const int n = a.num_seqs;
  const int tid = threadIdx.x;
  const int chunk = (n + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(tid * chunk, n), s1 = min(s0 + chunk, n);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (clamped_len(a, s) + kUnit - 1) / kUnit;
  csum[tid] = local;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off *= 2) {
    const int v = tid >= off ? csum[tid - off] : 0;
    __syncthreads();
    csum[tid] += v;
    __syncthreads();
  }
  int run = csum[tid] - local;
  if (tid == 0) a.ws_pref[0] = 0;
  for (int s = s0; s < s1; ++s) {
    run += (clamped_len(a, s) + kUnit - 1) / kUnit;
    a.ws_pref[s + 1] = run;
  }
}

// ---- stream decode -----------------------------------------------------------------------------
// Position in a unit stream: KV head slot hh of the stream, sequence, unit j of nj in the sequence.
struct Cursor {
  int hh, seq, j, nj;
};

// The cursor at stream position r (the sequence holding unit r % useq of KV head slot r / useq).
__device__ __forceinline__ Cursor locate(const int32_t* pref, int n, int useq, int r) {
  Cursor c;
  c.hh = r / useq;
  const int rem = r - c.hh * useq;
  int lo = 0, hi = n - 1;                 // largest s with pref[s] <= rem; then pref[s + 1] > rem
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= rem) lo = mid; else hi = mid - 1;
  }
  c.seq = lo;
  c.j = rem - pref[lo];
  c.nj = pref[lo + 1] - pref[lo];
  return c;
}

// Next stream position (sequences without units are skipped).  Only called while a next position exists.
__device__ __forceinline__ void advance(Cursor& c, const int32_t* pref, int n) {
  if (++c.j < c.nj) return;
  c.j = 0;
  do {
    if (++c.seq == n) {
      c.seq = 0;
      ++c.hh;
    }
    c.nj = pref[c.seq + 1] - pref[c.seq];
  } while (c.nj == 0);
}

template <int KV, int D, int BS>
__device__ __forceinline__ SeqView seq_view(const DecodeArgs& a, int seq, int kvh) {
  constexpr int TILE = BS * D * Elem<KV>::kBytes;      // bytes of one (block, head) tile
  SeqView sv;
  sv.kbase = static_cast<const char*>(a.k_pool) + static_cast<int64_t>(kvh) * TILE;
  sv.vbase = static_cast<const char*>(a.v_pool) + static_cast<int64_t>(kvh) * TILE;
  sv.tab = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  sv.blk_stride = static_cast<int64_t>(a.num_kv_heads) * TILE;
  sv.nblk = (clamped_len(a, seq) + BS - 1) / BS;
  return sv;
}

// Q^T operands of (seq, KV head): column i holds query head kvh*G + i (zeros for i >= G); the k-slots
// of lane group kg follow the dims of its K loads.
template <int KV, int D, int G, typename QArr>
__device__ __forceinline__ void load_q(QArr& qb, const DecodeArgs& a, int seq, int kvh, int i, int kg) {
  using QT = typename std::conditional<KV == kF32, float, uint16_t>::type;
  const bool live = i < G;
  const QT* qrow = static_cast<const QT*>(a.q) +
                   (static_cast<int64_t>(seq) * a.num_q_heads + kvh * G + (live ? i : 0)) * D;
  if constexpr (KV == kF32) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const float4 w = live ? *reinterpret_cast<const float4*>(qrow + 16 * c + 4 * kg) : make_float4(0.f, 0.f, 0.f, 0.f);
      qb[4 * c] = w.x; qb[4 * c + 1] = w.y; qb[4 * c + 2] = w.z; qb[4 * c + 3] = w.w;
    }
  } else {
    constexpr int DPC = KV == kBF16 ? 32 : 64;          // dims covered by one K load of the 4 lane groups
    constexpr int SUB = KV == kBF16 ? 1 : 2;            // MFMAs per K load
#pragma unroll
    for (int c = 0; c < D / DPC; ++c)
#pragma unroll
      for (int h = 0; h < SUB; ++h) {
        const int d0 = DPC * c + (DPC / 4) * kg + 8 * h;
        const uint4 w = live ? *reinterpret_cast<const uint4*>(qrow + d0) : make_uint4(0, 0, 0, 0);
        qb[SUB * c + h] = __builtin_bit_cast(bf16x8, w);
      }
  }
}

// Streams and slots.  Stream x holds the KV heads h with h % streams == x, head slot hh = h / streams;
// its positions are hh * useq + pref[seq] + j.  A piece is a maximal run of one wave's positions
// inside one partition of one segment; it is written to slot
//   (hh * num_seqs + seq) * max_parts + partition + (wave index in the stream)
// which is unique: along a stream, later pieces have a larger (segment, partition) term and a wave
// index at least as large.
struct StreamGeo {
  int x, nh, useq, wi;
  int64_t share;
};

// Writes the piece [j0, j0 + np) of segment (c.hh, c.seq): the final output when the piece is the
// whole segment, else its partial record.
template <int KV, int D, int G>
__device__ __forceinline__ void finish_piece(const DecodeArgs& a, int out_bf16, const StreamGeo& geo,
                                             DecodeState<KV, D, G>& st, const Cursor& c, int j0, int np, int PU,
                                             int i, int kg) {
  float l = st.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  const int kvh = geo.x + a.streams * c.hh;
  if (i >= G) return;
  if (j0 == 0 && np == c.nj) {
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    const int64_t base = (static_cast<int64_t>(c.seq) * a.num_q_heads + kvh * G + i) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int d = 16 * t + 4 * kg;
      const float x0 = st.o[t][0] * inv, x1 = st.o[t][1] * inv, x2 = st.o[t][2] * inv, x3 = st.o[t][3] * inv;
      if (out_bf16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + base + d) =
            make_uint2(f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16), f32_to_bf16_bits(x2) | (f32_to_bf16_bits(x3) << 16));
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + base + d) = make_float4(x0, x1, x2, x3);
      }
    }
  } else {
    const int64_t slot = geo.x * a.stream_slots +
                         (static_cast<int64_t>(c.hh) * a.num_seqs + c.seq) * a.max_parts + j0 / PU + geo.wi;
    float* rec = a.ws_part + (slot * G + i) * (D + 4);
    if (kg == 0) *reinterpret_cast<float4*>(rec) = make_float4(st.m, l, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      *reinterpret_cast<float4*>(rec + 4 + 16 * t + 4 * kg) = make_float4(st.o[t][0], st.o[t][1], st.o[t][2], st.o[t][3]);
  }
}

// Moves the load cursor to the next stream position and issues that unit's loads into R (at the
// wave's last position it reloads that unit, unused); entering a new segment also loads the
// segment's Q operands into qnext.
template <int KV, int D, int BS, int G, typename QArr>
__device__ __forceinline__ void load_step(const DecodeArgs& a, const StreamGeo& geo, UnitRegs<KV, D>& R, Cursor& lc,
                                          SeqView& lv, int& lpos, int last, QArr& qnext, int i, int kg) {
  if (lpos < last) {
    ++lpos;
    advance(lc, a.ws_pref, a.num_seqs);
    if (lc.j == 0) {
      const int kvh = geo.x + a.streams * lc.hh;
      lv = seq_view<KV, D, BS>(a, lc.seq, kvh);
      load_q<KV, D, G>(qnext, a, lc.seq, kvh, i, kg);
    }
  }
  const int U = lc.j * kUnit;
  load_unit<KV, D, BS>(R, lv, unit_blocks<BS>(lv, U), i, kg);
  __builtin_amdgcn_sched_barrier(0);
}

// Consumes the np units of one piece (keys from U0 on); R holds the first of them on entry and the
// unit after the piece on exit: each consume is followed by the loads of the next stream position.
template <int KV, int D, int BS, int G, typename QArr>
__device__ __forceinline__ void run_piece(const DecodeArgs& a, const StreamGeo& geo, DecodeState<KV, D, G>& st,
                                          UnitRegs<KV, D>& R, Cursor& lc, SeqView& lv, int& lpos, int last,
                                          QArr& qnext, int U0, int L, int np, int i, int kg) {
#pragma unroll 1
  for (int q = 0; q < np; ++q) {
    st.consume(R, U0 + kUnit * q, L, kg, i, a.qk_scale);
    load_step<KV, D, BS, G>(a, geo, R, lc, lv, lpos, last, qnext, i, kg);
  }
}

// Persistent grid of waves over the unit streams.  Every wave takes an equal contiguous share of its
// stream (so the work is balanced to one unit) and runs one register ring across the segments of
// its share, with the next segment's Q and table entries fetched while the current one is consumed:
// no wave ever waits for a fresh start.  With streams == 8 the KV heads of stream x are served by
// the workgroups on XCD x (initial dispatch is round-robin over the 8 XCDs), so blocks shared by many
// sequences (a common prefix) are re-read from that XCD's L2, not from HBM.
template <int KV, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads, (Pipe<KV, D>::kOcc)) decode_stream_kernel(DecodeArgs a, int out_bf16) {
  using St = DecodeState<KV, D, G>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;         // row of an MFMA operand / column (head) of an accumulator
  const int kg = lane >> 4;        // k-group of an operand / row group of an accumulator
  const int n = a.num_seqs;
  const int32_t* pref = a.ws_pref;

  StreamGeo geo;
  geo.x = blockIdx.x % a.streams;
  geo.nh = a.num_kv_heads / a.streams;
  geo.useq = pref[n];
  geo.wi = (blockIdx.x / a.streams) * kWaves + wave;
  const int total = geo.nh * geo.useq;
  geo.share = (static_cast<int64_t>(total) + a.stream_waves - 1) / a.stream_waves;
  const int r0 = static_cast<int>(min(static_cast<int64_t>(total), geo.wi * geo.share));
  const int r1 = static_cast<int>(min(static_cast<int64_t>(total), (geo.wi + 1) * geo.share));
  if (r0 >= r1) return;
  const int PU = a.part_tokens / kUnit;

  St st;
  typename St::QOp qnext[St::NQB];
  Cursor cc = locate(pref, n, geo.useq, r0);            // consume cursor
  Cursor lc = cc;                                      // load cursor
  int lpos = r0;
  SeqView lv = seq_view<KV, D, BS>(a, lc.seq, geo.x + a.streams * lc.hh);
  load_q<KV, D, G>(st.qb, a, cc.seq, geo.x + a.streams * cc.hh, i, kg);
  UnitRegs<KV, D> R;
  load_unit<KV, D, BS>(R, lv, unit_blocks<BS>(lv, lc.j * kUnit), i, kg);

#pragma unroll 1
  for (int p = r0; p < r1;) {
    // the piece: the rest of this partition of this segment, within the wave's share
    const int np = min(min(r1 - p, cc.nj - cc.j), PU - cc.j % PU);
    const int L = clamped_len(a, cc.seq);
    st.reset();
    run_piece<KV, D, BS, G>(a, geo, st, R, lc, lv, lpos, r1 - 1, qnext, cc.j * kUnit, L, np, i, kg);
    finish_piece<KV, D, G>(a, out_bf16, geo, st, cc, cc.j, np, PU, i, kg);
    p += np;
    if (p < r1) {
      const bool new_seg = cc.j + np == cc.nj;
#pragma unroll 1
      for (int k = 0; k < np; ++k) advance(cc, pref, n);
      if (new_seg) {
#pragma unroll
        for (int c = 0; c < St::NQB; ++c) st.qb[c] = qnext[c];
      }
    }
  }
}

// Merge of the partial records of every (sequence, query head) whose segment was split into
// pieces: out = sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M) * v_scale, M = max_p m_p.  Segments
// served by one piece were written by the stream kernel; empty sequences (L = 0) get zeros here.
template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(DecodeArgs a, int out_bf16) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int h = blockIdx.x % a.num_q_heads;
  const int seq = blockIdx.x / a.num_q_heads;
  const int kvh = h / G, g = h % G;
  const int d = threadIdx.x;
  const int32_t* pref = a.ws_pref;
  const int n = a.num_seqs;
  const int nj = pref[seq + 1] - pref[seq];
  const int64_t oi = (static_cast<int64_t>(seq) * a.num_q_heads + h) * D + d;
  if (nj == 0) {
    store_out(a.out, oi, 0.f, out_bf16 != 0);
    return;
  }
  const int x = kvh % a.streams, hh = kvh / a.streams;
  const int useq = pref[n];
  const int64_t total = static_cast<int64_t>(a.num_kv_heads / a.streams) * useq;
  const int64_t share = (total + a.stream_waves - 1) / a.stream_waves;
  const int64_t S = static_cast<int64_t>(hh) * useq + pref[seq];
  const int PU = a.part_tokens / kUnit;
  const int nparts = (nj + PU - 1) / PU;
  if (nparts == 1 && S / share == (S + nj - 1) / share) return;
  const int64_t seg = (static_cast<int64_t>(hh) * n + seq) * a.max_parts + x * a.stream_slots;
  float mm = -INFINITY;
  for (int k = 0; k < nparts; ++k) {
    const int64_t u0 = S + static_cast<int64_t>(k) * PU, u1 = S + min((k + 1) * PU, nj) - 1;
    for (int64_t w = u0 / share; w <= u1 / share; ++w)
      mm = fmaxf(mm, a.ws_part[((seg + k + w) * G + g) * (D + 4)]);
  }
  const float ms = mm == -INFINITY ? 0.f : mm;
  float lsum = 0.f, o = 0.f;
  for (int k = 0; k < nparts; ++k) {
    const int64_t u0 = S + static_cast<int64_t>(k) * PU, u1 = S + min((k + 1) * PU, nj) - 1;
    for (int64_t w = u0 / share; w <= u1 / share; ++w) {
      const float* rec = a.ws_part + ((seg + k + w) * G + g) * (D + 4);
      const float f = __builtin_amdgcn_exp2f(rec[0] - ms);
      lsum += rec[1] * f;
      o += rec[4 + d] * f;
    }
  }
  store_out(a.out, oi, lsum > 0.f ? o / lsum * a.v_scale : 0.f, out_bf16 != 0);
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  return n;
}

constexpr int kMaxOcc = 3;   // the largest Pipe<>::kOcc

template <int KV, int D, int BS, int G>
int launch_one(const DecodeArgs& a0, int out_bf16, hipStream_t s) {
  DecodeArgs a = a0;
  const int64_t wgs = static_cast<int64_t>(device_cus()) * Pipe<KV, D>::kOcc / 8 * 8;   // resident, multiple of 8
  a.streams = a.num_kv_heads % 8 == 0 ? 8 : 1;
  a.stream_waves = static_cast<int32_t>(wgs / a.streams * kWaves);
  a.stream_slots = static_cast<int64_t>(a.num_kv_heads / a.streams) * a.num_seqs * a.max_parts + a.stream_waves;
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  hipLaunchKernelGGL((decode_stream_kernel<KV, D, BS, G>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
                     a, out_bf16);
  e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  const int64_t rw = static_cast<int64_t>(a.num_q_heads) * a.num_seqs;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(static_cast<unsigned>(rw)), dim3(D), 0, s, a, out_bf16);
  return static_cast<int>(hipGetLastError());
}

template <int KV, int D, int BS>
int pick_group(const DecodeArgs& a, int out_bf16, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_one<KV, D, BS, 1>(a, out_bf16, s);
    case 2: return launch_one<KV, D, BS, 2>(a, out_bf16, s);
    case 4: return launch_one<KV, D, BS, 4>(a, out_bf16, s);
    case 8: return launch_one<KV, D, BS, 8>(a, out_bf16, s);
    default: return -1;
  }
}

template <int KV, int D>
int pick_block(const DecodeArgs& a, int bs, int out_bf16, hipStream_t s) {
  switch (bs) {
    case 8: return pick_group<KV, D, 8>(a, out_bf16, s);
    case 16: return pick_group<KV, D, 16>(a, out_bf16, s);
    case 32: return pick_group<KV, D, 32>(a, out_bf16, s);
    default: return -1;
  }
}

template <int KV>
int pick_dim(const DecodeArgs& a, int bs, int d, int out_bf16, hipStream_t s) {
  switch (d) {
    case 64: return pick_block<KV, 64>(a, bs, out_bf16, s);
    case 128: return pick_block<KV, 128>(a, bs, out_bf16, s);
    default: return -1;
  }
}

}  // namespace

int decode_max_waves() { return device_cus() * kMaxOcc * kWaves; }

size_t decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_parts,
                              int64_t waves) {
  const int64_t pref = ((num_seqs + 1) * 4 + 255) / 256 * 256;
  const int64_t g = num_q_heads < 8 ? num_q_heads : 8;   // G <= 8 and G <= num_q_heads
  const int64_t records = num_q_heads * num_seqs * max_parts + waves * g;
  return static_cast<size_t>(pref + records * (head_dim + 4) * 4);
}

int launch_decode(const DecodeArgs& a, int kv_dtype, int q_dtype, int out_dtype, int block_size,
                  int head_dim, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ob = out_dtype == kBF16;
  if (a.part_tokens % kUnit != 0 || a.part_tokens <= 0) return -1;
  if (kv_dtype == kF32 && q_dtype == kF32) return pick_dim<kF32>(a, block_size, head_dim, ob, s);
  if (kv_dtype == kBF16 && q_dtype == kBF16) return pick_dim<kBF16>(a, block_size, head_dim, ob, s);
  if (kv_dtype == kFP8 && q_dtype == kBF16) return pick_dim<kFP8>(a, block_size, head_dim, ob, s);
  return -1;
}

}  // namespace pa
