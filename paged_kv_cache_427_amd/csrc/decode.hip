// Paged decode attention for gfx950: one query token per sequence over its block-table-mapped K/V.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» §三 3.1-3.2: the kernel gets
// the sequence's scattered K/V through its block table -- one indirection per block, contiguous
// coalesced reads inside it -- and dots the query with every cached key; §七 notes the indirection
// costs a little.  softmax(scale * q K^T) V is the textbook form of what the pages describe in words.
//
// Design (HBM-bound: at most 8 flop per byte of K/V, far below the MI355X ridge, so the goal is to
// keep HBM busy and the vector ALUs out of the way of the loads):
//  * two launches, the stream kernel and a merge kernel; the stream kernel plans the launch itself
//    (per-sequence unit counts as a prefix sum in LDS, each wave's start by a binary search), and
//    only a batch of more than 4096 sequences takes a one-workgroup plan kernel first.
//  * a unit is 32 keys of one (sequence, KV head) segment, for all G query heads of the group, so
//    each K/V byte is read once.  The units of all segments form one stream per XCD (KV head h in
//    stream h % 8; initial dispatch is round-robin over the 8 XCDs), so blocks shared by many
//    sequences -- a common prefix -- are re-read from that XCD's L2, not from HBM.
//  * a persistent grid of wave64s (one workgroup of four per CU; three for contexts of at most 64
//    tokens) walks the streams; each wave takes one contiguous share of its stream, so every wave
//    does the same number of units and the K/V of a segment is read in order.  The unit's physical blocks come from wave-uniform scalar reads of
//    the block table: one lookup per block, prepared one unit ahead so they overlap the loads.
//  * both products of a unit run on 16x16 MFMA tiles fed straight from the loads, no LDS staging:
//      S^T[key][head] = K[key][:] . Q[head][:]       A = K rows (token-major tile), B = Q^T
//      O^T[dim][head] += V^T[dim][key] P^T[key][head]   A = V^T rows (dim-major tile), B = P^T
//    The G query heads occupy columns 0..G-1 of the 16.  The keys of a unit are ordered inside its
//    two S^T tiles so that lane l holds keys 8*(l/16)..+7 for head l%16; after rounding to bf16 that
//    is exactly the B operand of the 16x16x32 P.V product over the unit's 32 keys, so the scores
//    never cross lanes, and the matching V^T operand is 8 consecutive keys of one dim-major V row.
//  * bf16 pools use v_mfma_f32_16x16x32_bf16 for both products; fp8 codes widen exactly to bf16
//    first (v_cvt_scalef32_pk_bf16_fp8, scales kept in fp32); fp32 pools use
//    v_mfma_f32_16x16x4_f32.  The probabilities are rounded to bf16 for the bf16/fp8 products and
//    the running sum uses the same rounded values; the fp32 path keeps fp32 probabilities.
//  * base-2 online softmax with one running max per head.  The max is raised only when a logit
//    exceeds it by more than 2^8 (so every exp stays <= 256); that test is one wave-wide ballot, and
//    only then are the lanes' maxima exchanged and the accumulators rescaled.
//  * one unit of K/V is in flight per wave while the previous one is consumed.  Blocks that no other
//    sequence of the launch reads (the caller's shared_blocks hint says which are shared) are
//    streamed with non-temporal loads, V always and K for fp8 pools, so that they do not push the
//    shared ones out of L2.
//  * a piece is a wave's run of units inside one partition of one segment.  A piece that is a whole
//    segment writes the output directly; any other piece writes (max, sum, unnormalised partial
//    output) to its own slot, and the merge kernel combines the pieces of each (sequence, head).

#include <hip/hip_runtime.h>

#include <mutex>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "decode_records.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

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

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = kDecodeUnit; // keys per unit of one wave (two 16x16 S^T tiles)
constexpr float kSlack = 8.0f;     // log2 of the growth allowed before the accumulators are rescaled

template <int KV>
struct Elem {
  static constexpr int kBytes = KV == kF32 ? 4 : KV == kBF16 ? 2 : 1;
};

// Workgroups per CU that the register budget of a kernel allows (the launch bound).
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

// Tables, lengths and the plan are read through ro() (the constant address space): the compiler
// keeps uniform reads of them on the scalar unit even where the kernel also stores or counts
// atomically, so they never wait behind the K/V loads in flight.

// Key order inside a unit.  Row i of the unit's S^T tile t is key 8*(i/4) + 4t + i%4, so the
// accumulator rows 4kg..4kg+3 of both tiles -- what lane group kg holds -- are keys 8kg..8kg+7: the
// probabilities of a lane are 8 consecutive keys, and so is its slice of the P.V operand, one
// contiguous piece of a dim-major V row.
__device__ __forceinline__ int tile_row_key(int t, int i) { return 8 * (i >> 2) + 4 * t + (i & 3); }

// Raw registers of one 32-key unit, as loaded by one lane (i = lane % 16, kg = lane / 16).
//  k[t][c]: key tile_row_key(t, i) of the unit, 16 bytes at byte 64c + 16kg of its row
//           (bf16: dims 32c+8kg..+8; fp8: dims 64c+16kg..+16; fp32: dims 16c+4kg..+4)
//  v[d]:    dim 16d + i, keys 8kg .. 8kg+7 of the unit (VW dwords)
template <int KV, int D>
struct UnitRegs {
  static constexpr int E = Elem<KV>::kBytes;
  static constexpr int KL = D * E / 64;   // 16-byte K loads per 16-key tile
  static constexpr int VW = 2 * E;        // dwords of 8 keys of one V row
  uint4 k[2][KL];
  uint32_t v[D / 16][VW];
};

// K/V loads.  NT: non-temporal (streamed: a block that no other sequence of the launch reads is read
// once, and should not push the shared ones out of L2); otherwise through the caches.  Streaming
// applies to the V loads of unshared blocks, and to their K loads only for fp8 pools.  Measured on
// MI355X, decode launch inside the step (copy, write, decode), bf16: streaming V only 1.371 ms on
// the shared-prefix decode (all through the caches 1.466, K and V streamed 1.490), 0.562 / 0.609 /
// 0.587 ms on the GQA decode, 0.210 / 0.230 / 0.208 ms on the Llama-7B-shaped one; fp8 (mixed
// step): K and V streamed 0.294 ms, V only 0.316, none 0.323.  A bf16 K row is two cache lines
// that consecutive loads read in halves, and the second half is then refetched when the first
// was not kept.
typedef uint32_t ld_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t ld_u32x2 __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint4 ld16(const char* p) {
  if constexpr (NT) {
    const ld_u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const ld_u32x4*>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ uint2 ld8(const char* p) {
  if constexpr (NT) {
    const ld_u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const ld_u32x2*>(p));
    return make_uint2(w.x, w.y);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}

template <int VW, bool NT>
__device__ __forceinline__ void load_piece(uint32_t (&dst)[VW], const char* p) {
  if constexpr (VW == 2) {
    const uint2 w = ld8<NT>(p);
    dst[0] = w.x; dst[1] = w.y;
  } else {
#pragma unroll
    for (int h = 0; h < VW / 4; ++h) {
      const uint4 w = ld16<NT>(p + 16 * h);
      dst[4 * h] = w.x; dst[4 * h + 1] = w.y; dst[4 * h + 2] = w.z; dst[4 * h + 3] = w.w;
    }
  }
}

// One (sequence, KV head) segment as the loads see it.
struct SeqView {
  const char* kbase;       // K pool + this KV head's tile offset
  const char* vbase;
  ro_i32 tab;              // this sequence's block table
  int64_t blk_stride;      // bytes of one block of one pool (all KV heads)
  int nblk;                // valid table entries: ceil(L / BS)
  int shared_units;        // units touching the sequence's shared leading blocks: read through the caches
  int pool_blocks;         // blocks of the pool (table entries are clamped below it)
};

// Physical blocks of the unit starting at key U (32 keys: 4, 2 or 1 blocks of 8, 16 or 32 tokens).
// A block past the sequence's last one (only in a unit that ends the sequence) is replaced by the
// last one; its keys are masked afterwards.
template <int BS>
struct UnitBlocks {
  static constexpr int N = kUnit / BS;
  int32_t b[N];   // physical block ids
};

// ub.b[q] for a per-lane q, as selects of wave-uniform values (the compiler must not turn the
// selects back into an indexed read, which would keep the block ids in scratch memory).
template <int N>
__device__ __forceinline__ int32_t pick_block(const int32_t (&b)[N], int q) {
  int32_t r = __builtin_amdgcn_readfirstlane(b[0]);
#pragma unroll
  for (int k = 1; k < N; ++k) r = q == k ? __builtin_amdgcn_readfirstlane(b[k]) : r;
  return r;
}

template <int BS>
__device__ __forceinline__ UnitBlocks<BS> unit_blocks(const SeqView& sv, int U) {
  const int j0 = U / BS;
  UnitBlocks<BS> ub;
#pragma unroll
  for (int q = 0; q < UnitBlocks<BS>::N; ++q) {
    // a table entry outside the pool is clamped into it: a wrong result for this sequence, but no
    // read outside the pool
    const int e = sv.tab[min(j0 + q, sv.nblk - 1)];
    ub.b[q] = min(max(e, 0), sv.pool_blocks - 1);
  }
  return ub;
}

// Issues the loads of the unit starting at key U (a multiple of 32) from its blocks `ub`.
template <int KV, int D, int BS, bool NT>
__device__ __forceinline__ void load_unit(UnitRegs<KV, D>& R, const SeqView& sv, const UnitBlocks<BS>& ub, int i,
                                          int kg) {
  using R_t = UnitRegs<KV, D>;
  constexpr int E = R_t::E, KL = R_t::KL, VW = R_t::VW;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = tile_row_key(t, i);                 // the unit's key in row i of tile t
    const char* krow = sv.kbase + static_cast<int64_t>(pick_block(ub.b, key / BS)) * sv.blk_stride + (key % BS) * (D * E);
#pragma unroll
    for (int c = 0; c < KL; ++c) R.k[t][c] = ld16<NT && KV == kFP8>(krow + 64 * c + 16 * kg);
  }
  const int key0 = 8 * kg;                              // keys 8kg .. 8kg+7: one block, consecutive
  const char* vrow = sv.vbase + static_cast<int64_t>(pick_block(ub.b, key0 / BS)) * sv.blk_stride + (key0 % BS) * E;
#pragma unroll
  for (int d = 0; d < D / 16; ++d) load_piece<VW, NT>(R.v[d], vrow + (16 * d + i) * BS * E);
}

template <int KV, int D, int G>
struct DecodeState {
  static constexpr int NQB = KV == kF32 ? D / 4 : D / 32;   // MFMAs per 16-key S^T tile
  typedef typename std::conditional<KV == kF32, float, bf16x8>::type QOp;
  f32x4 o[D / 16];     // O^T: lane holds dims 16t + 4kg + r for head lane % 16
  float m;             // running max (base-2 logits) of head lane % 16; equal across the 4 lane groups
  float l;             // this lane's partial exp-sum

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  // qb: the Q^T operand of each S^T MFMA (column i holds query head min(i, G - 1) of the group;
  // columns >= G are computed and never used).
  __device__ __forceinline__ void consume(UnitRegs<KV, D>& R, const QOp (&qb)[NQB], int U, int t1, int kg, int col,
                                          float qk_scale) {
    using R_t = UnitRegs<KV, D>;
    constexpr int KL = R_t::KL;
    // ---- S^T of the unit's two 16-key tiles: lane holds keys 8kg + 4t + r for head col ----
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
    float x[8];   // x[e]: key 8kg + e of the unit (e = 4t + r)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * t + r] = s[t][r] * qk_scale;
    if (U + kUnit > t1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (U + 8 * kg + 4 * t + r >= t1) x[4 * t + r] = -INFINITY;
      // masked keys may hold any bits (even NaN): zero their values so that 0 * v stays 0
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (U + 8 * kg + e < t1) continue;
#pragma unroll
        for (int d = 0; d < D / 16; ++d) {
          if constexpr (KV == kF32) {
            R.v[d][e] = 0u;
          } else if constexpr (KV == kBF16) {
            R.v[d][e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          } else {
            R.v[d][e / 4] &= ~(0xffu << (8 * (e % 4)));
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
    // ---- O^T += V^T P^T: k-slot e of lane group kg is key 8kg + e ----
    if constexpr (KV == kF32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) l += p[e];
#pragma unroll
      for (int d = 0; d < D / 16; ++d)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[d] = mma_s(__uint_as_float(R.v[d][e]), p[e], o[d]);
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
          va = as_bf16x8(R.v[d][0], R.v[d][1], R.v[d][2], R.v[d][3]);
        } else {
          va = as_bf16x8(fp8x2_to_bf16x2<false>(R.v[d][0]), fp8x2_to_bf16x2<true>(R.v[d][0]),
                         fp8x2_to_bf16x2<false>(R.v[d][1]), fp8x2_to_bf16x2<true>(R.v[d][1]));
        }
        o[d] = mma_s(va, pb, o[d]);
      }
    }
  }
};

// A length outside [0, max_ctx] is clamped so that table, workspace and output stay in bounds.
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int seq) { return min(max(ro(a.lens)[seq], 0), a.max_ctx); }

// ---- work plan ---------------------------------------------------------------------------------
// The units (32 keys) of every (KV head, sequence) segment form one stream per XCD, in the order
// (head slot, sequence, unit).  Wave v of a stream takes the contiguous static share [v S, (v + 1) S)
// of it, S = ceil(units / waves), so no wave has more than S units and the shares need no counter.
// (Measured on MI355X: handing part of each stream out dynamically, to the waves that finish
// first, was slower -- each extra share costs a cold start on a new segment's table entries and Q
// and adds a partial record.)  All streams have the same shape (the same sequences,
// num_kv_heads / streams heads each), so one schedule serves them all.  A batch of at most
// kSelfPlanMax sequences is planned by every workgroup of the stream kernel itself: the prefix of
// per-sequence unit counts in LDS, each wave's start cursor by a binary search in it (no plan
// launch, whose few microseconds and launch gap are a few percent of a short decode).  A larger
// batch is planned by the one-workgroup plan kernel, which also writes every share's start cursor.
constexpr int kPlanThreads = 1024;
constexpr int kPlanLds = 8192;        // prefix entries searched in LDS (larger batches search global memory)
constexpr int kSelfPlanMax = 4096;    // batches the stream kernel plans itself (a multiple of its threads)
static_assert(kSelfPlanMax % kThreads == 0, "a thread's run of sequences has a fixed bound");
constexpr int kSharesPerWave = 1;
constexpr int kSchedInts = 64;
// schedule header: [0] S (units per share), [1] V (shares)

struct Sched {
  int S, V;
  __device__ __forceinline__ int start(int v) const { return v * S; }
  __device__ __forceinline__ int share_of(int p) const { return p / S; }
};

// The schedule of `total` stream positions over `waves` waves.
__device__ __forceinline__ Sched make_sched(int total, int waves) {
  Sched sc;
  sc.S = max(1, (total + waves - 1) / waves);
  sc.V = (total + sc.S - 1) / sc.S;
  return sc;
}

// Prefix of per-sequence unit counts, read from LDS (stream kernel that planned itself) or from the
// plan kernel's table.
struct PrefView {
  const int* lds;
  const int32_t* g;
  bool in_lds;
  __device__ __forceinline__ int operator[](int k) const {
    return in_lds ? lds[k] : ro(g)[k];
  }
};

// Largest s with pref[s] <= r (then pref[s + 1] > r: sequence s holds unit r of its head slot).
template <typename P>
__device__ __forceinline__ int find_seq(const P& pref, int n, int r) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One workgroup: pref[s] = sum over sequences s' < s of ceil(L_s' / 32); the schedule header; the
// start cursor (head slot, sequence, unit, units of the sequence) of every share.
__global__ void __launch_bounds__(kPlanThreads) decode_plan_kernel(DecodeArgs a) {
  __shared__ int csum[kPlanThreads];
  __shared__ int spref[kPlanLds];
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
  const bool in_lds = n + 1 <= kPlanLds;
  int run = csum[tid] - local;
  if (tid == 0) {
    a.ws_pref[0] = 0;
    if (in_lds) spref[0] = 0;
  }
  for (int s = s0; s < s1; ++s) {
    run += (clamped_len(a, s) + kUnit - 1) / kUnit;
    a.ws_pref[s + 1] = run;
    if (in_lds) spref[s + 1] = run;
  }
  const int useq = csum[kPlanThreads - 1];
  const int total = (a.num_kv_heads / a.streams) * useq;
  const Sched sc = make_sched(total, a.stream_waves);
  if (tid == 0) {
    a.ws_sched[0] = sc.S;
    a.ws_sched[1] = sc.V;
  }
  __syncthreads();   // the prefix written above is read back by other threads of this workgroup
  for (int v = tid; v < sc.V; v += kPlanThreads) {
    const int p = sc.start(v);
    const int hh = p / useq, rem = p - hh * useq;
    int seq, base, next;
    if (in_lds) {
      seq = find_seq(spref, n, rem);
      base = spref[seq];
      next = spref[seq + 1];
    } else {
      seq = find_seq(a.ws_pref, n, rem);
      base = a.ws_pref[seq];
      next = a.ws_pref[seq + 1];
    }
    *reinterpret_cast<int4*>(a.ws_share + 4 * v) = make_int4(hh, seq, rem - base, next - base);
  }
}

// ---- stream decode -----------------------------------------------------------------------------
// Position in a unit stream: KV head slot hh of the stream, sequence, unit j of nj in the sequence.
struct Cursor {
  int hh, seq, j, nj;
};

// Next stream position (sequences without units are skipped).  Only called while a next position exists.
__device__ __forceinline__ void advance(Cursor& c, const PrefView& pref, int n) {
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
  sv.tab = ro(a.tables) + static_cast<int64_t>(seq) * a.max_blocks;
  sv.blk_stride = static_cast<int64_t>(a.num_kv_heads) * TILE;
  sv.nblk = (clamped_len(a, seq) + BS - 1) / BS;
  sv.pool_blocks = a.num_blocks;
  sv.shared_units = a.shared_blocks ? (max(ro(a.shared_blocks)[seq], 0) * BS + kUnit - 1) / kUnit : 0;
  return sv;
}

// Q^T operands of (seq, KV head): column i holds query head kvh*G + min(i, G - 1), so that every
// lane loads a real row (the columns >= G are never used); the k-slots of lane group kg follow the
// dims of its K loads.
template <int KV, int D, int G, typename QArr>
__device__ __forceinline__ void load_q(QArr& qb, const DecodeArgs& a, int seq, int kvh, int i, int kg) {
  using QT = typename std::conditional<KV == kF32, float, uint16_t>::type;
  const QT* qrow = static_cast<const QT*>(a.q) + seq * a.q_sseq + kvh * a.q_skv + min(i, G - 1) * a.q_sg;
  if constexpr (KV == kF32) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const float4 w = *reinterpret_cast<const float4*>(qrow + 16 * c + 4 * kg);
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
        qb[SUB * c + h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + d0));
      }
  }
}

// Pieces and slots.  A piece is a maximal run of one share's positions inside one partition of one
// segment; a piece that is not a whole segment is written to slot
//   x * stream_slots + (hh * num_seqs + seq) * max_parts + partition + share
// which is unique: along a stream both terms are non-decreasing from one piece to the next, and one
// of them grows.
template <int KV, int D, int G>
__device__ __forceinline__ void finish_piece(const DecodeArgs& a, int out_bf16, int x, int share,
                                             DecodeState<KV, D, G>& st, const Cursor& c, int np, int PU,
                                             int i, int kg) {
  float l = st.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  const int kvh = x + a.streams * c.hh;
  if (i >= G) return;
  if (!a.records_only && c.j == 0 && np == c.nj) {
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    const int64_t base = c.seq * a.o_sseq + kvh * a.o_skv + i * a.o_sg;
    if (a.lse && kg == 0) a.lse[base / D] = (st.m + __log2f(l)) * 0.6931471805599453f;
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
    const int64_t slot = segment_slot(a, x, c.hh, c.seq) + c.j / PU + share;
    float* rec = a.ws_part + (slot * G + i) * (D + 4);
    if (kg == 0) *reinterpret_cast<float4*>(rec) = make_float4(st.m, l, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      *reinterpret_cast<float4*>(rec + 4 + 16 * t + 4 * kg) = make_float4(st.o[t][0], st.o[t][1], st.o[t][2], st.o[t][3]);
  }
}

// A stream position prepared for loading: its cursor, the view of its segment, its blocks, its
// share, and whether it enters a segment or a share (its Q must be loaded with it).  `live` is false once the wave has no position left: the position then stays on
// the wave's last unit, which is loaded again (in bounds, unused).
template <int BS>
struct Pos {
  Cursor c;
  SeqView v;
  UnitBlocks<BS> ub;
  int pos, end, share;
  bool enter, live;
};

// Points P at the first unit of share v: its start cursor from the plan table, or found in the LDS
// prefix (useq units per head slot).
template <int KV, int D, int BS>
__device__ __forceinline__ void enter_share(const DecodeArgs& a, int x, int total, int useq, const Sched& sc,
                                            const PrefView& pref, Pos<BS>& P, int v) {
  if (pref.in_lds) {
    const int p = sc.start(v);
    const int hh = p / useq, rem = p - hh * useq;
    const int seq = find_seq(pref, a.num_seqs, rem);
    P.c.hh = hh;
    P.c.seq = seq;
    P.c.j = rem - pref[seq];
    P.c.nj = pref[seq + 1] - pref[seq];
  } else {
    const ro_i32 e = ro(a.ws_share) + 4 * v;
    P.c.hh = e[0];
    P.c.seq = e[1];
    P.c.j = e[2];
    P.c.nj = e[3];
  }
  P.share = v;
  P.pos = sc.start(v);
  P.end = min(total, sc.start(v + 1));
  P.v = seq_view<KV, D, BS>(a, P.c.seq, x + a.streams * P.c.hh);
  P.enter = true;
}

// Moves P to the next unit of the wave's share and reads that position's block-table entries.  It
// runs right after the loads of the current position are issued, so these dependent scalar reads
// overlap the loads in flight instead of delaying the next issue.
template <int KV, int D, int BS>
__device__ __forceinline__ void prepare_next(const DecodeArgs& a, int x, const PrefView& pref, Pos<BS>& P) {
  P.enter = false;
  if (P.pos + 1 < P.end) {
    ++P.pos;
    advance(P.c, pref, a.num_seqs);
    if (P.c.j == 0) {
      P.v = seq_view<KV, D, BS>(a, P.c.seq, x + a.streams * P.c.hh);
      P.enter = true;
    }
    P.ub = unit_blocks<BS>(P.v, P.c.j * kUnit);
  } else {
    P.live = false;
  }
}

// Issues the loads of the prepared position P into R (and its segment's Q into qnext when P enters
// a segment or a share: the only write of qnext, which the consumes of earlier units no longer need).
template <int KV, int D, int BS, int G, typename QArr>
__device__ __forceinline__ void issue(const DecodeArgs& a, int x, const Pos<BS>& P, UnitRegs<KV, D>& R, QArr& qnext,
                                      int i, int kg) {
  if (P.enter) load_q<KV, D, G>(qnext, a, P.c.seq, x + a.streams * P.c.hh, i, kg);
  if (P.c.j < P.v.shared_units)
    load_unit<KV, D, BS, false>(R, P.v, P.ub, i, kg);
  else
    load_unit<KV, D, BS, true>(R, P.v, P.ub, i, kg);
  __builtin_amdgcn_sched_barrier(0);
}

// Persistent grid of waves over the unit streams.  Wave v of stream x walks share v; one register
// ring runs across all the segments of its share: each consume is followed by the loads of the next position, and the
// position after that is prepared while those loads are in flight.  With streams == 8 the KV heads
// of stream x are served by the workgroups on XCD x (initial dispatch is round-robin over the 8
// XCDs), so blocks shared by many sequences (a common prefix) are re-read from that XCD's L2.
template <int KV, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads, (Pipe<KV, D>::kOcc)) decode_stream_kernel(DecodeArgs a, int out_bf16) {
  using St = DecodeState<KV, D, G>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;         // row of an MFMA operand / column (head) of an accumulator
  const int kg = lane >> 4;        // k-group of an operand / row group of an accumulator
  const int x = blockIdx.x % a.streams;
  const int wi = (blockIdx.x / a.streams) * kWaves + wave;
  const int n = a.num_seqs;
  const bool self_plan = a.self_plan != 0;
  __shared__ int spref[kSelfPlanMax + 1];
  __shared__ int scan_s[kThreads];
  int useq;
  Sched sc;
  if (self_plan) {
    // spref[s] = units of the sequences before s: a block-wide scan of per-thread runs
    // (a thread's run is at most kSelfPlanMax / kThreads sequences, loaded all at once)
    constexpr int kRun = kSelfPlanMax / kThreads;
    const int tid = threadIdx.x;
    const int chunk = (n + kThreads - 1) / kThreads;
    const int s0 = min(tid * chunk, n), s1 = min(s0 + chunk, n);
    int units[kRun];
#pragma unroll
    for (int k = 0; k < kRun; ++k) units[k] = s0 + k < s1 ? (clamped_len(a, s0 + k) + kUnit - 1) / kUnit : 0;
    int local = 0;
#pragma unroll
    for (int k = 0; k < kRun; ++k) local += units[k];
    scan_s[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off *= 2) {
      const int v = tid >= off ? scan_s[tid - off] : 0;
      __syncthreads();
      scan_s[tid] += v;
      __syncthreads();
    }
    int run = scan_s[tid] - local;
    if (tid == 0) spref[0] = 0;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      run += units[k];
      if (s0 + k < s1) spref[s0 + k + 1] = run;
    }
    __syncthreads();
    useq = spref[n];
    sc = make_sched((a.num_kv_heads / a.streams) * useq, a.stream_waves);
    if (blockIdx.x == 0) {   // the merge kernel reads the prefix and the schedule
      for (int s = tid; s <= n; s += kThreads) a.ws_pref[s] = spref[s];
      if (tid == 0) {
        a.ws_sched[0] = sc.S;
        a.ws_sched[1] = sc.V;
      }
    }
    if (a.fill_empty) {      // no merge launch: zeros (and -inf log-sum-exps) of empty sequences here
      const int hq = a.num_kv_heads * G;
      for (int seq = blockIdx.x; seq < n; seq += gridDim.x) {
        if (spref[seq + 1] != spref[seq]) continue;
        for (int k = tid; k < hq * D; k += kThreads) {
          const int hd = k / D, kvh = hd / G, g = hd % G;
          const int64_t row = seq * a.o_sseq + kvh * a.o_skv + g * a.o_sg;
          store_out(a.out, row + k % D, 0.f, out_bf16 != 0);
          if (a.lse && k % D == 0) a.lse[row / D] = -INFINITY;
        }
      }
    }
  } else {
    useq = ro(a.ws_pref)[n];
    sc.S = ro(a.ws_sched)[0];
    sc.V = ro(a.ws_sched)[1];
  }
  if (wi >= sc.V) return;
  const int total = (a.num_kv_heads / a.streams) * useq;
  const PrefView pref{spref, a.ws_pref, self_plan};
  const int PU = a.part_tokens / kUnit;

  St st;
  typename St::QOp qnext[St::NQB];
  UnitRegs<KV, D> R;
  Pos<BS> P;
  P.live = true;
  enter_share<KV, D, BS>(a, x, total, useq, sc, pref, P, wi);
  P.ub = unit_blocks<BS>(P.v, P.c.j * kUnit);
  issue<KV, D, BS, G>(a, x, P, R, qnext, i, kg);
  Cursor cc = P.c;                      // the position whose unit R holds
  int share = P.share, pos = P.pos, end = P.end;
  prepare_next<KV, D, BS>(a, x, pref, P);

#pragma unroll 1
  for (;;) {
    // the piece: the rest of this partition of this segment, within the share
    const Cursor c0 = cc;
    const int share0 = share, end0 = end;
    const int np = min(min(end0 - pos, c0.nj - c0.j), PU - c0.j % PU);
    const int L = clamped_len(a, c0.seq);
    bool more = true;
    st.reset();
#pragma unroll 1
    for (int q = 0; q < np; ++q) {
      st.consume(R, qnext, (c0.j + q) * kUnit, L, kg, i, a.qk_scale);
      more = P.live;
      issue<KV, D, BS, G>(a, x, P, R, qnext, i, kg);
      cc = P.c;
      share = P.share;
      pos = P.pos;
      end = P.end;
      prepare_next<KV, D, BS>(a, x, pref, P);
    }
    finish_piece<KV, D, G>(a, out_bf16, x, share0, st, c0, np, PU, i, kg);
    if (!more) break;   // the last issue was a reload: the wave's share is done
  }
}

// Merge of the partial records of the segments that were split into pieces:
// out = sum_r o_r 2^(m_r - M) / sum_r l_r 2^(m_r - M) * v_scale, M = max_r m_r.  One wave per
// (sequence, KV head) segment and HW of its G query heads (they share the segment's pieces), four
// waves per workgroup: a segment served by one piece (written by the stream kernel) leaves after
// reading the plan; an empty one gets zeros (and a -inf log-sum-exp); a split one is merged with its
// records' (max, sum) loaded across the lanes, 64 pieces at a time, for the wave's HW heads at once
// (the maximum and weighted sum of each head are wave reductions), and each lane then adds its
// slice of the output dims of every head over the records with many loads in flight.  The records
// of partition k are those of the shares v0(k)..v1(k) that overlap it, read in that order, so
// results do not depend on timing (nor on how many heads a wave serves).
constexpr int kMergeThreads = 256;

template <int D, int HW>
__global__ void __launch_bounds__(kMergeThreads) decode_merge_kernel(DecodeArgs a, int out_bf16) {
  constexpr int DPL = D / 64;   // output dims per lane
  constexpr int kRec = D + 4;   // floats of one head's record
  const int lane = threadIdx.x & 63;
  // workgroup i serves stream i % streams (with 8 streams, the XCD whose stream kernel workgroups
  // wrote that stream's records, so they are read from its L2); its waves are numbered (head slot,
  // sequence, slice of HW heads in the group) with the slice fastest
  const int G = a.num_q_heads / a.num_kv_heads;
  const int slices = G / HW;
  const int x = static_cast<int>(blockIdx.x % a.streams);
  const int64_t q = static_cast<int64_t>(blockIdx.x / a.streams) * (kMergeThreads / 64) + (threadIdx.x >> 6);
  const int hpx = a.num_kv_heads / a.streams;
  if (q >= static_cast<int64_t>(hpx) * a.num_seqs * slices) return;
  const int g0 = static_cast<int>(q % slices) * HW;
  const int seq = static_cast<int>((q / slices) % a.num_seqs);
  const int hh = static_cast<int>(q / (static_cast<int64_t>(slices) * a.num_seqs));
  const int kvh = hh * a.streams + x;
  const ro_i32 pref = ro(a.ws_pref);
  const int n = a.num_seqs;
  const int nj = pref[seq + 1] - pref[seq];
  const int64_t orow0 = seq * a.o_sseq + kvh * a.o_skv + g0 * a.o_sg;
  if (nj == 0) {
#pragma unroll
    for (int g = 0; g < HW; ++g) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) store_out(a.out, orow0 + g * a.o_sg + DPL * lane + e, 0.f, out_bf16 != 0);
      if (a.lse && lane == 0) a.lse[(orow0 + g * a.o_sg) / D] = -INFINITY;
    }
    return;
  }
  Sched sc;
  sc.S = ro(a.ws_sched)[0];
  sc.V = ro(a.ws_sched)[1];
  const int P0 = hh * pref[n] + pref[seq];   // stream position of the segment's first unit
  const int PU = a.part_tokens / kUnit;
  const int nparts = (nj + PU - 1) / PU;
  if (nparts == 1 && sc.share_of(P0) == sc.share_of(P0 + nj - 1)) return;   // one piece
  float M[HW], lsum[HW], o[HW][DPL];
#pragma unroll
  for (int g = 0; g < HW; ++g) {
    M[g] = -INFINITY;
    lsum[g] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[g][e] = 0.f;
  }
  PieceWalk walk;
  walk.init(segment_slot(a, x, hh, seq), P0, nj, PU, sc.S);
  while (!walk.done()) {
    int64_t my_off = 0;   // head g0 of the lane's piece
    int cnt = 0;
    for (; cnt < 64 && !walk.done(); ++cnt) {
      const int64_t slot = walk.next();
      if (lane == cnt) my_off = (slot * G + g0) * kRec;
    }
    float m_r[HW], l_r[HW];
#pragma unroll
    for (int g = 0; g < HW; ++g) {
      m_r[g] = lane < cnt ? a.ws_part[my_off + g * kRec] : -INFINITY;
      l_r[g] = lane < cnt ? a.ws_part[my_off + g * kRec + 1] : 0.f;
    }
    uint32_t w_bits[HW];
#pragma unroll
    for (int g = 0; g < HW; ++g) {
      float mb = m_r[g];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mb = fmaxf(mb, shfl_xor(mb, off));
      const float Mn = fmaxf(M[g], mb);
      const float alpha = M[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[g] - Mn);
      const float w_r = lane < cnt ? __builtin_amdgcn_exp2f(m_r[g] - Mn) : 0.f;
      float ls = l_r[g] * w_r;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ls += shfl_xor(ls, off);
      lsum[g] = lsum[g] * alpha + ls;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[g][e] *= alpha;
      w_bits[g] = __builtin_bit_cast(uint32_t, w_r);
      M[g] = Mn;
    }
    const uint32_t off_lo = static_cast<uint32_t>(my_off), off_hi = static_cast<uint32_t>(my_off >> 32);
    // up to 16 records' loads in flight at a time over the HW heads (slots past cnt load nothing)
    constexpr int kFly = HW >= 16 ? 1 : 16 / HW;
    for (int c0 = 0; c0 < cnt; c0 += kFly) {
      float val[kFly][HW][DPL], wt[kFly][HW];
#pragma unroll
      for (int j = 0; j < kFly; ++j) {
#pragma unroll
        for (int g = 0; g < HW; ++g) {
          wt[j][g] = 0.f;
#pragma unroll
          for (int e = 0; e < DPL; ++e) val[j][g][e] = 0.f;
        }
        if (c0 + j < cnt) {
          const int c = c0 + j;
          const int64_t r = (static_cast<int64_t>(__builtin_amdgcn_readlane(off_hi, c)) << 32) |
                            __builtin_amdgcn_readlane(off_lo, c);
#pragma unroll
          for (int g = 0; g < HW; ++g) {
            wt[j][g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(w_bits[g], c));
            if constexpr (DPL == 2) {
              const float2 t = *reinterpret_cast<const float2*>(a.ws_part + r + g * kRec + 4 + 2 * lane);
              val[j][g][0] = t.x;
              val[j][g][1] = t.y;
            } else {
              val[j][g][0] = a.ws_part[r + g * kRec + 4 + lane];
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kFly; ++j)
#pragma unroll
        for (int g = 0; g < HW; ++g)
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[g][e] += val[j][g][e] * wt[j][g];
    }
  }
#pragma unroll
  for (int g = 0; g < HW; ++g) {
    const int64_t orow = orow0 + g * a.o_sg;
    const float inv = lsum[g] > 0.f ? a.v_scale / lsum[g] : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_out(a.out, orow + DPL * lane + e, o[g][e] * inv, out_bf16 != 0);
    if (a.lse && lane == 0) a.lse[orow / D] = (M[g] + __log2f(lsum[g])) * 0.6931471805599453f;
  }
}

// Workgroups of the persistent grid: one per CU.  Measured on MI355X against three (what the
// register budget allows), 1.5 and two per CU: one is fastest on every workload (Llama-7B-shaped
// decode 236 -> 227 us, GQA long 630 -> 614 us, fp8 decode of the mixed step 339 -> 320 us, beam
// decode 691 -> 670 us, shared-prefix decode unchanged): each wave keeps a three times longer share,
// so fewer segment starts and fewer partial records, and one unit in flight per wave on every SIMD
// still keeps HBM busy.  Half a workgroup per CU is slower (260, 742, 482 us).
// Contexts of at most kShortCtx tokens are the exception: each wave then walks many one- or two-unit
// segments, each a cold start on its table entries and Q, so the launch is bound by latency and
// takes as many waves as the registers allow (the tails of the beam decode: 92 -> 76 us).
constexpr int kShortCtx = 2 * kUnit;
constexpr int kMaxOcc = 3;   // the largest Pipe<>::kOcc
int grid_workgroups(int per_cu) { return std::max(8, device_cus() * per_cu / 8 * 8); }

template <int KV, int D, int BS, int G>
int launch_one(const DecodeArgs& a0, int out_bf16, hipStream_t s) {
  DecodeArgs a = a0;
  const int64_t wgs = decode_launch_shape(a, KV);
  hipError_t e;
  if (!a.self_plan) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  hipLaunchKernelGGL((decode_stream_kernel<KV, D, BS, G>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
                     a, out_bf16);
  e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  if (a.fill_empty || a.records_only) return 0;
  // A wave merges all G heads of a segment when its rows are not partitioned (a few pieces each, at
  // share boundaries: the beam decode's shared part, G = 8, 20.8 -> 10.7 us), one head when they are
  // (rows of tens of pieces: whole groups per wave left too few waves for the long GQA decode, whose
  // decode launch went 564 -> 575 us).
  const int HW = a.max_parts == 1 ? G : 1;
  const int64_t waves = static_cast<int64_t>(a.num_kv_heads / a.streams) * a.num_seqs * (G / HW);   // per stream
  const int64_t mw = a.streams * ((waves + kMergeThreads / 64 - 1) / (kMergeThreads / 64));
  auto merge = HW == 1 ? decode_merge_kernel<D, 1> : decode_merge_kernel<D, G>;
  hipLaunchKernelGGL(merge, dim3(static_cast<unsigned>(mw)), dim3(kMergeThreads), 0, s, a, out_bf16);
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

int decode_max_waves() { return grid_workgroups(kMaxOcc) * kWaves; }

int64_t decode_launch_shape(DecodeArgs& a, int kv_dtype) {
  const int occ = kv_dtype == kF32 ? Pipe<kF32, 128>::kOcc : Pipe<kBF16, 128>::kOcc;
  const int64_t wgs = grid_workgroups(a.max_ctx <= kShortCtx ? occ : 1);   // resident, multiple of 8
  a.streams = a.num_kv_heads % 8 == 0 ? 8 : 1;
  a.stream_waves = static_cast<int32_t>(wgs / a.streams * kWaves);
  a.max_shares = kSharesPerWave * a.stream_waves;   // bounds the share count V
  a.self_plan = a.num_seqs <= kSelfPlanMax;
  // One-unit contexts are never split, so no piece needs merging: the stream kernel then writes the
  // zeros of empty sequences itself and the merge launch is left out.
  a.fill_empty = !a.records_only && a.self_plan && a.max_ctx <= kUnit;
  a.stream_slots = static_cast<int64_t>(a.num_kv_heads / a.streams) * a.num_seqs * a.max_parts + a.max_shares;
  return wgs;
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: share plan (pref, schedule header with the counters, share table), then the
// partial records.  Every share count is bounded by kSharesPerWave per wave of the launch.
size_t decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_parts,
                              int64_t waves) {
  const int64_t plan = align256((num_seqs + 1) * 4) + align256(kSchedInts * 4) + align256(16 * kSharesPerWave * waves);
  const int64_t g = num_q_heads < 8 ? num_q_heads : 8;   // G <= 8 and G <= num_q_heads
  const int64_t records = num_q_heads * num_seqs * max_parts + kSharesPerWave * waves * g;
  return static_cast<size_t>(plan + records * (head_dim + 4) * 4);
}

// The workspace of pa_decode_noalloc: one copy per GPU, reserved by the code object loader when the
// library is loaded on that GPU and held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: every use goes through the device address that
// hipGetSymbolAddress returns, looked up once per device with that device current.
static __device__ __align__(256) char scratch[PA_DECODE_STATIC_WORKSPACE_BYTES];

int decode_static_workspace(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  *ptr = nullptr;
  *bytes = PA_DECODE_STATIC_WORKSPACE_BYTES;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  std::lock_guard<std::mutex> guard(lock);
  if (dev >= 0 && dev < kMaxDevices && addr[dev]) {
    *ptr = addr[dev];
    return 0;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return static_cast<int>(e);
  if (!p) return static_cast<int>(hipErrorInvalidSymbol);
  if (dev >= 0 && dev < kMaxDevices) addr[dev] = p;
  *ptr = p;
  return 0;
}

void decode_workspace_carve(DecodeArgs& a, void* workspace) {
  char* p = static_cast<char*>(workspace);
  a.ws_pref = reinterpret_cast<int32_t*>(p);
  p += align256((static_cast<int64_t>(a.num_seqs) + 1) * 4);
  a.ws_sched = reinterpret_cast<int32_t*>(p);
  p += align256(kSchedInts * 4);
  a.ws_share = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<int64_t>(16) * kSharesPerWave * decode_max_waves());
  a.ws_part = reinterpret_cast<float*>(p);
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
