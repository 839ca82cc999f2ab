// Chunked causal prefill over paged K/V on gfx950 bf16 MFMA.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» FAQ Q4: prefill K/V live in pool
// blocks like decode's, and chunked prefill slices a long prompt and runs it next to decode; FAQ Q1:
// attention is computed tile by tile in on-chip memory without writing the score matrix to HBM.
// Query i of a chunk sits at position P + i and sees keys 0 .. P + i (the causal boundary is a
// reading; the pages state attention only in words).
//
// Design.  This is the one dense contraction of the path, so it runs on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * a workgroup of W = 4 or 8 wave64s owns 32 W (query, head) rows of one KV-head group: 32 W / G
//    queries of the G query heads that share the KV head, so one K/V tile in LDS serves every head
//    of the group; each wave owns 32 rows;
//  * key tiles of 64 positions are gathered through the block table and stored in LDS as bf16 (fp8
//    e4m3 codes convert exactly; scales stay in fp32), two K and two V^T buffers, one register stage
//    each for K and V, loads issued about one iteration before their LDS store;
//  * software pipeline: step t issues the score MFMAs of tile t + 1 beside the exponentials of tile
//    t, then the O MFMAs of tile t beside the LDS stores and loads of later tiles, so each MFMA
//    phase has independent vector work beside it; two steps per trip let the two score arrays
//    trade roles without register copies;
//  * every load instruction of a wave reads inside one pool block, so the table entries are
//    wave-uniform scalar loads, and every load is issued unconditionally, so that the only wait for
//    them is the one before the LDS store.  K tiles are stored [key][dim]; the V pool's dim-major
//    tiles give [dim][key] rows directly, so V needs no transposition, only a fixed permutation of
//    the keys inside each 16-key group;
//  * scores are formed transposed, S^T = K Q^T (A = K rows from LDS, B = Q held in registers), so the
//    fp32 result layout (each lane owns one query row and 16 keys) becomes, after bf16 rounding,
//    exactly the B operand of O^T = V^T P^T; softmax statistics need one cross-half lane exchange
//    (v_permlane32_swap);
//  * logits are scaled and shifted by one fma before the exp; the rescale of the output accumulators
//    is skipped while the running max has grown by less than 2^8 (base-2 logits), which keeps every
//    exp bounded by 256;
//  * work order: sequences longest first (when there are at most 64), the query tiles of each
//    (sequence, KV head) from the last (longest) to the first, and all tiles of one KV head on one
//    XCD so that they share its L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
// A plain vector type for 16-byte register stages: copies of the uint4 struct go through memcpy,
// which can leave the loader's array in scratch memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head_dim
constexpr int kKT = 64;          // keys per tile
// Workgroups of W = 4 or 8 waves own 32 W (query, head) rows; 8 waves share each widened K/V tile
// among twice the rows, and are used when the chunks are long enough to fill 256-row tiles.
constexpr int kKStride = kD * 2 + 16;    // bytes per K row in LDS (the padding spreads banks)
constexpr int kVStride = kKT * 2 + 16;   // bytes per V^T row in LDS
constexpr int kKBytes = kKT * kKStride;
constexpr int kVBytes = kD * kVStride;
constexpr int kOStride = kD * 2 + 16;    // bytes per bf16 output row staged in LDS (8 waves x 32 rows fit the tiles)
static_assert(8 * 32 * kOStride <= 2 * (kKBytes + kVBytes), "output staging fits the tile buffers");
constexpr float kRescaleSlack = 8.0f;    // log2 of the largest unrescaled growth
constexpr int kMaxRanked = 64;           // sequences ordered by length when there are at most this many
constexpr int kMaxLdsTable = 16384;      // table entries the pipelined kernel holds in LDS (64 KiB)

// Inside each 16-key group of a V^T row, key k sits at LDS position k with bits 2 and 3 swapped:
// keys 0-3, 8-11 | 4-7, 12-15.  The P^T operand of lane half h holds keys 4h..4h+3 and 8+4h..8+4h+3
// of the group (the S^T accumulator layout), which are then the 8 contiguous positions 8h..8h+7.

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Combine of each lane with its partner lane ^ 32 through v_permlane32_swap (a VALU exchange, no LDS
// round trip): given x in both operands, the first result holds lanes 0-31's values in both halves
// and the second lanes 32-63's, so their max (sum) is the pair's max (sum) in every lane.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Global -> registers -> LDS for one 64-key tile.
//   K: 16-byte chunks of pool rows; chunk id = u * 256 + thread -> key id / CPR, chunk id % CPR.
//   V: 16-key pieces of a dim row; piece id = u * 256 + thread -> key group id / 128, dim id % 128.
// Both id orders keep each wave's loads of one instruction inside one pool block.
template <int KV, int BS, int W>
struct TileLoader {
  static constexpr int kThreads = 64 * W;
  static constexpr int kE = KV == kBF16 ? 2 : 1;
  static constexpr int kRowBytes = kD * kE;
  static constexpr int kCPR = kRowBytes / 16;           // K chunks per key row
  static constexpr int kKU = kKT * kCPR / kThreads;     // K chunks per thread (fp8 2, bf16 4)
  static constexpr int kVU = 4 * kD / kThreads;         // V pieces per thread (2)
  static constexpr int kVW = 16 * kE / 4;               // dwords of one 16-key piece (fp8 4, bf16 8)
  u32x4 k[kKU];
  uint32_t v[kVU][kVW];
  int max_blocks;    // entries of a table row: lookups stay inside it
  int pool_blocks;   // blocks of the pool: a table entry outside it is clamped into it (wrong result, no
                     // read outside the pool)
  __device__ __forceinline__ int64_t clamp_blk(int e) const { return min(max(e, 0), pool_blocks - 1); }

  // K or V of tile keys [key0, key0 + 64).  Every load is issued unconditionally, so that the only
  // wait for them is the one before the matching store; a block past the last one holding a key
  // < n_keys is read as that last block (its keys are masked: scores by the causal mask, values
  // zeroed in store_v()).
  __device__ __forceinline__ void load_k(const char* kpool, const int32_t* tab, int64_t blk_stride, int64_t head_off,
                                         int key0, int n_keys, int wave, int lane) {
    const int jlast = min((n_keys - 1) / BS, max_blocks - 1);
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      // keys of this wave's instruction: key0 + (u*256 + 64*wave) / CPR .. + 64/CPR (one block)
      const int kw = key0 + (u * kThreads + 64 * wave) / kCPR;
      const int key = key0 + (u * kThreads + 64 * wave + lane) / kCPR;
      const int ch = lane % kCPR;
      const int64_t phys = clamp_blk(tab[min(kw / BS, jlast)]);
      k[u] = *reinterpret_cast<const u32x4*>(kpool + phys * blk_stride + head_off +
                                             static_cast<int64_t>(key % BS) * kRowBytes + ch * 16);
    }
  }

  __device__ __forceinline__ void load_v(const char* vpool, const int32_t* tab, int64_t blk_stride, int64_t head_off,
                                         int key0, int n_keys, int wave, int lane) {
    const int jlast = min((n_keys - 1) / BS, max_blocks - 1);
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
      const int g16 = (W / 2) * u + (wave >> 1);              // 16-key group of the tile
      const int dim = 64 * (wave & 1) + lane;
      const int kg = key0 + 16 * g16;                   // first key of the group
      if constexpr (BS >= 16) {
        const int64_t phys = clamp_blk(tab[min(kg / BS, jlast)]);
        const char* row = vpool + phys * blk_stride + head_off + static_cast<int64_t>(dim) * BS * kE +
                          (kg % BS) * kE;
#pragma unroll
        for (int j = 0; j < kVW / 4; ++j) {
          const uint4 w = reinterpret_cast<const uint4*>(row)[j];
          v[u][4 * j] = w.x; v[u][4 * j + 1] = w.y; v[u][4 * j + 2] = w.z; v[u][4 * j + 3] = w.w;
        }
      } else {
        // two 8-key blocks
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int64_t phys = clamp_blk(tab[min(kg / 8 + hb, jlast)]);
          const char* row = vpool + phys * blk_stride + head_off + static_cast<int64_t>(dim) * 8 * kE;
          if constexpr (kE == 1) {
            const uint2 w = *reinterpret_cast<const uint2*>(row);
            v[u][2 * hb] = w.x; v[u][2 * hb + 1] = w.y;
          } else {
            const uint4 w = *reinterpret_cast<const uint4*>(row);
            v[u][4 * hb] = w.x; v[u][4 * hb + 1] = w.y; v[u][4 * hb + 2] = w.z; v[u][4 * hb + 3] = w.w;
          }
        }
      }
    }
  }

  // The loads above, split in two: fetch_*() reads the tile's physical block ids from a table (for
  // the pipelined kernel, its copy in LDS), load_*_fetched() issues the loads at those blocks.  A
  // caller fetches a few instructions before loading, so that the loads never wait on the table.
  static constexpr int kVB = BS >= 16 ? 1 : 2;          // blocks one 16-key V piece spans
  int pk[kKU];
  int pvb[kVU][kVB];
  __device__ __forceinline__ void fetch_k(const int32_t* tab, int key0, int n_keys, int wave) {
    const int jlast = min((n_keys - 1) / BS, max_blocks - 1);
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int kw = key0 + (u * kThreads + 64 * wave) / kCPR;
      pk[u] = tab[min(kw / BS, jlast)];
    }
  }
  __device__ __forceinline__ void fetch_v(const int32_t* tab, int key0, int n_keys, int wave) {
    const int jlast = min((n_keys - 1) / BS, max_blocks - 1);
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
      const int kg = key0 + 16 * ((W / 2) * u + (wave >> 1));
#pragma unroll
      for (int hb = 0; hb < kVB; ++hb) pvb[u][hb] = tab[min(kg / BS + hb, jlast)];
    }
  }
  __device__ __forceinline__ void load_k_fetched(const char* kpool, int64_t blk_stride, int64_t head_off, int key0,
                                                 int wave, int lane) {
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int key = key0 + (u * kThreads + 64 * wave + lane) / kCPR;
      const int ch = lane % kCPR;
      const int64_t phys = __builtin_amdgcn_readfirstlane(pk[u]);
      k[u] = *reinterpret_cast<const u32x4*>(kpool + phys * blk_stride + head_off +
                                             static_cast<int64_t>(key % BS) * kRowBytes + ch * 16);
    }
  }
  __device__ __forceinline__ void load_v_fetched(const char* vpool, int64_t blk_stride, int64_t head_off, int key0,
                                                 int wave, int lane) {
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
      const int g16 = (W / 2) * u + (wave >> 1);
      const int dim = 64 * (wave & 1) + lane;
      const int kg = key0 + 16 * g16;
      if constexpr (BS >= 16) {
        const int64_t phys = __builtin_amdgcn_readfirstlane(pvb[u][0]);
        const char* row = vpool + phys * blk_stride + head_off + static_cast<int64_t>(dim) * BS * kE +
                          (kg % BS) * kE;
#pragma unroll
        for (int j = 0; j < kVW / 4; ++j) {
          const uint4 w = reinterpret_cast<const uint4*>(row)[j];
          v[u][4 * j] = w.x; v[u][4 * j + 1] = w.y; v[u][4 * j + 2] = w.z; v[u][4 * j + 3] = w.w;
        }
      } else {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int64_t phys = __builtin_amdgcn_readfirstlane(pvb[u][hb]);
          const char* row = vpool + phys * blk_stride + head_off + static_cast<int64_t>(dim) * 8 * kE;
          if constexpr (kE == 1) {
            const uint2 w = *reinterpret_cast<const uint2*>(row);
            v[u][2 * hb] = w.x; v[u][2 * hb + 1] = w.y;
          } else {
            const uint4 w = *reinterpret_cast<const uint4*>(row);
            v[u][4 * hb] = w.x; v[u][4 * hb + 1] = w.y; v[u][4 * hb + 2] = w.z; v[u][4 * hb + 3] = w.w;
          }
        }
      }
    }
  }

  // K rows widened to bf16, [key][dim] with stride kKStride.
  __device__ __forceinline__ void store_k(char* ks, int wave, int lane) const {
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int id = u * kThreads + 64 * wave + lane;
      const int key = id / kCPR;
      const int ch = id % kCPR;
      char* dst = ks + key * kKStride;
      if constexpr (kE == 2) {
        *reinterpret_cast<u32x4*>(dst + ch * 16) = k[u];
      } else {
        const u32x4 c = k[u];
        *reinterpret_cast<uint4*>(dst + ch * 32) = make_uint4(fp8x2_lo(c.x), fp8x2_hi(c.x), fp8x2_lo(c.y), fp8x2_hi(c.y));
        *reinterpret_cast<uint4*>(dst + ch * 32 + 16) =
            make_uint4(fp8x2_lo(c.z), fp8x2_hi(c.z), fp8x2_lo(c.w), fp8x2_hi(c.w));
      }
    }
  }

  // store_v() with the masking of keys >= n_keys done by a scalar-computed mask per dword instead
  // of a branch (keys below n_keys keep every bit), so that a caller's instruction schedule is one
  // basic block.
  __device__ __forceinline__ void store_v_masked(char* vt, int key0, int n_keys, int wave, int lane) {
    constexpr int kPer = 4 / kE;   // elements per dword: fp8 4, bf16 2
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
      const int g16 = (W / 2) * u + (wave >> 1);
      // keys of the group below n_keys (wave-uniform: the masks are computed on the scalar unit)
      const int valid = __builtin_amdgcn_readfirstlane(n_keys - (key0 + 16 * g16));
#pragma unroll
      for (int m = 0; m < kVW; ++m) {
        const int nv = min(max(valid - kPer * m, 0), kPer);
        const uint32_t keep = nv >= kPer ? 0xffffffffu : ((1u << (8 * kE * nv)) - 1u);
        v[u][m] &= keep;
      }
    }
    store_v(vt, 0, 1 << 30, wave, lane);
  }

  // V^T rows widened to bf16, [dim][key position] with stride kVStride.  Values of keys >= n_keys
  // may hold any bits (even NaN, or another block's data): they are zeroed so that 0 * v stays 0.
  __device__ __forceinline__ void store_v(char* vt, int key0, int n_keys, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
      const int g16 = (W / 2) * u + (wave >> 1);
      const int dim = 64 * (wave & 1) + lane;
      const int valid = n_keys - (key0 + 16 * g16);      // keys of the group below n_keys
      if (valid < 16) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (e < valid) continue;
          if constexpr (kE == 1)
            v[u][e / 4] &= ~(0xffu << (8 * (e % 4)));
          else
            v[u][e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
      uint32_t d[8];   // bf16 pairs: d[m] = keys 2m, 2m+1 of the group
      if constexpr (kE == 2) {
#pragma unroll
        for (int m = 0; m < 8; ++m) d[m] = v[u][m];
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          d[2 * m] = fp8x2_lo(v[u][m]);
          d[2 * m + 1] = fp8x2_hi(v[u][m]);
        }
      }
      char* dst = vt + dim * kVStride + g16 * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[4], d[5]);        // keys 0-3, 8-11
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(d[2], d[3], d[6], d[7]);   // keys 4-7, 12-15
    }
  }
};

// The sequence a workgroup of rank r serves, with its chunk's first query row, chunk length and prior
// context.  With at most kMaxRanked sequences, rank 0 is the one with the most keys (ties by index):
// lane s loads sequence s's sizes once and the ranking compares registers across lanes, so the
// lookup is one round trip to memory.  Larger batches are served in index order.
struct SeqInfo {
  int seq, q_base, C, P;
};

__device__ __forceinline__ SeqInfo seq_info(const PrefillArgs& a, int r, int lane) {
  const int n = a.num_seqs;
  SeqInfo si;
  if (n <= kMaxRanked) {
    int q0 = 0, q1 = 0, pr = 0;
    if (lane < n) {
      q0 = a.qsl[lane];
      q1 = a.qsl[lane + 1];
      pr = a.prior[lane];
    }
    const int mine = lane < n ? pr + q1 - q0 : -1;
    int rank = 0;
    for (int s = 0; s < n; ++s) {
      const int other = __builtin_amdgcn_readlane(mine, s);
      rank += (other > mine) || (other == mine && s < lane);
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < n && rank == r);
    si.seq = hit ? static_cast<int>(__builtin_ctzll(hit)) : 0;
    si.q_base = __builtin_amdgcn_readlane(q0, si.seq);
    si.C = __builtin_amdgcn_readlane(q1, si.seq) - si.q_base;
    si.P = __builtin_amdgcn_readlane(pr, si.seq);
  } else {
    si.seq = r;
    si.q_base = a.qsl[r];
    si.C = a.qsl[r + 1] - si.q_base;
    si.P = a.prior[r];
  }
  return si;
}

template <int KV, int BS, int G, int W>
__global__ void __launch_bounds__(64 * W, W == 4 ? 2 : 1) prefill_kernel(PrefillArgs a, int out_bf16, int num_qtiles,
                                                              int xcd_remap) {
  constexpr int kRows = 32 * W;      // (query, head) rows per workgroup
  constexpr int QT = kRows / G;      // queries per workgroup
  __shared__ __attribute__((aligned(16))) char smem[2 * (kKBytes + kVBytes)];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- which (sequence, KV head, query tile) ----
  int rank, kvh, qt;
  if (xcd_remap) {
    // workgroup i runs on XCD i % 8; that XCD takes the KV heads congruent to it, so all query
    // tiles of one (sequence, KV head) share its L2
    const int x = blockIdx.x % 8;
    const int j = blockIdx.x / 8;
    qt = num_qtiles - 1 - j % num_qtiles;   // longest tiles first
    const int rr = j / num_qtiles;
    const int hpx = a.num_kv_heads / 8;
    rank = rr / hpx;
    kvh = (rr % hpx) * 8 + x;
  } else {
    qt = num_qtiles - 1 - blockIdx.x % num_qtiles;
    const int rr = blockIdx.x / num_qtiles;
    rank = rr / a.num_kv_heads;
    kvh = rr % a.num_kv_heads;
  }
  if (rank >= a.num_seqs) return;
  const SeqInfo si = seq_info(a, rank, lane);
  const int seq = si.seq, q_base = si.q_base, C = si.C, P = si.P;
  const int q0 = qt * QT;
  if (q0 >= C) return;
  const int q_end = min(q0 + QT, C);
  const int n_keys = P + q_end;
  const int n_tiles = (n_keys + kKT - 1) / kKT;

  const int h = lane >> 5;
  const int row = wave * 32 + (lane & 31);
  const int g = row / QT;
  const int qi = q0 + row % QT;
  const bool row_ok = qi < C;
  const int qpos = P + qi;
  const int head = kvh * G + g;

  // Q slice as the B operand: lane (row, h) holds dims 16c + 8h .. +8 of its query row
  bf16x8 qb[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(q_base + qi) * a.num_q_heads + head) * kD;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 w = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * c + 8 * h) : make_uint4(0, 0, 0, 0);
      qb[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  const int32_t* tab = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  constexpr int kTile = BS * TileLoader<KV, BS, W>::kRowBytes;   // bytes of one (block, head) tile
  const int64_t head_off = static_cast<int64_t>(kvh) * kTile;
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * kTile;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;   // running max (base-2 logits) of this row, the one the accumulators use
  float l_run = 0.f;
  const float c2 = a.qk_scale;

  // LDS: two K buffers and two V^T buffers.  Tile t's K sits in kbuf[t & 1], its V^T in vbuf[t & 1].
  char* const kbuf0 = smem;
  char* const kbuf1 = smem + kKBytes;
  char* const vbuf0 = smem + 2 * kKBytes;
  char* const vbuf1 = smem + 2 * kKBytes + kVBytes;
  const int last = n_tiles - 1;
  TileLoader<KV, BS, W> ld;
  ld.max_blocks = a.max_blocks;
  ld.pool_blocks = a.num_blocks;

  // S^T = K Q^T of the tile whose K rows are in kb, as two 32-key halves.
  auto scores = [&](const char* kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
      const char* krow = kb + (sb * 32 + (lane & 31)) * kKStride + 16 * h;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 32 * c);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[c], s[sb], 0, 0, 0);
      }
    }
  };

  // Software pipeline.  On entry to step t: sc = S(t); K(t + 1) and V(t) are in LDS; the registers
  // hold V(t + 1) and K(t + 2) (loaded, or in flight).  Step t
  //   1. masks tile t (tiles crossing the diagonal only), takes its max, rescales if needed;
  //   2. issues the MFMAs of S(t + 1) into sn beside the exponentials of tile t, then stores V(t + 1)
  //      into vbuf[(t + 1) & 1] and issues the loads of V(t + 2);
  //   3. issues O += V(t) P(t) beside the store of K(t + 2) into kbuf[t & 1] (K(t) is done) and the
  //      loads of K(t + 3);
  //   4. waits at the barrier, after which every buffer written in 2 and 3 is visible and every
  //      buffer read in 2 and 3 may be overwritten.
  // Tiles past the last one are read as the last one (their results are unused).
  auto step = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
    const bool odd = t & 1;
    const int key_base = t * kKT;
    if (key_base + kKT - 1 > P + q0) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key_base + sb * 32 + 8 * (r / 4) + 4 * h + (r % 4);
          sc[sb][r] = key <= qpos ? sc[sb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[sb][r]);
    mx = half_max(mx) * c2;     // base-2 logit units (c2 > 0)
    // rescale only when the max moved by more than the slack (wave-uniform decision)
    const bool grow = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;

    scores(odd ? kbuf0 : kbuf1, sn);
    bf16x8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // the row sum adds the bf16-rounded probability that the P.V product uses
        const __bf16 p = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[c / 2][8 * (c % 2) + e], c2, nm)));
        lsum += static_cast<float>(p);
        pb[c][e] = p;
      }
    l_run += half_sum(lsum);
    ld.store_v(odd ? vbuf0 : vbuf1, min(t + 1, last) * kKT, n_keys, wave, lane);
    ld.load_v(vpool, tab, blk_stride, head_off, min(t + 2, last) * kKT, n_keys, wave, lane);

#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const char* vrow = (odd ? vbuf1 : vbuf0) + (dt * 32 + (lane & 31)) * kVStride + 16 * h;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrow + 32 * c);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], o[dt], 0, 0, 0);
      }
    }
    ld.store_k(odd ? kbuf1 : kbuf0, wave, lane);
    ld.load_k(kpool, tab, blk_stride, head_off, min(t + 3, last) * kKT, n_keys, wave, lane);
    __syncthreads();
  };

  // Prologue: K(0), V(0) to LDS; S(0); K(1) to LDS; V(1) and K(2) left in registers.
  ld.load_k(kpool, tab, blk_stride, head_off, 0, n_keys, wave, lane);
  ld.load_v(vpool, tab, blk_stride, head_off, 0, n_keys, wave, lane);
  ld.store_k(kbuf0, wave, lane);
  ld.store_v(vbuf0, 0, n_keys, wave, lane);
  ld.load_k(kpool, tab, blk_stride, head_off, min(1, last) * kKT, n_keys, wave, lane);
  ld.load_v(vpool, tab, blk_stride, head_off, min(1, last) * kKT, n_keys, wave, lane);
  __syncthreads();
  f32x16 sa[2], sb2[2];
  scores(kbuf0, sa);
  ld.store_k(kbuf1, wave, lane);
  ld.load_k(kpool, tab, blk_stride, head_off, min(2, last) * kKT, n_keys, wave, lane);
  __syncthreads();

  // Two steps per trip so that the score arrays trade roles without register copies.
  int t = 0;
#pragma unroll 1
  for (; t + 1 < n_tiles; t += 2) {
    step(t, sa, sb2);
    step(t + 1, sb2, sa);
  }
  if (t < n_tiles) step(t, sa, sb2);

  // ---- out[token][head][d] = O^T[d][row] / l ----
  if (!row_ok) return;
  const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
  const int64_t obase = (static_cast<int64_t>(q_base + qi) * a.num_q_heads + head) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = dt * 32 + 8 * rr + 4 * h;
      const float x0 = o[dt][4 * rr] * inv, x1 = o[dt][4 * rr + 1] * inv;
      const float x2 = o[dt][4 * rr + 2] * inv, x3 = o[dt][4 * rr + 3] * inv;
      if (out_bf16) {
        uint16_t* op = static_cast<uint16_t*>(a.out) + obase + d;
        *reinterpret_cast<uint2*>(op) = make_uint2(f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16),
                                                   f32_to_bf16_bits(x2) | (f32_to_bf16_bits(x3) << 16));
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + d) = make_float4(x0, x1, x2, x3);
      }
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
// a + b + c of a packed bf16 pair and an fp32 sum (one v_dot2c against (1, 1))
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// The 8-wave kernel as one balanced software pipeline.  Step t of a workgroup issues 32 MFMAs, each
// in a chunk of its own: even chunks the products O^T += V^T(t - 1) P^T(t - 1) (the probabilities
// of the previous tile), odd chunks S^T(t + 1) = K(t + 1) Q^T (the scores of the next one).  Beside
// each MFMA a wave computes one probability of tile t (an fma and an exp2; every second one also
// packs the pair to bf16 and adds it to the row sum with a bf16 dot), so that every MFMA of a wave
// has about as much vector work beside it as the MFMA itself takes (MI355X issues 32 x 32 x 16 bf16
// MFMAs every 32 cycles per SIMD; an exp2 takes 8 cycles of the vector unit, an fma 2).  LDS
// fragments are read kAhead chunks before their MFMA; the tile loads and LDS stores sit in the
// first chunks; one barrier ends the step.
//
// Probabilities are exp2(c2 s - m) against the row's reference max m, with no per-tile max: a lane
// whose 32 probabilities of the tile sum above 2^8 (so one may exceed 2^8), or to NaN, sends its wave
// to a rare path that takes the tile's true row max, rescales O and the sums to it and recomputes the
// tile.  The row sum adds the bf16-rounded probabilities that the P.V product uses.
template <int KV, int BS, int G, int W>
__global__ void __launch_bounds__(64 * W, 1) prefill_pipe_kernel(PrefillArgs a, int out_bf16, int num_qtiles,
                                                                 int xcd_remap) {
  constexpr int kRows = 32 * W;      // (query, head) rows per workgroup
  constexpr int QT = kRows / G;      // queries per workgroup
  constexpr int kAhead = 3;          // chunks between an LDS fragment read and its MFMA
  constexpr float kSumBound = 256.f;
  __shared__ __attribute__((aligned(16))) char smem[2 * (kKBytes + kVBytes)];
  extern __shared__ int32_t tab_s[];   // the sequence's block-table row (dynamic, max_blocks entries)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Lane s of every wave holds sequence s's chunk start, chunk end, prior context and, for a batch
  // of at most kMaxRanked sequences, its rank by key count (0 = most keys, ties by index): one round
  // trip to memory for the whole workgroup, and each item's lookup is then register-only.
  const int n_seqs = a.num_seqs;
  const bool ranked = n_seqs <= kMaxRanked;
  int s_q0 = 0, s_q1 = 0, s_pr = 0, s_rank = -1;
  if (ranked) {
    if (lane < n_seqs) {
      s_q0 = a.qsl[lane];
      s_q1 = a.qsl[lane + 1];
      s_pr = a.prior[lane];
    }
    const int mine = lane < n_seqs ? s_pr + s_q1 - s_q0 : -1;
    int rk = 0;
    for (int s2 = 0; s2 < n_seqs; ++s2) {
      const int other = __builtin_amdgcn_readlane(mine, s2);
      rk += (other > mine) || (other == mine && s2 < lane);
    }
    s_rank = lane < n_seqs ? rk : -1;
  }
  // The item list (rank, KV head, query tile), ranks in order and the longest query tile first: with
  // the XCD remap, workgroup i serves the KV heads congruent to i % 8 (the XCD it runs on), so the
  // items of one (sequence, KV head) share that XCD's L2.  The nb workgroups of a list take its
  // items in snake order: round R gives item R nb + b to workgroup b (R even) or to nb - 1 - b (R
  // odd), which evens out the decreasing sizes along the list without any shared counter.
  const int xq = xcd_remap ? static_cast<int>(blockIdx.x % 8) : 0;
  const int nb = xcd_remap ? static_cast<int>(gridDim.x / 8) : static_cast<int>(gridDim.x);
  const int wb = xcd_remap ? static_cast<int>(blockIdx.x / 8) : static_cast<int>(blockIdx.x);
  const int heads = xcd_remap ? a.num_kv_heads / 8 : a.num_kv_heads;
  const int64_t n_items = static_cast<int64_t>(n_seqs) * heads * num_qtiles;

#pragma unroll 1
  for (int R = 0;; ++R) {
  const int64_t item = static_cast<int64_t>(R) * nb + ((R & 1) ? nb - 1 - wb : wb);
  if (item >= n_items) break;
  const int qt = num_qtiles - 1 - static_cast<int>(item % num_qtiles);
  const int64_t grp = item / num_qtiles;   // (rank, KV head of the list)
  const int rank = static_cast<int>(grp / heads);
  const int kvh = xcd_remap ? static_cast<int>(grp % heads) * 8 + xq : static_cast<int>(grp % heads);
  int seq, q_base, C, P;
  if (ranked) {
    const uint64_t hit = __builtin_amdgcn_ballot_w64(s_rank == rank);
    seq = hit ? static_cast<int>(__builtin_ctzll(hit)) : 0;
    q_base = __builtin_amdgcn_readlane(s_q0, seq);
    C = __builtin_amdgcn_readlane(s_q1, seq) - q_base;
    P = __builtin_amdgcn_readlane(s_pr, seq);
  } else {
    seq = rank;
    q_base = a.qsl[rank];
    C = a.qsl[rank + 1] - q_base;
    P = a.prior[rank];
  }
  const int q0 = qt * QT;
  if (q0 >= C) continue;
  const int q_end = min(q0 + QT, C);
  const int n_keys = P + q_end;
  const int n_tiles = (n_keys + kKT - 1) / kKT;

  const int h = lane >> 5;
  const int row = wave * 32 + (lane & 31);
  const int g = row / QT;
  const int qi = q0 + row % QT;
  const bool row_ok = qi < C;
  const int qpos = P + qi;
  const int head = kvh * G + g;

  bf16x8 qb[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(q_base + qi) * a.num_q_heads + head) * kD;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 w = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * c + 8 * h) : make_uint4(0, 0, 0, 0);
      qb[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  constexpr int kTile = BS * TileLoader<KV, BS, W>::kRowBytes;
  const int64_t head_off = static_cast<int64_t>(kvh) * kTile;
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * kTile;
  {
    // the table entries of this workgroup's keys, into LDS (ready after the prologue's first barrier)
    const int32_t* tab_g = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    const int nblk = min((n_keys + BS - 1) / BS, a.max_blocks);
    for (int i = threadIdx.x; i < nblk; i += 64 * W) tab_s[i] = min(max(tab_g[i], 0), a.num_blocks - 1);
  }
  const int32_t* const tab = tab_s;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;   // reference max (base-2 logits) of this row
  float l_lane = 0.f;        // this lane's share of the row's probability sum (its half of the keys)
  const float c2 = a.qk_scale;

  char* const kbuf0 = smem;
  char* const kbuf1 = smem + kKBytes;
  char* const vbuf0 = smem + 2 * kKBytes;
  char* const vbuf1 = smem + 2 * kKBytes + kVBytes;
  const int last = n_tiles - 1;
  TileLoader<KV, BS, W> ld;
  ld.max_blocks = a.max_blocks;
  ld.pool_blocks = a.num_blocks;

  // One step; on entry: sc = S(t); pp = P(t - 1) (bf16 pairs); LDS holds K(t + 1) and V(t - 1);
  // the register stage holds K(t + 2) and V(t).
  auto step = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2], uint32_t (&pp)[4][4], uint32_t (&pn)[4][4])
      __attribute__((always_inline)) {
    const bool odd = t & 1;
    const char* const kread = odd ? kbuf0 : kbuf1;     // K(t + 1)
    const char* const vread = odd ? vbuf0 : vbuf1;     // V(t - 1)
    char* const kwrite = odd ? kbuf1 : kbuf0;          // K(t + 2) replaces K(t)
    char* const vwrite = odd ? vbuf1 : vbuf0;          // V(t) replaces V(t - 2)
    const int key_base = t * kKT;
    if (key_base + kKT - 1 > P + q0) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key_base + sb * 32 + 8 * (r / 4) + 4 * h + (r % 4);
          sc[sb][r] = key <= qpos ? sc[sb][r] : -INFINITY;
        }
    }
    const float nm = -m_run;
    float lsum2[2] = {0.f, 0.f};   // two accumulators halve the dependent chain of row-sum dots
    bf16x8 frag[32];
    // MFMA order: even chunks the O products (dt, c) with dt fastest, odd chunks the S products
    // (sb, c) with sb fastest, so an accumulator recurs only every 8 (O) or 4 (S) chunks
    auto read_frag = [&](int i) __attribute__((always_inline)) {
      const int k = i >> 1;
      const char* src = (i & 1) ? kread + ((k & 1) * 32 + (lane & 31)) * kKStride + 16 * h + 32 * (k >> 1)
                                : vread + ((k & 3) * 32 + (lane & 31)) * kVStride + 16 * h + 32 * (k >> 2);
      frag[i] = *reinterpret_cast<const bf16x8*>(src);
    };
    // score j of tile t: P^T operand c = j / 8, element e = j % 8
    auto score = [&](int j) __attribute__((always_inline)) {
      const int c = j >> 3, e = j & 7;
      return sc[c >> 1][8 * (c & 1) + e];
    };
    float x[32], pr[32];
    uint32_t wp[16];
    x[0] = __builtin_fmaf(score(0), c2, nm);
#pragma unroll
    for (int i = 0; i < kAhead; ++i) read_frag(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + kAhead < 32) read_frag(i + kAhead);
      const int k = i >> 1;
      if (i & 1) {
        const int sb = k & 1, c = k >> 1;
        if (c == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          sn[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[i], qb[c], z, 0, 0, 0);
        } else {
          sn[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[i], qb[c], sn[sb], 0, 0, 0);
        }
      } else {
        const int dt = k & 3, c = k >> 2;
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            frag[i], as_bf16x8(pp[c][0], pp[c][1], pp[c][2], pp[c][3]), o[dt], 0, 0, 0);
      }
      // softmax of tile t, lagged so that no instruction waits on the one before it: the logit of
      // score i + 1, the probability of score i, the bf16 pair of scores i - 4, i - 3, and the row
      // sum of the pair packed two chunks earlier
      if (i + 1 < 32) x[i + 1] = __builtin_fmaf(score(i + 1), c2, nm);
      pr[i] = __builtin_amdgcn_exp2f(x[i]);
      if (i >= 4 && ((i - 3) & 1)) {
        const int jp = i - 3;
        wp[jp >> 1] = pack_bf16(pr[jp - 1], pr[jp]);
        pn[jp >> 3][(jp & 7) >> 1] = wp[jp >> 1];
      }
      if (i >= 6 && ((i - 5) & 1)) {
        const int jd = i - 5;
        lsum2[(jd >> 1) & 1] = add_pair(wp[jd >> 1], lsum2[(jd >> 1) & 1]);
      }
      if (i == 0) ld.fetch_v(tab, min(t + 1, last) * kKT, n_keys, wave);
      if (i == 1) ld.fetch_k(tab, min(t + 3, last) * kKT, n_keys, wave);
      if (i == 4) ld.store_v_masked(vwrite, t * kKT, n_keys, wave, lane);
      if (i == 5) ld.load_v_fetched(vpool, blk_stride, head_off, min(t + 1, last) * kKT, wave, lane);
      if (i == 8) ld.store_k(kwrite, wave, lane);
      if (i == 9) ld.load_k_fetched(kpool, blk_stride, head_off, min(t + 3, last) * kKT, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the pairs and sums the lag left: pairs (28, 29), (30, 31); sums of pairs 13, 14, 15
#pragma unroll
    for (int jp = 29; jp < 32; jp += 2) {
      wp[jp >> 1] = pack_bf16(pr[jp - 1], pr[jp]);
      pn[jp >> 3][(jp & 7) >> 1] = wp[jp >> 1];
    }
#pragma unroll
    for (int jd = 27; jd < 32; jd += 2) lsum2[(jd >> 1) & 1] = add_pair(wp[jd >> 1], lsum2[(jd >> 1) & 1]);
    float lsum = lsum2[0] + lsum2[1];
    if (__builtin_amdgcn_ballot_w64(row_ok && !(lsum <= kSumBound)) != 0) {
      // the tile's true row max; rescale everything accumulated so far to it and recompute the tile
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[sb][r]);
      mx = half_max(mx) * c2;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      const float nm2 = m_new == -INFINITY ? 0.f : -m_new;
      lsum = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c >> 1][8 * (c & 1) + e], c2, nm2));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c >> 1][8 * (c & 1) + e + 1], c2, nm2));
          const uint32_t w = pack_bf16(p0, p1);
          pn[c][e >> 1] = w;
          lsum = add_pair(w, lsum);
        }
    }
    l_lane += lsum;
    __syncthreads();
  };

  // Prologue: S(0) from K(0); K(1) in kbuf1; V(-1) = zeros in vbuf1 with P(-1) = 0 (O(-1) adds 0);
  // the register stage then holds K(2) and V(0).  K(0), V(0) and K(1) are loaded together (K(1)
  // through a second register stage), then K(2), so the prologue waits on memory twice.
  __syncthreads();   // the table in LDS
  {
    TileLoader<KV, BS, W> ld1;
    ld1.max_blocks = a.max_blocks;
    ld1.pool_blocks = a.num_blocks;
    ld.load_k(kpool, tab, blk_stride, head_off, 0, n_keys, wave, lane);
    ld.load_v(vpool, tab, blk_stride, head_off, 0, n_keys, wave, lane);
    ld1.load_k(kpool, tab, blk_stride, head_off, min(1, last) * kKT, n_keys, wave, lane);
    for (int i = threadIdx.x; i < kVBytes / 16; i += 64 * W)
      reinterpret_cast<uint4*>(vbuf1)[i] = make_uint4(0, 0, 0, 0);
    ld.store_k(kbuf0, wave, lane);
    ld.load_k(kpool, tab, blk_stride, head_off, min(2, last) * kKT, n_keys, wave, lane);
    ld1.store_k(kbuf1, wave, lane);
  }
  __syncthreads();
  f32x16 sa[2], sb2[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[sb][r] = 0.f;
    const char* krow = kbuf0 + (sb * 32 + (lane & 31)) * kKStride + 16 * h;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      sa[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(krow + 32 * c), qb[c],
                                                       sa[sb], 0, 0, 0);
  }
  __syncthreads();   // every wave's S(0) has read kbuf0 before the first step overwrites it

  uint32_t pA[4][4], pB[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) pA[c][w] = 0u;
  int t = 0;
#pragma unroll 1
  for (; t + 1 < n_tiles; t += 2) {
    step(t, sa, sb2, pA, pB);
    step(t + 1, sb2, sa, pB, pA);
  }
  // V(last) was stored into vbuf[last & 1] by the last step
  const char* const vlast = (last & 1) ? vbuf1 : vbuf0;
  if (t < n_tiles) {
    step(t, sa, sb2, pA, pB);
    // the last tile's O products: P(last) in pB
    const char* vread = vlast;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const char* vrow = vread + (dt * 32 + (lane & 31)) * kVStride + 16 * h;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(vrow + 32 * c),
                                                        as_bf16x8(pB[c][0], pB[c][1], pB[c][2], pB[c][3]), o[dt],
                                                        0, 0, 0);
    }
  } else {
    const char* vread = vlast;                       // P(last) in pA
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const char* vrow = vread + (dt * 32 + (lane & 31)) * kVStride + 16 * h;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(vrow + 32 * c),
                                                        as_bf16x8(pA[c][0], pA[c][1], pA[c][2], pA[c][3]), o[dt],
                                                        0, 0, 0);
    }
  }

  const float l = half_sum(l_lane);
  const float inv = l > 0.f ? a.v_scale / l : 0.f;
  if (out_bf16) {
    // bf16 rows leave through LDS so that every store writes whole rows: wave w stages its 32 rows
    // [row][dim] (stride kOStride) in its own slice of the tile buffers, once every wave's last
    // products have read them, and stores 4 rows x 256 B per instruction.
    __syncthreads();
    char* const ost = smem + wave * (32 * kOStride);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = dt * 32 + 8 * rr + 4 * h;
        *reinterpret_cast<uint2*>(ost + (lane & 31) * kOStride + 2 * d) =
            make_uint2(f32_to_bf16_bits(o[dt][4 * rr] * inv) | (f32_to_bf16_bits(o[dt][4 * rr + 1] * inv) << 16),
                       f32_to_bf16_bits(o[dt][4 * rr + 2] * inv) | (f32_to_bf16_bits(o[dt][4 * rr + 3] * inv) << 16));
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wr = 4 * j + (lane >> 4);            // row of the wave
      const int srow = wave * 32 + wr;
      const int sq = q0 + srow % QT;
      const uint4 w = *reinterpret_cast<const uint4*>(ost + wr * kOStride + 16 * (lane & 15));
      if (sq < C) {
        uint16_t* op = static_cast<uint16_t*>(a.out) +
                       (static_cast<int64_t>(q_base + sq) * a.num_q_heads + kvh * G + srow / QT) * kD;
        *reinterpret_cast<uint4*>(op + 8 * (lane & 15)) = w;
      }
    }
  } else if (row_ok) {
    const int64_t obase = (static_cast<int64_t>(q_base + qi) * a.num_q_heads + head) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = dt * 32 + 8 * rr + 4 * h;
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + d) =
            make_float4(o[dt][4 * rr] * inv, o[dt][4 * rr + 1] * inv, o[dt][4 * rr + 2] * inv,
                        o[dt][4 * rr + 3] * inv);
      }
  }
  }   // items
}

template <int KV, int BS, int G, int W>
int launch_g(const PrefillArgs& a, int out_bf16, hipStream_t s) {
  constexpr int QT = 32 * W / G;
  const int num_qtiles = (a.max_chunk + QT - 1) / QT;
  const int64_t groups = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int xcd_remap = a.num_kv_heads % 8 == 0;
  const int64_t wgs = groups * num_qtiles;
  if (wgs > 0x7fffffff) return -1;
  // The pipelined kernel keeps the sequence's table row in LDS beside its 70 KiB of tiles; rows
  // longer than kMaxLdsTable entries take the kernel that reads the table from memory.
  const size_t tab_bytes = (static_cast<size_t>(a.max_blocks) * 4 + 15) / 16 * 16;
  // 8-wave tiles only: with 4 waves the pipelined kernel measured 4% slower on the mixed fp8 step,
  // and its bf16 instances spill.
  if constexpr (W == 8) {
    if (a.max_blocks <= kMaxLdsTable) {
      constexpr int kMaxDevices = 64;
      static bool attr_set[kMaxDevices] = {};
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return static_cast<int>(e);
      if (dev < 0 || dev >= kMaxDevices || !attr_set[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_pipe_kernel<KV, BS, G, W>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsTable * 4);
        if (e != hipSuccess) return static_cast<int>(e);
        if (dev >= 0 && dev < kMaxDevices) attr_set[dev] = true;
      }
      // persistent: one workgroup per compute unit (what the registers allow), each walking its
      // share of the item list; never more workgroups than items
      const int64_t cus = device_cus();
      int64_t grid;
      if (xcd_remap) {
        const int64_t per_list = static_cast<int64_t>(a.num_seqs) * (a.num_kv_heads / 8) * num_qtiles;
        grid = 8 * std::max<int64_t>(1, std::min<int64_t>(cus / 8, per_list));
      } else {
        grid = std::max<int64_t>(1, std::min<int64_t>(cus, wgs));
      }
      hipLaunchKernelGGL((prefill_pipe_kernel<KV, BS, G, W>), dim3(static_cast<unsigned>(grid)), dim3(64 * W),
                         tab_bytes, s, a, out_bf16, num_qtiles, xcd_remap);
      return static_cast<int>(hipGetLastError());
    }
  }
  hipLaunchKernelGGL((prefill_kernel<KV, BS, G, W>), dim3(static_cast<unsigned>(wgs)), dim3(64 * W), 0, s, a,
                     out_bf16, num_qtiles, xcd_remap);
  return static_cast<int>(hipGetLastError());
}

template <int KV, int BS, int W>
int launch_w(const PrefillArgs& a, int out_bf16, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<KV, BS, 1, W>(a, out_bf16, s);
    case 2: return launch_g<KV, BS, 2, W>(a, out_bf16, s);
    case 4: return launch_g<KV, BS, 4, W>(a, out_bf16, s);
    case 8: return launch_g<KV, BS, 8, W>(a, out_bf16, s);
    default: return -1;
  }
}

// 256-row tiles (8 waves) when the longest chunk fills at least four of them, else 128-row tiles:
// 8 waves measured 3% faster on 512-query chunks of 4-head groups, but short chunks would leave
// more of a 256-row tile masked.
template <int KV, int BS>
int launch_bs(const PrefillArgs& a, int out_bf16, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.max_chunk) * (a.num_q_heads / a.num_kv_heads);
  return rows >= 1024 ? launch_w<KV, BS, 8>(a, out_bf16, s) : launch_w<KV, BS, 4>(a, out_bf16, s);
}

template <int KV>
int launch_kv(const PrefillArgs& a, int bs, int out_bf16, hipStream_t s) {
  switch (bs) {
    case 8: return launch_bs<KV, 8>(a, out_bf16, s);
    case 16: return launch_bs<KV, 16>(a, out_bf16, s);
    case 32: return launch_bs<KV, 32>(a, out_bf16, s);
    default: return -1;
  }
}

}  // namespace

int launch_prefill(const PrefillArgs& a, int kv_dtype, int out_dtype, int block_size, int head_dim,
                   void* stream) {
  if (head_dim != kD) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ob = out_dtype == kBF16;
  if (kv_dtype == kBF16) return launch_kv<kBF16>(a, block_size, ob, s);
  if (kv_dtype == kFP8) return launch_kv<kFP8>(a, block_size, ob, s);
  return -1;
}

}  // namespace pa
