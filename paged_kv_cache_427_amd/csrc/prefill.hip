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
constexpr float kRescaleSlack = 8.0f;    // log2 of the largest unrescaled growth
constexpr int kMaxRanked = 64;           // sequences ordered by length when there are at most this many

// Inside each 16-key group of a V^T row, key k sits at LDS position k with bits 2 and 3 swapped:
// keys 0-3, 8-11 | 4-7, 12-15.  The P^T operand of lane half h holds keys 4h..4h+3 and 8+4h..8+4h+3
// of the group (the S^T accumulator layout), which are then the 8 contiguous positions 8h..8h+7.

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

  // K or V of tile keys [key0, key0 + 64).  Every load is issued unconditionally, so that the only
  // wait for them is the one before the matching store; a block past the last one holding a key
  // < n_keys is read as that last block (its keys are masked: scores by the causal mask, values
  // zeroed in store_v()).
  __device__ __forceinline__ void load_k(const char* kpool, const int32_t* tab, int64_t blk_stride, int64_t head_off,
                                         int key0, int n_keys, int wave, int lane) {
    const int jlast = (n_keys - 1) / BS;
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      // keys of this wave's instruction: key0 + (u*256 + 64*wave) / CPR .. + 64/CPR (one block)
      const int kw = key0 + (u * kThreads + 64 * wave) / kCPR;
      const int key = key0 + (u * kThreads + 64 * wave + lane) / kCPR;
      const int ch = lane % kCPR;
      const int64_t phys = tab[min(kw / BS, jlast)];
      k[u] = *reinterpret_cast<const u32x4*>(kpool + phys * blk_stride + head_off +
                                             static_cast<int64_t>(key % BS) * kRowBytes + ch * 16);
    }
  }

  __device__ __forceinline__ void load_v(const char* vpool, const int32_t* tab, int64_t blk_stride, int64_t head_off,
                                         int key0, int n_keys, int wave, int lane) {
    const int jlast = (n_keys - 1) / BS;
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
      const int g16 = (W / 2) * u + (wave >> 1);              // 16-key group of the tile
      const int dim = 64 * (wave & 1) + lane;
      const int kg = key0 + 16 * g16;                   // first key of the group
      if constexpr (BS >= 16) {
        const int64_t phys = tab[min(kg / BS, jlast)];
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
          const int64_t phys = tab[min(kg / 8 + hb, jlast)];
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

// Sequence of length rank r (0 = most keys; ties by index), for num_seqs <= kMaxRanked.  Every wave
// computes it on its own: lane s ranks sequence s against all others.
__device__ __forceinline__ int seq_of_rank(const PrefillArgs& a, int r, int lane) {
  const int n = a.num_seqs;
  int mine = -1;
  if (lane < n) mine = a.prior[lane] + a.qsl[lane + 1] - a.qsl[lane];
  int rank = 0;
  for (int s = 0; s < n; ++s) {
    const int other = a.prior[s] + a.qsl[s + 1] - a.qsl[s];
    rank += (other > mine) || (other == mine && s < lane);
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < n && rank == r);
  return hit ? static_cast<int>(__builtin_ctzll(hit)) : 0;
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
  const int seq = a.num_seqs <= kMaxRanked ? seq_of_rank(a, rank, lane) : rank;
  const int q_base = a.qsl[seq];
  const int C = a.qsl[seq + 1] - q_base;
  const int q0 = qt * QT;
  if (q0 >= C) return;
  const int P = a.prior[seq];
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
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c / 2][8 * (c % 2) + e], c2, nm));
        lsum += p;
        pb[c][e] = static_cast<__bf16>(p);
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

template <int KV, int BS, int G, int W>
int launch_g(const PrefillArgs& a, int out_bf16, hipStream_t s) {
  constexpr int QT = 32 * W / G;
  const int num_qtiles = (a.max_chunk + QT - 1) / QT;
  const int64_t groups = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int xcd_remap = a.num_kv_heads % 8 == 0;
  const int64_t wgs = groups * num_qtiles;
  if (wgs > 0x7fffffff) return -1;
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
