// Paged decode attention for gfx950: one query token per sequence over its block-table-mapped K/V.
//
// «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» §三 3.1-3.2: the kernel gets
// the sequence's scattered K/V through its block table -- one indirection per block, contiguous
// coalesced reads inside it -- and dots the query with every cached key; §七 notes the indirection
// costs a little.  softmax(scale * q K^T) V is the textbook form of what the pages describe in words.
//
// Design (HBM-bound: at most 8 flop per byte of K/V, far below the MI355X ridge):
//  * one workgroup of 4 wave64s owns one context partition of one KV head and serves all G query
//    heads of that group, so each K/V byte is read once.  Workgroups are numbered so that all work
//    of one KV head lands on one XCD (dispatch is round-robin over the 8 XCDs): blocks shared by
//    many sequences (a common prefix) are then re-read from that XCD's L2, not from HBM.
//  * waves take the partition's blocks round-robin; the table entry is a wave-uniform scalar load.
//  * a block tile (block_size rows x head_dim) is read with 16-byte loads in which every group of NL
//    lanes covers 16*NL contiguous bytes of one token row (whole 128-byte lines); the next block's
//    K/V is in flight while the current one is consumed (two register stages, unrolled by two).
//  * bf16 and fp8 pools: q.k and p.v run on packed bf16 dot products (v_dot2_f32_bf16, fp32
//    accumulation); fp8 codes widen exactly to bf16.  The probabilities fed to p.v are rounded to
//    bf16, and the running sum uses the same rounded values, as MFMA attention kernels do.
//    fp32 pools keep exact fp32 FMAs.
//  * logits are reduced over the NL lanes of a row with DPP; every lane keeps its own running max,
//    exp-sum and output partial (base-2 online softmax) for the tokens it saw.  The running max is
//    raised only when a logit exceeds it by more than 2^8 (so exp stays <= 256), which makes the
//    rescale of the accumulators rare.  Lanes, then waves (through LDS), merge once per partition.
//  * a sequence with several partitions writes (max, sum, normalised partial) per partition and a
//    second kernel merges them; a single-partition sequence writes its output directly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kSlack = 8.0f;   // log2 of the growth allowed before the accumulators are rescaled

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
  // packed bf16 pairs: pair i = elements (2i, 2i+1)
  __device__ static void pairs(const uint4& c, uint32_t* p) {
    p[0] = c.x; p[1] = c.y; p[2] = c.z; p[3] = c.w;
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
  __device__ static void pairs(const uint4& c, uint32_t* p) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
      p[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    }
  }
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Partner value across lanes `MASK` apart (lane ^ MASK).
template <int MASK>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (MASK == 8) {
    return dpp<0x128>(x);               // row_ror:8 -- lane i <- lane i+8 within each 16
  } else {
    return shfl_xor(x, MASK);
  }
}

// Per-lane running state and one block's worth of work.
template <int KV, int D, int BS, int G>
struct DecodeLane {
  using Gm = Geo<KV, D, BS>;
  static constexpr int NL = Gm::kNL, TPI = Gm::kTPI, TG = Gm::kTG, CPL = Gm::kCPL, EPC = Gm::kEPC,
                       DL = Gm::kDL, ROW = Gm::kRow;
  static constexpr bool kPacked = KV != kF32;
  static constexpr int PPC = EPC / 2;                 // bf16 pairs per chunk (packed path)

  float qf[G][kPacked ? 1 : DL];                      // fp32 path: q * scale
  uint32_t qp[G][kPacked ? CPL * PPC : 1];            // packed path: raw bf16 pairs of q
  float m[G], l[G], acc[G][DL];

  __device__ __forceinline__ void consume(uint4 (&kc)[TG][CPL], uint4 (&vc)[TG][CPL], int row0, int t1,
                                          int tokset, float qk_scale) {
    // ---- logits of this lane's rows, reduced over the NL lanes that share each row ----
    float s[G][TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
      for (int g = 0; g < G; ++g) s[g][tg] = 0.f;
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr) {
        if constexpr (kPacked) {
          uint32_t kp[PPC];
          KvChunk<KV>::pairs(kc[tg][cr], kp);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < PPC; ++i) s[g][tg] = dot2(qp[g][cr * PPC + i], kp[i], s[g][tg]);
        } else {
          float kf[EPC];
          KvChunk<KV>::cvt(kc[tg][cr], kf);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPC; ++e) s[g][tg] = fmaf(qf[g][cr * EPC + e], kf[e], s[g][tg]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s[g][tg] = group_sum<NL>(s[g][tg]);
        if constexpr (kPacked) s[g][tg] *= qk_scale;
      }
    }
    // ---- rows past the partition end (only in its last block): -inf logits, zero values ----
    if (row0 + BS > t1) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const bool ok = row0 + tg * TPI + tokset < t1;
#pragma unroll
        for (int g = 0; g < G; ++g) s[g][tg] = ok ? s[g][tg] : -INFINITY;
#pragma unroll
        for (int cr = 0; cr < CPL; ++cr)
          if (!ok) vc[tg][cr] = make_uint4(0, 0, 0, 0);
      }
    }
    // ---- running max: raised only when a logit exceeds it by more than the slack ----
    bool grow = false;
    float mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mx[g] = s[g][0];
#pragma unroll
      for (int tg = 1; tg < TG; ++tg) mx[g] = fmaxf(mx[g], s[g][tg]);
      grow |= mx[g] > m[g] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = mx[g] > m[g] + kSlack ? mx[g] : m[g];
        const float alpha = mn == m[g] ? 1.f : fast_exp2(m[g] - mn);   // 0 when m was -inf
        m[g] = mn;
        l[g] *= alpha;
#pragma unroll
        for (int i = 0; i < DL; ++i) acc[g][i] *= alpha;
      }
    }
    // ---- probabilities and the value accumulation ----
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float ms = m[g] == -INFINITY ? 0.f : m[g];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) s[g][tg] = fast_exp2(s[g][tg] - ms);   // 0 for -inf logits
    }
    if constexpr (kPacked) {
      // round p to bf16 once; the sum and the p.v products use the same rounded value
      uint32_t pb[G][TG];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          pb[g][tg] = f32_to_bf16_bits(s[g][tg]);
          l[g] += __uint_as_float(pb[g][tg] << 16);
        }
#pragma unroll
      for (int tg = 0; tg + 1 < TG; tg += 2) {
        uint32_t pp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g] = pb[g][tg] | (pb[g][tg + 1] << 16);
#pragma unroll
        for (int cr = 0; cr < CPL; ++cr) {
          uint32_t va[PPC], vb[PPC];
          KvChunk<KV>::pairs(vc[tg][cr], va);
          KvChunk<KV>::pairs(vc[tg + 1][cr], vb);
#pragma unroll
          for (int i = 0; i < PPC; ++i) {
            const uint32_t even = __builtin_amdgcn_perm(vb[i], va[i], 0x05040100u);  // dim 2i of both rows
            const uint32_t odd = __builtin_amdgcn_perm(vb[i], va[i], 0x07060302u);   // dim 2i+1
#pragma unroll
            for (int g = 0; g < G; ++g) {
              acc[g][cr * EPC + 2 * i] = dot2(even, pp[g], acc[g][cr * EPC + 2 * i]);
              acc[g][cr * EPC + 2 * i + 1] = dot2(odd, pp[g], acc[g][cr * EPC + 2 * i + 1]);
            }
          }
        }
      }
      if constexpr (TG % 2 == 1) {
        constexpr int tg = TG - 1;
#pragma unroll
        for (int cr = 0; cr < CPL; ++cr) {
          float vf[EPC];
          KvChunk<KV>::cvt(vc[tg][cr], vf);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float p = __uint_as_float(pb[g][tg] << 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[g][cr * EPC + e] = fmaf(p, vf[e], acc[g][cr * EPC + e]);
          }
        }
      }
    } else {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
        for (int g = 0; g < G; ++g) l[g] += s[g][tg];
#pragma unroll
        for (int cr = 0; cr < CPL; ++cr) {
          float vf[EPC];
          KvChunk<KV>::cvt(vc[tg][cr], vf);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[g][cr * EPC + e] = fmaf(s[g][tg], vf[e], acc[g][cr * EPC + e]);
        }
      }
    }
  }
};

template <int TG, int CPL>
__device__ __forceinline__ void load_tile(uint4 (&kc)[TG][CPL], uint4 (&vc)[TG][CPL], const char* kb,
                                          const char* vb, const int (&off)[TG][CPL]) {
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int cr = 0; cr < CPL; ++cr) {
      kc[tg][cr] = *reinterpret_cast<const uint4*>(kb + off[tg][cr]);
      vc[tg][cr] = *reinterpret_cast<const uint4*>(vb + off[tg][cr]);
    }
}

// Work item of workgroup `id`: (partition, KV head, sequence), partitions fastest.  With xcd_map
// the KV head's index within its group of 8 equals id % 8, so every workgroup of one KV head runs on
// the same XCD; each XCD walks its heads one at a time, sequence by sequence, so blocks shared by the
// sequences of that head stay in its L2 while reads of private blocks keep HBM busy.
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int xcd_map, int& part, int& kvh, int& seq) {
  const int id = blockIdx.x;
  if (xcd_map) {
    const int x = id % 8;
    const int j = id / 8;
    part = j % a.max_parts;
    const int r = j / a.max_parts;
    seq = r % a.num_seqs;
    kvh = (r / a.num_seqs) * 8 + x;
  } else {
    part = id % a.max_parts;
    const int r = id / a.max_parts;
    kvh = r % a.num_kv_heads;
    seq = r / a.num_kv_heads;
  }
}

template <int KV, int D, int BS, int G, typename QT>
__global__ void __launch_bounds__(kThreads) decode_part_kernel(DecodeArgs a, int out_bf16, int xcd_map) {
  using Lane = DecodeLane<KV, D, BS, G>;
  constexpr int NL = Lane::NL, TPI = Lane::TPI, TG = Lane::TG, CPL = Lane::CPL, EPC = Lane::EPC,
                DL = Lane::DL, ROW = Lane::ROW, PPC = Lane::PPC;
  constexpr int TILE = BS * ROW;                      // bytes of one (block, head) tile

  int part, kvh, seq;
  decode_item(a, xcd_map, part, kvh, seq);
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

  Lane st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const QT* qrow = static_cast<const QT*>(a.q) + (static_cast<int64_t>(seq) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int cr = 0; cr < CPL; ++cr) {
      const int d0 = (cr * NL + cl) * EPC;
      if constexpr (Lane::kPacked) {
        const uint32_t* q32 = reinterpret_cast<const uint32_t*>(qrow + d0);
#pragma unroll
        for (int i = 0; i < PPC; ++i) st.qp[g][cr * PPC + i] = q32[i];
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) st.qf[g][cr * EPC + e] = static_cast<float>(qrow[d0 + e]) * a.qk_scale;
      }
    }
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) st.acc[g][i] = 0.f;
  }

  const char* kbase = static_cast<const char*>(a.k_pool) + static_cast<int64_t>(kvh) * TILE;
  const char* vbase = static_cast<const char*>(a.v_pool) + static_cast<int64_t>(kvh) * TILE;
  const int32_t* tab = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * TILE;
  int off[TG][CPL];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int cr = 0; cr < CPL; ++cr) off[tg][cr] = (tg * TPI + tokset) * ROW + (cr * NL + cl) * 16;

  // two register stages, unrolled so that no stage is copied into the other
  uint4 ka[TG][CPL], va[TG][CPL], kb2[TG][CPL], vb2[TG][CPL];
  int b = blk0 + wave;
  if (b < blk1) {
    const int64_t base = tab[b] * blk_stride;
    load_tile<TG, CPL>(ka, va, kbase + base, vbase + base, off);
  }
  for (; b < blk1; b += 2 * kWaves) {
    const int b1 = b + kWaves;
    if (b1 < blk1) {
      const int64_t base = tab[b1] * blk_stride;
      load_tile<TG, CPL>(kb2, vb2, kbase + base, vbase + base, off);
    }
    st.consume(ka, va, b * BS, t1, tokset, a.qk_scale);
    if (b1 >= blk1) break;
    const int b2 = b1 + kWaves;
    if (b2 < blk1) {
      const int64_t base = tab[b2] * blk_stride;
      load_tile<TG, CPL>(ka, va, kbase + base, vbase + base, off);
    }
    st.consume(kb2, vb2, b1 * BS, t1, tokset, a.qk_scale);
  }

  // ---- merge the lanes of different row sets (same dims) inside the wave ----
#pragma unroll
  for (int g = 0; g < G; ++g) {
    auto merge = [&](auto mask_tag) {
      constexpr int MASK = decltype(mask_tag)::value;
      const float mo = xor_lane<MASK>(st.m[g]);
      const float lo = xor_lane<MASK>(st.l[g]);
      const float mn = fmaxf(st.m[g], mo);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float a1 = fast_exp2(st.m[g] - ms);
      const float a2 = fast_exp2(mo - ms);
      st.l[g] = st.l[g] * a1 + lo * a2;
#pragma unroll
      for (int i = 0; i < DL; ++i) st.acc[g][i] = st.acc[g][i] * a1 + xor_lane<MASK>(st.acc[g][i]) * a2;
      st.m[g] = mn;
    };
    if constexpr (NL <= 4) merge(std::integral_constant<int, 4>());
    if constexpr (NL <= 8) merge(std::integral_constant<int, 8>());
    merge(std::integral_constant<int, 16>());
    merge(std::integral_constant<int, 32>());
  }

  // ---- merge the waves through LDS ----
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[wave][g] = st.m[g];
      sm_l[wave][g] = st.l[g];
    }
  }
  if (tokset == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int cr = 0; cr < CPL; ++cr)
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm_o[wave][g][(cr * NL + cl) * EPC + e] = st.acc[g][cr * EPC + e];
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
      const float f = fast_exp2(sm_m[w][g] - ms);
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
  const int h = blockIdx.x % a.num_q_heads;
  const int seq = blockIdx.x / a.num_q_heads;
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
    const float w = lp[p] * fast_exp2(mp[p] - ms);
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
    const int64_t wgs = static_cast<int64_t>(a.max_parts) * a.num_kv_heads * a.num_seqs;
    if (wgs > 0x7fffffff) return -1;
    const int xcd_map = a.num_kv_heads % 8 == 0;
    hipLaunchKernelGGL((decode_part_kernel<KV, D, BS, G, QT>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
                       a, out_bf16, xcd_map);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
    if (a.max_parts > 1) {
      const int64_t rw = static_cast<int64_t>(a.num_q_heads) * a.num_seqs;
      hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(static_cast<unsigned>(rw)), dim3(D), 0, s, a, out_bf16);
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
