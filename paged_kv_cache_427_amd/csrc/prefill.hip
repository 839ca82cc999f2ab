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
//  * a workgroup of 4 wave64s owns 128 (query, head) rows of one KV-head group: 128/G queries of
//    the G query heads that share the KV head, so one K/V tile in LDS serves every head of the group;
//    each wave owns 32 rows;
//  * key tiles of 64 positions are gathered through the block table (one lookup per block row),
//    widened to bf16 (fp8 e4m3 codes convert exactly; scales stay in fp32) and stored in LDS: K as
//    [key][dim], V transposed as [dim][key], double-buffered so the next tile's global loads are in
//    flight during the current tile's MFMAs;
//  * scores are formed transposed, S^T = K Q^T (A = K rows from LDS, B = Q held in registers), so the
//    fp32 result layout (each lane owns one query row and 16 keys) becomes, after bf16 rounding,
//    exactly the B operand of O^T = V^T P^T; softmax statistics need one cross-half lane exchange;
//  * the rescale of the output accumulators is skipped while the running max has grown by less than
//    2^8 (base-2 logits), which keeps every exp bounded by 256;
//  * the grid is remapped so all query tiles of one (sequence, KV head) run on the same XCD and share
//    its L2.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;          // head_dim
constexpr int kKT = 64;          // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 128;       // (query, head) rows per workgroup
constexpr int kKStride = kD * 2 + 16;    // bytes per K row in LDS (padding spreads banks)
constexpr int kVStride = kKT * 2 + 8;    // bytes per V^T row in LDS
constexpr int kKBytes = kKT * kKStride;
constexpr int kVBytes = kD * kVStride;
constexpr int kBufBytes = kKBytes + kVBytes;
constexpr float kRescaleSlack = 8.0f;    // log2 of the largest unrescaled growth

template <int KV>
struct Src;
template <>
struct Src<kBF16> {
  static constexpr int kElem = 2, kEPC = 8;     // elements per 16-byte chunk
};
template <>
struct Src<kFP8> {
  static constexpr int kElem = 1, kEPC = 16;
};

// Global -> registers for one key tile: each thread owns `kUnits` (key pair, 16-byte chunk) units.
template <int KV, int BS>
struct TileLoader {
  static constexpr int kRowBytes = kD * Src<KV>::kElem;
  static constexpr int kChunks = kRowBytes / 16;             // chunks per key row
  static constexpr int kUnits = (kKT / 2) * kChunks / kThreads;
  uint4 k0[kUnits], k1[kUnits], v0[kUnits], v1[kUnits];

  __device__ void load(const char* kpool, const char* vpool, const int32_t* tab, int64_t blk_stride,
                       int64_t head_off, int tile, int n_keys) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int unit = threadIdx.x + kThreads * u;
      const int kp = unit / kChunks;
      const int ch = unit % kChunks;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = tile * kKT + 2 * kp + half;
        uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (key < n_keys) {
          const int64_t off = static_cast<int64_t>(tab[key / BS]) * blk_stride + head_off +
                              static_cast<int64_t>(key % BS) * kRowBytes + ch * 16;
          kk = *reinterpret_cast<const uint4*>(kpool + off);
          vv = *reinterpret_cast<const uint4*>(vpool + off);
        }
        if (half == 0) { k0[u] = kk; v0[u] = vv; } else { k1[u] = kk; v1[u] = vv; }
      }
    }
  }

  // Widen to bf16 and store: K row-major, V transposed (one dword = the two keys of a pair).
  __device__ void store(char* buf) const {
    char* ks = buf;
    char* vt = buf + kKBytes;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int unit = threadIdx.x + kThreads * u;
      const int kp = unit / kChunks;
      const int ch = unit % kChunks;
      constexpr int EPC = Src<KV>::kEPC;
      uint32_t kb0[EPC / 2], kb1[EPC / 2], vb0[EPC / 2], vb1[EPC / 2];
      widen(k0[u], kb0);
      widen(k1[u], kb1);
      widen(v0[u], vb0);
      widen(v1[u], vb1);
      const int d0 = ch * EPC;
#pragma unroll
      for (int i = 0; i < EPC / 8; ++i) {
        *reinterpret_cast<uint4*>(ks + (2 * kp) * kKStride + (d0 + 8 * i) * 2) =
            make_uint4(kb0[4 * i], kb0[4 * i + 1], kb0[4 * i + 2], kb0[4 * i + 3]);
        *reinterpret_cast<uint4*>(ks + (2 * kp + 1) * kKStride + (d0 + 8 * i) * 2) =
            make_uint4(kb1[4 * i], kb1[4 * i + 1], kb1[4 * i + 2], kb1[4 * i + 3]);
      }
#pragma unroll
      for (int i = 0; i < EPC / 2; ++i) {
        const uint32_t lo = (vb0[i] & 0xffffu) | (vb1[i] << 16);           // dim d0 + 2i
        const uint32_t hi = (vb0[i] >> 16) | (vb1[i] & 0xffff0000u);       // dim d0 + 2i + 1
        *reinterpret_cast<uint32_t*>(vt + (d0 + 2 * i) * kVStride + 4 * kp) = lo;
        *reinterpret_cast<uint32_t*>(vt + (d0 + 2 * i + 1) * kVStride + 4 * kp) = hi;
      }
    }
  }

  // 16 bytes of stored codes -> packed bf16 pairs (element 2i in the low half of out[i]).
  __device__ static void widen(const uint4& c, uint32_t* out) {
    if constexpr (KV == kBF16) {
      out[0] = c.x; out[1] = c.y; out[2] = c.z; out[3] = c.w;
    } else {
      const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
        auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
        out[2 * i] = __builtin_bit_cast(uint32_t, lo);
        out[2 * i + 1] = __builtin_bit_cast(uint32_t, hi);
      }
    }
  }
};

template <int KV, int BS, int G>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(PrefillArgs a, int out_bf16, int num_qtiles,
                                                              int xcd_remap) {
  constexpr int QT = kRows / G;      // queries per workgroup
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];

  // ---- which (sequence, KV head, query tile) ----
  const int groups = a.num_seqs * a.num_kv_heads;
  int grp, qt;
  if (xcd_remap) {
    // workgroup i runs on XCD i % 8; give that XCD whole groups so their tiles share its L2
    const int x = blockIdx.x % 8;
    const int j = blockIdx.x / 8;
    grp = x + 8 * (j / num_qtiles);
    qt = num_qtiles - 1 - j % num_qtiles;   // longest tiles first
  } else {
    grp = blockIdx.x / num_qtiles;
    qt = num_qtiles - 1 - blockIdx.x % num_qtiles;
  }
  if (grp >= groups) return;
  const int seq = grp / a.num_kv_heads;
  const int kvh = grp % a.num_kv_heads;
  const int q_base = a.qsl[seq];
  const int C = a.qsl[seq + 1] - q_base;
  const int q0 = qt * QT;
  if (q0 >= C) return;
  const int P = a.prior[seq];
  const int q_end = min(q0 + QT, C);
  const int n_keys = P + q_end;
  const int n_tiles = (n_keys + kKT - 1) / kKT;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  constexpr int kRowBytes = TileLoader<KV, BS>::kRowBytes;
  const int64_t head_off = static_cast<int64_t>(kvh) * BS * kRowBytes;
  const int64_t blk_stride = static_cast<int64_t>(a.num_kv_heads) * BS * kRowBytes;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;   // running max (base-2 logits) of this row, the one the accumulators use
  float l_run = 0.f;

  TileLoader<KV, BS> ld;
  ld.load(kpool, vpool, tab, blk_stride, head_off, 0, n_keys);
  ld.store(smem);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    char* buf = smem + (t & 1) * kBufBytes;
    if (t + 1 < n_tiles) ld.load(kpool, vpool, tab, blk_stride, head_off, t + 1, n_keys);

    // ---- S^T = K Q^T for two 32-key halves ----
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
      const char* krow = buf + (sb * 32 + (lane & 31)) * kKStride + 16 * h;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 32 * c);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[c], s[sb], 0, 0, 0);
      }
    }

    // ---- scale, causal mask, running max ----
    const int key_base = t * kKT;
    const bool diag = key_base + kKT - 1 > P + q0;
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[sb][r] * a.qk_scale;
        if (diag) {
          const int key = key_base + sb * 32 + 8 * (r / 4) + 4 * h + (r % 4);
          x = key <= qpos ? x : -INFINITY;
        }
        s[sb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // rescale only when the max moved by more than the slack (wave-uniform decision)
    const bool grow = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const float ms = m_run == -INFINITY ? 0.f : m_run;

    // ---- P^T = 2^(S^T - m) as bf16 B operands; row sums ----
    bf16x8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2f(s[c / 2][8 * (c % 2) + e] - ms);
        lsum += p;
        pb[c][e] = static_cast<__bf16>(p);
      }
    l_run += lsum + shfl_xor(lsum, 32);

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const char* vrow = buf + kKBytes + (dt * 32 + (lane & 31)) * kVStride;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // k-slots 0..3 <- keys 16c + 4h + 0..3, slots 4..7 <- keys 16c + 8 + 4h + 0..3
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (16 * c + 4 * h) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (16 * c + 8 + 4 * h) * 2);
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], o[dt], 0, 0, 0);
      }
    }

    if (t + 1 < n_tiles) ld.store(smem + ((t + 1) & 1) * kBufBytes);
    __syncthreads();
  }

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

template <int KV, int BS, int G>
int launch_g(const PrefillArgs& a, int out_bf16, hipStream_t s) {
  constexpr int QT = kRows / G;
  const int num_qtiles = (a.max_chunk + QT - 1) / QT;
  const int64_t groups = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int xcd_remap = groups % 8 == 0;
  const int64_t wgs = groups * num_qtiles;
  if (wgs > 0x7fffffff) return -1;
  hipLaunchKernelGGL((prefill_kernel<KV, BS, G>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s, a,
                     out_bf16, num_qtiles, xcd_remap);
  return static_cast<int>(hipGetLastError());
}

template <int KV, int BS>
int launch_bs(const PrefillArgs& a, int out_bf16, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<KV, BS, 1>(a, out_bf16, s);
    case 2: return launch_g<KV, BS, 2>(a, out_bf16, s);
    case 4: return launch_g<KV, BS, 4>(a, out_bf16, s);
    case 8: return launch_g<KV, BS, 8>(a, out_bf16, s);
    default: return -1;
  }
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
