// The partial records of a decode whose segments were split into pieces: where they live in the
// workspace and the order in which they are combined.  The decode's merge kernel and the beam
// decode's tail kernel both walk a segment's pieces this way («GPU 学习日报 Day 28：vLLM 与
// PagedAttention：GPU Memory 管理的艺术», §六 question 3: the shared prompt part of every branch is
// such a segment).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

constexpr int kDecodeUnit = 32;   // keys per unit of one decode wave

// Integer inputs that no kernel of a launch writes while it runs (tables, lengths, the plan of an
// earlier launch), read through the constant address space so that uniform reads stay on the
// scalar unit.
typedef const int32_t __attribute__((address_space(4)))* ro_i32;
__device__ __forceinline__ ro_i32 ro(const int32_t* p) { return (ro_i32)p; }
typedef const float __attribute__((address_space(4)))* ro_f32;
__device__ __forceinline__ ro_f32 ro(const float* p) { return (ro_f32)p; }

// Slot of piece (partition 0, share 0) of segment (head slot hh, sequence seq) of stream x; piece
// (partition k, share v) of the segment is at that slot + k + v.
__device__ __forceinline__ int64_t segment_slot(const DecodeArgs& a, int x, int hh, int seq) {
  return (static_cast<int64_t>(hh) * a.num_seqs + seq) * a.max_parts + x * a.stream_slots;
}

// The pieces of one segment in order: piece (k, v) ends at the nearer of partition k's end and share
// v's end, found without divisions.  P0 is the segment's first stream position, nj its units, PU
// the units of a partition and S those of a share.
struct PieceWalk {
  int64_t seg;
  int k, vv, pe, nb, seg_end, nparts, PU, S;
  __device__ __forceinline__ void init(int64_t seg_slot, int P0, int nj, int pu, int s) {
    seg = seg_slot;
    PU = pu;
    S = s;
    nparts = (nj + PU - 1) / PU;
    k = 0;
    vv = P0 / S;
    pe = P0 + min(PU, nj);
    nb = (vv + 1) * S;
    seg_end = P0 + nj;
  }
  __device__ __forceinline__ bool done() const { return k >= nparts; }
  // The slot of the current piece; then steps to the next one.
  __device__ __forceinline__ int64_t next() {
    const int64_t slot = seg + k + vv;
    const int e = min(pe, nb);
    if (e == nb) {
      ++vv;
      nb += S;
    }
    if (e == pe) {
      ++k;
      pe = min(pe + PU, seg_end);
    }
    return slot;
  }
};

}  // namespace pa
