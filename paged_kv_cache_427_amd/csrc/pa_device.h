// Device helpers for the gfx950 kernels of libpa: number conversions and in-wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---- bf16 ------------------------------------------------------------------------------------
// A dword holding two bf16 values: element 0 in the low half, element 1 in the high half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- fp8 e4m3 (OCP "FN": bias 7, no infinities, S.1111.111 = NaN, max 448) ---------------------
// Bytes 0,1 (HI=false) or 2,3 (HI=true) of `w` -> two floats, by the gfx950 conversion unit.
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
  a = r[0];
  b = r[1];
}

// Nearest e4m3 code to an fp32 value: clamp to +-448, then round to nearest, ties to the even code.
// NaN -> 0x7F.  Written from the format definition with integer arithmetic so that the result does
// not depend on the conversion unit's rounding or saturation modes.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  if (y != y) return 0x7fu;
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    // below the smallest normal 2^-6: multiples of 2^-9; a * 512 is exact, rint rounds half to even
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t e = (ua >> 23) - 120u;          // biased e4m3 exponent, 1..15
    const uint32_t man = ua & 0x7fffffu;
    const uint32_t m3 = man >> 20;
    const uint32_t rem = man & 0xfffffu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (m3 & 1u));
    code = (e << 3) + m3 + up;                      // a carry moves into the exponent
  }
  return code | sign;
}

// ---- DPP lane exchange ------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each 16

// Sum over aligned groups of N lanes (N in {1, 2, 4, 8, 16}); every lane of a group gets the sum.
// All 64 lanes must be active.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

}  // namespace pa
