// Device helpers shared by the OSDN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osdn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Element access for the two storage types of q, k, v, k~, o.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p) { return *p; }
  static __device__ __forceinline__ void store(float *p, float x) { *p = x; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float load(const bf16 *p) { return (float)(*p); }
  // round to nearest even (the hardware conversion on gfx950)
  static __device__ __forceinline__ void store(bf16 *p, float x) { *p = (bf16)x; }
};

// Sum over the 64 lanes of a wave; every lane receives the total.
// Quad butterflies and row mirrors via DPP, then the four 16-lane rows are
// combined through lane reads (gfx9 DPP cannot cross rows symmetrically).
__device__ __forceinline__ float wave_sum(float v) {
  // DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
  // row_half_mirror = 0x141, row_mirror = 0x140.
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return (r0 + r1) + (r2 + r3);
}

// Maximum over the 64 lanes of a wave, every lane receives it (the same DPP
// steps as wave_sum; a maximum does not depend on the order).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over the four lanes l % 16 + 16 r (r = 0..3) of a wave, every one of
// them receiving it: the row swap then the lane-half swap (gfx950), adding
// in the order of xor-16 then xor-32 shuffles.
__device__ __forceinline__ float column_sum4(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// A power of two >= x (x >= 0 and finite; 1 for 0).  Values divided by it keep
// their significand exactly, so it moves a vector into fp16's normal range
// without changing how it rounds.
// Waits here for a load into x's registers to arrive (an empty asm that reads
// them), so that a branch that uses x after this point holds no wait of its own.
__device__ __forceinline__ void arrived(const uint4 &x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}
__device__ __forceinline__ void arrived(float x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ float pow2_above(float x) {
  if (!(x > 0.f)) return 1.0f;
  int e;
  frexpf(x, &e);  // x = f 2^e with f in [0.5, 1)
  return ldexpf(1.0f, e);
}

// 1 / p for p a power of two, exactly (the bits 1.0f / p gives, without the
// division's refinement steps)
__device__ __forceinline__ float pow2_inv(float p) {
  int e;
  frexpf(p, &e);  // p = 0.5 * 2^e
  return ldexpf(1.0f, 1 - e);
}

// Input transforms of the raw-input flags (include/osdn.h): the scale that
// normalises a vector of squared norm n (a zero vector stays zero), and the
// logistic sigmoid of a gate logit.
__device__ __forceinline__ float unit_scale(float n) { return n > 0.f ? 1.0f / sqrtf(n) : 0.f; }
__device__ __forceinline__ float sigmoid_gate(float x) { return 1.0f / (1.0f + expf(-x)); }


// Sum over aligned groups of G lanes (G = 2..64, power of two); every lane of
// the group receives the group's total.  Steps within a 16-lane row are DPP
// moves: the quad permutations [1,0,3,2] and [2,3,0,1] (xor 1, xor 2), then the
// half-row and row mirrors, which pair the same partial sums as xor 4 and xor 8
// once the quads (and half-rows) hold equal values, so the result is the xor
// butterfly's bit for bit.  Wider steps are xor shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) {
    if (m == 1)
      v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    else if (m == 2)
      v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    else if (m == 4)
      v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    else if (m == 8)
      v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    else
      v += __shfl_xor(v, m, 64);
  }
  return v;
}

}  // namespace osdn
