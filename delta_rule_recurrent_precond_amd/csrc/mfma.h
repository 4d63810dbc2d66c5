// Matrix-core and lane helpers shared by the bf16/fp16 kernels (gfx950, wave64).
//
// Operand layouts of the 16x16 matrix-core products used here (checked on the
// device): for 16x16x32 f16 the A operand of lane l holds row l & 15, k slots
// 8(l >> 4) .. +7; the B operand column l & 15, the same k slots; the result
// column l & 15, rows 4(l >> 4) .. +3.  16x16x16 (f16, bf16) has the same
// pattern with 4 k slots per lane.  "Paired" k order: a result tile feeds the
// next product from registers when the partner operand reads k slots
// kb + 4g .. +3 and kb + 16 + 4g .. +3 of its row (ldpk below).
#pragma once

#include "device.h"

namespace osdn {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16bf(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// fp32 -> fp16 rounding a materialised fp32 value.  The empty asm keeps the
// compiler from fusing the conversion into the producing FMA (a mixed-precision
// FMA rounds once, straight to fp16), so equal fp32 values give equal fp16
// values on every code path -- needed for bitwise-reproducible continuation.
__device__ __forceinline__ f16 h(float x) {
  asm("" : "+v"(x));
  return (f16)x;
}
__device__ __forceinline__ f16x4 h4(f32x4 v) { return f16x4{h(v[0]), h(v[1]), h(v[2]), h(v[3])}; }
__device__ __forceinline__ f16x8 cat(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ float bf2f(unsigned short u) {
  return __builtin_bit_cast(float, ((unsigned)u) << 16);
}
__device__ __forceinline__ f16x4 ld4(const f16 *p) { return *(const f16x4 *)p; }
__device__ __forceinline__ f16x8 ld8(const f16 *p) { return *(const f16x8 *)p; }
// 16x16x32 operand in the paired k order from a row-major f16 row:
// halves kb + 4g .. +3 and kb + 16 + 4g .. +3.
__device__ __forceinline__ f16x8 ldpk(const f16 *row, int kb, int g) {
  return cat(ld4(row + kb + 4 * g), ld4(row + kb + 16 + 4 * g));
}
// Sum of squares of 8 bf16 (16 bytes), fp32.
__device__ __forceinline__ float sqsum8(const uint4 &u) {
  const unsigned short *s = (const unsigned short *)&u;
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = bf2f(s[e]);
    a = fmaf(x, x, a);
  }
  return a;
}
// 8 bf16 times a scale (fp32), rounded once to fp16.
__device__ __forceinline__ f16x8 cvt8s(const uint4 &u, float sc) {
  const unsigned short *s = (const unsigned short *)&u;
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = h(bf2f(s[e]) * sc);
  return r;
}
// 8 bf16 (16 bytes) as fp16 (exact for |x| in fp16's normal range)
__device__ __forceinline__ f16x8 cvt8(const uint4 &u) {
  const unsigned short *s = (const unsigned short *)&u;
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16)bf2f(s[e]);
  return r;
}
// hardware 2^x and log2 x (about 1 ulp)
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }
// Lanes of one wave exchange data through LDS between the two sides of this
// call; it keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_wave_barrier(); }

// Lower-triangular 16x16 tile list of a 64x64 matrix (10 tiles).
__device__ __forceinline__ void tri_tile(int idx, int &rt, int &ct) {
  rt = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
  ct = idx - (rt * (rt + 1)) / 2;
}
// Off-diagonal lower tiles (row tile > col tile), 6 of them:
// (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__device__ __forceinline__ void off_tile(int idx, int &rt, int &ct) {
  rt = idx >= 3 ? 3 : idx >= 1 ? 2 : 1;
  ct = idx - (rt * (rt - 1)) / 2;
}

// Sum over the 4 lanes of an aligned quad (DPP quad permutations); all four
// lanes receive the same bits.
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  return v;
}
__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// (I + N)^-1 for a strictly lower 16x16 fp32 block N in LDS (row stride ld;
// entries on and above the diagonal must be zero), by one wave.  Lanes
// 4c..4c+3 solve column c by forward substitution: lane q keeps rows q, q+4,
// q+8, q+12 and their share of each dot product, and quad sums join the
// shares.  On return x[j] holds row q + 4j of column c.
__device__ __forceinline__ void tri16_inverse_quad(const float *N, int ld, int lane,
                                                   float (&x)[4]) {
  const int col = lane >> 2, q = lane & 3;
  float nv[16][4];
#pragma unroll
  for (int t = 1; t < 16; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) nv[t][j] = N[t * ld + q + 4 * j];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    float p = 0.f;
    if (t > 0) {
      const float p0 = fmaf(nv[t][0], x[0], nv[t][1] * x[1]);
      const float p1 = fmaf(nv[t][2], x[2], nv[t][3] * x[3]);
      p = quad_sum(p0 + p1);
    }
    const float xt = (t == col ? 1.f : 0.f) - p;
    if (q == (t & 3)) x[t >> 2] = xt;
  }
}

}  // namespace osdn
