// Device helpers shared by the gfx950 kernels of the INT8-KV attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8a {

constexpr int kHeadDim = 256;
constexpr int kPage = 16;          // tokens per page
constexpr int kBlockBytes = 4096;  // codes per (page, kv head)
constexpr int kGroup = 6;          // query heads per KV head (v1 contract)
constexpr float kLog2e = 1.4426950408889634f;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Workgroup barrier that orders LDS only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}


// Lane permutations inside a 16-lane row (DPP): lane ^ 1, lane ^ 2, mirror of each
// 8-lane half, mirror of the row. Applied in that order they bring every lane of a row
// the row's reduction.
__device__ __forceinline__ float dpp(float v, int ctrl_sel) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true); break;   // [1,0,3,2]
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true); break;   // [2,3,0,1]
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true); break;  // half mirror
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true); break; // mirror
  }
  return __builtin_bit_cast(float, r);
}

// Reductions over the 4 lanes {n, n+16, n+32, n+48} that share one column of a
// 16x16 matrix-core accumulator (the column index is lane % 16). gfx950's lane swaps
// stay in the VALU: permlane16_swap exchanges 16-lane rows 1<->0 and 3<->2 between its
// two operands, permlane32_swap the two 32-lane halves, so combining the pair of results
// of each swap reduces over lane xor 16 and then lane xor 32.
__device__ __forceinline__ void swap16(float v, float* a, float* b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float* a, float* b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float col_max(float v) {
  float a, b;
  swap16(v, &a, &b);
  swap32(fmaxf(a, b), &a, &b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float col_sum(float v) {
  float a, b;
  swap16(v, &a, &b);
  swap32(a + b, &a, &b);
  return a + b;
}

// col_max for values whose bit patterns order like the values (non-negative floats).
__device__ __forceinline__ uint32_t col_max_u(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const uint32_t a = max(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  return max(r[0], r[1]);
}

// Whole-wave max / sum without LDS: DPP inside each 16-lane row, then the row swaps.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v = fmaxf(v, dpp(v, k));
  return col_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v += dpp(v, k);
  return col_sum(v);
}

// Whole-wave max of values whose bit patterns order like the values (non-negative
// floats), as unsigned integers: no NaN canonicalisation between the steps, and each DPP
// step is one fused max.
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));  // half mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));  // mirror
  return col_max_u(v);
}

// amax / 127 rounded to nearest even, as the IEEE fp32 division gives it. Inside
// [2^-90, 2^127): q = RN(amax RN(1/127)) is within an ulp of the quotient, the remainder
// amax - 127 q is exact in one fma (a normal number or 0 there), and one more fma with
// RN(1/127) rounds q + rem / 127 correctly (Markstein's correction step). The rounding
// pattern repeats per binade inside the range; checked against the division for every
// significand of a binade and for values across the range. Outside it (tiny, huge, inf,
// NaN) the division itself.
__device__ __forceinline__ float div127(float amax) {
  constexpr float kR = 1.0f / 127.0f;
  if (amax >= 0x1p-90f && amax < 0x1p127f) {
    const float q = amax * kR;
    const float rem = fmaf(-q, 127.0f, amax);
    return fmaf(rem, kR, q);
  }
  return amax / 127.0f;
}

// Row quantizer for one row of 256 values spread over a wave, 4 per lane (lane l holds
// elements 4l..4l+3). Rule: amax = max|x|, scale = amax/127 (IEEE fp32 division),
// code = clamp(rint(x/scale), -127, 127) with x/scale the correctly rounded quotient and
// rint half to even; scale == 0 gives all-zero codes. Returns the 4 codes packed
// little-endian. The quotient is formed by a reciprocal multiply wherever that provably
// rounds to the same code, and by the IEEE division elsewhere (below).
// ("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §2.1.)
__device__ __forceinline__ uint32_t quantize4(float x0, float x1, float x2, float x3,
                                              float* scale_out) {
  const uint32_t m = 0x7fffffffu;
  const uint32_t a = max(max(__float_as_uint(x0) & m, __float_as_uint(x1) & m),
                         max(__float_as_uint(x2) & m, __float_as_uint(x3) & m));
  const float amax = __uint_as_float(wave_max_u(a));
  const float scale = div127(amax);
  *scale_out = scale;
  if (scale == 0.0f) return 0u;
  // |x / scale| <= 127 (1 + 2^-23), so the codes need no clamp, and rint(v) of such a v
  // is fl(v + 1.5 * 2^23) - 1.5 * 2^23, whose fp32 bits carry the code's two's complement
  // in their low byte. The product x * rcp(scale) (reciprocal within an ulp) lies within
  // 1.5 * 2^-23 * 127 < 2^-15 of the correctly rounded x / scale, so the two round to the
  // same integer unless the product is within 2^-15 of a half-integer; the lane divides
  // when it is within 2^-14 (and with a denormal scale, whose reciprocal is not finite).
  constexpr float kM = 12582912.0f;  // 1.5 * 2^23
  const float x[4] = {x0, x1, x2, x3};
  float t[4];
  bool slow = !(scale >= 0x1p-126f);
  const float r = __builtin_amdgcn_rcpf(scale);
  float e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[i] = fmaf(x[i], r, kM);                  // rint(x r) + 1.5 * 2^23
    e[i] = fmaf(x[i], r, -(t[i] - kM));        // x r minus its nearest integer
  }
  // One compare for the lane's four.
  slow |= fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3]))) >= 0.5f - 0x1p-14f;
  if (slow) {
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = x[i] / scale + kM;
  }
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t[1]), __float_as_uint(t[0]), 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t[3]), __float_as_uint(t[2]), 0x04000c0cu);
  return lo | hi;
}

// Four signed int8 codes (one dword) -> their exact values as fp16, in two halves of
// two. 1024 + (b + 128) is exact in fp16; subtracting 1152 leaves b. `bias` must be
// 0x80808080 (it is a parameter so that a caller can pass it through memory and keep
// the conversion from being scheduled ahead of a barrier).
__device__ __forceinline__ void i8x4_to_f16(uint32_t a, h2* lo, h2* hi, uint32_t bias) {
  const uint32_t u = a ^ bias;
  const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  *lo = __builtin_bit_cast(h2, p0) - off;
  *hi = __builtin_bit_cast(h2, p1) - off;
}

__device__ __forceinline__ v8h i8x8_to_f16(uint32_t a0, uint32_t a1, uint32_t bias) {
  h2 r0, r1, r2, r3;
  i8x4_to_f16(a0, &r0, &r1, bias);
  i8x4_to_f16(a1, &r2, &r3, bias);
  v8h o;
  o[0] = r0[0]; o[1] = r0[1]; o[2] = r1[0]; o[3] = r1[1];
  o[4] = r2[0]; o[5] = r2[1]; o[6] = r3[0]; o[7] = r3[1];
  return o;
}

}  // namespace i8a
