// Device-side helpers shared by the gfx950 kernels of libtilemix.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace tilemix {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;          // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;

#define TM_DEV __device__ __forceinline__

TM_DEV int lane_id() { return __lane_id(); }

// Value of the first active lane (a wave-uniform value), bit for bit: the
// builtin is int-typed, so other 32-bit types go through a bit cast, never a
// numeric conversion.
template <typename T>
TM_DEV T uniform(T x) {
  static_assert(sizeof(T) == 4, "uniform() takes a 32-bit value");
  return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
// A wave-uniform float pinned to a scalar register.  (The compiler drops a
// readfirstlane of a value it already knows to be uniform and may then keep
// the value in a vector register; long-lived per-wave constants belong in SGPRs.)
// The compiler's hazard recognizer does not look inside an asm block, so the
// block carries its own wait states: a VALU write of x just before (1 needed),
// and VALU (2) or VMEM (5) reads of the result just after.
TM_DEV float sgpr_f32(float x) {
  float r;
  asm volatile("s_nop 1\n\tv_readfirstlane_b32 %0, %1\n\ts_nop 4" : "=s"(r) : "v"(x));
  return r;
}
TM_DEV uint64_t uniform64(uint64_t x) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Reductions over the four lanes l, l^16, l^32, l^48 (one lane per 16-lane
// row): gfx950's row-swapping permutes exchange rows 0<->1, 2<->3, then the two
// halves of the wave, in registers with no LDS round trip.  With both operands
// holding x, v_permlane16_swap leaves (x0 x0 x2 x2) in its first register and
// (x1 x1 x3 x3) in its second (by 16-lane rows); v_permlane32_swap leaves
// (x_lo x_lo) and (x_hi x_hi).  Combining the two registers after each swap
// leaves every lane with (x0 op x1) op (x2 op x3).
//
// The swaps are written as asm: ROCm 7.2's builtins for them return the first
// register twice.  The asm carries the wait states a permute needs after a
// VALU write of its operands (the hazard recognizer does not look inside asm).
TM_DEV void permlane16_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
TM_DEV void permlane32_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
template <typename Op>
TM_DEV float rows4_reduce(float x, Op op) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane16_swap(a, b);
  const float y = op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  uint32_t c = __builtin_bit_cast(uint32_t, y), d = c;
  permlane32_swap(c, d);
  return op(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
TM_DEV float rows4_max(float x) {
  return rows4_reduce(x, [](float u, float v) { return __builtin_elementwise_maximum(u, v); });
}
TM_DEV float rows4_sum(float x) {
  return rows4_reduce(x, [](float u, float v) { return u + v; });
}

TM_DEV uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// ---- blockwise symmetric INT8 quantisation, bit-exact with the definition
//   a = max|x|, scale = fl32(a/127), q = clamp(rint_half_even(fl32(x/scale)), +-127),
//   an all-zero block taking scale 1 and q = 0.
//  * a is taken on the fp16 bit patterns (|x| bits order like the values), two
//    per packed u16 max;
//  * scale and r = fl32(1/scale) are correctly rounded divisions, once per
//    block; per element q0 = fl32(x r), e = x - q0 scale (one fma, exact) and
//    q1 = fl32(q0 + e r) is the correctly rounded quotient fl32(x/scale) (the
//    correction step of Markstein's division).  tests/quant_division_exhaustive.c
//    replays these steps for every finite fp16 x with |x| <= a against every
//    scale a fp16 block can produce: the only difference is the sign of a zero
//    quotient, which does not reach the int8;
//  * adding 1.5 * 2^23 rounds q1 to an integer with ties to even, and the low
//    byte of the sum's bit pattern is that integer in two's complement;
//  * |q1| <= 127 (1 + 2^-23) because scale >= a/127 (1 - 2^-24), so the clamp
//    never binds and is not applied.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// running max of |x| over 8 fp16 (one 16-byte chunk), as two packed u16 lanes
TM_DEV u16x2 absmax_acc(u16x2 mx, const u32x4 v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, v[e] & 0x7FFF7FFFu));
  return mx;
}
TM_DEV uint32_t absmax_bits(u16x2 mx) { return max((uint32_t)mx[0], (uint32_t)mx[1]); }

// block scale from the fp16 bits of a = max|x|
TM_DEV float block_scale(uint32_t abits) {
  const float amax = (float)__builtin_bit_cast(f16, (unsigned short)abits);
  return (abits == 0) ? 1.0f : __fdiv_rn(amax, 127.0f);
}

// 8 fp16 -> 8 int8 (two dwords, element 0 in the lowest byte); rs = fl32(1/scale)
TM_DEV u32x2 quant8(const u32x4 v, float scale, float rs) {
  const f16x8 hv = __builtin_bit_cast(f16x8, v);
  uint32_t byte[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xf = (float)hv[e];
    const float q0 = xf * rs;
    const float er = __builtin_fmaf(-q0, scale, xf);
    const float q1 = __builtin_fmaf(er, rs, q0);
    byte[e] = __builtin_bit_cast(uint32_t, q1 + 12582912.0f);
  }
  const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(byte[3], byte[2], 0x0c0c0400u),
                                            __builtin_amdgcn_perm(byte[1], byte[0], 0x0c0c0400u), 0x05040100u);
  const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(byte[7], byte[6], 0x0c0c0400u),
                                            __builtin_amdgcn_perm(byte[5], byte[4], 0x0c0c0400u), 0x05040100u);
  return u32x2{lo, hi};
}

// Four int8 (one dword) -> four fp16 (two dwords) times 2^E, exact: bias the
// bytes to unsigned, splice them under the fp16 exponent of 1024 (bits 0x64uu
// encode 1024 + u), then (1024 + u) 2^E - 1152 2^E = v 2^E in one packed fp16
// fma per pair (scale = 2^E, bias = -1152 2^E, both exact in fp16 for E in
// [-24, 5]; the fma's exact result v 2^E is a multiple of 2^-24 below 65504).
TM_DEV u32x2 i8x4_to_f16x4(uint32_t w, f16x2 scale = f16x2{(f16)1.0f, (f16)1.0f},
                           f16x2 bias = f16x2{(f16)-1152.0f, (f16)-1152.0f}) {
  const uint32_t t = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, t, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, t, 0x04030402u);
  const f16x2 a = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, lo), scale, bias);
  const f16x2 b = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, hi), scale, bias);
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Sixteen int8 -> two 16-byte chunks of fp16 (channels 0..7 and 8..15), times 2^E.
TM_DEV void i8x16_to_f16x16(const u32x4 w, u32x4& c0, u32x4& c1, f16x2 scale = f16x2{(f16)1.0f, (f16)1.0f},
                            f16x2 bias = f16x2{(f16)-1152.0f, (f16)-1152.0f}) {
  const u32x2 a = i8x4_to_f16x4(w.x, scale, bias), b = i8x4_to_f16x4(w.y, scale, bias);
  const u32x2 c = i8x4_to_f16x4(w.z, scale, bias), d = i8x4_to_f16x4(w.w, scale, bias);
  c0 = u32x4{a.x, a.y, b.x, b.y};
  c1 = u32x4{c.x, c.y, d.x, d.y};
}

}  // namespace tilemix
