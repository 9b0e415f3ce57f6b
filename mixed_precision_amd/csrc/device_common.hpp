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

template <typename T>
TM_DEV T uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}
TM_DEV uint64_t uniform64(uint64_t x) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

TM_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// XOR swizzle of 16-byte chunks inside an LDS row so that the 16 lanes of an
// MFMA operand read (16 consecutive rows, same logical chunk) hit distinct banks.
// row_bytes in {64, 128, 256}.
template <int ROW_BYTES>
TM_DEV int swz_chunk(int row, int chunk) {
  constexpr int cpr = ROW_BYTES / 16;      // chunks per row
  constexpr int rpp = 256 / ROW_BYTES;     // rows per 256-byte bank period
  return chunk ^ ((row / rpp) % cpr);
}

// V^T rows hold 64 keys = 16 units of 8 bytes; swizzle of the unit index.
TM_DEV int swz_vt(int d, int unit) { return unit ^ (d & 14); }

// Four int8 (one dword) -> four fp16 (two dwords), exact: bias the bytes to
// unsigned, splice them under the fp16 exponent of 1024 (bits 0x64uu encode
// 1024 + u), then subtract 1152 with one packed fp16 add per pair.
TM_DEV u32x2 i8x4_to_f16x4(uint32_t w) {
  const uint32_t t = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, t, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, t, 0x04030402u);
  const f16x2 bias = {(f16)1152.0f, (f16)1152.0f};
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
  const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Sixteen int8 -> two 16-byte chunks of fp16 (channels 0..7 and 8..15).
TM_DEV void i8x16_to_f16x16(const u32x4 w, u32x4& c0, u32x4& c1) {
  const u32x2 a = i8x4_to_f16x4(w.x), b = i8x4_to_f16x4(w.y);
  const u32x2 c = i8x4_to_f16x4(w.z), d = i8x4_to_f16x4(w.w);
  c0 = u32x4{a.x, a.y, b.x, b.y};
  c1 = u32x4{c.x, c.y, d.x, d.y};
}

// Transpose a 4-key x 8-channel fp16 block: rows r0..r3 hold channels 0..7 of
// keys 0..3; column x (channel x of keys 0..3, 8 bytes) is returned per x.
TM_DEV u32x2 vt_column(const u32x4& r0, const u32x4& r1, const u32x4& r2, const u32x4& r3, int x) {
  const int w = x >> 1;
  const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
  return u32x2{__builtin_amdgcn_perm(r1[w], r0[w], sel), __builtin_amdgcn_perm(r3[w], r2[w], sel)};
}

}  // namespace tilemix
