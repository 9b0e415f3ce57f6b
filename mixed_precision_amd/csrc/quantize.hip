// Blockwise symmetric INT8 quantiser (quantize-once operand preparation).
//
// One wavefront owns one (head, sequence, token block): it streams the block's
// rows with 16-byte loads (consecutive lanes read consecutive 16-byte chunks of
// a row, so each row is one coalesced segment), keeps them in registers, reduces
// the absolute maximum across the wave, derives the block scale and writes the
// int8 values with 8-byte stores.  HBM-bound: 2 bytes read and 1 byte written
// per element plus one float per block.
//
// Definition (paperlayer.ai summary of arXiv 2608.17336, "TileMix: Tile-Centric
// Mixed-Precision Attention for LLM Inference Acceleration", §3 Preliminaries and
// App. C: blockwise symmetric INT8 for Q and K, made once per attention call):
//   a = max|x|, scale = fl32(a/127), q = clamp(rint_half_even(fl32(x/scale)), +-127);
//   a zero block gets scale 1 and q = 0.
//
// Exactness at a few instructions per element:
//  * a = max|x| is taken on the fp16 bit patterns (|x| bits order like the
//    values), two per packed u16 max;
//  * scale and its reciprocal r = fl32(1/scale) are correctly rounded divisions,
//    once per block; per element q0 = fl32(x r), e = x - q0 scale (one fma, exact)
//    and q1 = fl32(q0 + e r) is the correctly rounded quotient fl32(x/scale)
//    (the correction step of Markstein's division; checked for every finite
//    fp16 x with |x| <= a against every scale a fp16 block can produce: the
//    only difference is the sign of a zero quotient, which does not reach the
//    int8 value);
//  * adding 1.5 * 2^23 rounds q1 to an integer with ties to even, and the low
//    byte of the sum's bit pattern is that integer in two's complement;
//  * |q1| <= 127 (1 + 2^-23) because scale >= a/127 (1 - 2^-24), so the clamp
//    never binds and is not applied.
#include "device_common.hpp"
#include "internal.hpp"

namespace tilemix {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

TM_DEV uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void quantize_blockwise_kernel(QuantArgs a) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int CPL = BLK * CPR / 64;   // chunks per lane
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  if (h >= a.num_heads) return;
  const int nb = (a.max_seqlen + BLK - 1) / BLK;
  const int b = blockIdx.x / nb;
  const int kb = blockIdx.x % nb;
  const int s0 = a.cu[b];
  const int L = a.cu[b + 1] - s0;
  const int r0 = kb * BLK;
  float* sc = a.scales + ((int64_t)h * a.batch + b) * nb + kb;
  if (r0 >= L) {
    if (lane == 0) *sc = 0.0f;
    return;
  }
  const int rows = min(BLK, L - r0);
  const f16* x = static_cast<const f16*>(a.x);

  u32x4 v[CPL];
  u16x2 mx = {0, 0};
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int id = lane + 64 * i;
    const int row = id / CPR, col = id % CPR;
    if (row < rows) {
      v[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)(s0 + r0 + row) * a.stride_tok +
                                             (int64_t)h * a.stride_head + col * 8);
    } else {
      v[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, v[i][e] & 0x7FFF7FFFu));
  }
  const uint32_t abits = wave_max_u32(max((uint32_t)mx[0], (uint32_t)mx[1]));
  const float amax = (float)__builtin_bit_cast(f16, (unsigned short)abits);
  const float scale = (abits == 0) ? 1.0f : __fdiv_rn(amax, 127.0f);
  const float rs = __fdiv_rn(1.0f, scale);
  if (lane == 0) *sc = scale;

#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int id = lane + 64 * i;
    const int row = id / CPR, col = id % CPR;
    if (row < rows) {
      const f16x8 hv = __builtin_bit_cast(f16x8, v[i]);
      uint32_t byte[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xf = (float)hv[e];
        const float q0 = xf * rs;
        const float er = __builtin_fmaf(-q0, scale, xf);
        const float q1 = __builtin_fmaf(er, rs, q0);
        byte[e] = __builtin_bit_cast(uint32_t, q1 + 12582912.0f);
      }
      // low bytes of 8 words -> two dwords
      const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(byte[3], byte[2], 0x0c0c0400u),
                                                __builtin_amdgcn_perm(byte[1], byte[0], 0x0c0c0400u), 0x05040100u);
      const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(byte[7], byte[6], 0x0c0c0400u),
                                                __builtin_amdgcn_perm(byte[5], byte[4], 0x0c0c0400u), 0x05040100u);
      *reinterpret_cast<u32x2*>(a.xq + ((int64_t)(s0 + r0 + row) * a.num_heads + h) * D + col * 8) =
          u32x2{lo, hi};
    }
  }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int nb = (a.max_seqlen + a.blk - 1) / a.blk;
  dim3 grid((unsigned)((int64_t)nb * a.batch), (unsigned)((a.num_heads + 3) / 4));
  dim3 block(256);
  if (a.head_dim == 128 && a.blk == 64)
    hipLaunchKernelGGL((quantize_blockwise_kernel<128, 64>), grid, block, 0, s, a);
  else if (a.head_dim == 128 && a.blk == 128)
    hipLaunchKernelGGL((quantize_blockwise_kernel<128, 128>), grid, block, 0, s, a);
  else if (a.head_dim == 64 && a.blk == 64)
    hipLaunchKernelGGL((quantize_blockwise_kernel<64, 64>), grid, block, 0, s, a);
  else if (a.head_dim == 64 && a.blk == 128)
    hipLaunchKernelGGL((quantize_blockwise_kernel<64, 128>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tilemix
