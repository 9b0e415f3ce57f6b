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
//   a zero block gets scale 1 and q = 0.  Both divisions are correctly rounded
//   (__fdiv_rn), rint is v_rndne_f32, so the result is bit-exact with the CPU
//   definition.
#include "device_common.hpp"
#include "internal.hpp"

namespace tilemix {

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

  f16x8 v[CPL];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int id = lane + 64 * i;
    const int row = id / CPR, col = id % CPR;
    if (row < rows) {
      v[i] = *reinterpret_cast<const f16x8*>(x + (int64_t)(s0 + r0 + row) * a.stride_tok +
                                             (int64_t)h * a.stride_head + col * 8);
    } else {
      v[i] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[i][e]));
  }
  amax = wave_max(amax);
  const float scale = (amax == 0.0f) ? 1.0f : __fdiv_rn(amax, 127.0f);
  if (lane == 0) *sc = scale;

#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int id = lane + 64 * i;
    const int row = id / CPR, col = id % CPR;
    if (row < rows) {
      uint32_t w[2] = {0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qv = __builtin_rintf(__fdiv_rn((float)v[i][e], scale));
        qv = fminf(fmaxf(qv, -127.0f), 127.0f);
        const uint32_t byte = (uint32_t)(int32_t)qv & 0xffu;
        w[e >> 2] |= byte << (8 * (e & 3));
      }
      *reinterpret_cast<u32x2*>(a.xq + ((int64_t)(s0 + r0 + row) * a.num_heads + h) * D + col * 8) =
          u32x2{w[0], w[1]};
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
