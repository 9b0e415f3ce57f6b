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
// The exact division and rounding are those of quant8() and block_scale()
// (device_common.hpp), shared with the attention kernel's on-the-fly mode.
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
    mx = absmax_acc(mx, v[i]);
  }
  const float scale = block_scale(wave_max_u32(absmax_bits(mx)));
  const float rs = __fdiv_rn(1.0f, scale);
  if (lane == 0) *sc = scale;

#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int id = lane + 64 * i;
    const int row = id / CPR, col = id % CPR;
    if (row < rows) {
      *reinterpret_cast<u32x2*>(a.xq + ((int64_t)(s0 + r0 + row) * a.num_heads + h) * D + col * 8) =
          quant8(v[i], scale, rs);
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
