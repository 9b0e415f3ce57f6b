// Instantiations of the fused attention kernel for head_dim 128 with three
// query heads per work item (GQA groups of 3): FP16 or INT8 K/V, and FP16 K/V
// with Q quantised on the fly.  This file is compiled with the
// instruction-level-parallelism scheduling strategy (the build's per-source
// flags): at 3 heads the kernel sits at the register limit, and that schedule
// interleaves the MFMAs with the softmax arithmetic more densely (and keeps the
// INT8 K/V kernel free of spills).
#include "attn_kernel.hpp"

namespace tilemix {

hipError_t launch_attn_d128_qb3(const AttnArgs& a, bool kv_int8, int64_t nslots, bool debug, hipStream_t s) {
  if (kv_int8)
    return debug ? launch_attn_inst<128, 3, true, kOtfNone, true>(a, nslots, s)
                 : launch_attn_inst<128, 3, true, kOtfNone, false>(a, nslots, s);
  if (a.otf == kOtfQ)
    return debug ? launch_attn_inst<128, 3, false, kOtfQ, true>(a, nslots, s)
                 : launch_attn_inst<128, 3, false, kOtfQ, false>(a, nslots, s);
  return debug ? launch_attn_inst<128, 3, false, kOtfNone, true>(a, nslots, s)
               : launch_attn_inst<128, 3, false, kOtfNone, false>(a, nslots, s);
}

}  // namespace tilemix
