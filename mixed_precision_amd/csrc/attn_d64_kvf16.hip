// Instantiations of the fused attention kernel for head_dim 64, FP16 K/V.
#include "attn_kernel.hpp"

namespace tilemix {

hipError_t launch_attn_d64_kv0(const AttnArgs& a, int64_t nslots, bool debug, hipStream_t s) {
  switch (a.hc * 2 + (debug ? 1 : 0)) {
    case 2: return launch_attn_inst<64, 1, false, kOtfNone, false>(a, nslots, s);
    case 3: return launch_attn_inst<64, 1, false, kOtfNone, true>(a, nslots, s);
    case 4: return launch_attn_inst<64, 2, false, kOtfNone, false>(a, nslots, s);
    case 5: return launch_attn_inst<64, 2, false, kOtfNone, true>(a, nslots, s);
    case 6: return launch_attn_inst<64, 3, false, kOtfNone, false>(a, nslots, s);
    case 7: return launch_attn_inst<64, 3, false, kOtfNone, true>(a, nslots, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tilemix
