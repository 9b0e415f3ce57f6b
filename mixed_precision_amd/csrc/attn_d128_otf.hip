// Instantiations of the fused attention kernel for head_dim 128, FP16 K/V, with
// Q and K quantised on the fly inside the kernel.
#include "attn_kernel.hpp"

namespace tilemix {

hipError_t launch_attn_d128_otf(const AttnArgs& a, int64_t nslots, bool debug, hipStream_t s) {
  switch (a.hc * 2 + (debug ? 1 : 0)) {
    case 2: return launch_attn_inst<128, 1, false, true, false>(a, nslots, s);
    case 3: return launch_attn_inst<128, 1, false, true, true>(a, nslots, s);
    case 4: return launch_attn_inst<128, 2, false, true, false>(a, nslots, s);
    case 5: return launch_attn_inst<128, 2, false, true, true>(a, nslots, s);
    case 6: return launch_attn_inst<128, 3, false, true, false>(a, nslots, s);
    case 7: return launch_attn_inst<128, 3, false, true, true>(a, nslots, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tilemix
