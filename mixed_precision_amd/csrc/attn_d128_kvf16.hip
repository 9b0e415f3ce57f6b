// Instantiations of the fused attention kernel for head_dim 128, FP16 K/V.
#include "attn_kernel.hpp"

namespace tilemix {

hipError_t launch_attn_d128_qb3(const AttnArgs& a, bool kv_int8, int64_t nslots, bool debug, hipStream_t s);

hipError_t launch_attn_d128_kv0(const AttnArgs& a, int64_t nslots, bool debug, hipStream_t s) {
  switch (a.hc * 2 + (debug ? 1 : 0)) {
    case 2: return launch_attn_inst<128, 1, false, kOtfNone, false>(a, nslots, s);
    case 3: return launch_attn_inst<128, 1, false, kOtfNone, true>(a, nslots, s);
    case 4: return launch_attn_inst<128, 2, false, kOtfNone, false>(a, nslots, s);
    case 5: return launch_attn_inst<128, 2, false, kOtfNone, true>(a, nslots, s);
    case 6:
    case 7: return launch_attn_d128_qb3(a, false, nslots, debug, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tilemix
