// Instantiations of the decode kernel (one query per sequence and head over a KV cache).
#include "attn_decode.hpp"

namespace tilemix {

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return a.kv_int8 ? launch_decode_inst<64, true>(a, s) : launch_decode_inst<64, false>(a, s);
  return a.kv_int8 ? launch_decode_inst<128, true>(a, s) : launch_decode_inst<128, false>(a, s);
}

}  // namespace tilemix
