// Decode kernel instantiations for fp8 KV pools with f32 queries.
#include "decode_kernel.h"

namespace pkv {
kv_status_t launch_decode_fp8_f32(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s) {
  return launch_decode<fp8_t, f32_t>(p, D, G, mfma, s);
}
}  // namespace pkv
