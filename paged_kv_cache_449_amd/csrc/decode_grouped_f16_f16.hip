// Prefix-grouped decode instantiations for f16 KV pools with f16 queries.
#include "decode_grouped.h"

namespace pkv {
kv_status_t launch_grouped_f16_f16(const DecodeParams& p, int D, int G, const int32_t* gs, const int32_t* gsh, int ng,
                                 hipStream_t s) {
  return launch_grouped<f16_t, f16_t>(p, D, G, gs, gsh, ng, s);
}
}  // namespace pkv
