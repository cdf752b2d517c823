// Prefix-grouped decode instantiations for bf16 KV pools with bf16 queries.
#include "decode_grouped.h"

namespace pkv {
kv_status_t launch_grouped_bf16_bf16(const DecodeParams& p, int D, int G, const int32_t* gs, const int32_t* gsh, int ng,
                                 hipStream_t s) {
  return launch_grouped<bf16_t, bf16_t>(p, D, G, gs, gsh, ng, s);
}
}  // namespace pkv
