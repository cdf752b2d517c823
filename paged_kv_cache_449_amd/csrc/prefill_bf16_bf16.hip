// Multi-token paged attention instantiations for bf16 KV pools with bf16 queries.
#include "prefill_kernel.h"

namespace pkv {
kv_status_t launch_prefill_bf16_bf16(const DecodeParams& p, int D, int G, int mode, hipStream_t s) {
  return launch_prefill<bf16_t, bf16_t>(p, D, G, mode, s);
}
}  // namespace pkv
