// Multi-token paged attention instantiations for f16 KV pools with f16 queries.
#include "prefill_kernel.h"

namespace pkv {
kv_status_t launch_prefill_f16_f16(const DecodeParams& p, int D, int G, int mode, hipStream_t s) {
  return launch_prefill<f16_t, f16_t>(p, D, G, mode, s);
}
}  // namespace pkv
