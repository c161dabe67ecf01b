// hq_prefill_attn: causal hybrid-precision prefill attention (gfx950).
// (kernels pending; the entry point reports HQ_ERR_UNSUPPORTED until then)
#include "hq_internal.h"

namespace hq {

size_t prefill_ws_bytes(int32_t, int32_t, int32_t, int32_t, const hq_policy&) { return 256; }

hipError_t launch_prefill(const void*, const void*, const void*, int32_t, int32_t, int32_t, int32_t, bool,
                          const hq_policy&, const int32_t*, const int32_t*, int32_t, float, void*, hq_dtype, void*,
                          hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace hq
