// fp8 (e4m3) attention: not built yet; the entry point reports it as unsupported.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {

bool fp8_attention_available() { return false; }

size_t fp8_scratch_bytes(int, int, int, int) { return 0; }

hipError_t launch_attn_fp8(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int64_t,
                           int64_t, int64_t, int64_t, const int32_t*, const int32_t*,
                           const int32_t*, int64_t, int, int, int, int, float, int, float,
                           int32_t*, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace h3
