#include "device_common.h"
namespace gqa {
hipError_t launch_gqa_prefill(const void*, const void*, const void*, int32_t, int32_t, int32_t,
                              int32_t, int32_t, float, const RopeDev&, void*, void*, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace gqa
