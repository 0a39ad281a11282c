#include "device_common.h"
namespace gqa {
SparseLayout sparse_layout(int32_t B, int32_t H, int32_t S_max, int32_t top_k) {
    SparseLayout l{};
    l.scores_bytes = ((size_t)B * S_max * 4 + 255) & ~(size_t)255;
    l.total = l.scores_bytes;
    return l;
}
hipError_t launch_topk_sparse_decode(const void*, const void*, const void*, const void*,
                                     const int32_t*, int32_t, int32_t, int32_t, int32_t, float,
                                     int32_t*, void*, void*, const SparseLayout&, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace gqa
