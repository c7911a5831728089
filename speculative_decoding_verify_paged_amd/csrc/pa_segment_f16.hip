// pa_segment_f16.hip — segment-kernel instances for a f16 KV cache.
#include "pa_kernels_impl.h"

namespace pav {

hipError_t launch_segment_f16(const SegmentArgs& a, int D, int bs, int rb, dim3 grid,
                               hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return dispatch_d<kF16, kF16>(a, D, bs, rb, grid, st, e0, e1);
}

}  // namespace pav
