// pa_segment_u8.hip — segment-kernel instances for a u8 KV cache (f16 or
// bf16 queries).
#include "pa_kernels_impl.h"

namespace pav {

hipError_t launch_segment_u8(const SegmentArgs& a, int q_dtype, int D, int bs, int rb, dim3 grid,
                             hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (q_dtype == kF16) return dispatch_d<kF16, kU8>(a, D, bs, rb, grid, st, e0, e1);
  if (q_dtype == kBF16) return dispatch_d<kBF16, kU8>(a, D, bs, rb, grid, st, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace pav
