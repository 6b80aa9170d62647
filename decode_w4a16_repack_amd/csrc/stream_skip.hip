// Small-M fused W4A16 GEMM/GEMV for gfx950 (at most 4 rows) with the skip +
// RMSNorm prologue in registers (residual fragments loaded with the
// activations, the sum written out once): the instantiations of
// stream_kernel.h that carry it.  Above 4 rows the prologue is staged.
#include "stream_kernel.h"

namespace w4a16 {

hipError_t launch_stream_skip(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                              bool gate_up, hipStream_t stream) {
  return launch_stream_cfg<2>(a, pl, group, scale_f32, gate_up, stream);
}

}  // namespace w4a16
