// Small-M fused W4A16 GEMM/GEMV for gfx950 (M <= 16) with the RMSNorm
// prologue in registers (gamma read back from LDS): the instantiations of
// stream_kernel.h that carry it.
#include "stream_kernel.h"

namespace w4a16 {

hipError_t launch_stream_rms(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                             bool gate_up, hipStream_t stream) {
  return launch_stream_cfg<1>(a, pl, group, scale_f32, gate_up, stream);
}

}  // namespace w4a16
