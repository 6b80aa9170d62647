// Small-M fused W4A16 GEMM/GEMV for gfx950 (M <= 16): the plain kernels
// (no RMSNorm prologue, or the prologue staged by stage.hip) and the
// configuration table the planner reads.  The kernel and its design notes
// are in stream_kernel.h.
#include "stream_kernel.h"

namespace w4a16 {

const StreamCfg kStreamCfgs[kNumStreamCfgs] = {
#define W4A16_CFG_ROW(cpw, kpw, nwk, pd) {cpw, kpw, nwk, pd},
    W4A16_STREAM_CFGS(W4A16_CFG_ROW)
#undef W4A16_CFG_ROW
};

hipError_t launch_stream(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                         bool gate_up, hipStream_t stream) {
  if (a.gamma != nullptr)
    return a.resid != nullptr ? launch_stream_skip(a, pl, group, scale_f32, gate_up, stream)
                              : launch_stream_rms(a, pl, group, scale_f32, gate_up, stream);
  return launch_stream_cfg<0>(a, pl, group, scale_f32, gate_up, stream);
}

}  // namespace w4a16
