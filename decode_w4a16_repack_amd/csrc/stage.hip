// Activation staging for the RMSNorm prologue where the product kernel does
// not run it itself: the tile kernel (M > 32), the panel kernel with a
// residual or a k split across workgroups, and the streaming kernel with a
// residual above 4 rows or a deep slice.
//
// The onnx-genai pull request's "fused RMS-norm" update normalizes the
// activation before the fused product, staging the normalized rows through
// scratch memory.  Here the staged tensor is x * gamma rounded once to fp16,
// plus each row's fp32 sum of squares; the GEMM then runs its plain kernel on
// the staged rows and multiplies row m of the result by
// 1 / sqrt(ss[m] / K + eps) in its epilogue.  With the skip prologue
// (SkipSimplifiedLayerNormalization, "Stage 2 of spec-capture" update) the
// row is first replaced by A + residual, rounded once to fp16, which is also
// written out.
//
// Why not inside the tile kernel: its wavefronts read every activation
// fragment from the shared LDS stage, so each of the four column quarters
// would repeat the x * gamma multiply and the sums of squares of every row;
// one pass over the M x K activations costs less.  The streaming and panel
// kernels, which load each fragment once, run the prologue themselves.
#include "common.h"

namespace w4a16 {

namespace {

// One workgroup of 256 threads per row; 8 consecutive k per thread and step.
// Sum of squares: fp32 per thread (products of fp16 values are exact in
// fp32), then a fixed-order tree (wavefront butterfly, wavefronts in order):
// run-to-run identical.
__global__ void __launch_bounds__(256)
rms_stage_kernel(const f16 *__restrict__ A, const f16 *__restrict__ resid,
                 f16 *__restrict__ resid_out, const f16 *__restrict__ gamma, int K,
                 f16 *__restrict__ x_out, float *__restrict__ ss_out) {
  __shared__ float part[4];
  const int m = blockIdx.x;
  const size_t row = (size_t)m * K;
  float ss = 0.f;
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    f16x8 x = *reinterpret_cast<const f16x8 *>(A + row + k);
    if (resid != nullptr) {
      x = x + *reinterpret_cast<const f16x8 *>(resid + row + k);  // one rounding
      if (resid_out != nullptr) *reinterpret_cast<f16x8 *>(resid_out + row + k) = x;
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f16x2 x2 = {x[2 * h], x[2 * h + 1]};
      ss = __builtin_amdgcn_fdot2(x2, x2, ss, false);
    }
    // the packed fp16 multiply rounds the exact product once
    *reinterpret_cast<f16x8 *>(x_out + row + k) = x * *reinterpret_cast<const f16x8 *>(gamma + k);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ss_out[m] = ((part[0] + part[1]) + part[2]) + part[3];
}

}  // namespace

hipError_t launch_rms_stage(const f16 *A, const f16 *resid, f16 *resid_out, const f16 *gamma,
                            int M, int K, f16 *x_out, float *ss_out, hipStream_t stream) {
  hipLaunchKernelGGL(rms_stage_kernel, dim3(M), dim3(256), 0, stream, A, resid, resid_out,
                     gamma, K, x_out, ss_out);
  return hipGetLastError();
}

}  // namespace w4a16
