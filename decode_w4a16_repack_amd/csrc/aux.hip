// Measurement aids: the separate passes of the unfused chain, streaming
// probes for the achievable HBM rate, and two probes of a compute unit's
// own data paths (LDS reads, and global-to-LDS copies of data held in L2)
// that bound the MFMA-tile kernel.
//
// The "Fusion benchmark" page measures a fused kernel against the unfused
// chain at the same shape: matmul, then a bias pass, then a ReLU pass, each
// reading and writing memory.  These kernels are those passes (and the
// RMSNorm pass that stages a normalized activation before a plain GEMM).  They
// are deliberately plain one-pass kernels: vectorized 16-byte accesses, one
// read and one write per element.
#include "common.h"

namespace w4a16 {

namespace {

__global__ void __launch_bounds__(256)
add_bias_kernel(const f16 *__restrict__ in, const f16 *__restrict__ bias,
                int N, size_t vecs, f16 *__restrict__ out) {
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < vecs;
       v += (size_t)gridDim.x * blockDim.x) {
    const size_t e = v * 8;
    const int n = (int)(e % (size_t)N);
    const f16x8 x = *reinterpret_cast<const f16x8 *>(in + e);
    const f16x8 b = *reinterpret_cast<const f16x8 *>(bias + n);
    f16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (f16)((float)x[i] + (float)b[i]);
    *reinterpret_cast<f16x8 *>(out + e) = y;
  }
}

__global__ void __launch_bounds__(256)
relu_kernel(const f16 *__restrict__ in, size_t vecs, f16 *__restrict__ out) {
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < vecs;
       v += (size_t)gridDim.x * blockDim.x) {
    const f16x8 x = *reinterpret_cast<const f16x8 *>(in + v * 8);
    f16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] > (f16)0.0f ? x[i] : (f16)0.0f;
    *reinterpret_cast<f16x8 *>(out + v * 8) = y;
  }
}

// One workgroup per row: sum of squares with a fixed-order tree, then
// out = fp16(a * gamma / sqrt(mean + eps)).
__global__ void __launch_bounds__(256)
rmsnorm_kernel(const f16 *__restrict__ A, const f16 *__restrict__ gamma,
               float eps, int K, f16 *__restrict__ out) {
  __shared__ float part[256];
  const int m = blockIdx.x;
  const f16 *a = A + (size_t)m * K;
  float ss = 0.f;
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const f16x8 x = *reinterpret_cast<const f16x8 *>(a + k);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += (float)x[i] * (float)x[i];
  }
  part[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float r = 1.0f / sqrtf(part[0] / (float)K + eps);
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const f16x8 x = *reinterpret_cast<const f16x8 *>(a + k);
    const f16x8 g = *reinterpret_cast<const f16x8 *>(gamma + k);
    f16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (f16)((float)x[i] * (float)g[i] * r);
    *reinterpret_cast<f16x8 *>(out + (size_t)m * K + k) = y;
  }
}

// Streaming read: four independent 16-byte loads per thread per iteration,
// folded with xor so the loads cannot be removed; one word per workgroup.
__global__ void __launch_bounds__(256)
probe_read_kernel(const u32x4 *__restrict__ buf, size_t vecs,
                  uint32_t *__restrict__ sink) {
  __shared__ uint32_t red[256];
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; v + 3 * stride < vecs; v += 4 * stride) {
    const u32x4 a = buf[v], b = buf[v + stride], c = buf[v + 2 * stride],
                d = buf[v + 3 * stride];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^
           c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; v < vecs; v += stride) {
    const u32x4 a = buf[v];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] ^= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(256)
probe_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                  size_t vecs) {
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < vecs;
       v += (size_t)gridDim.x * blockDim.x)
    dst[v] = src[v];
}

// LDS read rate: each 512-thread workgroup fills 64 KiB of LDS, then every
// wavefront reads 16 chunks of 16 bytes per iteration (lane l of read r:
// chunk (l + 64 * ((r + wave + it) mod 64)) mod 4096, conflict-free) and
// folds them into one word per thread, written to sink[workgroup * 512 +
// thread].
__global__ void __launch_bounds__(512) probe_lds_read_kernel(int iters, uint32_t *sink) {
  __shared__ u32x4 buf[4096];
  const int t = threadIdx.x;
  for (int i = t; i < 4096; i += 512) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  const int lane = t & 63, w = t >> 6;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc ^= buf[(lane + 64 * ((r + w + it) & 63)) & 4095];
  }
  sink[(size_t)blockIdx.x * 512 + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Issue probe: how far independent VALU work overlaps the matrix cores.
// Every wavefront runs iters rounds of 8 v_mfma_f32_16x16x32_f16 (four
// accumulators, two MFMAs each) and X independent fp32 FMAs (sixteen
// registers; X / 8 after each MFMA), then folds its registers into one value
// per thread in sink.  The time per round against X, at one and at two
// wavefronts per SIMD, gives the MFMA time alone and what each VALU
// instruction adds to it.
template <int X>
__global__ void __launch_bounds__(512) probe_mfma_valu_kernel(int iters, float s, float *sink) {
  f32x4 acc[4] = {};
  const f16x8 a = {(f16)((float)threadIdx.x * 0.001f)};
  const f16x8 b = {(f16)1.0f};
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (float)(threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      acc[m & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[m & 3], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < X / 8; ++x) v[(m * 7 + x) & 15] = __builtin_fmaf(v[(m * 7 + x) & 15], s, 1.0f);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += v[i];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r + acc[0][0] + acc[1][1] + acc[2][2] + acc[3][3];
}

// Global-to-LDS copy rate of activation-like rows held in L2: buf is a
// 64-row fp16 matrix of K = bytes / 128 columns.  Per step, wavefront
// (wc, ks) of a 512-thread workgroup copies a quarter (four 1 KiB copies of
// four whole 256-byte row segments each, the MFMA-tile kernel's activation
// copy) of the 64 x 128 k tile 2 * step + ks + workgroup (mod K / 128) into a
// two-step ring, waits for the previous step's copies, meets the workgroup,
// and reads 16 bytes per lane back; one word per thread goes to sink.
__global__ void __launch_bounds__(512) probe_lds_copy_kernel(const uint8_t *buf, int KC, int steps,
                                                             uint32_t *sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[8 * 2 * 4096];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wc = w & 3, ks = w >> 2;
  const size_t K = (size_t)KC * 128;
  uint32_t off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int sl = (wc + 4 * q) * 64 + lane;
    const int row = sl >> 4, chunk = (sl & 15) ^ (row & 15);
    off[q] = (uint32_t)((row * K + 8 * chunk) * 2);
  }
  uint8_t *mine = ring + w * 2 * 4096;
  auto issue = [&](int step, int slot) {
    const int kt = (int)((2u * (unsigned)step + (unsigned)ks + blockIdx.x) % (unsigned)KC);
    const uint8_t *base = buf + (size_t)kt * 256;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(base + off[q]),
                                       (void __attribute__((address_space(3))) *)(mine + slot * 4096 + q * 1024),
                                       16, 0, 0);
  };
  u32x4 acc = {0, 0, 0, 0};
  issue(0, 0);
  for (int s = 0; s < steps; ++s) {
    issue(s + 1, (s + 1) & 1);  // (the last step's extra copy is waited for below)
    __builtin_amdgcn_s_waitcnt((4 & 15) | (7 << 4) | (15 << 8));  // vmcnt(4): step s landed
    __builtin_amdgcn_s_barrier();
    acc ^= *reinterpret_cast<const u32x4 *>(mine + (s & 1) * 4096 + lane * 16);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read back before the slot is refilled
    __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_s_waitcnt(0);
  sink[(size_t)blockIdx.x * 512 + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Plain reads of one packed weight matrix (KC = K/128 tiles of 1 KiB per
// 16-column tile, tile u = t*KC + kc at u*1024) under two decompositions of
// its NT*KC tiles over 512-thread workgroups, with the same load loop (one
// 16-byte load per lane per tile, eight tiles per batch, the next batch in
// flight while one is folded):
//  MODE 0: the streaming kernel's: workgroup g takes column tiles 4g..4g+3
//          over all of K, wavefront w the k tiles w*KPW .. w*KPW + KPW - 1
//          (KPW = ceil(KC/8)) of each;
//  MODE 1: the tiles split evenly over nwg workgroups: workgroup g takes the
//          contiguous range [g*U/nwg, (g+1)*U/nwg) of U = NT*KC, its
//          wavefronts dealt the range round-robin.
// One word per thread goes to sink[g * 512 + thread].
template <int MODE>
__global__ void __launch_bounds__(512) probe_tiles_kernel(const uint8_t *w, int NT, int KC, int nwg,
                                                          uint32_t *sink) {
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = blockIdx.x;
  int n, nk = 1, ct0 = 0, kb = 0;
  size_t u0 = 0;
  if constexpr (MODE == 0) {
    const int kpw = (KC + 7) / 8;
    kb = wv * kpw;
    const int nkr = max(0, min(kpw, KC - kb));  // k tiles of this slice (none past K)
    nk = max(nkr, 1);
    ct0 = 4 * g;
    n = nkr > 0 ? min(4, NT - ct0) * nkr : 0;
  } else {
    const size_t U = (size_t)NT * KC;
    u0 = (size_t)g * U / (size_t)nwg;
    const size_t cnt = (size_t)(g + 1) * U / (size_t)nwg - u0;
    n = cnt > (size_t)wv ? (int)((cnt - wv + 7) / 8) : 0;
  }
  auto unit = [&](int j) __attribute__((always_inline)) -> size_t {
    if constexpr (MODE == 0)
      return (size_t)(ct0 + j / nk) * KC + kb + j % nk;
    else
      return u0 + wv + (size_t)8 * j;
  };
  auto load8 = [&](int base, u32x4 (&v)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = base + i < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w + unit(base + i) * 1024) + lane)
                          : u32x4{0, 0, 0, 0};
  };
  u32x4 cur[8], nxt[8];
  u32x4 acc = {0, 0, 0, 0};
  load8(0, cur);
  for (int b = 0; b < n; b += 8) {
    load8(b + 8, nxt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc ^= cur[i];
      cur[i] = nxt[i];
    }
  }
  sink[(size_t)g * 512 + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

unsigned grid_for(size_t vecs, unsigned cap) {
  size_t b = (vecs + 255) / 256;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_add_bias(const f16 *in, const f16 *bias, int M, int N,
                           f16 *out, hipStream_t stream) {
  const size_t vecs = (size_t)M * N / 8;
  hipLaunchKernelGGL(add_bias_kernel, dim3(grid_for(vecs, 8192)), dim3(256), 0,
                     stream, in, bias, N, vecs, out);
  return hipGetLastError();
}

hipError_t launch_relu(const f16 *in, int M, int N, f16 *out,
                       hipStream_t stream) {
  const size_t vecs = (size_t)M * N / 8;
  hipLaunchKernelGGL(relu_kernel, dim3(grid_for(vecs, 8192)), dim3(256), 0,
                     stream, in, vecs, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const f16 *A, const f16 *gamma, float eps, int M,
                          int K, f16 *out, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, stream, A, gamma,
                     eps, K, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink,
                             hipStream_t stream) {
  const size_t vecs = bytes / 16;
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid_for(vecs / 4, 4096)), dim3(256),
                     0, stream, reinterpret_cast<const u32x4 *>(buf), vecs, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes,
                             hipStream_t stream) {
  const size_t vecs = bytes / 16;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(grid_for(vecs / 4, 8192)), dim3(256),
                     0, stream, reinterpret_cast<const u32x4 *>(src),
                     reinterpret_cast<u32x4 *>(dst), vecs);
  return hipGetLastError();
}

hipError_t launch_probe_lds_read(int workgroups, int iters, uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_lds_read_kernel, dim3(workgroups), dim3(512), 0, stream, iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_lds_copy(const void *buf, size_t bytes, int workgroups, int steps,
                                 uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_lds_copy_kernel, dim3(workgroups), dim3(512), 0, stream,
                     static_cast<const uint8_t *>(buf), (int)(bytes / 16384), steps, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_valu(int valu, int threads, int workgroups, int iters, float *sink,
                                  hipStream_t stream) {
  const float s = 0.999f;
  switch (valu) {
    case 0: hipLaunchKernelGGL(probe_mfma_valu_kernel<0>, dim3(workgroups), dim3(threads), 0, stream, iters, s, sink); break;
    case 8: hipLaunchKernelGGL(probe_mfma_valu_kernel<8>, dim3(workgroups), dim3(threads), 0, stream, iters, s, sink); break;
    case 16: hipLaunchKernelGGL(probe_mfma_valu_kernel<16>, dim3(workgroups), dim3(threads), 0, stream, iters, s, sink); break;
    case 32: hipLaunchKernelGGL(probe_mfma_valu_kernel<32>, dim3(workgroups), dim3(threads), 0, stream, iters, s, sink); break;
    case 48: hipLaunchKernelGGL(probe_mfma_valu_kernel<48>, dim3(workgroups), dim3(threads), 0, stream, iters, s, sink); break;
    case 64: hipLaunchKernelGGL(probe_mfma_valu_kernel<64>, dim3(workgroups), dim3(threads), 0, stream, iters, s, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

unsigned probe_tiles_grid(int N, int mode, int workgroups) {
  return mode == 0 ? (unsigned)((N / kTileN + 3) / 4) : (unsigned)workgroups;
}

hipError_t launch_probe_tiles(const void *w, int K, int N, int mode, int workgroups, uint32_t *sink,
                              hipStream_t stream) {
  const uint8_t *b = static_cast<const uint8_t *>(w);
  const int NT = N / kTileN, KC = K / kTileK;
  const unsigned grid = probe_tiles_grid(N, mode, workgroups);
  if (mode == 0)
    hipLaunchKernelGGL(probe_tiles_kernel<0>, dim3(grid), dim3(512), 0, stream, b, NT, KC, 0, sink);
  else
    hipLaunchKernelGGL(probe_tiles_kernel<1>, dim3(grid), dim3(512), 0, stream, b, NT, KC, workgroups, sink);
  return hipGetLastError();
}

}  // namespace w4a16
