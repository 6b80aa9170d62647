// One-time repack of canonical int4 weights into the packed layout
// (layout version 1, described in include/w4a16.h).
//
// Following the onnx-genai pull request "Marlin-style fused fp16xint4
// tensor-core GEMM" ("What's landed"), the weights are reordered once,
// without loss, so that every weight load is coalesced; the bytes written
// here must equal those of the oracle's host repack.  The reorder itself is
// this library's, designed for gfx950: one 16-byte load per lane
// (1 KiB per 64-lane wavefront) delivers, in each 32-bit word, the eight codes
// one v_mfma_f32_16x16x32_f16 B operand slot needs, in the bit order that the
// in-register exponent-bias unpack turns into fp16 pairs with two mask
// operations and one shift.
#include "common.h"

namespace w4a16 {

// One thread per packed 32-bit word.  Word o = ((t*KC + kc)*64 + lane)*4 + d
// holds codes k = 128*kc + 32*d + 8*(lane/16) + j (j = 0..7) of column
// n = 16*t + lane%16.  Those eight codes are one aligned 32-bit word of the
// canonical row n (code j in bits 4j); code j moves to nibble
// pos(j) = 4*(j%2) + j/2 of the packed word.
__global__ void __launch_bounds__(256)
repack_weights_kernel(const uint32_t *__restrict__ q, uint32_t *__restrict__ out,
                      int K, int /*N: implied by words*/, size_t words) {
  size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= words) return;
  const int d = (int)(o & 3);
  const int lane = (int)((o >> 2) & 63);
  const size_t tile = o >> 8;
  const int KC = K / kTileK;
  const int kc = (int)(tile % (size_t)KC);
  const size_t t = tile / (size_t)KC;
  const size_t n = t * kTileN + (size_t)(lane & 15);
  const int k0 = kc * kTileK + 32 * d + 8 * (lane >> 4);
  // byte offset n*K/2 + k0/2 is a multiple of 4 (K % 128 == 0, k0 % 8 == 0)
  const uint32_t x = q[(n * (size_t)K / 2 + (size_t)k0 / 2) / 4];
  uint32_t y = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t code = (x >> (4 * j)) & 0xFu;
    const int pos = 4 * (j & 1) + (j >> 1);
    y |= code << (4 * pos);
  }
  out[o] = y;
}

// Writes the metadata tail of the packed buffer byte by byte: scales in
// [N/16][G][16] element order, zero-points in [N/16][G][16]-nibble order, and
// zero pad bytes.  One-time work (a few MB at most), kept simple.
__global__ void __launch_bounds__(256)
repack_meta_kernel(const uint8_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
                   int /*N: implied by the byte counts*/, int G, int sb, size_t s_bytes,
                   size_t z_off, size_t z_bytes,
                   uint8_t *__restrict__ tail, size_t tail_bytes) {
  const size_t zrow = (size_t)(G + 1) / 2;
  for (size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x; b < tail_bytes;
       b += (size_t)gridDim.x * blockDim.x) {
    uint8_t v = 0;
    if (b < s_bytes) {
      const size_t e = b / sb;  // packed element (t, i, c)
      const size_t t = e / ((size_t)G * 16);
      const size_t i = (e / 16) % G;
      const size_t n = t * 16 + e % 16;
      v = scales[(n * G + i) * sb + b % sb];
    } else if (zeros != nullptr && b >= z_off && b < z_off + z_bytes) {
      const size_t zb = b - z_off;  // packed byte: nibbles 2p, 2p+1 of (t, i)
      const size_t t = zb / ((size_t)G * 8);
      const size_t i = (zb / 8) % G;
      const size_t n0 = t * 16 + 2 * (zb % 8);
      const uint8_t lo = (zeros[n0 * zrow + i / 2] >> (4 * (i & 1))) & 15;
      const uint8_t hi = (zeros[(n0 + 1) * zrow + i / 2] >> (4 * (i & 1))) & 15;
      v = (uint8_t)(lo | (hi << 4));
    }
    tail[b] = v;
  }
}

hipError_t launch_repack(const uint8_t *qweight, const void *scales,
                         const uint8_t *zeros, int K, int N, int group,
                         int scale_bytes, uint8_t *packed, hipStream_t stream) {
  const PackedOffsets off = packed_offsets(K, N, group, scale_bytes, zeros != nullptr);
  const size_t words = (size_t)K * (size_t)N / 8;
  const unsigned blocks = (unsigned)((words + 255) / 256);
  hipLaunchKernelGGL(repack_weights_kernel, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t *>(qweight),
                     reinterpret_cast<uint32_t *>(packed), K, N, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int G = K / group;
  const size_t s_bytes = (size_t)N * G * scale_bytes;
  const size_t tail_bytes = off.total - off.scales;
  const size_t z_off = zeros ? off.zeros - off.scales : 0;
  const size_t z_bytes = zeros ? (size_t)N * G / 2 : 0;
  unsigned mblocks = (unsigned)((tail_bytes + 255) / 256);
  if (mblocks > 8192) mblocks = 8192;
  hipLaunchKernelGGL(repack_meta_kernel, dim3(mblocks), dim3(256), 0, stream,
                     static_cast<const uint8_t *>(scales), zeros, N, G, scale_bytes, s_bytes,
                     z_off, z_bytes, packed + off.scales, tail_bytes);
  return hipGetLastError();
}

}  // namespace w4a16
