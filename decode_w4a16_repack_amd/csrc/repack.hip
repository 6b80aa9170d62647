// One-time repack of canonical int4 weights into the packed layout
// (layout version 1, described in include/w4a16.h).
//
// The onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core GEMM"
// ("What's landed") repacks the weights once into a bijective reorder built
// for coalesced loads and keeps the device repack byte-identical to the host
// reference.  This reorder is designed for gfx950: one 16-byte load per lane
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
                      int K, int N, size_t words) {
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

// Copies the scale and zero-point arrays into their regions and zero-fills
// the pad words, so the whole metadata tail of the packed buffer is written.
__global__ void __launch_bounds__(256)
repack_meta_kernel(const uint32_t *__restrict__ scales, size_t s_words,
                   const uint32_t *__restrict__ zeros, size_t z_words,
                   uint32_t *__restrict__ tail, size_t z_start_word,
                   size_t tail_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < tail_words;
       i += (size_t)gridDim.x * blockDim.x) {
    uint32_t v = 0;
    if (i < s_words) {
      v = scales[i];
    } else if (zeros != nullptr && i >= z_start_word && i < z_start_word + z_words) {
      v = zeros[i - z_start_word];
    }
    tail[i] = v;
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

  const size_t G = (size_t)(K / group);
  const size_t s_words = (size_t)N * G * (size_t)scale_bytes / 4;
  const size_t z_words = zeros ? (size_t)N * ((G + 1) / 2) / 4 : 0;
  const size_t tail_words = (off.total - off.scales) / 4;
  const size_t z_start = zeros ? (off.zeros - off.scales) / 4 : 0;
  unsigned mblocks = (unsigned)((tail_words + 255) / 256);
  if (mblocks > 4096) mblocks = 4096;
  hipLaunchKernelGGL(repack_meta_kernel, dim3(mblocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t *>(scales), s_words,
                     reinterpret_cast<const uint32_t *>(zeros), z_words,
                     reinterpret_cast<uint32_t *>(packed + off.scales), z_start,
                     tail_words);
  return hipGetLastError();
}

}  // namespace w4a16
