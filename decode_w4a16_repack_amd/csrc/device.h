// Device-side building blocks shared by the GEMM kernels.
#pragma once

#include <atomic>
#include <type_traits>

#include "common.h"

namespace w4a16 {

// Raises a kernel's dynamic-LDS limit on the current device to `bytes` when a
// plan needs more than the default 64 KiB.  `limit` is the kernel's own
// per-device record of the largest size already set, so repeated launches
// (also under stream capture) make no attribute call; concurrent first
// launches from several host threads may both set it, which is harmless.
inline hipError_t raise_lds_limit(const void *kern, size_t bytes,
                                  std::atomic<size_t> (&limit)[kMaxDevices]) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return hipErrorInvalidDevice;
  }
  if (limit[dev].load(std::memory_order_acquire) >= bytes) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next launch
    return e;
  }
  size_t cur = limit[dev].load(std::memory_order_acquire);
  while (cur < bytes && !limit[dev].compare_exchange_weak(cur, bytes, std::memory_order_acq_rel)) {
  }
  return hipSuccess;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at
// compile time whatever the body's size (a #pragma unroll may give up on a
// large body, and arrays indexed by the loop variable then go to scratch).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) {
  return __builtin_bit_cast(f16x2, v);
}

// Eight codes of one packed word -> fp16 (q - z), exact.  Code j of the word
// sits in bits 4*(j/2) (even j) or 16 + 4*(j/2) (odd j).  OR-ing a nibble into
// the mantissa of fp16 1024.0 gives 1024 + q (bits 0-3 of a half) or
// 1024 + 16q (bits 4-7); subtracting 1024 + z, or scaling by 1/16 and
// subtracting 64 + z, leaves the integer q - z in [-15, 15], exact in fp16.
// zlo = -(1024 + z), zhi = -(64 + z) in both halves.
// (x & m) | o in one VALU instruction.  Written out because the compiler
// splits it into v_and + v_or when both constants are literals (GFX9 VOP3
// encodings take no literal): m goes in an SGPR, o in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
  return r;
}

__device__ __forceinline__ f16x8 unpack8(uint32_t w, f16x2 zlo, f16x2 zhi) {
  const uint32_t magic = 0x64006400u;  // fp16 1024.0 in both halves
  const uint32_t w8 = w >> 8;
  const f16x2 t0 = as_f16x2(and_or(w, 0x000F000Fu, magic));   // j = 0, 1
  const f16x2 t1 = as_f16x2(and_or(w, 0x00F000F0u, magic));   // j = 2, 3 (x16)
  const f16x2 t2 = as_f16x2(and_or(w8, 0x000F000Fu, magic));  // j = 4, 5
  const f16x2 t3 = as_f16x2(and_or(w8, 0x00F000F0u, magic));  // j = 6, 7 (x16)
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 h0 = t0 + zlo;
  const f16x2 h1 = t1 * sixteenth + zhi;
  const f16x2 h2 = t2 + zlo;
  const f16x2 h3 = t3 * sixteenth + zhi;
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const f16x4 lo = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
  const f16x4 hi = __builtin_shufflevector(h2, h3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp16 constants -(1024 + z) and -(64 + z) in both halves, for z in 0..15,
// built from their bit patterns: 1024 + z has exponent field 25 and
// mantissa z (0x6400 | z); 64 + z has exponent field 21 and mantissa 16z
// (0x5400 | z << 4); the sign bit makes them negative.
// (The OR of disjoint bit fields is written as an add so that each constant
// is one multiply-add.)
__device__ __forceinline__ void zero_consts(uint32_t z, f16x2 &zlo, f16x2 &zhi) {
  zlo = as_f16x2(z * 0x00010001u + 0xE400E400u);
  zhi = as_f16x2(z * 0x00100010u + 0xD400D400u);
}

// D = A(16x32 fp16) x B(32x16 fp16) + C, fp32.  Lane l supplies A row l%16 and
// B column l%16 at k slots 8*(l/16)..+7 (any k order works as long as A and
// B agree, which the packed layout and the LDS reads guarantee); lane l gets
// D rows 4*(l/16)+e, e = 0..3, of column l%16.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// ---------------------------------------------------------------------------
// Contraction with the zero-point taken out of the weights.
//
// (q - z) * a summed over a group equals sum(q * a) - z * sum(a), so the
// weights can enter the matrix core as the bare codes q and the zero-point
// is applied per group with the group's activation row sums U:
//   acc += s * sum_k q*a  -  s * z * U.
// The codes are placed into fp16 without any arithmetic: masking nibble
// pairs into the low mantissa bits of a zero exponent gives the fp16
// subnormals q * 2^-24 (bits 0-3) or 16q * 2^-24 (bits 4-7), exact.  The
// activation slots that meet a 16q code (slots 2, 3, 6, 7 of each 8) are
// pre-scaled by 1/16 (exact for normal fp16 values), so every product is
// q * a * 2^-24, exact in the fp32 accumulator; the group scale carries
// the 2^24 back.  U comes from the same activation fragments times a
// constant B of 1 (or 16 in the pre-scaled slots), one MFMA per 32-k step,
// shared by every column tile that uses the fragments.

// Eight codes of one packed word -> fp16 q * 2^-24 (slots 0, 1, 4, 5) and
// 16q * 2^-24 (slots 2, 3, 6, 7).
__device__ __forceinline__ f16x8 unpack8_sub(uint32_t w) {
  const uint32_t w8 = w >> 8;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
  return __builtin_bit_cast(f16x8, v);
}

// Activation fragment pre-scaled for unpack8_sub: slots 2, 3, 6, 7 times 1/16.
__device__ __forceinline__ f16x8 prescale_frag(f16x8 x) {
  const f16x8 m = {(f16)1.0f, (f16)1.0f, (f16)0.0625f, (f16)0.0625f,
                   (f16)1.0f, (f16)1.0f, (f16)0.0625f, (f16)0.0625f};
  return x * m;
}

// Group row sums of a pre-scaled activation k tile (128 k): ug[gl] holds,
// for this lane's output rows 4*(l/16)+e, the sum of the activations of
// group gl (0 .. 128/G - 1) of the tile.
template <int G>
__device__ __forceinline__ void group_row_sums(f32x4 (&ug)[128 / G], const f16x8 (&a)[4], int kq) {
  const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)16.0f, (f16)16.0f,
                      (f16)1.0f, (f16)1.0f, (f16)16.0f, (f16)16.0f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (G >= 32) {
    constexpr int SPG = G / 32;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      ug[d / SPG] = mfma16(a[d], ones, (d % SPG == 0) ? zero4 : ug[d / SPG]);
  } else {
    const f16x8 zero8 = {};
    const f16x8 olo = (kq < 2) ? ones : zero8;
    const f16x8 ohi = (kq < 2) ? zero8 : ones;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      ug[2 * d] = mfma16(a[d], olo, zero4);
      ug[2 * d + 1] = mfma16(a[d], ohi, zero4);
    }
  }
}

// An empty asm that reads and writes an accumulator: the scaled group sums
// are added where they are made.  Left to itself the compiler may defer the
// adds of a whole loop to its end, keep every group sum and scale alive until
// then and spill them (two weight streams, or many groups per k tile).
__device__ __forceinline__ void pin_acc(f32x4 &acc) { asm volatile("" : "+v"(acc)); }

// Contract one packed k tile of one 16-column weight tile with one 16-row
// tile of pre-scaled activation fragments a[d] (d = 32-k step), given the
// tile's group row sums ug; zp_of(gl) / scale_of(gl) as for contract_tile.
// PIN: pin the accumulator after each group (pin_acc).
template <int G, bool PIN = false, class ZpOf, class ScaleOf>
__device__ __forceinline__ void contract_tile_sub(f32x4 &acc, const u32x4 &w, const f16x8 (&a)[4],
                                                  const f32x4 (&ug)[128 / G], int kq, ZpOf zp_of,
                                                  ScaleOf scale_of) {
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  auto apply = [&](const f32x4 &part, int gl) __attribute__((always_inline)) {
    const float s = scale_of(gl);
    const float s24 = s * 16777216.0f;  // 2^24: the codes entered as q * 2^-24
    const float sz = -s * (float)zp_of(gl);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc[e] = __builtin_fmaf(ug[gl][e], sz, __builtin_fmaf(part[e], s24, acc[e]));
    if constexpr (PIN) pin_acc(acc);
  };
  if constexpr (G >= 32) {
    constexpr int SPG = G / 32;
    f32x4 accg;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      accg = mfma16(a[d], unpack8_sub(w[d]), (d % SPG == 0) ? zero4 : accg);
      if ((d + 1) % SPG == 0) apply(accg, d / SPG);
    }
  } else {
    const f16x8 zero8 = {};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f16x8 b = unpack8_sub(w[d]);
      const f32x4 p0 = mfma16(a[d], (kq < 2) ? b : zero8, zero4);
      const f32x4 p1 = mfma16(a[d], (kq < 2) ? zero8 : b, zero4);
      apply(p0, 2 * d);
      apply(p1, 2 * d + 1);
    }
  }
}

// One lane's 16 bytes of a packed weight tile.  Where the weights are read
// once per call (STREAMING), the load is marked non-temporal: it streams
// through L2 without displacing the lines that are reused (activation rows,
// scales), and the HBM stream runs faster (M=1 K=5120 N=13824: 9.0 -> 8.35
// us).  A kernel whose row blocks re-read the same weights keeps them in L2.
template <bool STREAMING = true>
__device__ __forceinline__ u32x4 load_weights(const uint8_t *tile_base, int lane) {
  if constexpr (STREAMING)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(tile_base) + lane);
  else
    return reinterpret_cast<const u32x4 *>(tile_base)[lane];
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes at src land at lds_base + 16 * l.  lds_base must be the
// same for the whole wavefront.  Completion is tracked by the vector-memory
// counter, like any load.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                   (void __attribute__((address_space(3))) *)lds_base, 16, 0, 0);
}

// Same with 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes land
// at lds_base + 4 * l.
__device__ __forceinline__ void copy4_to_lds(const void *src, void *lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                   (void __attribute__((address_space(3))) *)lds_base, 4, 0, 0);
}

// The same copies as buffer loads (buffer_load_dword[x4] ... lds) from a
// raw byte range: lane l's bytes at base + voff + soff land at lds_base +
// size * l.  A kernel that keeps issuing copies while it uses registers
// loaded by plain loads takes these: the compiler counts a buffer copy in
// order with the plain loads and waits for exactly the load a register needs,
// whereas a global_load_lds still in flight makes it wait for every load
// (vmcnt(0)) before each such use.  Offsets are 32-bit; a read at or past
// `bytes` returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
  // word 3: 32-bit data format, the raw (unswizzled, stride 0) form
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds_base, 16,
                                           voff, soff, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                             void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds_base, 4,
                                           voff, soff, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited to n (< 64); the
// other counters at their maximum (no wait).  GFX9 encoding: vmcnt[3:0] in
// bits 3:0, expcnt in 6:4, lgkmcnt in 11:8, vmcnt[5:4] in 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Cross-workgroup exchange through global memory.  Agent-scope atomic
// loads and stores are coherent across the XCDs (each has its own L2) on
// their own, so split-K partials go through them; wait_stores() makes a
// wavefront's earlier stores complete (and the compiler keep them before
// it) before it signals arrival with count_arrival().
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ unsigned count_arrival(uint32_t *c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_arrival(uint32_t *c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight (a plain __syncthreads also waits for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier that leaves global loads and global-to-LDS copies in
// flight: this wavefront's LDS reads and writes are waited for (lgkmcnt(0);
// vmcnt and expcnt untouched), the compiler may not move memory accesses
// across it, and no cache or vector-memory wait is emitted (a release fence
// on LDS would also wait for the copies still in flight).
__device__ __forceinline__ void lds_only_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace w4a16
