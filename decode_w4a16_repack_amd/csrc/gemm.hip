// Fused fp16 x int4 group-quantized GEMM for gfx950 (CDNA4).
//
// Method (onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
// GEMM"): the weights arrive repacked once ("What's landed"), the int4 codes
// are unpacked in registers, the zero-point is subtracted, the matrix cores
// contract fp16 activations with the exact integers (q - zp), and each
// group's fp32 partial is multiplied by its scale after the contraction.
// Split-K ("P2 - widen the win: split-K") partitions the k tiles over
// workgroups; the partial sums are reduced in a fixed order by the last
// workgroup to arrive, so results are deterministic.  Epilogues: bias and
// bias + ReLU ("Fusion benchmark" page), the RMSNorm prologue ("fused RMS-norm"
// update) and the paired gate/up SwiGLU ("gate_up SwiGLU MLP fusion" update).
//
// gfx950 design (not the page's SM80 mma.sync design):
//  * one workgroup = 4 wavefronts of 64 lanes; wavefront w owns the 16-column
//    weight tile 4*blockIdx.x + w and MT 16-row m tiles;
//  * each lane streams its own 16 bytes of every 1 KiB packed tile
//    (global_load_dwordx4, fully coalesced) through a register ring DW tiles
//    deep, so HBM sees many independent 1 KiB requests per wavefront;
//  * activations are staged through LDS in rounds of DA k tiles, double
//    buffered (one barrier per round), rows padded by 16 bytes so the
//    ds_read_b128 fragment reads of 16 rows are conflict-free;
//  * one packed 32-bit word becomes the eight fp16 values (q - zp) of one
//    v_mfma_f32_16x16x32_f16 B operand with two mask-or operations, one
//    shift and four packed fp16 adds/fmas (exponent-bias trick: OR a nibble
//    into the mantissa of 1024.0, then subtract 1024 + zp);
//  * the group accumulator starts each group from an inline zero, so the
//    scale step is 4 fp32 FMAs per lane per group; group 16 (half of one
//    32-deep MFMA) issues two MFMAs with the other half's B lanes zeroed.
#include "common.h"

namespace w4a16 {

namespace {

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) {
  return __builtin_bit_cast(f16x2, v);
}

// Eight codes of one packed word -> fp16 (q - z), exact.  Code j of the word
// sits in bits 4*(j/2) (even j) or 16 + 4*(j/2) (odd j); zlo = -(1024 + z),
// zhi = -(64 + z) in both halves.
__device__ __forceinline__ f16x8 unpack8(uint32_t w, f16x2 zlo, f16x2 zhi) {
  const uint32_t magic = 0x64006400u;  // fp16 1024.0 in both halves
  const uint32_t w8 = w >> 8;
  const f16x2 t0 = as_f16x2((w & 0x000F000Fu) | magic);   // 1024 + q, j = 0, 1
  const f16x2 t1 = as_f16x2((w & 0x00F000F0u) | magic);   // 1024 + 16q, j = 2, 3
  const f16x2 t2 = as_f16x2((w8 & 0x000F000Fu) | magic);  // j = 4, 5
  const f16x2 t3 = as_f16x2((w8 & 0x00F000F0u) | magic);  // 16x, j = 6, 7
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

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// Per (column, k tile) metadata of one lane: the scales of the 128/G groups
// of the tile, raw, and their zero-point nibbles, raw.
template <int G, bool SF32>
struct Meta {
  static constexpr int GPC = 128 / G;
  static constexpr int SW = (GPC * (SF32 ? 4 : 2) + 3) / 4;
  uint32_t s[SW];
  uint32_t z;
};

template <int G, bool SF32>
__device__ __forceinline__ void load_meta(Meta<G, SF32> &m,
                                          const uint8_t *__restrict__ srow,
                                          const uint8_t *__restrict__ zrow,
                                          int kc, bool has_zp) {
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  const uint8_t *sp = srow + (size_t)kc * GPC * SB;
  constexpr int bytes = GPC * SB;
  if constexpr (bytes == 2) {
    m.s[0] = *reinterpret_cast<const uint16_t *>(sp);
  } else if constexpr (bytes == 4) {
    m.s[0] = *reinterpret_cast<const uint32_t *>(sp);
  } else if constexpr (bytes == 8) {
    const u32x2 v = *reinterpret_cast<const u32x2 *>(sp);
    m.s[0] = v[0];
    m.s[1] = v[1];
  } else if constexpr (bytes == 16) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(sp);
    m.s[0] = v[0]; m.s[1] = v[1]; m.s[2] = v[2]; m.s[3] = v[3];
  } else {
    const u32x4 v0 = *reinterpret_cast<const u32x4 *>(sp);
    const u32x4 v1 = *reinterpret_cast<const u32x4 *>(sp + 16);
    m.s[0] = v0[0]; m.s[1] = v0[1]; m.s[2] = v0[2]; m.s[3] = v0[3];
    m.s[4] = v1[0]; m.s[5] = v1[1]; m.s[6] = v1[2]; m.s[7] = v1[3];
  }
  if (has_zp) {
    if constexpr (G == 128) {
      m.z = zrow[kc >> 1];
    } else if constexpr (G == 64) {
      m.z = zrow[kc];
    } else if constexpr (G == 32) {
      m.z = *reinterpret_cast<const uint16_t *>(zrow + 2 * (size_t)kc);
    } else {
      m.z = *reinterpret_cast<const uint32_t *>(zrow + 4 * (size_t)kc);
    }
  } else {
    m.z = 0x88888888u;  // symmetric: zero-point 8 everywhere
  }
}

template <int G, bool SF32>
__device__ __forceinline__ float scale_of(const Meta<G, SF32> &m, int gl) {
  if constexpr (SF32) {
    return __builtin_bit_cast(float, m.s[gl]);
  } else {
    const uint16_t h = (uint16_t)(m.s[gl >> 1] >> (16 * (gl & 1)));
    return (float)__builtin_bit_cast(f16, h);
  }
}

// Contract one k tile (4 MFMA steps of 32 k) of one weight tile with MT m
// tiles of staged activations and add the scaled group sums into acc.
template <int MT, int G, bool SF32>
__device__ __forceinline__ void mma_tile(f32x4 (&acc)[MT], const u32x4 &w,
                                         const Meta<G, SF32> &meta, int kc,
                                         const f16 *__restrict__ lds_tile,
                                         int lds_stride, int lane, int mrows) {
  const int kq = lane >> 4;
  const int arow = lane & 15;
  f32x4 accg[MT];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const f16x8 zero8 = {};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // zero-point of this lane's B slot (k = 32d + 8kq .. +7 of the tile)
    const int gl_b = (G == 16) ? (2 * d + (kq >> 1)) : (32 * d) / G;
    const int znib = (G == 128) ? (kc & 1) : gl_b;
    const int z = (int)((meta.z >> (4 * znib)) & 15u);
    const f16 zl = (f16)(float)(-(1024 + z));
    const f16 zh = (f16)(float)(-(64 + z));
    const f16x2 zlo = {zl, zl};
    const f16x2 zhi = {zh, zh};
    const f16x8 b = unpack8(w[d], zlo, zhi);
    f16x8 a[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int row = 16 * t + arow;
      a[t] = zero8;
      if (row < mrows)
        a[t] = *reinterpret_cast<const f16x8 *>(lds_tile + row * lds_stride +
                                                32 * d + 8 * kq);
    }
    if constexpr (G >= 32) {
      constexpr int SPG = G / 32;  // MFMA steps per group
#pragma unroll
      for (int t = 0; t < MT; ++t)
        accg[t] = mfma16(a[t], b, (d % SPG == 0) ? zero4 : accg[t]);
      if ((d + 1) % SPG == 0) {
        const float s = scale_of<G, SF32>(meta, (32 * d) / G);
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] += accg[t] * s;
      }
    } else {
      // group 16: k slots kq = 0, 1 belong to group 2d, kq = 2, 3 to 2d + 1
      const f16x8 blo = (kq < 2) ? b : zero8;
      const f16x8 bhi = (kq < 2) ? zero8 : b;
      const float s0 = scale_of<G, SF32>(meta, 2 * d);
      const float s1 = scale_of<G, SF32>(meta, 2 * d + 1);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const f32x4 p0 = mfma16(a[t], blo, zero4);
        const f32x4 p1 = mfma16(a[t], bhi, zero4);
        acc[t] += p0 * s0;
        acc[t] += p1 * s1;
      }
    }
  }
}

// Tile parameters per MT: DA k tiles of activations per LDS round, DW k
// tiles in flight per weight stream.
template <int MT> struct Cfg;
template <> struct Cfg<1> { static constexpr int DA = 4, DW = 8; };
template <> struct Cfg<2> { static constexpr int DA = 2, DW = 8; };
template <> struct Cfg<4> { static constexpr int DA = 1, DW = 4; };

template <int MT, int G, bool SF32, bool GU>
__global__ void __launch_bounds__(256)
gemm_kernel(const GemmArgs p) {
  constexpr int NW = GU ? 2 : 1;             // weight streams
  constexpr int DA = Cfg<MT>::DA;
  constexpr int DW = GU ? Cfg<MT>::DW / 2 : Cfg<MT>::DW;
  static_assert(DW % DA == 0, "ring depth must hold whole LDS rounds");
  constexpr int MR = 16 * MT;                // LDS rows
  constexpr int LDS_STRIDE = DA * kTileK + 8;  // halves per LDS row (+16 B pad)
  constexpr int TPR = 256 / MR;              // staging threads per row
  constexpr int SEG = DA * 16 / TPR;         // 16-byte segments per thread per round

  __shared__ __attribute__((aligned(16))) f16 lds_a[2][MR * LDS_STRIDE];
  __shared__ float rms_sum[MR];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int NTL = p.N / kTileN;
  const int KC = p.K / kTileK;
  const int ct = blockIdx.x * 4 + wave;
  const bool active = ct < NTL;
  const int s = blockIdx.y;
  const int S = p.split;
  const int m0 = blockIdx.z * MR;
  const int mrows = min(MR, p.M - m0);
  const int kc_begin = s * p.cps;
  const int nch = min(KC, kc_begin + p.cps) - kc_begin;
  const int nrounds = (nch + DA - 1) / DA;
  const bool rms = p.gamma != nullptr;
  const bool has_zp = p.has_zp != 0;
  const int G_all = p.K / G;
  const size_t zrow_bytes = (size_t)(G_all + 1) / 2;
  const int ncol = ct * kTileN + (lane & 15);  // this lane's column

  // weight and metadata streams of this lane
  const uint8_t *wbase[NW];
  const uint8_t *srow[NW];
  const uint8_t *zrow[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    wbase[i] = p.w[i] + (size_t)ct * KC * kTileBytes + (size_t)lane * 16;
    srow[i] = reinterpret_cast<const uint8_t *>(p.scales[i]) +
              (size_t)ncol * G_all * (SF32 ? 4 : 2);
    zrow[i] = has_zp ? p.zeros[i] + (size_t)ncol * zrow_bytes : nullptr;
  }

  u32x4 ring_w[NW][DW];
  Meta<G, SF32> ring_m[NW][DW];

  // prologue: fill the weight ring
  if (active) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      if (j < nch) {
        const int kc = kc_begin + j;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          ring_w[i][j] = *reinterpret_cast<const u32x4 *>(wbase[i] + (size_t)kc * kTileBytes);
          load_meta<G, SF32>(ring_m[i][j], srow[i], zrow[i], kc, has_zp);
        }
      }
    }
  }

  // activation staging: thread -> (row, segments)
  const int srow_a = tid / TPR;
  const int su = tid % TPR;
  const bool stage_row = srow_a < mrows;
  const f16 *arow_g = p.A + (size_t)(m0 + (stage_row ? srow_a : 0)) * p.K;
  u32x4 areg[SEG];
  u32x4 greg[SEG];
  float ss = 0.f;  // this thread's share of the row's sum of squares

  auto stage_load = [&](int r) {
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int seg = su + TPR * i;
      const int c = r * DA + seg / 16;
      if (stage_row && c < nch) {
        const size_t k = (size_t)(kc_begin + c) * kTileK + (seg % 16) * 8;
        areg[i] = *reinterpret_cast<const u32x4 *>(arow_g + k);
        if (rms) greg[i] = *reinterpret_cast<const u32x4 *>(p.gamma + k);
      }
    }
  };
  auto stage_store = [&](int r, f16 *buf) {
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int seg = su + TPR * i;
      const int c = r * DA + seg / 16;
      if (stage_row && c < nch) {
        u32x4 v = areg[i];
        if (rms) {
          const f16x8 a = __builtin_bit_cast(f16x8, v);
          const f16x8 g = __builtin_bit_cast(f16x8, greg[i]);
          f16x8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float af = (float)a[e];
            ss += af * af;
            x[e] = (f16)(af * (float)g[e]);
          }
          v = __builtin_bit_cast(u32x4, x);
        }
        *reinterpret_cast<u32x4 *>(buf + srow_a * LDS_STRIDE + seg * 8) = v;
      }
    }
  };

  stage_load(0);
  stage_store(0, lds_a[0]);
  __syncthreads();
  if (nrounds > 1) stage_load(1);

  f32x4 acc[NW][MT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int base = 0; base < nch; base += DW) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const int c = base + j;
      if (c < nch) {
        const int r = c / DA;
        const int jj = j % DA;  // == c % DA since DW % DA == 0
        if (active) {
          u32x4 wv[NW];
          Meta<G, SF32> mv[NW];
#pragma unroll
          for (int i = 0; i < NW; ++i) {
            wv[i] = ring_w[i][j];
            mv[i] = ring_m[i][j];
          }
          if (c + DW < nch) {
            const int kc2 = kc_begin + c + DW;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
              ring_w[i][j] = *reinterpret_cast<const u32x4 *>(wbase[i] + (size_t)kc2 * kTileBytes);
              load_meta<G, SF32>(ring_m[i][j], srow[i], zrow[i], kc2, has_zp);
            }
          }
          const f16 *tile = lds_a[r & 1] + jj * kTileK;
#pragma unroll
          for (int i = 0; i < NW; ++i)
            mma_tile<MT, G, SF32>(acc[i], wv[i], mv[i], kc_begin + c, tile,
                                  LDS_STRIDE, lane, mrows);
        }
        if (jj == DA - 1 || c == nch - 1) {  // end of LDS round r
          if (r + 1 < nrounds) stage_store(r + 1, lds_a[(r + 1) & 1]);
          __syncthreads();
          if (r + 2 < nrounds) stage_load(r + 2);
        }
      }
    }
  }

  // sum of squares of each staged row over this split's k range
  if (rms) {
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, TPR);
    if (su == 0 && stage_row) rms_sum[srow_a] = ss;
  }

  const int blk = blockIdx.z * gridDim.x + blockIdx.x;
  if (S > 1) {
    // publish this split's partial sums, then let the last arrival reduce
    if (active) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * t + 4 * (lane >> 4) + e;
          if (row < mrows) {
#pragma unroll
            for (int i = 0; i < NW; ++i)
              p.ws_part[(((size_t)s * NW + i) * p.M + m0 + row) * p.N + ncol] = acc[i][t][e];
          }
        }
    }
    if (rms && su == 0 && stage_row)
      p.ws_rms[((size_t)blk * S + s) * 64 + srow_a] = ss;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&p.ws_cnt[blk], 1u);
      is_last = (prev == (unsigned)(S - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (active) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * t + 4 * (lane >> 4) + e;
          if (row < mrows) {
#pragma unroll
            for (int i = 0; i < NW; ++i) {
              float v = 0.f;
              for (int s2 = 0; s2 < S; ++s2) {
                v += (s2 == s) ? acc[i][t][e]
                               : p.ws_part[(((size_t)s2 * NW + i) * p.M + m0 + row) * p.N + ncol];
              }
              acc[i][t][e] = v;
            }
          }
        }
    }
    if (rms && tid < mrows) {
      float v = 0.f;
      for (int s2 = 0; s2 < S; ++s2)
        v += (s2 == s) ? rms_sum[tid] : p.ws_rms[((size_t)blk * S + s2) * 64 + tid];
      rms_sum[tid] = v;  // rows are only read after the barrier below
    }
    if (tid == 0) p.ws_cnt[blk] = 0u;  // ready for the next call
  }
  __syncthreads();

  // epilogue: lane holds column ncol, rows 16t + 4*(lane/16) + e
  if (!active) return;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * t + 4 * (lane >> 4) + e;
      if (row < mrows) {
        float rs = 1.0f;
        if (rms) rs = 1.0f / sqrtf(rms_sum[row] / (float)p.K + p.eps);
        float y;
        if constexpr (GU) {
          const float g = acc[0][t][e] * rs;
          const float u = acc[1][t][e] * rs;
          y = silu(g) * u;
        } else {
          y = acc[0][t][e] * rs;
          if (p.epilogue != 0) y += (float)p.bias[ncol];
          if (p.epilogue == 2) y = y > 0.f ? y : 0.f;
        }
        p.out[(size_t)(m0 + row) * p.N + ncol] = (f16)y;
      }
    }
}

template <int MT, int G, bool SF32, bool GU>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<MT, G, SF32, GU>), dim3(pl.gx, pl.gy, pl.gz),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int MT, int G>
hipError_t launch_mg(const GemmArgs &a, const Plan &pl, bool sf32, bool gu,
                     hipStream_t st) {
  if (sf32) return gu ? launch_t<MT, G, true, true>(a, pl, st) : launch_t<MT, G, true, false>(a, pl, st);
  return gu ? launch_t<MT, G, false, true>(a, pl, st) : launch_t<MT, G, false, false>(a, pl, st);
}

template <int MT>
hipError_t launch_m(const GemmArgs &a, const Plan &pl, int group, bool sf32,
                    bool gu, hipStream_t st) {
  switch (group) {
    case 16: return launch_mg<MT, 16>(a, pl, sf32, gu, st);
    case 32: return launch_mg<MT, 32>(a, pl, sf32, gu, st);
    case 64: return launch_mg<MT, 64>(a, pl, sf32, gu, st);
    default: return launch_mg<MT, 128>(a, pl, sf32, gu, st);
  }
}

}  // namespace

Plan make_plan(int M, int K, int N, int group, bool gate_up) {
  (void)group;
  Plan p{};
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int NTL = N / kTileN;
  const int KC = K / kTileK;
  const int NW = gate_up ? 2 : 1;
  p.gx = (NTL + 3) / 4;
  p.gz = (M + 16 * p.mt - 1) / (16 * p.mt);
  const int base = p.gx * p.gz;
  // Aim for about four workgroups per CU (256 CUs), but keep the fp32
  // partial-sum traffic (written and read once: 8*S*M*N*NW bytes) under a
  // tenth of the int4 weight bytes (K*N/2 per stream).
  int S = (1024 + base - 1) / base;
  const long cap = (long)K / (160L * M);
  if (S > cap) S = (int)cap;
  if (S > 8) S = 8;
  if (S > KC) S = KC;
  if (S < 1) S = 1;
  p.cps = (KC + S - 1) / S;
  p.split = (KC + p.cps - 1) / p.cps;
  p.gy = p.split;
  size_t off = 0;
  if (p.split > 1) {
    p.ws_part_off = off;
    off = align256(off + (size_t)p.split * NW * M * N * 4);
    p.ws_rms_off = off;
    off = align256(off + (size_t)base * p.split * 64 * 4);
    p.ws_cnt_off = off;
    off = align256(off + (size_t)base * 4);
  }
  p.ws_total = off;
  return p;
}

hipError_t launch_gemm(const GemmArgs &a, const Plan &pl, int group,
                       bool scale_f32, bool gate_up, hipStream_t stream) {
  switch (pl.mt) {
    case 1: return launch_m<1>(a, pl, group, scale_f32, gate_up, stream);
    case 2: return launch_m<2>(a, pl, group, scale_f32, gate_up, stream);
    default: return launch_m<4>(a, pl, group, scale_f32, gate_up, stream);
  }
}

}  // namespace w4a16
