// Small-M fused W4A16 GEMM/GEMV for gfx950: the HBM-bound decode regime.
//
// Method as in ring.hip (onnx-genai pull request "Marlin-style fused
// fp16xint4 tensor-core GEMM": repacked weights, in-register unpack, matrix
// core contraction with the exact integers (q - zp), per-group scale after
// the accumulate; split-K with a fixed-order reduction, "P2 - widen the win:
// split-K": small M is limited by the weight loads in flight).
//
// gfx950 design, for shapes whose activation rows fit in LDS whole:
//  * a workgroup is NWC 16-column weight tiles x NWK slices of k (split-K
//    inside the workgroup, reduced through LDS in slice order);
//  * first, the workgroup's activation rows (rows < M only) are copied into
//    LDS with direct global-to-LDS loads (global_load_lds_dwordx4), in
//    "fragment order" so the 16 rows one MFMA operand reads are 16
//    consecutive 16-byte slots;
//  * then every wavefront issues ALL of its weight tiles (one 16-byte load
//    per lane per 1 KiB tile) and their scale / zero-point loads - CW tiles,
//    unconditionally, so the count is a compile-time constant;
//  * one exact wait (vmcnt <= the weight loads just issued) covers the
//    activation copies, then an LDS-only barrier;
//  * tile j is contracted as soon as its own load has landed (the compiler's
//    wait before tile j allows the later tiles to stay in flight), so the
//    arithmetic overlaps the HBM stream and no barrier sits in the loop.
#include "device.h"

namespace w4a16 {

namespace {

template <int MT, int NWC, int NWK, int CW, int PD, int G, bool SF32, bool GU>
__global__ void __launch_bounds__(64 * NWC * NWK)
oneshot_kernel(const GemmArgs p) {
  static_assert(PD >= 1 && PD <= CW, "prefetch depth");
  constexpr int NWAVE = NWC * NWK;
  constexpr int NT = 64 * NWAVE;
  constexpr int NW = GU ? 2 : 1;
  constexpr int MR = 16 * MT;
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int LOADS_PER_TILE = NW;  // one 16-byte weight load per tile and stream

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wc = wave % NWC;
  const int wk = wave / NWC;
  const int NTL = p.N / kTileN;
  const int KC = p.K / kTileK;
  const int Gall = p.K / G;
  const int ct = blockIdx.x * NWC + wc;
  const bool active = ct < NTL;
  const int ctc = active ? ct : NTL - 1;
  const int s = blockIdx.y;
  const int S = p.split;
  const int m0 = blockIdx.z * MR;
  const int mrows = min(MR, p.M - m0);
  const int R = p.rows_pow2;
  const int kb = s * p.cps;
  const int nkc = min(KC, kb + p.cps) - kb;
  const int cpw = (nkc + NWK - 1) / NWK;
  const int my_kb = kb + wk * cpw;
  const int my_n = max(0, min(cpw, nkc - wk * cpw));
  const bool rms = p.gamma != nullptr;
  const bool has_zp = p.has_zp != 0;
  const int ncol = ctc * kTileN + (lane & 15);

  // LDS: activation slots (fragment order, whole k range of the workgroup;
  // aliased by the slice reduction at the end), gamma, scales, zero-points,
  // sums of squares.
  uint8_t *lA = smem;
  f16 *lG = reinterpret_cast<f16 *>(smem + p.lds_g);
  uint8_t *lS = smem + p.lds_s;  // [NW][NWC] x scopy: [group][16 columns] scales
  uint8_t *lZ = smem + p.lds_z;  // [NW][NWC] x zcopy: [group][8 bytes] zero-points
  const int GRC = p.gr;          // staged groups per column tile (capacity)
  const int scopy = (GRC * 16 * SB + 1023) / 1024 * 1024;
  const int zcopy = (GRC * 8 + 255) / 256 * 256;
  float *lRms = reinterpret_cast<float *>(smem + p.lds_r);  // [NT] + [MR]
  float *lRow = lRms + NT;
  float *lRed = reinterpret_cast<float *>(smem);

  // 1. activation rows -> LDS, direct global-to-LDS copies, before any
  //    weight load.  Slot (((tt * 4 + d) * 4 + kq) * R + row), tt = slice
  //    tile (sl * cpw + t), holds A[row][k(tt) + 32d + 8kq .. +7].
  const int n_slots = NWK * cpw * 16 * R;
  const int n_copies = (n_slots + 63) / 64;
  for (int q = wave; q < n_copies; q += NWAVE) {
    const int slot = min(q * 64 + lane, n_slots - 1);
    const int row = slot % R;
    const int rest = slot / R;
    const int kq = rest & 3;
    const int d = (rest >> 2) & 3;
    const int tt = rest >> 4;
    const int sl = tt / cpw;
    const int kc = min(kb + sl * cpw + (tt - sl * cpw), KC - 1);
    const int rg = m0 + min(row, mrows - 1);
    const f16 *src = p.A + (size_t)rg * p.K + (size_t)kc * kTileK + 32 * d + 8 * kq;
    copy16_to_lds(src, lA + (size_t)q * 1024);
  }
  if (rms) {
    const int n_g = (nkc * kTileK * 2 + 1023) / 1024;  // 1 KiB copies of gamma
    for (int q = wave; q < n_g; q += NWAVE) {
      const int e = min(q * 64 + lane, nkc * 16 - 1);
      const f16 *src = p.gamma + (size_t)kb * kTileK + e * 8;
      copy16_to_lds(src, reinterpret_cast<uint8_t *>(lG) + (size_t)q * 1024);
    }
  }

  // 2. scales and zero-points of the workgroup's column tiles and groups:
  //    contiguous runs in the packed layout, copied straight into LDS
  const int gb = kb * GPC;
  const int ngr = nkc * GPC;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    for (int w = 0; w < NWC; ++w) {
      const int tw = min(blockIdx.x * NWC + w, NTL - 1);
      const size_t first = (size_t)tw * Gall + gb;  // first (tile, group) record
      const int sbytes = ngr * 16 * SB;
      const uint8_t *ssrc = reinterpret_cast<const uint8_t *>(p.scales[i]) + first * 16 * SB;
      uint8_t *sdst = lS + (size_t)(i * NWC + w) * scopy;
      for (int q = wave; q * 1024 < sbytes; q += NWAVE)
        copy16_to_lds(ssrc + min(q * 1024 + lane * 16, sbytes - 16), sdst + q * 1024);
      uint8_t *zdst = lZ + (size_t)(i * NWC + w) * zcopy;
      if (has_zp) {
        const int zbytes = ngr * 8;
        const uint8_t *zsrc = p.zeros[i] + first * 8;
        for (int q = wave; q * 256 < zbytes; q += NWAVE)
          copy4_to_lds(zsrc + min(q * 256 + lane * 4, zbytes - 4), zdst + q * 256);
      } else {
        for (int e = tid; e * 4 < zcopy; e += NT)  // symmetric: every zero-point is 8
          reinterpret_cast<uint32_t *>(zdst)[e] = 0x88888888u;
      }
    }
  }

  // 3'. the first PD weight tiles of this wavefront (one 16-byte load per
  //     lane per tile and stream, unconditional: tail tiles re-read a valid
  //     tile); tile j + PD is issued when tile j is contracted, so each
  //     wavefront keeps PD tiles in flight and its arithmetic follows its
  //     own arrivals instead of bunching up after the whole stream.
  const uint8_t *wbase[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    wbase[i] = p.w[i] + (size_t)ctc * KC * kTileBytes + (size_t)lane * 16;
  u32x4 wv[NW][CW];
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    const int kc = min(my_kb + min(j, max(my_n - 1, 0)), KC - 1);
#pragma unroll
    for (int i = 0; i < NW; ++i)
      wv[i][j] = *reinterpret_cast<const u32x4 *>(wbase[i] + (size_t)kc * kTileBytes);
  };
#pragma unroll
  for (int j = 0; j < PD; ++j) issue_tile(j);

  // 3. the copies into LDS (issued before the PD tiles) have landed; with
  //    more than 63 loads in flight the issue itself waited, which already
  //    retired the copies (completion is in issue order)
  wait_vmcnt<(PD * LOADS_PER_TILE < 63 ? PD * LOADS_PER_TILE : 63)>();
  lds_barrier();

  // 4. RMSNorm prologue: per-row sums of squares (fixed order), x * gamma
  //    in place; the 1/sqrt(mean + eps) factor waits for the epilogue.
  float ss = 0.f;
  if (rms) {
    for (int slot = tid; slot < n_slots; slot += NT) {
      const int row = slot % R;  // == tid % R: NT is a multiple of R
      const int rest = slot / R;
      const int kq = rest & 3;
      const int d = (rest >> 2) & 3;
      const int tt = rest >> 4;
      const int sl = tt / cpw;
      const int t = tt - sl * cpw;
      const int sl_n = max(0, min(cpw, nkc - sl * cpw));
      if (row < mrows && t < sl_n) {
        f16x8 x = *reinterpret_cast<const f16x8 *>(lA + (size_t)slot * 16);
        const f16x8 g = *reinterpret_cast<const f16x8 *>(
            lG + (size_t)(sl * cpw + t) * kTileK + 32 * d + 8 * kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xf = (float)x[e];
          ss += xf * xf;
          x[e] = (f16)(xf * (float)g[e]);
        }
        *reinterpret_cast<f16x8 *>(lA + (size_t)slot * 16) = x;
      }
    }
    lRms[tid] = ss;
    lds_barrier();
  }

  // 5. contraction, tile by tile as the loads land
  f32x4 acc[NW][MT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // activation slot of this lane: rows beyond M read a valid row instead
  // (an A row feeds only its own output row, and those are never written)
  const int kq = lane >> 4;
  const int c = lane & 15;
  const int zshift = 4 * (c & 1);
  const int dstride = 64 * R;   // bytes between 32-k steps of a tile
  const int tstride = 256 * R;  // bytes per packed k tile
  int lane_off[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) lane_off[t] = (kq * R + min(16 * t + c, mrows - 1)) * 16;
  const uint8_t *a_slice = lA + (size_t)wk * cpw * tstride;
  if (active) {
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      if (j + PD < CW) issue_tile(j + PD);
      if (j < my_n) {
        const int gi0 = (wk * cpw + j) * GPC;  // first group of tile j, split-relative
        const uint8_t *a_lane[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) a_lane[t] = a_slice + j * tstride + lane_off[t];
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const uint8_t *st = lS + (size_t)(i * NWC + wc) * scopy + ((size_t)gi0 * 16 + c) * SB;
          const uint8_t *zt = lZ + (size_t)(i * NWC + wc) * zcopy + (size_t)gi0 * 8 + (c >> 1);
          contract_tile_frag<MT, G>(
              acc[i], wv[i][j], a_lane, dstride, kq,
              [&](int gl) __attribute__((always_inline)) {
                return (zt[gl * 8] >> zshift) & 15;
              },
              [&](int gl) __attribute__((always_inline)) {
                if constexpr (SF32)
                  return *reinterpret_cast<const float *>(st + gl * 16 * SB);
                else
                  return (float)*reinterpret_cast<const f16 *>(st + gl * 16 * SB);
              });
        }
      }
    }
  }
  __syncthreads();  // all tiles done: the activation slots become reduction scratch

  // 6. slices -> slice 0, in order
  if constexpr (NWK > 1) {
    constexpr int PER = NW * MT * 4;
    if (wk > 0 && active) {
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lRed[(((wk - 1) * NWC + wc) * PER + (i * MT + t) * 4 + e) * 64 + lane] = acc[i][t][e];
    }
    __syncthreads();
    if (wk == 0 && active) {
      for (int w2 = 1; w2 < NWK; ++w2) {
#pragma unroll
        for (int i = 0; i < NW; ++i)
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][t][e] += lRed[(((w2 - 1) * NWC + wc) * PER + (i * MT + t) * 4 + e) * 64 + lane];
      }
    }
  }
  if (rms && tid < mrows) {
    float v = 0.f;
    for (int j = tid; j < NT; j += R) v += lRms[j];
    lRow[tid] = v;
  }
  const bool owner = (wk == 0) && active;

  // 7. k splits across workgroups (narrow grids only): partials, then the
  //    last arrival sums them in split order.
  const int blk = blockIdx.z * gridDim.x + blockIdx.x;
  if (S > 1) {
    if (owner) {
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
    __syncthreads();
    if (rms && tid < mrows) p.ws_rms[((size_t)blk * S + s) * 64 + tid] = lRow[tid];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&p.ws_cnt[blk], 1u);
      is_last = (prev == (unsigned)(S - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (owner) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * t + 4 * (lane >> 4) + e;
          if (row < mrows) {
#pragma unroll
            for (int i = 0; i < NW; ++i) {
              float v = 0.f;
              for (int s2 = 0; s2 < S; ++s2)
                v += (s2 == s) ? acc[i][t][e]
                               : p.ws_part[(((size_t)s2 * NW + i) * p.M + m0 + row) * p.N + ncol];
              acc[i][t][e] = v;
            }
          }
        }
    }
    if (rms && tid < mrows) {
      float v = 0.f;
      for (int s2 = 0; s2 < S; ++s2)
        v += (s2 == s) ? lRow[tid] : p.ws_rms[((size_t)blk * S + s2) * 64 + tid];
      lRow[tid] = v;
    }
    if (tid == 0) p.ws_cnt[blk] = 0u;
  }
  __syncthreads();

  // 8. epilogue
  if (!owner) return;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * t + 4 * (lane >> 4) + e;
      if (row < mrows) {
        float rsc = 1.0f;
        if (rms) rsc = 1.0f / sqrtf(lRow[row] / (float)p.K + p.eps);
        float y;
        if constexpr (GU) {
          y = silu(acc[0][t][e] * rsc) * (acc[1][t][e] * rsc);
        } else {
          y = acc[0][t][e] * rsc;
          if (p.epilogue != 0) y += (float)p.bias[ncol];
          if (p.epilogue == 2) y = y > 0.f ? y : 0.f;
        }
        p.out[(size_t)(m0 + row) * p.N + ncol] = (f16)y;
      }
    }
}

template <int MT, int NWC, int NWK, int CW, int PD, int G, bool SF32, bool GU>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = oneshot_kernel<MT, NWC, NWK, CW, PD, G, SF32, GU>;
  // Raise the kernel's dynamic-LDS limit when a plan needs more than the
  // default 64 KiB; only the first launch that needs a larger size makes the
  // attribute call, so repeated launches (also under stream capture) make none.
  static size_t lds_limit = 64 * 1024;
  if (pl.lds_bytes > lds_limit) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)pl.lds_bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error for the caller's next launch
      return e;
    }
    lds_limit = pl.lds_bytes;
  }
  hipLaunchKernelGGL(kern, dim3(pl.gx, pl.gy, pl.gz), dim3(64 * NWC * NWK), pl.lds_bytes,
                     stream, a);
  return hipGetLastError();
}

template <int MT, int NWC, int NWK, int CW, int PD, int G>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (sf32) return gu ? launch_t<MT, NWC, NWK, CW, PD, G, true, true>(a, pl, st)
                      : launch_t<MT, NWC, NWK, CW, PD, G, true, false>(a, pl, st);
  return gu ? launch_t<MT, NWC, NWK, CW, PD, G, false, true>(a, pl, st)
            : launch_t<MT, NWC, NWK, CW, PD, G, false, false>(a, pl, st);
}

template <int MT, int NWC, int NWK, int CW, int PD>
hipError_t launch_c(const GemmArgs &a, const Plan &pl, int group, bool sf32, bool gu,
                    hipStream_t st) {
  switch (group) {
    case 16: return launch_g<MT, NWC, NWK, CW, PD, 16>(a, pl, sf32, gu, st);
    case 32: return launch_g<MT, NWC, NWK, CW, PD, 32>(a, pl, sf32, gu, st);
    case 64: return launch_g<MT, NWC, NWK, CW, PD, 64>(a, pl, sf32, gu, st);
    default: return launch_g<MT, NWC, NWK, CW, PD, 128>(a, pl, sf32, gu, st);
  }
}

}  // namespace

const OneshotCfg kOneshotCfgs[kNumOneshotCfgs] = {
    {1, 1, 4, 10, 2},  // 0: M <= 16, one column tile, four k slices, <= 10 tiles each
    {1, 1, 8, 10, 2},  // 1: eight k slices (512 threads) for narrow N / long K
    {1, 2, 2, 10, 2},  // 2: two column tiles share the activations
};

hipError_t launch_oneshot(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                          bool gate_up, hipStream_t stream) {
  switch (pl.cfg) {
    case 0: return launch_c<1, 1, 4, 10, 2>(a, pl, group, scale_f32, gate_up, stream);
    case 1: return launch_c<1, 1, 8, 10, 2>(a, pl, group, scale_f32, gate_up, stream);
    default: return launch_c<1, 2, 2, 10, 2>(a, pl, group, scale_f32, gate_up, stream);
  }
}

}  // namespace w4a16
