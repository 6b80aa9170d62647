// Small-M fused W4A16 GEMM/GEMV for gfx950 (M <= 16 per 16-row tile): the
// HBM-bound decode regime, where the whole cost is streaming the packed
// weights once.
//
// Method (onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
// GEMM", "What's landed"): repacked weights, in-register unpack to the exact
// integers (q - zp), matrix-core contraction, per-group scale after the
// accumulate; split-K with a fixed-order reduction ("P2 - widen the win:
// split-K" and "Small-M split-K retune": at small M the weight loads in
// flight set the speed, so k is split to put more of them in flight).
//
// gfx950 design:
//  * a workgroup is NWK wavefronts, one per k slice; each wavefront owns
//    KPW consecutive 128-k tiles of the workgroup's k range for the same
//    CPW 16-column weight tiles, so the workgroup covers CPW column tiles
//    over its whole k range and reduces the NWK slices in LDS in slice order
//    (no partial sums leave the workgroup unless the k range itself is split
//    across workgroups, which only narrow or very deep shapes need);
//  * each lane keeps its activation fragments for the wavefront's k slice in
//    registers for the whole kernel (row l%16, k slots 8*(l/16)..+7 of every
//    32-k step: one 16-byte global load each), so the CPW column tiles reuse
//    them and no activation staging, LDS traffic or barrier sits in the loop;
//  * the wavefront streams its CPW x KPW weight tiles (one 16-byte load per
//    lane per 1 KiB tile), PD tiles ahead of the contraction, k tile outer
//    and column tile inner so consecutive MFMA chains are independent;
//  * scales and zero-points of the workgroup's column tiles are contiguous
//    runs in the packed layout, copied into LDS with direct global-to-LDS
//    loads before the stream starts;
//  * wavefront c < CPW finishes column tile c: slice sum, RMSNorm factor,
//    epilogue, one fp16 write.
#include "device.h"

namespace w4a16 {

namespace {

template <int CPW, int KPW, int NWK, int PD, int G, bool SF32, bool GU>
__global__ void __launch_bounds__(64 * NWK)
stream_kernel(const GemmArgs p) {
  static_assert(CPW <= NWK, "one finishing wavefront per column tile");
  static_assert(PD >= 1 && PD <= CPW * KPW, "prefetch depth");
  constexpr int NT = 64 * NWK;
  constexpr int NW = GU ? 2 : 1;
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int NTILE = CPW * KPW;
  // loads issued after the metadata copies that may still be in flight at
  // the first barrier: the activation fragments and the first PD tiles
  constexpr int AFTER_COPIES = 4 * KPW + PD * NW;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NTL = p.N / kTileN;
  const int KC = p.K / kTileK;
  const int Gall = p.K / G;
  const int ct0 = blockIdx.x * CPW;
  const int s = blockIdx.y;
  const int S = p.split;
  const int m0 = blockIdx.z * 16;
  const int mrows = min(16, p.M - m0);
  const int kb = s * p.cps;
  const int nkc = min(KC, kb + p.cps) - kb;
  const int my_kb = kb + wk * KPW;
  const int my_n = max(0, min(KPW, nkc - wk * KPW));  // valid k tiles of this slice
  const bool rms = p.gamma != nullptr;
  const bool has_zp = p.has_zp != 0;
  const int kq = lane >> 4;
  const int c = lane & 15;

  // LDS: scales and zero-points [NW][CPW] runs, slice partial sums, sums of
  // squares.
  const int GRC = p.gr;  // staged groups per column tile (capacity)
  const int scopy = (GRC * 16 * SB + 1023) / 1024 * 1024;
  const int zcopy = (GRC * 8 + 255) / 256 * 256;
  uint8_t *lS = smem + p.lds_s;
  uint8_t *lZ = smem + p.lds_z;
  float *lRed = reinterpret_cast<float *>(smem);            // [NWK][NW*CPW][4][64]
  float *lRms = reinterpret_cast<float *>(smem + p.lds_r);  // [NWK][64] + [16]
  float *lRow = lRms + NT;

  // 1. scales and zero-points of the column tiles over the workgroup's
  //    groups: contiguous runs in the packed layout, copied straight to LDS
  const int gb = kb * GPC;
  const int ngr = nkc * GPC;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
#pragma unroll
    for (int w = 0; w < CPW; ++w) {
      const int tw = min(ct0 + w, NTL - 1);
      const size_t first = (size_t)tw * Gall + gb;  // first (tile, group) record
      const int sbytes = ngr * 16 * SB;
      const uint8_t *ssrc = reinterpret_cast<const uint8_t *>(p.scales[i]) + first * 16 * SB;
      uint8_t *sdst = lS + (i * CPW + w) * scopy;
      for (int q = wk; q * 1024 < sbytes; q += NWK)
        copy16_to_lds(ssrc + min(q * 1024 + lane * 16, sbytes - 16), sdst + q * 1024);
      uint8_t *zdst = lZ + (i * CPW + w) * zcopy;
      if (has_zp) {
        const int zbytes = ngr * 8;
        const uint8_t *zsrc = p.zeros[i] + first * 8;
        for (int q = wk; q * 256 < zbytes; q += NWK)
          copy4_to_lds(zsrc + min(q * 256 + lane * 4, zbytes - 4), zdst + q * 256);
      } else {
        for (int e = tid; e * 4 < zcopy; e += NT)  // symmetric: every zero-point is 8
          reinterpret_cast<uint32_t *>(zdst)[e] = 0x88888888u;
      }
    }
  }

  // 2. activation fragments of this slice, in registers.  Rows past M read
  //    row M-1 (an A row feeds only its own output row, never written); k
  //    tiles past the slice read a valid tile and are zeroed, so they add
  //    nothing.
  const int arow = m0 + min(c, mrows - 1);
  f16x8 a[KPW][4][1];
  {
    const f16 *arow_p = p.A + (size_t)arow * p.K + 8 * kq;
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        a[t][d][0] = *reinterpret_cast<const f16x8 *>(arow_p + kc * kTileK + 32 * d);
    }
  }
  f16x8 gam[KPW][4];
  if (rms) {
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        gam[t][d] = *reinterpret_cast<const f16x8 *>(p.gamma + kc * kTileK + 32 * d + 8 * kq);
    }
  }

  // 3. the first PD weight tiles; tile f = t * CPW + w (k tile t, column
  //    tile w) is issued PD tiles before it is contracted.  Tiles past the
  //    slice or past N re-read a valid tile.
  const uint8_t *wbase[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) wbase[i] = p.w[i] + (size_t)lane * 16;
  u32x4 wv[NW][NTILE];
  auto issue_tile = [&](int f) __attribute__((always_inline)) {
    const int t = f / CPW, w = f % CPW;
    const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
    const size_t tile = (size_t)min(ct0 + w, NTL - 1) * KC + kc;
#pragma unroll
    for (int i = 0; i < NW; ++i)
      wv[i][f] = *reinterpret_cast<const u32x4 *>(wbase[i] + tile * kTileBytes);
  };
#pragma unroll
  for (int f = 0; f < PD; ++f) issue_tile(f);

  // 4. the metadata copies (issued first) have landed
  wait_vmcnt<(AFTER_COPIES < 63 ? AFTER_COPIES : 63)>();
  lds_barrier();

  // 5. RMSNorm prologue on the fragments: per-lane sum of squares (row l%16,
  //    this lane's k slots), x * gamma rounded once to fp16; the factor
  //    1/sqrt(mean + eps) is applied in the epilogue.  Zeroing of the k
  //    tiles past the slice happens here too.
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < KPW; ++t) {
    const bool valid = t < my_n;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f16x8 x = valid ? a[t][d][0] : f16x8{};
      if (rms) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xf = (float)x[e];
          ss += xf * xf;
          x[e] = (f16)(xf * (float)gam[t][d][e]);
        }
      }
      a[t][d][0] = x;
    }
  }

  // 6. contraction, k tile outer, column tile inner
  f32x4 acc[NW][CPW][1];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int w = 0; w < CPW; ++w) acc[i][w][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int zshift = 4 * (c & 1);
#pragma unroll
  for (int f = 0; f < NTILE; ++f) {
    if (f + PD < NTILE) issue_tile(f + PD);
    const int t = f / CPW, w = f % CPW;
    // first group of k tile t in the workgroup's staged runs (clamped to a
    // staged group for k tiles past the slice, whose activations are zero)
    const int gi0 = min(wk * KPW + t, max(nkc - 1, 0)) * GPC;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint8_t *st = lS + (i * CPW + w) * scopy + (gi0 * 16 + c) * SB;
      const uint8_t *zt = lZ + (i * CPW + w) * zcopy + gi0 * 8 + (c >> 1);
      contract_tile<1, G>(
          acc[i][w], wv[i][f], a[t], kq,
          [&](int gl) __attribute__((always_inline)) { return (zt[gl * 8] >> zshift) & 15; },
          [&](int gl) __attribute__((always_inline)) {
            if constexpr (SF32)
              return *reinterpret_cast<const float *>(st + gl * 16 * SB);
            else
              return (float)*reinterpret_cast<const f16 *>(st + gl * 16 * SB);
          });
    }
  }

  // 7. slice partial sums -> LDS; wavefront w < CPW sums column tile w over
  //    the slices in slice order
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int w = 0; w < CPW; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lRed[((wk * NW * CPW + i * CPW + w) * 4 + e) * 64 + lane] = acc[i][w][0][e];
  if (rms) lRms[wk * 64 + lane] = ss;
  lds_barrier();
  const int wfin = wk;  // the column tile this wavefront finishes (if < CPW)
  const bool owner = wfin < CPW && ct0 + wfin < NTL;
  f32x4 fin[NW];
  if (wfin < CPW) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      for (int w2 = 0; w2 < NWK; ++w2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] += lRed[((w2 * NW * CPW + i * CPW + wfin) * 4 + e) * 64 + lane];
      fin[i] = v;
    }
  }
  // row sums of squares: row r is held by lanes r, r+16, r+32, r+48 of
  // every slice
  if (rms && tid < mrows) {
    float v = 0.f;
    for (int w2 = 0; w2 < NWK; ++w2)
#pragma unroll
      for (int g = 0; g < 4; ++g) v += lRms[w2 * 64 + 16 * g + tid];
    lRow[tid] = v;
  }
  const int ncol = (ct0 + wfin) * kTileN + c;

  // 8. k splits across workgroups (narrow grids and very deep k only):
  //    partials, then the last arrival sums them in split order
  const int blk = blockIdx.z * gridDim.x + blockIdx.x;
  if (S > 1) {
    lds_barrier();  // lRow complete
    if (owner) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * kq + e;
        if (row < mrows) {
#pragma unroll
          for (int i = 0; i < NW; ++i)
            p.ws_part[(((size_t)s * NW + i) * p.M + m0 + row) * p.N + ncol] = fin[i][e];
        }
      }
    }
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
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * kq + e;
        if (row < mrows) {
#pragma unroll
          for (int i = 0; i < NW; ++i) {
            float v = 0.f;
            for (int s2 = 0; s2 < S; ++s2)
              v += (s2 == s) ? fin[i][e]
                             : p.ws_part[(((size_t)s2 * NW + i) * p.M + m0 + row) * p.N + ncol];
            fin[i][e] = v;
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
  lds_barrier();  // lRow final

  // 9. epilogue, one fp16 write per output
  if (!owner) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * kq + e;
    if (row < mrows) {
      float rsc = 1.0f;
      if (rms) rsc = 1.0f / sqrtf(lRow[row] / (float)p.K + p.eps);
      float y;
      if constexpr (GU) {
        y = silu(fin[0][e] * rsc) * (fin[1][e] * rsc);
      } else {
        y = fin[0][e] * rsc;
        if (p.epilogue != 0) y += (float)p.bias[ncol];
        if (p.epilogue == 2) y = y > 0.f ? y : 0.f;
      }
      p.out[(size_t)(m0 + row) * p.N + ncol] = (f16)y;
    }
  }
}

template <int CPW, int KPW, int NWK, int PD, int G, bool SF32, bool GU>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = stream_kernel<CPW, KPW, NWK, PD, G, SF32, GU>;
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
  hipLaunchKernelGGL(kern, dim3(pl.gx, pl.gy, pl.gz), dim3(64 * NWK), pl.lds_bytes, stream, a);
  return hipGetLastError();
}

template <int CPW, int KPW, int NWK, int PD, int G>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (sf32) return gu ? launch_t<CPW, KPW, NWK, PD, G, true, true>(a, pl, st)
                      : launch_t<CPW, KPW, NWK, PD, G, true, false>(a, pl, st);
  return gu ? launch_t<CPW, KPW, NWK, PD, G, false, true>(a, pl, st)
            : launch_t<CPW, KPW, NWK, PD, G, false, false>(a, pl, st);
}

template <int CPW, int KPW, int NWK, int PD>
hipError_t launch_c(const GemmArgs &a, const Plan &pl, int group, bool sf32, bool gu,
                    hipStream_t st) {
  switch (group) {
    case 16: return launch_g<CPW, KPW, NWK, PD, 16>(a, pl, sf32, gu, st);
    case 32: return launch_g<CPW, KPW, NWK, PD, 32>(a, pl, sf32, gu, st);
    case 64: return launch_g<CPW, KPW, NWK, PD, 64>(a, pl, sf32, gu, st);
    default: return launch_g<CPW, KPW, NWK, PD, 128>(a, pl, sf32, gu, st);
  }
}

}  // namespace

const StreamCfg kStreamCfgs[kNumStreamCfgs] = {
    {4, 5, 8, 8},  // 0: 4 column tiles x 8 slices of 5 k tiles (K <= 5120)
    {2, 5, 8, 6},  // 1: 2 column tiles, for narrower N
    {1, 5, 8, 4},  // 2: 1 column tile, for narrow N
};

hipError_t launch_stream(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                         bool gate_up, hipStream_t stream) {
  switch (pl.cfg) {
    case 0: return launch_c<4, 5, 8, 8>(a, pl, group, scale_f32, gate_up, stream);
    case 1: return launch_c<2, 5, 8, 6>(a, pl, group, scale_f32, gate_up, stream);
    default: return launch_c<1, 5, 8, 4>(a, pl, group, scale_f32, gate_up, stream);
  }
}

}  // namespace w4a16
