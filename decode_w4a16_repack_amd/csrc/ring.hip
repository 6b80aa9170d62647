// Fused fp16 x int4 group-quantized GEMM/GEMV for gfx950 (CDNA4).
//
// Method (onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
// GEMM"): weights repacked once ("What's landed"), int4 codes unpacked in
// registers, zero-point subtracted, fp16 matrix-core contraction with the
// exact integers (q - zp), each group's fp32 partial multiplied by its scale
// after the contraction, split-K with a fixed-order reduction ("P2 - widen
// the win: split-K"; small M is limited by weight loads in flight, and
// deeper k splitting raises weight throughput).  Epilogues: bias and
// bias + ReLU ("Fusion benchmark" page), RMSNorm prologue ("fused RMS-norm"
// update), paired gate/up with SwiGLU ("gate_up SwiGLU MLP fusion" update).
//
// gfx950 design.  A workgroup is NWC x NWK wavefronts: NWC 16-column weight
// tiles times NWK slices of the k range (split-K inside the workgroup,
// reduced through LDS in slice order: deterministic, no fences, no
// atomics).  Each wavefront walks its slice in rounds of DA packed k tiles:
//  * weights (one 16-byte load per lane per tile, a fully coalesced 1 KiB per
//    wavefront) and their scales / zero-points are loaded two rounds ahead
//    into a three-round register ring;
//  * the activations of the next round are loaded into registers at the top
//    of a round and written to the other half of a double-buffered LDS tile
//    at its end, in "fragment order" ([slice][tile][step][k slot][row]) so
//    that the 16 rows an MFMA operand reads sit in 16 consecutive 16-byte
//    slots (conflict-free ds_read_b128, no padding);
//  * rounds are separated by an LDS-only barrier, so weight loads in flight
//    are never drained by a barrier;
//  * every load is issued unconditionally (tail tiles re-read a valid tile
//    and are not used), so the compiler's per-load wait counts are exact and
//    a wavefront waits only for the data it is about to use.
// Rows >= M are never loaded; their operand registers are zero.
#include <type_traits>

#include "device.h"

namespace w4a16 {

namespace {

template <int MT, int NWC, int NWK, int DA, int G, bool SF32, bool GU>
__global__ void __launch_bounds__(64 * NWC * NWK)
ring_kernel(const GemmArgs p) {
  constexpr int NWAVE = NWC * NWK;
  constexpr int NT = 64 * NWAVE;
  constexpr int NW = GU ? 2 : 1;
  constexpr int MR = 16 * MT;
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int NSLOT = 3;                       // rounds in the register ring
  constexpr int SEGMAX = (NWK * DA * MR * 16 + NT - 1) / NT;  // staging loads / thread

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
  const int ctc = active ? ct : NTL - 1;  // clamped: loads stay in bounds
  const int s = blockIdx.y;
  const int S = p.split;
  const int m0 = blockIdx.z * MR;
  const int mrows = min(MR, p.M - m0);
  const int R = p.rows_pow2;  // staged rows, a power of two >= min(M, MR)
  const int kb = s * p.cps;
  const int nkc = min(KC, kb + p.cps) - kb;
  const int cpw = (nkc + NWK - 1) / NWK;           // tiles per slice
  const int nr = (cpw + DA - 1) / DA;              // rounds
  const int my_kb = kb + wk * cpw;                 // first tile of this slice
  const int my_n = max(0, min(cpw, nkc - wk * cpw));  // tiles of this slice
  const bool rms = p.gamma != nullptr;
  const bool has_zp = p.has_zp != 0;
  const int ncol = ctc * kTileN + (lane & 15);

  const size_t abuf = (size_t)NWK * DA * 4 * 4 * R * 16;  // bytes per LDS buffer
  uint8_t *lA0 = smem;
  uint8_t *lA1 = smem + abuf;
  float *lRms = reinterpret_cast<float *>(smem + p.lds_r);   // [NT] partial sums of squares
  float *lRed = reinterpret_cast<float *>(smem);             // aliases the A buffers at the end

  // scales and zero-points of the workgroup's column tiles and groups, copied
  // straight into LDS once (contiguous runs in the packed layout)
  uint8_t *lS = smem + p.lds_s;
  uint8_t *lZ = smem + p.lds_z;
  const int GRC = p.gr;
  const int scopy = (GRC * 16 * SB + 1023) / 1024 * 1024;
  const int zcopy = (GRC * 8 + 255) / 256 * 256;
  {
    const int gb = kb * GPC;
    const int ngr = nkc * GPC;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      for (int w = 0; w < NWC; ++w) {
        const int tw = min(blockIdx.x * NWC + w, NTL - 1);
        const size_t first = (size_t)tw * Gall + gb;
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
  }

  // weight stream of this lane
  const uint8_t *wbase[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    wbase[i] = p.w[i] + (size_t)ctc * KC * kTileBytes + (size_t)lane * 16;

  // register ring: NSLOT rounds x DA tiles
  u32x4 rw[NW][NSLOT][DA];

  auto tile_of = [&](int r, int c) __attribute__((always_inline)) {  // clamped k tile
    int t = r * DA + c;
    t = min(t, max(my_n - 1, 0));
    return min(my_kb + t, KC - 1);
  };
  auto issue_round = [&](int r, auto slot_c) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int c = 0; c < DA; ++c) {
      const int kc = tile_of(r, c);
#pragma unroll
      for (int i = 0; i < NW; ++i)
        rw[i][SL][c] = *reinterpret_cast<const u32x4 *>(wbase[i] + (size_t)kc * kTileBytes);
    }
  };

  // activation staging: thread -> fixed row (tid % R), segments of that row
  const int srow = tid % R;
  const int scol = tid / R;                // first segment index of this thread
  constexpr int SPR = NWK * DA * 16;       // 16-byte segments per row per round
  const bool srow_ok = srow < mrows;
  const f16 *arow = p.A + (size_t)(m0 + (srow_ok ? srow : 0)) * p.K;
  u32x4 areg[SEGMAX];
  u32x4 greg[SEGMAX];
  float ss = 0.f;

  auto stage_load = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SEGMAX; ++i) {
      const int sg_all = scol + (NT / R) * i;     // segment within the row's round
      if (sg_all < SPR) {
        const int sl = sg_all / (DA * 16);
        const int c = (sg_all / 16) % DA;
        const int sg = sg_all % 16;
        int t = r * DA + c;
        const int sl_n = max(0, min(cpw, nkc - sl * cpw));
        t = min(t, max(sl_n - 1, 0));
        const int kc = min(kb + sl * cpw + t, KC - 1);
        const size_t k = (size_t)kc * kTileK + sg * 8;
        if (srow_ok) {
          areg[i] = *reinterpret_cast<const u32x4 *>(arow + k);
          if (rms) greg[i] = *reinterpret_cast<const u32x4 *>(p.gamma + k);
        }
      }
    }
  };
  auto stage_store = [&](int r, uint8_t *buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SEGMAX; ++i) {
      const int sg_all = scol + (NT / R) * i;
      if (sg_all < SPR && srow_ok) {
        const int sl = sg_all / (DA * 16);
        const int c = (sg_all / 16) % DA;
        const int sg = sg_all % 16;
        u32x4 v = areg[i];
        if (rms) {
          // sum of squares of real (not tail re-read) tiles only
          const int sl_n = max(0, min(cpw, nkc - sl * cpw));
          const bool real = (r * DA + c) < sl_n;
          const f16x8 a = __builtin_bit_cast(f16x8, v);
          const f16x8 g = __builtin_bit_cast(f16x8, greg[i]);
          f16x8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float af = (float)a[e];
            if (real) ss += af * af;
            x[e] = (f16)(af * (float)g[e]);
          }
          v = __builtin_bit_cast(u32x4, x);
        }
        const int slot = ((((sl * DA + c) * 4 + (sg >> 2)) * 4 + (sg & 3)) * R) + srow;
        *reinterpret_cast<u32x4 *>(buf + (size_t)slot * 16) = v;
      }
    }
  };

  f32x4 acc[NW][MT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // activation slot of this lane: rows beyond M read a valid row instead
  // (an A row feeds only its own output row, and those are never written)
  const int kq = lane >> 4;
  const int cc = lane & 15;
  const int zshift = 4 * (cc & 1);
  const int dstride = 64 * R;   // bytes between 32-k steps of a tile
  const int tstride = 256 * R;  // bytes per packed k tile
  int lane_off[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) lane_off[t] = (kq * R + min(16 * t + cc, mrows - 1)) * 16;

  auto compute_round = [&](int r, auto slot_c, const uint8_t *buf) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    if (!active) return;
#pragma unroll
    for (int c = 0; c < DA; ++c) {
      if (r * DA + c < my_n) {
        // split-relative first group of this tile
        const int gi0 = (wk * cpw + r * DA + c) * GPC;
        const uint8_t *a_lane[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) a_lane[t] = buf + (wk * DA + c) * tstride + lane_off[t];
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const uint8_t *st = lS + (size_t)(i * NWC + wc) * scopy + ((size_t)gi0 * 16 + cc) * SB;
          const uint8_t *zt = lZ + (size_t)(i * NWC + wc) * zcopy + (size_t)gi0 * 8 + (cc >> 1);
          contract_tile_frag<MT, G>(
              acc[i], rw[i][SL][c], a_lane, dstride, kq,
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
  };

  // prologue: rounds 0 and 1 of weights, round 0 of activations
  issue_round(0, std::integral_constant<int, 0>{});
  issue_round(1, std::integral_constant<int, 1>{});
  stage_load(0);
  stage_store(0, lA0);
  wait_vmcnt<0>();  // this wavefront's metadata copies into LDS have landed
  lds_barrier();

  // main loop, unrolled by the ring size so every register index is static
  auto step = [&](int r, auto slot_c, auto nslot_c, uint8_t *cur, uint8_t *nxt) __attribute__((always_inline)) {
    stage_load(r + 1);                 // next round's activations (clamped)
    issue_round(r + 2, nslot_c);       // weights two rounds ahead (clamped)
    compute_round(r, slot_c, cur);
    stage_store(r + 1, nxt);
    lds_barrier();
  };
  for (int r = 0; r < nr; r += 3) {
    step(r, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{},
         (r & 1) ? lA1 : lA0, (r & 1) ? lA0 : lA1);
    if (r + 1 < nr)
      step(r + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{},
           (r & 1) ? lA0 : lA1, (r & 1) ? lA1 : lA0);
    if (r + 2 < nr)
      step(r + 2, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{},
           (r & 1) ? lA1 : lA0, (r & 1) ? lA0 : lA1);
  }

  // sum of squares per staged row: thread partials, then a fixed-order sum
  if (rms) lRms[tid] = ss;
  __syncthreads();  // also: every wavefront is done with the A buffers

  // in-workgroup reduction of the NWK slices, slice 0 first
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
  // row sums of squares: contributors of row r are threads r, r + R, ...
  float *lRow = lRms + NT;  // [MR]
  if (rms && tid < mrows) {
    float v = 0.f;
    for (int j = tid; j < NT; j += R) v += lRms[j];
    lRow[tid] = v;
  }
  const bool owner = (wk == 0) && active;

  // k splits across workgroups (only for grids too small to fill the chip):
  // publish partials; the last arrival sums them in split order.
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
    __syncthreads();  // lRow complete
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

  // epilogue: lane holds column ncol, rows 16t + 4*(lane/16) + e
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

template <int MT, int NWC, int NWK, int DA, int G, bool SF32, bool GU>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = ring_kernel<MT, NWC, NWK, DA, G, SF32, GU>;
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

template <int MT, int NWC, int NWK, int DA, int G>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (sf32) return gu ? launch_t<MT, NWC, NWK, DA, G, true, true>(a, pl, st)
                      : launch_t<MT, NWC, NWK, DA, G, true, false>(a, pl, st);
  return gu ? launch_t<MT, NWC, NWK, DA, G, false, true>(a, pl, st)
            : launch_t<MT, NWC, NWK, DA, G, false, false>(a, pl, st);
}

template <int MT, int NWC, int NWK, int DA>
hipError_t launch_c(const GemmArgs &a, const Plan &pl, int group, bool sf32, bool gu,
                    hipStream_t st) {
  switch (group) {
    case 16: return launch_g<MT, NWC, NWK, DA, 16>(a, pl, sf32, gu, st);
    case 32: return launch_g<MT, NWC, NWK, DA, 32>(a, pl, sf32, gu, st);
    case 64: return launch_g<MT, NWC, NWK, DA, 64>(a, pl, sf32, gu, st);
    default: return launch_g<MT, NWC, NWK, DA, 128>(a, pl, sf32, gu, st);
  }
}

}  // namespace

// Tile configurations compiled in (index = Plan::cfg).
const RingCfg kRingCfgs[kNumRingCfgs] = {
    {1, 1, 4, 2},  // 0: M <= 16, one column tile, four k slices
    {1, 2, 2, 2},  // 1: M <= 16, two column tiles, two k slices
    {1, 1, 8, 2},  // 2: M <= 16, eight k slices (512 threads) for narrow N
    {2, 2, 2, 1},  // 3: M <= 32
    {4, 2, 2, 1},  // 4: M <= 64 per m block
};

hipError_t launch_ring(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                       bool gate_up, hipStream_t stream) {
  switch (pl.cfg) {
    case 0: return launch_c<1, 1, 4, 2>(a, pl, group, scale_f32, gate_up, stream);
    case 1: return launch_c<1, 2, 2, 2>(a, pl, group, scale_f32, gate_up, stream);
    case 2: return launch_c<1, 1, 8, 2>(a, pl, group, scale_f32, gate_up, stream);
    case 3: return launch_c<2, 2, 2, 1>(a, pl, group, scale_f32, gate_up, stream);
    default: return launch_c<4, 2, 2, 1>(a, pl, group, scale_f32, gate_up, stream);
  }
}

}  // namespace w4a16
