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
//    32-k step), so the CPW column tiles reuse them and no activation
//    traffic or barrier sits in the loop;
//  * the wavefront streams its CPW x KPW weight tiles (one 16-byte load per
//    lane per 1 KiB tile), PD tiles ahead of the contraction, k tile outer
//    and column tile inner so consecutive MFMA chains are independent;
//  * each wavefront copies the scales and zero-points of its slice (runs of
//    the packed layout) into a private LDS region with direct global-to-LDS
//    loads, and for M <= 4 also its activation rows (unique data, then read
//    back as fragments); nothing is shared between wavefronts until the
//    final reduction, so the only barrier is the one before it;
//  * the slice partial sums go through the same private regions; wavefront
//    c < CPW finishes column tile c: slice sum in slice order, RMSNorm
//    factor, epilogue, one fp16 write.  With a residual and more than 4 rows
//    the skip + RMSNorm prologue is staged instead (stage.hip): every column
//    block would otherwise read both activation slices.
//
// This header holds the kernel template and its launch helpers; stream.hip
// instantiates the plain kernels and stream_rms.hip the ones with the
// RMSNorm prologue, so the two sets compile in parallel.
#pragma once

#include "device.h"

namespace w4a16 {

namespace {

// Occupancy: the NWK wavefronts of a workgroup need NWK / 4 per SIMD, and a
// second workgroup would need twice that, which neither the registers of
// this loop nor the plan allow; so the compiler is told that NWK / 4 is the
// occupancy, and spends the registers a higher target would have reserved
// on keeping more loads in flight (M=1: 8.9 -> 8.3 us).
// RMS: 0 no prologue, 1 RMSNorm of A, 2 RMSNorm of A + residual.
template <int CPW, int KPW, int NWK, int PD, bool ALDS, int G, bool SF32, bool GU, int RMS>
__global__ void __launch_bounds__(64 * NWK) __attribute__((amdgpu_waves_per_eu(NWK / 4, NWK / 4)))
stream_kernel(const GemmArgs p) {
  static_assert(CPW <= NWK, "one finishing wavefront per column tile");
  static_assert(PD >= 1 && PD <= CPW * KPW, "prefetch depth");
  constexpr int NW = GU ? 2 : 1;
  // tiles in flight: gate_up loads two per tile, so half as many tiles
  constexpr int PDE = GU ? (PD + 1) / 2 : PD;
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int NTILE = CPW * KPW;
  constexpr int GPW = KPW * GPC;                 // groups of one wavefront's k slice
  constexpr int MS_BYTES = CPW * GPW * 16 * SB;  // its scales, [CPW][GPW][16]
  constexpr int MZ_BYTES = CPW * GPW * 8;        // its zero-points, [CPW][GPW][8 bytes]
  constexpr int MZ_PAD = (MZ_BYTES + 15) / 16 * 16;
  constexpr int SU = GPW * SB;                   // 16-byte scale units per column tile
  constexpr int ZU = GPW * 2;                    // 4-byte zero-point units per column tile
  constexpr bool RES = RMS == 2;  // residual added before the norm
  // k tiles whose activation fragments are loaded with the first PDE weight
  // tiles (each k tile's just before its first weight tile)
  constexpr int A_EARLY = (PDE - 1) / CPW + 1 < KPW ? (PDE - 1) / CPW + 1 : KPW;
  // (the skip prologue loads the whole slice before the weights: more loads
  // after the copies than counted here, which only makes the wait stricter)
  // weight tiles issued before the direct-to-LDS copies (LDS-staged rows,
  // several column tiles per wavefront; measured: a single-column
  // configuration is slower with them, K=4096 N=4096 M=4 5.5 -> 5.8 us)
  constexpr int F0 = (ALDS && CPW >= 2) ? (PDE < 2 ? PDE : 2) : 0;
  // loads issued after the direct-to-LDS copies that may still be in
  // flight when the copies are waited for (at least): the register
  // activation fragments of the first k tiles (unless they come through
  // LDS) and the first PDE tiles but the F0 issued before the copies
  constexpr int AFTER_COPIES = (ALDS ? 0 : 4 * A_EARLY) + (PDE - F0) * NW;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

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
  // the RMSNorm prologue is its own instantiation, so the plain kernel holds
  // none of its registers
  constexpr bool rms = RMS != 0;
  const bool has_zp = p.has_zp != 0;
  const int kq = lane >> 4;
  const int c = lane & 15;
  const int R = p.rows_pow2;  // activation rows staged in LDS (ALDS)

  // LDS: one private region per wavefront (its scales, zero-points and,
  // with ALDS, activation slots; reused for its partial sums at the end),
  // then the per-slice row sums of squares.  No region is shared before
  // the final reduction, so nothing waits for another wavefront until then.
  uint8_t *region = smem + wk * p.lds_s;
  uint8_t *ms = region;                   // [NW] x MS_BYTES
  uint8_t *mz = region + NW * MS_BYTES;   // [NW] x MZ_PAD
  uint8_t *mg = mz + NW * MZ_PAD;         // the slice's gamma, [KPW][128] fp16
  uint8_t *aslots = mg + KPW * kTileK * 2;  // ALDS: KPW * 16 * R slots of 16 bytes
  float *lRms = reinterpret_cast<float *>(smem + p.lds_r);  // [NWK][16]

  // 0. weight tiles: tile f = t * CPW + w (k tile t, column tile w) is issued
  //    PDE tiles before it is contracted, the activations of k tile t from
  //    registers just before tile (t, 0) (below: where they come from).
  //    Tiles past the slice or past N re-read a valid tile.  With the
  //    activation rows staged in LDS, the first F0 tiles go out before the
  //    copies of steps 1-2, so that the weight stream starts as early as it
  //    can (K=5120 N=13824 M=1: 8.05 -> 7.83 us); they then land before the
  //    copies, which the wait of step 4 covers all the same.
  const int arow = min(c, mrows - 1);
  f16x8 a[KPW][4][1];
  // Without LDS staging the fragments of k tile t are loaded just before the
  // first weight tile of t: loads complete in issue order, so a slice loaded
  // up front made the first tile wait for all of it.  The skip prologue (at
  // most 4 rows) loads the slice and its residual up front and adds them
  // before the loop: a conditional store of the sum inside the loop would
  // split it into branches and spill.
  const f16 *arow_p = p.A + (size_t)(m0 + arow) * p.K + 8 * kq;
  auto load_a = [&](int t) __attribute__((always_inline)) {
    const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
#pragma unroll
    for (int d = 0; d < 4; ++d)
      a[t][d][0] = *reinterpret_cast<const f16x8 *>(arow_p + kc * kTileK + 32 * d);
  };
  constexpr bool A_PROGRESSIVE = !ALDS && !RES;
  u32x4 wv[NW][NTILE];
  auto issue_tile = [&](int f) __attribute__((always_inline)) {
    const int t = f / CPW, w = f % CPW;
    if (A_PROGRESSIVE && w == 0) load_a(t);
    const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
    const size_t tile = (size_t)min(ct0 + w, NTL - 1) * KC + kc;
#pragma unroll
    for (int i = 0; i < NW; ++i)
      wv[i][f] = load_weights(p.w[i] + tile * kTileBytes, lane);
  };
#pragma unroll
  for (int f = 0; f < F0; ++f) issue_tile(f);

  // 1. this slice's scales and zero-points of the CPW column tiles: runs of
  //    the packed layout, copied straight into the region (reads clamped to
  //    the column tile's own groups; lanes past the copy write nothing)
  const int g0 = my_kb * GPC;
  const size_t srun = (size_t)Gall * 16 * SB;  // scale bytes of one column tile
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    uint8_t *msi = ms + i * MS_BYTES;
    uint8_t *mzi = mz + i * MZ_PAD;
    const uint8_t *sbase = reinterpret_cast<const uint8_t *>(p.scales[i]);
#pragma unroll
    for (int q = 0; q < (CPW * SU + 63) / 64; ++q) {
      const int u = q * 64 + lane;
      if (u < CPW * SU) {
        const int w = u / SU, o = u - w * SU;
        const size_t tw = (size_t)min(ct0 + w, NTL - 1);
        const size_t off = min((size_t)g0 * 16 * SB + (size_t)o * 16, srun - 16);
        copy16_to_lds(sbase + tw * srun + off, msi + q * 1024);
      }
    }
    if (has_zp) {
      const size_t zrun = (size_t)Gall * 8;
#pragma unroll
      for (int q = 0; q < (CPW * ZU + 63) / 64; ++q) {
        const int u = q * 64 + lane;
        if (u < CPW * ZU) {
          const int w = u / ZU, o = u - w * ZU;
          const size_t tw = (size_t)min(ct0 + w, NTL - 1);
          const size_t off = min((size_t)g0 * 8 + (size_t)o * 4, zrun - 4);
          copy4_to_lds(p.zeros[i] + tw * zrun + off, mzi + q * 256);
        }
      }
    } else {
      for (int e = lane; e * 4 < MZ_BYTES; e += 64)  // symmetric: every zero-point is 8
        reinterpret_cast<uint32_t *>(mzi)[e] = 0x88888888u;
    }
  }

  if constexpr (rms) {
    // the slice's gamma (positions past the slice copy a valid tile): read
    // back from LDS by the prologue, so it holds no registers while the
    // activations, the residual and the first weight tiles are in flight
#pragma unroll
    for (int q = 0; q < (KPW * 16 + 63) / 64; ++q) {
      const int u = q * 64 + lane;
      if (u < KPW * 16) {
        const int kc = min(my_kb + min(u >> 4, max(my_n - 1, 0)), KC - 1);
        copy16_to_lds(p.gamma + kc * kTileK + (u & 15) * 8, mg + q * 1024);
      }
    }
  }

  // 2. activation fragments of this slice (row l%16, k slots 8*(l/16)..+7 of
  //    each 32-k step).  Rows past M read row M-1 (an A row feeds only its
  //    own output row, never written); k tiles past the slice read a valid
  //    tile and are zeroed below, so they add nothing.
  //    ALDS: the slice's rows are first copied into the region in fragment
  //    order (slot ((t*4 + d)*4 + kq)*R + row), unique data only.
  if constexpr (ALDS) {
    const int lr = __builtin_ctz(R);
    const int n_slots = KPW * 16 * R;
    for (int q = 0; q * 64 < n_slots; ++q) {
      const int sl = q * 64 + lane;
      if (sl < n_slots) {
        const int row = sl & (R - 1);
        const int rest = sl >> lr;
        const int kqs = rest & 3, d = (rest >> 2) & 3, t = rest >> 4;
        const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
        const f16 *src = p.A + (size_t)(m0 + min(row, mrows - 1)) * p.K + kc * kTileK + 32 * d + 8 * kqs;
        copy16_to_lds(src, aslots + q * 1024);
      }
    }
  }
  // activation fragment (t, d) from the slots (ALDS), once the copies landed
  const uint8_t *aslot_p = aslots + (kq * R + arow) * 16;
  auto read_slot = [&](int t, int d) __attribute__((always_inline)) {
    return *reinterpret_cast<const f16x8 *>(aslot_p + (t * 4 + d) * 64 * R);
  };
  f16x8 rr[RES ? KPW : 1][4];
  if constexpr (RES) {
    const f16 *rrow_p = p.resid + (size_t)(m0 + arow) * p.K + 8 * kq;
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      if constexpr (!ALDS) load_a(t);
      const int kc = min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        rr[t][d] = *reinterpret_cast<const f16x8 *>(rrow_p + kc * kTileK + 32 * d);
    }
  }

  // 3. the other weight tiles in flight
#pragma unroll
  for (int f = F0; f < PDE; ++f) issue_tile(f);

  // 4. this wavefront's copies into its region have landed (completion is
  //    in issue order); no other wavefront reads the region before the end
  wait_vmcnt<(AFTER_COPIES < 63 ? AFTER_COPIES : 63)>();
  if constexpr (RES) {
    // s = A + resid rounded once to fp16; the workgroups of column block 0
    // write s out, each (row, k) once
    const bool write_res = p.resid_out != nullptr && blockIdx.x == 0 && c < mrows;
#pragma unroll
    for (int t = 0; t < KPW; ++t)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        a[t][d][0] = (ALDS ? read_slot(t, d) : a[t][d][0]) + rr[t][d];
    if (write_res) {
      f16 *orow = p.resid_out + (size_t)(m0 + c) * p.K + 8 * kq;
#pragma unroll
      for (int t = 0; t < KPW; ++t)
        if (t < my_n)
#pragma unroll
          for (int d = 0; d < 4; ++d)
            *reinterpret_cast<f16x8 *>(orow + (my_kb + t) * kTileK + 32 * d) = a[t][d][0];
    }
  }

  // 5. each k tile's fragments are prepared at their first use: k tiles past
  //    the slice are zeroed; with the RMSNorm prologue the per-lane sum of
  //    squares (row l%16, this lane's k slots; fp16 products are exact in
  //    fp32) and x * gamma rounded once to fp16 (the packed multiply rounds
  //    the exact product once), 1/sqrt(mean + eps) following in the
  //    epilogue; then the 1/16 pre-scale of the slots facing high nibbles.
  float ss = 0.f;
  auto prep_tile = [&](int t, const f16x8 (&src)[4], f16x8 (&at)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f16x8 x = src[d];
      if constexpr (rms) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const f16x2 x2 = {x[2 * h], x[2 * h + 1]};
          ss = __builtin_amdgcn_fdot2(x2, x2, ss, false);
        }
        x = x * *reinterpret_cast<const f16x8 *>(mg + (t * kTileK + 32 * d + 8 * kq) * 2);
      }
      at[d] = prescale_frag(x);
    }
  };
  // From LDS (M <= 4, slices of at most 5 k tiles) the fragments are ready
  // with the copies, and the whole slice is prepared before the loop
  // (measured faster: nothing waits for them, and the loop keeps only weight
  // work between its MFMAs); fragments loaded from memory are prepared at
  // their first use.
  //    (k tiles past the slice: zeroed by one uniform branch when the slice
  //    has any, ahead of the loop; per element at first use otherwise)
  static_assert(!ALDS || KPW <= 5, "LDS-staged rows only for shallow slices");
  constexpr bool PREP_AHEAD = ALDS;
  if constexpr (PREP_AHEAD) {
    if constexpr (!RES) {
#pragma unroll
      for (int t = 0; t < KPW; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) a[t][d][0] = read_slot(t, d);
    }
    if (my_n < KPW) {
#pragma unroll
      for (int t = 0; t < KPW; ++t)
        if (t >= my_n)
#pragma unroll
          for (int d = 0; d < 4; ++d) a[t][d][0] = f16x8{};
    }
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      f16x8 src[4], at0[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) src[d] = a[t][d][0];
      prep_tile(t, src, at0);
#pragma unroll
      for (int d = 0; d < 4; ++d) a[t][d][0] = at0[d];
    }
  }

  // 6. contraction, k tile outer, column tile inner.  The codes enter the
  //    matrix core bare (q * 2^-24); the activation slots facing 16q codes
  //    are pre-scaled by 1/16, and each k tile's group row sums serve its
  //    CPW column tiles for the zero-point term.
  f32x4 acc[NW][CPW][1];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int w = 0; w < CPW; ++w) acc[i][w][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int zshift = 4 * (c & 1);
  f32x4 ug[GPC];
  f16x8 at[4];
#pragma unroll
  for (int f = 0; f < NTILE; ++f) {
    if (f + PDE < NTILE) issue_tile(f + PDE);
    const int t = f / CPW, w = f % CPW;
    if (w == 0) {
      if constexpr (PREP_AHEAD) {
#pragma unroll
        for (int d = 0; d < 4; ++d) at[d] = a[t][d][0];
      } else {
        f16x8 src[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
          src[d] = t < my_n ? a[t][d][0] : f16x8{};
        prep_tile(t, src, at);
      }
      group_row_sums<G>(ug, at, kq);
    }
    const int gi0 = (w * KPW + t) * GPC;  // first group of the tile in the region
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint8_t *st = ms + i * MS_BYTES + (gi0 * 16 + c) * SB;
      const uint8_t *zt = mz + i * MZ_PAD + gi0 * 8 + (c >> 1);
      contract_tile_sub<G, GU>(
          acc[i][w][0], wv[i][f], at, ug, kq,
          [&](int gl) __attribute__((always_inline)) { return (zt[gl * 8] >> zshift) & 15; },
          [&](int gl) __attribute__((always_inline)) {
            if constexpr (SF32)
              return *reinterpret_cast<const float *>(st + gl * 16 * SB);
            else
              return (float)*reinterpret_cast<const f16 *>(st + gl * 16 * SB);
          });
    }
  }

  // 7. slice partial sums into the wavefront's own region ([i][w][lane],
  //    16 bytes per lane), row sums of squares of the slice; one barrier;
  //    wavefront w < CPW then sums column tile w over the slices in order
  f32x4 *red = reinterpret_cast<f32x4 *>(region);
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int w = 0; w < CPW; ++w) red[(i * CPW + w) * 64 + lane] = acc[i][w][0];
  if (rms) {
    // row l%16's k slots of this slice are spread over lanes l%16 + 16j
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 16) lRms[wk * 16 + lane] = ss;
  }
  const int wfin = wk;  // the column tile this wavefront finishes (if < CPW)
  const bool finisher = wfin < CPW && ct0 + wfin < NTL;
  const int ncol = (ct0 + wfin) * kTileN + c;
  // The epilogue's own inputs (bias, the staged rows' sums of squares) are
  // loaded before the barrier, so that their latency overlaps the wait for
  // the slowest slice instead of following the reduction: everything after
  // the barrier is on the kernel's critical path.
  float bias_v = 0.f;
  f32x4 row_ss = {0.f, 0.f, 0.f, 0.f};
  if (finisher) {
    if (!GU && p.epilogue != 0) bias_v = (float)p.bias[ncol];
    if (!rms && p.row_ss != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * kq + e < mrows) row_ss[e] = p.row_ss[m0 + 4 * kq + e];
    }
  }
  lds_barrier();
  if (!finisher) return;
  // all NWK slice partials are read before any is added (one LDS round
  // trip instead of a chain of them), then summed in slice order
  f32x4 fin[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    f32x4 part[NWK];
#pragma unroll
    for (int w2 = 0; w2 < NWK; ++w2)
      part[w2] = reinterpret_cast<const f32x4 *>(smem + w2 * p.lds_s)[(i * CPW + wfin) * 64 + lane];
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w2 = 0; w2 < NWK; ++w2) v += part[w2];
    fin[i] = v;
  }
  // sums of squares of this lane's output rows 4*(l/16) + e
  f32x4 rs = {0.f, 0.f, 0.f, 0.f};
  if (rms) {
    f32x4 part[NWK];
#pragma unroll
    for (int w2 = 0; w2 < NWK; ++w2) part[w2] = reinterpret_cast<const f32x4 *>(lRms + w2 * 16)[kq];
#pragma unroll
    for (int w2 = 0; w2 < NWK; ++w2) rs += part[w2];
  }

  // 8. k splits across workgroups (narrow grids and very deep k only): the
  //    finishing wavefronts store partials; the finishing wavefront of the
  //    last workgroup to arrive (counted per column tile) sums them in split
  //    order.  Partials, sums of squares and counters are agent-scope atomic
  //    accesses, coherent across the XCDs' separate L2 caches by themselves;
  //    the only ordering needed is that a wavefront's partial stores have
  //    completed before its arrival is counted (a wait on its own stores),
  //    and the last arrival reads them only after its count returned.  A
  //    device-wide fence instead would write back and invalidate the whole
  //    L2 of the XCD once per finishing wavefront.
  if (S > 1) {
    const size_t cnt = (size_t)blockIdx.z * NTL + ct0 + wfin;  // per column tile
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * kq + e;
      if (row < mrows) {
#pragma unroll
        for (int i = 0; i < NW; ++i)
          store_agent(&p.ws_part[(((size_t)s * NW + i) * p.M + m0 + row) * p.N + ncol], fin[i][e]);
        if (rms && c == 0) store_agent(&p.ws_rms[(cnt * S + s) * 16 + row], rs[e]);
      }
    }
    wait_stores();
    int last = 0;
    if (lane == 0) last = count_arrival(&p.ws_cnt[cnt]) == (unsigned)(S - 1);
    last = __shfl(last, 0);
    if (!last) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * kq + e;
      if (row < mrows) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          float v = 0.f;
          for (int s2 = 0; s2 < S; ++s2)
            v += (s2 == s) ? fin[i][e]
                           : load_agent(&p.ws_part[(((size_t)s2 * NW + i) * p.M + m0 + row) * p.N + ncol]);
          fin[i][e] = v;
        }
        if (rms) {
          float v = 0.f;
          for (int s2 = 0; s2 < S; ++s2)
            v += (s2 == s) ? rs[e] : load_agent(&p.ws_rms[(cnt * S + s2) * 16 + row]);
          rs[e] = v;
        }
      }
    }
    if (lane == 0) reset_arrival(&p.ws_cnt[cnt]);
  }

  // 9. epilogue, one fp16 write per output
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * kq + e;
    if (row < mrows) {
      float rsc = 1.0f;
      if (rms) rsc = 1.0f / sqrtf(rs[e] / (float)p.K + p.eps);
      else if (p.row_ss != nullptr)  // rows staged by stage.hip
        rsc = 1.0f / sqrtf(row_ss[e] / (float)p.K + p.eps);
      float y;
      if constexpr (GU) {
        y = silu(fin[0][e] * rsc) * (fin[1][e] * rsc);
      } else {
        y = fin[0][e] * rsc;
        if (p.epilogue != 0) y += bias_v;
        if (p.epilogue == 2) y = y > 0.f ? y : 0.f;
      }
      p.out[(size_t)(m0 + row) * p.N + ncol] = (f16)y;
    }
  }
}

template <int CPW, int KPW, int NWK, int PD, bool ALDS, int G, bool SF32, bool GU, int RMS>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = stream_kernel<CPW, KPW, NWK, PD, ALDS, G, SF32, GU, RMS>;
  static std::atomic<size_t> lds_limit[kMaxDevices];
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(kern), pl.lds_bytes, lds_limit);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.gx, pl.gy, pl.gz), dim3(64 * NWK), pl.lds_bytes, stream, a);
  return hipGetLastError();
}

template <int CPW, int KPW, int NWK, int PD, bool ALDS, int G, int RMS>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (sf32) return gu ? launch_t<CPW, KPW, NWK, PD, ALDS, G, true, true, RMS>(a, pl, st)
                      : launch_t<CPW, KPW, NWK, PD, ALDS, G, true, false, RMS>(a, pl, st);
  return gu ? launch_t<CPW, KPW, NWK, PD, ALDS, G, false, true, RMS>(a, pl, st)
            : launch_t<CPW, KPW, NWK, PD, ALDS, G, false, false, RMS>(a, pl, st);
}

template <int CPW, int KPW, int NWK, int PD, int G, int RMS>
hipError_t launch_a(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  // (deep slices never stage their rows through LDS: the planner does not
  // choose it, and the compiler would hoist every slot read of the slice)
  if constexpr (KPW <= 5) {
    if (pl.alds) return launch_g<CPW, KPW, NWK, PD, true, G, RMS>(a, pl, sf32, gu, st);
  }
  return launch_g<CPW, KPW, NWK, PD, false, G, RMS>(a, pl, sf32, gu, st);
}

template <int CPW, int KPW, int NWK, int PD, int RMS>
hipError_t launch_c(const GemmArgs &a, const Plan &pl, int group, bool sf32, bool gu,
                    hipStream_t st) {
  // the skip prologue in registers holds the whole slice: only shallow
  // slices take it (staged_prologue stages the others)
  if constexpr (RMS == 2 && KPW > 5) {
    return hipErrorInvalidValue;
  } else {
    switch (group) {
      case 16: return launch_a<CPW, KPW, NWK, PD, 16, RMS>(a, pl, sf32, gu, st);
      case 32: return launch_a<CPW, KPW, NWK, PD, 32, RMS>(a, pl, sf32, gu, st);
      case 64: return launch_a<CPW, KPW, NWK, PD, 64, RMS>(a, pl, sf32, gu, st);
      default: return launch_a<CPW, KPW, NWK, PD, 128, RMS>(a, pl, sf32, gu, st);
    }
  }
}


// (CPW, KPW, NWK, PD) of each configuration, in plan order: the planner
// takes the first one whose grid reaches 200 workgroups.
#define W4A16_STREAM_CFGS(X) \
  X(4, 5, 8, 8)   /* 4 column tiles x 8 slices of 5 k tiles (K <= 5120) */ \
  X(2, 5, 8, 6)   /* 2 column tiles, for narrower N */                     \
  X(1, 5, 8, 4)   /* 1 column tile, for narrow N */                        \
  X(1, 14, 8, 4)  /* 1 column tile x 8 slices of 14 k tiles (K <= 14336) */

// Launch the configuration the plan names with prologue mode RMS.
template <int RMS>
hipError_t launch_stream_cfg(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                             bool gate_up, hipStream_t stream) {
  int i = 0;
#define W4A16_CFG_CASE(cpw, kpw, nwk, pd) \
  if (pl.cfg == i++)                      \
    return launch_c<cpw, kpw, nwk, pd, RMS>(a, pl, group, scale_f32, gate_up, stream);
  W4A16_STREAM_CFGS(W4A16_CFG_CASE)
#undef W4A16_CFG_CASE
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace w4a16
