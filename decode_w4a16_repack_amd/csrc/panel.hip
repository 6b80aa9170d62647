// Fused W4A16 GEMM for gfx950 at 16 < M: blocks of MT 16-row tiles, where
// the weight stream from HBM still sets the pace (K=5120 N=13824 stays
// below the fp16 ridge up to M ~ 128) but each weight code now feeds
// several row tiles.
//
// Method (onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
// GEMM", "What's landed"): repacked weights, in-register unpack to the
// exact integers (q - zp), matrix-core contraction, each group's fp32
// partial multiplied by its scale after the contraction; k split with a
// fixed-order reduction ("P2 - widen the win: split-K").
//
// gfx950 design (the small-M stream kernel's, widened to MT row tiles):
//  * a workgroup is NWK wavefronts, one per k slice of KPW consecutive
//    128-k tiles, over the same CPW 16-column weight tiles and the same
//    16*MT rows; the slices are reduced in LDS in slice order;
//  * a wavefront streams its CPW x KPW weight tiles (one 16-byte load per
//    lane per 1 KiB tile) PD tiles ahead of the contraction;
//  * the activation fragments of one k tile (MT row tiles x four 32-k
//    steps) go from global memory (L2) straight into registers, each
//    fragment loaded by exactly one wavefront of the workgroup and used by
//    its CPW column tiles; with ADB the next k tile's fragments are loaded
//    while the current one is contracted;
//  * each 32-bit word of codes is unpacked once into the exact integers
//    q - z as fp16 and feeds MT matrix-core operations, so the unpack cost
//    per MFMA falls as 1/MT;
//  * scales and zero-points of the slice (and, with the RMSNorm prologue,
//    its gamma) are copied once into a private LDS region per wavefront; no
//    barrier sits in the loop, only the one before the slice reduction;
//  * with the RMSNorm prologue each k tile's fragments are turned into
//    x * gamma once, and their sums of squares kept per row;
//  * the (row tile, column tile) output blocks are shared out over the
//    wavefronts for the final sum: slice sum in slice order, the RMSNorm
//    row scale (from the slices' sums of squares, or from rows staged by
//    stage.hip), epilogue, one fp16 write.  Wide reductions (gate_up) go in
//    one pass per weight stream so the LDS need not hold both at once.
#include "device.h"

namespace w4a16 {

namespace {

// (occupancy NWK / 4 wavefronts per SIMD, as for the streaming kernel)
// RMS: the RMSNorm prologue in the kernel (no residual, no k split across
// workgroups): x * gamma rounded once to fp16 in the fragments, the row
// sums of squares in fp32, 1/sqrt(mean + eps) in the epilogue.
template <int MT, int CPW, int KPW, int NWK, int PD, bool ADB, int G, bool SF32, bool GU, bool RMS>
__global__ void __launch_bounds__(64 * NWK) __attribute__((amdgpu_waves_per_eu(NWK / 4, NWK / 4)))
panel_kernel(const GemmArgs p) {
  constexpr int NW = GU ? 2 : 1;
  constexpr int PDE = GU ? (PD + 1) / 2 : PD;  // tiles in flight per weight stream
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int NTILE = CPW * KPW;
  constexpr int GPW = KPW * GPC;                 // groups of one wavefront's k slice
  constexpr int MS_BYTES = CPW * GPW * 16 * SB;  // its scales, [CPW][GPW][16]
  constexpr int MZ_BYTES = CPW * GPW * 8;        // its zero-points, [CPW][GPW][8 bytes]
  constexpr int MZ_PAD = (MZ_BYTES + 15) / 16 * 16;
  constexpr int SU = GPW * SB;  // 16-byte scale units per column tile
  constexpr int ZU = GPW * 2;   // 4-byte zero-point units per column tile
  constexpr int NPAIR = MT * CPW;                   // output blocks of the workgroup
  constexpr int PPW = (NPAIR + NWK - 1) / NWK;      // output blocks finished per wavefront
  constexpr int NAB = ADB ? 2 : 1;                  // activation buffers
  constexpr bool A1_EARLY = ADB && KPW > 1;  // second k tile's activations before the loop
  // loads issued after the metadata copies that may still be in flight when
  // the copies are waited for: the first k tile's activations (and the
  // second's) and the first PDE tiles of each stream
  constexpr int AFTER_COPIES = MT * 4 * (A1_EARLY ? 2 : 1) + PDE * NW;
  static_assert(PDE >= 1 && PDE <= NTILE, "prefetch depth");

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
  const int m0 = blockIdx.z * (16 * MT);
  const int mrows = min(16 * MT, p.M - m0);
  const int kb = s * p.cps;
  const int nkc = min(KC, kb + p.cps) - kb;
  const int my_kb = kb + wk * KPW;
  const int my_n = max(0, min(KPW, nkc - wk * KPW));  // valid k tiles of this slice
  const bool has_zp = p.has_zp != 0;
  const int kq = lane >> 4;
  const int c = lane & 15;

  uint8_t *region = smem + wk * p.lds_s;
  uint8_t *ms = region;                  // [NW] x MS_BYTES
  uint8_t *mz = region + NW * MS_BYTES;  // [NW] x MZ_PAD
  uint8_t *mg = mz + NW * MZ_PAD;        // RMS: the slice's gamma, [KPW][128] fp16
  // RMS: the slices' row sums of squares, [NWK][16 * MT], after the split flag
  float *lRms = reinterpret_cast<float *>(smem + p.lds_r + 16);

  // 1. this slice's scales and zero-points of the CPW column tiles, copied
  //    straight into the private region (reads clamped to the column tile's
  //    own groups; lanes past the copy write nothing)
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
  if constexpr (RMS) {
    // the slice's gamma (positions past the slice copy a valid tile)
#pragma unroll
    for (int q = 0; q < (KPW * 16 + 63) / 64; ++q) {
      const int u = q * 64 + lane;
      if (u < KPW * 16) {
        const int kc = min(my_kb + min(u >> 4, max(my_n - 1, 0)), KC - 1);
        copy16_to_lds(p.gamma + kc * kTileK + (u & 15) * 8, mg + q * 1024);
      }
    }
  }

  // 2. activation fragments of k tile position t of the slice: row tile mt,
  //    row 16*mt + l%16 (rows past M read row M-1: an A row feeds only its
  //    own output row, never written), k slots 8*(l/16)..+7 of each 32-k
  //    step d.  Positions past the slice re-read a valid tile; their scales
  //    are taken as zero, so they add nothing.
  auto kc_of = [&](int t) __attribute__((always_inline)) {
    return min(my_kb + min(t, max(my_n - 1, 0)), KC - 1);
  };
  f16x8 a[NAB][MT][4];
  auto load_a = [&](int t, f16x8 (&ab)[MT][4]) __attribute__((always_inline)) {
    const int kc = kc_of(t);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const size_t off = (size_t)(m0 + min(16 * mt + c, mrows - 1)) * p.K + kc * kTileK + 8 * kq;
#pragma unroll
      for (int d = 0; d < 4; ++d) ab[mt][d] = *reinterpret_cast<const f16x8 *>(p.A + off + 32 * d);
    }
  };

  // 3. weight tiles: tile f = t * CPW + w (k tile position t, column tile
  //    w), issued PDE tiles before it is contracted; tiles past the slice or
  //    past N re-read a valid tile
  u32x4 wv[NW][NTILE];
  auto issue_tile = [&](int f) __attribute__((always_inline)) {
    const int t = f / CPW, w = f % CPW;
    const size_t tile = (size_t)min(ct0 + w, NTL - 1) * KC + kc_of(t);
#pragma unroll
    for (int i = 0; i < NW; ++i)
      wv[i][f] = load_weights(p.w[i] + tile * kTileBytes, lane);
  };

  // (the wait below counts on every later load being issued after the
  // copies: nothing may be scheduled above this point)
  __builtin_amdgcn_sched_barrier(0);
  load_a(0, a[0]);
#pragma unroll
  for (int f = 0; f < PDE; ++f) issue_tile(f);
  if constexpr (A1_EARLY) load_a(1, a[1 % NAB]);
  // 4. this wavefront's metadata copies have landed (completion is in issue
  //    order); no other wavefront reads its region before the reduction
  wait_vmcnt<(AFTER_COPIES < 63 ? AFTER_COPIES : 63)>();

  // 5. contraction, k tile outer, column tile inner: each unpacked word of
  //    codes feeds MT MFMAs, each activation fragment CPW
  f32x4 acc[NW][CPW][MT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int w = 0; w < CPW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][w][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int zshift = 4 * (c & 1);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  float ss[MT];  // RMS: this lane's part of the sums of squares of rows 16 mt + l%16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) ss[mt] = 0.f;
  static_for<NTILE>([&](auto fc) __attribute__((always_inline)) {
    constexpr int f = decltype(fc)::value;
    constexpr int t = f / CPW, w = f % CPW;
    f16x8 (&at)[MT][4] = a[t % NAB];
    // one weight tile at a time: the scheduler may not pull a later tile's
    // unpack or loads up into this one (the registers would run out)
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (w == 0) {
      if constexpr (!ADB && t > 0) {
        // (no earlier: the single activation buffer is still being read
        // by the previous k tile, and hoisting the loads above that would
        // need a second buffer's registers)
        __builtin_amdgcn_sched_barrier(0);
        load_a(t, at);
      }
      if constexpr (ADB && t > 0 && t + 1 < KPW) load_a(t + 1, a[(t + 1) % NAB]);
    }
    if constexpr (f + PDE < NTILE) issue_tile(f + PDE);
    if constexpr (RMS && w == 0) {
      // the k tile's fragments, once for its CPW column tiles: sums of
      // squares (fp16 products are exact in fp32), then x * gamma rounded
      // once to fp16 (tiles past the slice add nothing: their scales are 0)
      if (t < my_n) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const f16x8 x = at[mt][d];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const f16x2 x2 = {x[2 * h], x[2 * h + 1]};
              ss[mt] = __builtin_amdgcn_fdot2(x2, x2, ss[mt], false);
            }
            at[mt][d] = x * *reinterpret_cast<const f16x8 *>(mg + (t * kTileK + 32 * d + 8 * kq) * 2);
          }
      }
    }
    const float on = t < my_n ? 1.0f : 0.0f;
    const int gi0 = (w * KPW + t) * GPC;  // first group of the tile in the region
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const u32x4 wt = wv[i][f];
      const uint8_t *st = ms + i * MS_BYTES + (gi0 * 16 + c) * SB;
      const uint8_t *zt = mz + i * MZ_PAD + gi0 * 8 + (c >> 1);
      auto scale = [&](int gl) __attribute__((always_inline)) {
        if constexpr (SF32)
          return on * *reinterpret_cast<const float *>(st + gl * 16 * SB);
        else
          return on * (float)*reinterpret_cast<const f16 *>(st + gl * 16 * SB);
      };
      auto zconst = [&](int gl, f16x2 &zlo, f16x2 &zhi) __attribute__((always_inline)) {
        zero_consts((uint32_t)((zt[gl * 8] >> zshift) & 15), zlo, zhi);
      };
      if constexpr (G >= 32) {
        constexpr int SPG = G / 32;  // 32-k steps per group
        f32x4 accg[MT];
        f16x2 zlo, zhi;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          if (d % SPG == 0) zconst(d / SPG, zlo, zhi);
          const f16x8 b = unpack8(wt[d], zlo, zhi);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            accg[mt] = mfma16(at[mt][d], b, (d % SPG == 0) ? zero4 : accg[mt]);
          if ((d + 1) % SPG == 0) {
            const float sc = scale(d / SPG);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[i][w][mt][e] = __builtin_fmaf(accg[mt][e], sc, acc[i][w][mt][e]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) pin_acc(acc[i][w][mt]);
          }
        }
      } else {
        // group 16: the k slots of lanes kq < 2 are group 2d, the others 2d + 1
        const f16x8 zero8 = {};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          f16x2 zlo, zhi;
          zconst(2 * d + (kq >> 1), zlo, zhi);
          const f16x8 b = unpack8(wt[d], zlo, zhi);
          const f16x8 blo = (kq < 2) ? b : zero8;
          const f16x8 bhi = (kq < 2) ? zero8 : b;
          const float s0 = scale(2 * d), s1 = scale(2 * d + 1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const f32x4 p0 = mfma16(at[mt][d], blo, zero4);
            const f32x4 p1 = mfma16(at[mt][d], bhi, zero4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][w][mt][e] =
                  __builtin_fmaf(p1[e], s1, __builtin_fmaf(p0[e], s0, acc[i][w][mt][e]));
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) pin_acc(acc[i][w][mt]);
        }
      }
    }
  });

  // 6. the slice partial sums, one weight stream per pass, through the
  //    private regions; wavefront wk finishes output blocks wk, wk + NWK, ...
  //    (block = mt * CPW + w) in slice order
  if constexpr (RMS) {
    // row 16 mt + l%16's k slots of this slice are spread over lanes
    // l%16 + 16j; the first lds_barrier below publishes them
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float v = ss[mt];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) lRms[wk * (16 * MT) + 16 * mt + lane] = v;
    }
  }
  f32x4 fin[NW][PPW];
  f32x4 *red = reinterpret_cast<f32x4 *>(region);
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i > 0) lds_barrier();  // the previous pass's reads are done
#pragma unroll
    for (int w = 0; w < CPW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[(mt * CPW + w) * 64 + lane] = acc[i][w][mt];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int pr = wk + NWK * j;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (pr < NPAIR) {
        // every slice's partial read before any is added (one LDS round
        // trip), then summed in slice order
        f32x4 part[NWK];
#pragma unroll
        for (int w2 = 0; w2 < NWK; ++w2)
          part[w2] = reinterpret_cast<const f32x4 *>(smem + w2 * p.lds_s)[pr * 64 + lane];
#pragma unroll
        for (int w2 = 0; w2 < NWK; ++w2) v += part[w2];
      }
      fin[i][j] = v;
    }
  }

  // 7. k splits across workgroups (deep K, or a grid short of one
  //    workgroup per compute unit): every workgroup stores its partial sums
  //    and the last workgroup to arrive at this
  //    output tile (one counter per tile) sums them in split order.
  //    Agent-scope atomic accesses keep the exchange coherent across the
  //    XCDs' L2 caches without a device-wide fence; every wavefront waits
  //    for its own stores before the workgroup barrier that precedes the
  //    count.
  if (S > 1) {
    const size_t tile_id = (size_t)blockIdx.z * gridDim.x + blockIdx.x;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int pr = wk + NWK * j;
      if (pr >= NPAIR) break;
      const int mt = pr / CPW, w = pr % CPW;
      const int ncol = min(ct0 + w, NTL - 1) * kTileN + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mt + 4 * kq + e;
        if (row < mrows && ct0 + w < NTL) {
#pragma unroll
          for (int i = 0; i < NW; ++i)
            store_agent(&p.ws_part[(((size_t)s * NW + i) * p.M + m0 + row) * p.N + ncol], fin[i][j][e]);
        }
      }
    }
    wait_stores();
    int *flag = reinterpret_cast<int *>(smem + p.lds_r);
    __syncthreads();
    if (tid == 0) *flag = count_arrival(&p.ws_cnt[tile_id]) == (unsigned)(S - 1);
    __syncthreads();
    if (*flag == 0) return;
    // split by split, in order, all of the wavefront's outputs at once: one
    // round trip to memory per split (rows past M and columns past N read a
    // clamped slot and are never written)
    f32x4 sum[NW][PPW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int j = 0; j < PPW; ++j) sum[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < S; ++s2) {
      f32x4 v[NW][PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int pr = min(wk + NWK * j, NPAIR - 1);
        const int mt = pr / CPW, w = pr % CPW;
        const int ncol = min(ct0 + w, NTL - 1) * kTileN + c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = min(16 * mt + 4 * kq + e, mrows - 1);
#pragma unroll
          for (int i = 0; i < NW; ++i)
            v[i][j][e] = (s2 == s) ? fin[i][j][e]
                                   : load_agent(&p.ws_part[(((size_t)s2 * NW + i) * p.M + m0 + row) * p.N + ncol]);
        }
      }
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < PPW; ++j) sum[i][j] += v[i][j];
    }
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int j = 0; j < PPW; ++j) fin[i][j] = sum[i][j];
    if (tid == 0) reset_arrival(&p.ws_cnt[tile_id]);
  }

  // 8. epilogue (row scale of the RMSNorm prologue, SwiGLU or bias / ReLU),
  //    one fp16 write per output
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int pr = wk + NWK * j;
    if (pr >= NPAIR) break;
    const int mt = pr / CPW, w = pr % CPW;
    if (ct0 + w >= NTL) continue;
    const int ncol = (ct0 + w) * kTileN + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mt + 4 * kq + e;
      if (row < mrows) {
        float rsc = 1.0f;
        if constexpr (RMS) {
          // the slices' sums in slice order
          float rs = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < NWK; ++w2) rs += lRms[w2 * (16 * MT) + row];
          rsc = 1.0f / sqrtf(rs / (float)p.K + p.eps);
        } else if (p.row_ss != nullptr) {
          rsc = 1.0f / sqrtf(p.row_ss[m0 + row] / (float)p.K + p.eps);
        }
        float y;
        if constexpr (GU) {
          y = silu(fin[0][j][e] * rsc) * (fin[1][j][e] * rsc);
        } else {
          y = fin[0][j][e] * rsc;
          if (p.epilogue != 0) y += (float)p.bias[ncol];
          if (p.epilogue == 2) y = y > 0.f ? y : 0.f;
        }
        p.out[(size_t)(m0 + row) * p.N + ncol] = (f16)y;
      }
    }
  }
}

template <int MT, int CPW, int KPW, int NWK, int PD, bool ADB, int G, bool SF32, bool GU, bool RMS>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = panel_kernel<MT, CPW, KPW, NWK, PD, ADB, G, SF32, GU, RMS>;
  static std::atomic<size_t> lds_limit[kMaxDevices];
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(kern), pl.lds_bytes, lds_limit);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.gx, pl.gy, pl.gz), dim3(64 * NWK), pl.lds_bytes, stream, a);
  return hipGetLastError();
}

template <int MT, int CPW, int KPW, int NWK, int PD, bool ADB, int G, bool RMS>
hipError_t launch_r(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (gu)
    return sf32 ? launch_t<MT, CPW, KPW, NWK, PD, ADB, G, true, true, RMS>(a, pl, st)
                : launch_t<MT, CPW, KPW, NWK, PD, ADB, G, false, true, RMS>(a, pl, st);
  return sf32 ? launch_t<MT, CPW, KPW, NWK, PD, ADB, G, true, false, RMS>(a, pl, st)
              : launch_t<MT, CPW, KPW, NWK, PD, ADB, G, false, false, RMS>(a, pl, st);
}

// with a gamma (and so, by the plan, no residual and no k split across
// workgroups) the RMSNorm prologue runs in the kernel
template <int MT, int CPW, int KPW, int NWK, int PD, bool ADB, int G>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (a.gamma != nullptr) {
    if (a.resid != nullptr || pl.split > 1) return hipErrorInvalidValue;
    return launch_r<MT, CPW, KPW, NWK, PD, ADB, G, true>(a, pl, sf32, gu, st);
  }
  return launch_r<MT, CPW, KPW, NWK, PD, ADB, G, false>(a, pl, sf32, gu, st);
}

template <int MT, int CPW, int KPW, int NWK, int PD, bool ADB>
hipError_t launch_c(const GemmArgs &a, const Plan &pl, int group, bool sf32, bool gu,
                    hipStream_t st) {
  switch (group) {
    case 16: return launch_g<MT, CPW, KPW, NWK, PD, ADB, 16>(a, pl, sf32, gu, st);
    case 32: return launch_g<MT, CPW, KPW, NWK, PD, ADB, 32>(a, pl, sf32, gu, st);
    case 64: return launch_g<MT, CPW, KPW, NWK, PD, ADB, 64>(a, pl, sf32, gu, st);
    default: return launch_g<MT, CPW, KPW, NWK, PD, ADB, 128>(a, pl, sf32, gu, st);
  }
}

}  // namespace

// (MT, CPW, KPW, NWK, PD, ADB) of each configuration: 32 rows x 4 column
// tiles, the next k tile's activations loaded while the current one is
// contracted; narrow grids are filled by splitting k across workgroups.
#define W4A16_PANEL_CFGS(X) X(2, 4, 5, 8, 8, true)

const PanelCfg kPanelCfgs[kNumPanelCfgs] = {
#define W4A16_CFG_ROW(mt, cpw, kpw, nwk, pd, adb) {mt, cpw, kpw, nwk, pd},
    W4A16_PANEL_CFGS(W4A16_CFG_ROW)
#undef W4A16_CFG_ROW
};

hipError_t launch_panel(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                        bool gate_up, hipStream_t stream) {
  int i = 0;
#define W4A16_CFG_CASE(mt, cpw, kpw, nwk, pd, adb) \
  if (pl.cfg == i++)                               \
    return launch_c<mt, cpw, kpw, nwk, pd, adb>(a, pl, group, scale_f32, gate_up, stream);
  W4A16_PANEL_CFGS(W4A16_CFG_CASE)
#undef W4A16_CFG_CASE
  return hipErrorInvalidValue;
}

}  // namespace w4a16
