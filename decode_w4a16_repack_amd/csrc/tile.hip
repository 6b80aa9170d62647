// Fused W4A16 GEMM for gfx950 at M > 16: the matrix-core regime (at
// K=5120 N=13824 the arithmetic intensity passes the fp16 ridge near M=128).
//
// Method (onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
// GEMM", "What's landed"): repacked weights, in-register unpack to the exact
// integers (q - zp), matrix-core contraction, each group's fp32 partial
// multiplied by its scale after the contraction; the k range is split and
// reduced in a fixed order, so results are run-to-run identical.
//
// gfx950 design.  A workgroup computes a 64-row x (2*CT*16)-column output
// tile over the whole K with 8 wavefronts (4 when LDS is short):
//  * wavefront (wc, ks) owns column half wc (CT 16-column weight tiles) and
//    k slice ks: it takes every NKS-th 128-k tile, so the NKS slices walk K
//    side by side in steps;
//  * its output block is 64 x (CT*16) = MT x CT MFMA tiles: each unpacked
//    weight fragment feeds MT = 4 MFMAs and each activation fragment CT, which
//    keeps both the unpack (VALU) and the activation reads (LDS) below the
//    matrix-core time;
//  * per step and slice, the 64 x 128 activation tile goes straight from
//    global memory into a double-buffered LDS tile (direct global-to-LDS
//    loads of whole row segments; both column halves read it), its 16-byte
//    chunks XOR-swizzled by row so an MFMA operand read is conflict-free;
//    the wavefront's scales and zero-points of the step go the same way into
//    its own double-buffered LDS slot;
//  * the weights of the next step are loaded into registers (one 16-byte
//    load per lane per 1 KiB tile) while the current step computes;
//  * one barrier per step; after the last, the slices' partial sums meet in
//    LDS and wavefront (wc, ks) finishes row tiles ks, ks + NKS, ... of its
//    column half in slice order: RMSNorm factor, epilogue, one fp16 write.
#include "device.h"

namespace w4a16 {

namespace {

constexpr int kTileMT = 4;   // 16-row MFMA tiles per wavefront (64 rows per workgroup)
constexpr int kTileNWC = 2;  // column halves per workgroup

template <int G, bool SF32>
constexpr int tile_nks() {
  return (G == 16 && SF32) ? 2 : 4;  // k slices; fewer when the metadata slots need the LDS
}

template <int CT, int G, bool SF32, bool GU>
__global__ void __launch_bounds__((64 * kTileNWC * tile_nks<G, SF32>()))
tile_kernel(const GemmArgs p) {
  constexpr int MT = kTileMT;
  constexpr int NWC = kTileNWC;
  constexpr int NKS = tile_nks<G, SF32>();
  constexpr int NW = GU ? 2 : 1;
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int A_BYTES = 64 * kTileK * 2;            // one slice's 64 x 128 activation tile
  constexpr int MS = CT * GPC * 16 * SB;              // scales of one step, one stream
  constexpr int MZ = (CT * GPC * 8 + 15) / 16 * 16;   // zero-points of one step, one stream
  constexpr int GB = kTileK * 2;                       // gamma of one step (RMSNorm)
  constexpr int MB = NW * (MS + MZ) + GB;             // one metadata slot
  constexpr int SU = GPC * SB;                        // 16-byte scale units per column tile
  constexpr int ZU = GPC * 2;                         // 4-byte zero-point units per column tile
  constexpr int META_OFF = 2 * NKS * A_BYTES;
  constexpr int RMS_OFF = META_OFF + NWC * NKS * 2 * MB;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave % NWC;
  const int ks = wave / NWC;
  const int kq = lane >> 4;
  const int c = lane & 15;
  const int NTL = p.N / kTileN;
  const int KC = p.K / kTileK;
  const int Gall = p.K / G;
  const int m0 = blockIdx.z * 64;
  const int mrows = min(64, p.M - m0);
  const int ctw = blockIdx.x * NWC * CT + wc * CT;  // first column tile of this wavefront
  const int nsteps = (KC + NKS - 1) / NKS;
  const bool rms = p.gamma != nullptr;
  const bool has_zp = p.has_zp != 0;
  uint8_t *mslot = smem + META_OFF + wave * 2 * MB;
  float *lRms = reinterpret_cast<float *>(smem + RMS_OFF);  // [NKS][64 rows]

  // k tile of step j for this slice (clamped: steps past K re-read a valid
  // tile and are skipped)
  auto ktile = [&](int j) __attribute__((always_inline)) { return j * NKS + ks; };

  // direct-to-LDS copies of step j: this slice's activation tile (half of
  // it per column half) and this wavefront's scales / zero-points (and
  // gamma, with the RMSNorm prologue)
  auto issue_copies = [&](int j) __attribute__((always_inline)) {
    const int kt = min(ktile(j), KC - 1);
    uint8_t *abuf = smem + ((j & 1) * NKS + ks) * A_BYTES;
#pragma unroll
    for (int q = wc; q < A_BYTES / 1024; q += NWC) {
      // slot r * 16 + pos holds 16-byte chunk pos ^ (r % 16) of row r: one
      // copy reads four whole 256-byte row segments
      const int sl = q * 64 + lane;
      const int row = sl >> 4, chunk = (sl & 15) ^ (row & 15);
      const f16 *src = p.A + (size_t)(m0 + min(row, mrows - 1)) * p.K + kt * kTileK + 8 * chunk;
      copy16_to_lds(src, abuf + q * 1024);
    }
    uint8_t *slot = mslot + (j & 1) * MB;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint8_t *sbase = reinterpret_cast<const uint8_t *>(p.scales[i]);
#pragma unroll
      for (int q = 0; q < (CT * SU + 63) / 64; ++q) {
        const int u = q * 64 + lane;
        if (u < CT * SU) {
          const int w = u / SU, o = u - w * SU;
          const size_t t = (size_t)min(ctw + w, NTL - 1);
          copy16_to_lds(sbase + ((t * Gall + (size_t)kt * GPC) * 16) * SB + o * 16,
                        slot + i * MS + q * 1024);
        }
      }
      if (has_zp) {
#pragma unroll
        for (int q = 0; q < (CT * ZU + 63) / 64; ++q) {
          const int u = q * 64 + lane;
          if (u < CT * ZU) {
            const int w = u / ZU, o = u - w * ZU;
            const size_t t = (size_t)min(ctw + w, NTL - 1);
            copy4_to_lds(p.zeros[i] + (t * Gall + (size_t)kt * GPC) * 8 + o * 4,
                         slot + NW * MS + i * MZ + q * 256);
          }
        }
      }
    }
    if (rms && lane < 16) copy16_to_lds(p.gamma + kt * kTileK + lane * 8, slot + NW * (MS + MZ));
  };

  // symmetric weights: every zero-point is 8, in both slots
  if (!has_zp) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < NW; ++i)
        for (int e = lane; e * 4 < MZ; e += 64)
          reinterpret_cast<uint32_t *>(mslot + b * MB + NW * MS + i * MZ)[e] = 0x88888888u;
  }

  // weight tiles of step j (registers)
  auto load_w = [&](int j, u32x4 (&wv)[NW][CT]) __attribute__((always_inline)) {
    const int kt = min(ktile(j), KC - 1);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const size_t tile = (size_t)min(ctw + ct, NTL - 1) * KC + kt;
#pragma unroll
      for (int i = 0; i < NW; ++i)
        wv[i][ct] = reinterpret_cast<const u32x4 *>(p.w[i] + tile * kTileBytes)[lane];
    }
  };
  f32x4 acc[NW][MT][CT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[i][mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 ssq = {0.f, 0.f, 0.f, 0.f};  // sum of squares of row 16mt + c, per mt (column half 0)

  const int zshift = 4 * (c & 1);
  auto compute = [&](int j, const u32x4 (&wv)[NW][CT]) __attribute__((always_inline)) {
    // row 16mt + c, chunk 4d + kq sits at slot row * 16 + ((4d + kq) ^ c): the
    // 16 rows of one operand read land in 16 different chunk positions
    const uint8_t *abuf = smem + ((j & 1) * NKS + ks) * A_BYTES + c * 256;
    const uint8_t *slot = mslot + (j & 1) * MB;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // the step's activation fragments, all 4 x MT of them
    f16x8 a[4][MT];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f16x8 gam = {};
      if (rms) gam = *reinterpret_cast<const f16x8 *>(slot + NW * (MS + MZ) + (32 * d + 8 * kq) * 2);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        a[d][mt] = *reinterpret_cast<const f16x8 *>(abuf + mt * 4096 + ((4 * d + kq) ^ c) * 16);
        if (rms) {
          if (wc == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = (float)a[d][mt][e];
              ssq[mt] = __builtin_fmaf(x, x, ssq[mt]);
            }
          }
          a[d][mt] = a[d][mt] * gam;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint8_t *sp = slot + i * MS + ((ct * GPC) * 16 + c) * SB;     // scale of group 0
        const uint8_t *zp = slot + NW * MS + i * MZ + (ct * GPC) * 8 + (c >> 1);
        auto scale = [&](int g2) __attribute__((always_inline)) {
          if constexpr (SF32)
            return *reinterpret_cast<const float *>(sp + g2 * 16 * SB);
          else
            return (float)*reinterpret_cast<const f16 *>(sp + g2 * 16 * SB);
        };
        auto zconst = [&](int g2, f16x2 &zlo, f16x2 &zhi) __attribute__((always_inline)) {
          zero_consts((uint32_t)((zp[g2 * 8] >> zshift) & 15), zlo, zhi);
        };
        if constexpr (G >= 32) {
          constexpr int SPG = G / 32;  // 32-k steps per group
          f32x4 accg[MT];
          f16x2 zlo, zhi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            if (d % SPG == 0) zconst(d / SPG, zlo, zhi);
            const f16x8 b = unpack8(wv[i][ct][d], zlo, zhi);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              accg[mt] = mfma16(a[d][mt], b, (d % SPG == 0) ? zero4 : accg[mt]);
            if ((d + 1) % SPG == 0) {
              const float sc = scale(d / SPG);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  acc[i][mt][ct][e] = __builtin_fmaf(accg[mt][e], sc, acc[i][mt][ct][e]);
            }
          }
        } else {
          // group 16: k slots of lanes kq < 2 are group 2d, the others 2d + 1
          const f16x8 zero8 = {};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            f16x2 zlo, zhi;
            zconst(2 * d + (kq >> 1), zlo, zhi);
            const f16x8 b = unpack8(wv[i][ct][d], zlo, zhi);
            const f16x8 blo = (kq < 2) ? b : zero8;
            const f16x8 bhi = (kq < 2) ? zero8 : b;
            const float s0 = scale(2 * d), s1 = scale(2 * d + 1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const f32x4 p0 = mfma16(a[d][mt], blo, zero4);
              const f32x4 p1 = mfma16(a[d][mt], bhi, zero4);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[i][mt][ct][e] =
                    __builtin_fmaf(p1[e], s1, __builtin_fmaf(p0[e], s0, acc[i][mt][ct][e]));
            }
          }
        }
      }
    }
  };

  // Pipeline: copies and weights of step 0, then per step j: wait for its
  // copies, barrier (also frees the other buffers), issue step j + 1,
  // compute j.
  u32x4 w0[NW][CT], w1[NW][CT];
  issue_copies(0);
  load_w(0, w0);
  auto step = [&](int j, u32x4 (&wcur)[NW][CT], u32x4 (&wnext)[NW][CT])
      __attribute__((always_inline)) {
    // the copies of step j were issued before its weight loads
    wait_vmcnt<NW * CT>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (j + 1 < nsteps) {
      issue_copies(j + 1);
      load_w(j + 1, wnext);
    }
    if (ktile(j) < KC) compute(j, wcur);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  };
  for (int j = 0; j < nsteps; j += 2) {
    step(j, w0, w1);
    if (j + 1 < nsteps) step(j + 1, w1, w0);
  }
  __syncthreads();  // every step done: the activation tiles become reduction scratch

  // slice partial sums -> LDS ([wave][i][mt][ct][lane], 16 bytes per lane)
  f32x4 *red = reinterpret_cast<f32x4 *>(smem);
  constexpr int PER = NW * MT * CT;
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        red[((wave * NW + i) * MT + mt) * CT * 64 + ct * 64 + lane] = acc[i][mt][ct];
  if (rms && wc == 0) {
    // row 16mt + c's k slots are spread over lanes c + 16j
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float v = ssq[mt];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) lRms[ks * 64 + 16 * mt + lane] = v;
    }
  }
  __syncthreads();
  (void)PER;

  // wavefront (wc, ks) finishes row tiles ks, ks + NKS, ... of column half wc
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt % NKS != ks) continue;
    f32x4 rs = {0.f, 0.f, 0.f, 0.f};
    if (rms)
      for (int s2 = 0; s2 < NKS; ++s2)
        rs += reinterpret_cast<const f32x4 *>(lRms + s2 * 64 + 16 * mt)[kq];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (ctw + ct >= NTL) continue;
      f32x4 fin[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int s2 = 0; s2 < NKS; ++s2)
          v += red[(((s2 * NWC + wc) * NW + i) * MT + mt) * CT * 64 + ct * 64 + lane];
        fin[i] = v;
      }
      const int ncol = (ctw + ct) * kTileN + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mt + 4 * kq + e;
        if (row < mrows) {
          float rsc = 1.0f;
          if (rms) rsc = 1.0f / sqrtf(rs[e] / (float)p.K + p.eps);
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
  }
}

template <int CT, int G, bool SF32, bool GU>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = tile_kernel<CT, G, SF32, GU>;
  // Raise the kernel's dynamic-LDS limit above the default 64 KiB once; later
  // launches (also under stream capture) make no attribute call.
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
  hipLaunchKernelGGL(kern, dim3(pl.gx, pl.gy, pl.gz), dim3(64 * kTileNWC * tile_nks<G, SF32>()),
                     pl.lds_bytes, stream, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  if (sf32) return gu ? launch_t<2, G, true, true>(a, pl, st) : launch_t<4, G, true, false>(a, pl, st);
  return gu ? launch_t<2, G, false, true>(a, pl, st) : launch_t<4, G, false, false>(a, pl, st);
}

}  // namespace

int tile_k_slices(int group, bool scale_f32) {
  if (scale_f32 && group == 16) return tile_nks<16, true>();
  return 4;
}

size_t tile_lds_bytes(int group, int scale_bytes, bool gate_up) {
  const int nks = tile_k_slices(group, scale_bytes == 4);
  const int nw = gate_up ? 2 : 1;
  const int ct = gate_up ? 2 : 4;
  const int gpc = kTileK / group;
  const size_t ms = (size_t)ct * gpc * 16 * scale_bytes;
  const size_t mz = ((size_t)ct * gpc * 8 + 15) / 16 * 16;
  const size_t mb = nw * (ms + mz) + kTileK * 2;
  const size_t a = 2 * (size_t)nks * 64 * kTileK * 2;
  return a + (size_t)kTileNWC * nks * 2 * mb + (size_t)nks * 64 * 4;
}

int tile_columns(bool gate_up) { return kTileNWC * (gate_up ? 2 : 4) * kTileN; }

hipError_t launch_tile(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                       bool gate_up, hipStream_t stream) {
  switch (group) {
    case 16: return launch_g<16>(a, pl, scale_f32, gate_up, stream);
    case 32: return launch_g<32>(a, pl, scale_f32, gate_up, stream);
    case 64: return launch_g<64>(a, pl, scale_f32, gate_up, stream);
    default: return launch_g<128>(a, pl, scale_f32, gate_up, stream);
  }
}

}  // namespace w4a16
