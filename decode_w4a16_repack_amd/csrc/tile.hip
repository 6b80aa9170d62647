// Fused W4A16 GEMM for gfx950 at M > 16: the matrix-core regime (at
// K=5120 N=13824 the arithmetic intensity passes the fp16 ridge near M=128).
//
// Method (onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
// GEMM", "What's landed"): repacked weights, in-register unpack to the exact
// integers (q - zp), matrix-core contraction, each group's fp32 partial
// multiplied by its scale after the contraction; the k range is split and
// reduced in a fixed order, so results are run-to-run identical.
//
// gfx950 design.  A workgroup computes a 64-row x (4*CT*16)-column output
// tile over the whole K with 8 wavefronts, two per SIMD (one issues VALU
// work while the other's MFMAs run):
//  * wavefront (wc, ks) owns column quarter wc (CT 16-column weight tiles)
//    and k slice ks: it takes every other 128-k tile, so the two slices walk
//    K side by side in steps;
//  * its output block is 64 x (CT*16) = 4 x CT MFMA tiles: each unpacked
//    weight fragment feeds 4 MFMAs and each activation fragment CT, and the
//    activation tile of a step is shared by the four column quarters;
//  * the slice's 64 x 128 activation tile goes straight from global memory
//    (L2) into an LDS stage with buffer loads to LDS (whole row segments;
//    all four column quarters read it), its 16-byte chunks XOR-swizzled by
//    row so an MFMA operand read is conflict-free; ST stages, so the copies
//    of step j + ST - 1 are issued while step j computes; each wavefront's
//    scales and zero-points go the same way into its own LDS blocks, several
//    steps per copy (every copy costs issue time in the memory pipeline,
//    whatever its size);
//  * the weight tiles (the HBM stream: one 16-byte load per lane per 1 KiB
//    tile) go straight into registers D = 3 steps ahead (a ring of four,
//    the step loop unrolled by four);
//  * a step's copies and weight loads go out one per 32-k block of its
//    contraction, not as one burst after the barrier;
//  * the number of copies and loads per step is fixed (tail steps re-read
//    the last tile), which keeps the one wait per step exact;
//  * one barrier per step; after the last step, the slices' partial sums
//    meet in LDS and wavefront (wc, ks) finishes row tiles ks, ks + 2 of its
//    column quarter in slice order (the RMSNorm row scale of rows staged by
//    stage.hip, the epilogue), through an LDS tile to 16-byte fp16 stores.
#include <type_traits>

#include "device.h"

namespace w4a16 {

namespace {

constexpr int kTileMT = 4;   // 16-row MFMA tiles per wavefront (64 rows per workgroup)
constexpr int kTileNWC = 4;  // column quarters per workgroup
constexpr int kTileNKS = 2;  // k slices per workgroup
constexpr int kTileNWave = kTileNWC * kTileNKS;
constexpr int kTileABytes = 64 * kTileK * 2;  // one slice's 64 x 128 activation tile
constexpr int kLdsMax = 160 * 1024;

// Scales and zero-points of one wavefront go into LDS in blocks of
// tile_mbs() steps (one copy per stream and kind for a whole block), in a
// ring of tile_nbuf() blocks.
constexpr int tile_step_scale_bytes(int ct, int group, int sb) { return ct * (kTileK / group) * 16 * sb; }
constexpr int tile_step_zp_bytes(int ct, int group) { return ct * (kTileK / group) * 8; }
// (a divisor of the main loop's unroll of 4, so a block opens at a fixed
// position of the unrolled body)
constexpr int tile_mbs(int ct, int group, int sb) {
  return 1024 / tile_step_scale_bytes(ct, group, sb) >= 4   ? 4
         : 1024 / tile_step_scale_bytes(ct, group, sb) >= 2 ? 2
                                                             : 1;
}
constexpr int tile_meta_block_bytes(int ct, int group, int sb, int nw) {
  return nw * (tile_mbs(ct, group, sb) * tile_step_scale_bytes(ct, group, sb) +
               (tile_mbs(ct, group, sb) * tile_step_zp_bytes(ct, group) + 15) / 16 * 16);
}
constexpr int tile_stage_bytes() { return kTileNKS * kTileABytes; }
constexpr int tile_nbuf(int st, int mbs) { return (st - 1 + mbs - 1) / mbs + 1; }
constexpr int tile_lds(int st, int ct, int group, int sb, int nw) {
  return st * tile_stage_bytes() +
         kTileNWave * tile_nbuf(st, tile_mbs(ct, group, sb)) * tile_meta_block_bytes(ct, group, sb, nw);
}
constexpr int tile_stages(int ct, int group, int sb, int nw) {
  return tile_lds(4, ct, group, sb, nw) <= kLdsMax ? 4 : tile_lds(3, ct, group, sb, nw) <= kLdsMax ? 3 : 2;
}

// (occupancy: one workgroup of kTileNWave wavefronts per compute unit, which
// its LDS stages allow anyway)
template <int CT, int G, bool SF32, bool GU>
__global__ void __launch_bounds__(64 * kTileNWave)
    __attribute__((amdgpu_waves_per_eu(kTileNWave / 4, kTileNWave / 4)))
tile_kernel(const GemmArgs p) {
  constexpr int MT = kTileMT;
  constexpr int NWC = kTileNWC;
  constexpr int NKS = kTileNKS;
  constexpr int NW = GU ? 2 : 1;
  constexpr int GPC = 128 / G;
  constexpr int SB = SF32 ? 4 : 2;
  constexpr int PSS = CT * GPC * 16 * SB;  // scale bytes of one step, one stream
  constexpr int PSZ = CT * GPC * 8;        // zero-point bytes of one step, one stream
  constexpr int ST = tile_stages(CT, G, SB, NW);
  constexpr int MBS = tile_mbs(CT, G, SB);  // steps per metadata block
  constexpr int NBUF = tile_nbuf(ST, MBS);  // metadata blocks in the ring
  constexpr int BS = MBS * PSS;                        // scale bytes of a block, one stream
  constexpr int BZ = (MBS * PSZ + 15) / 16 * 16;       // zero-point bytes of a block, one stream
  constexpr int MBLK = tile_meta_block_bytes(CT, G, SB, NW);
  constexpr int STAGE = tile_stage_bytes();
  constexpr int META_OFF = ST * STAGE;
  constexpr int D = 3;  // steps the weight tiles are loaded ahead (ring of D + 1)
  static_assert(kTileNWave * NW * MT * CT * 1024 <= ST * STAGE, "reduction scratch");
  static_assert(D >= ST - 1, "weights at least as far ahead as the copies");
  static_assert(BS <= 1024 && BZ <= 256 + 15, "one copy per block, stream and kind");
  static_assert(MBS >= ST - 1 || NBUF * MBS >= ST, "metadata ring");
  // per step and wavefront at least: activation copies CL, then weight-tile
  // loads WL.  At the top of step j, the loads issued after the copies of
  // step j are the WL weight loads of the step that issued them and the
  // copies and weight loads of the ST - 2 steps after it; metadata copies
  // (one block every MBS steps) and the first steps' extra loads only add to
  // that, which makes the wait stricter, never looser.
  constexpr int CL = kTileABytes / 1024 / NWC;
  constexpr int WL = NW * CT;
  constexpr int AFTER = WL + (ST - 2) * (CL + WL);
  static_assert(AFTER < 64, "vmcnt range");

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
  const bool has_zp = p.has_zp != 0;

  auto ktile = [&](int j) __attribute__((always_inline)) { return j * NKS + ks; };
  auto abuf_of = [&](int st) __attribute__((always_inline)) {
    return smem + st * STAGE + ks * kTileABytes;
  };
  // metadata block b of this wavefront: scales [NW][MBS][CT][GPC][16],
  // then zero-points [NW][MBS][CT][GPC][8 bytes]
  auto mblk_of = [&](int b) __attribute__((always_inline)) {
    return smem + META_OFF + (wave * NBUF + b % NBUF) * MBLK;
  };

  // per-lane source offsets of the copies, fixed for the whole kernel (the
  // per-step part of each address is wavefront-uniform)
  constexpr int AQ = kTileABytes / 1024 / NWC;  // activation copies per wavefront
  uint32_t aoff[AQ];
#pragma unroll
  for (int qi = 0; qi < AQ; ++qi) {
    // slot r * 16 + pos holds 16-byte chunk pos ^ (r % 16) of row r: one
    // copy reads four whole 256-byte row segments
    const int sl = (wc + NWC * qi) * 64 + lane;
    const int row = sl >> 4, chunk = (sl & 15) ^ (row & 15);
    aoff[qi] = (uint32_t)(min(row, mrows - 1) * p.K + 8 * chunk) * 2u;
  }
  // metadata: lane u of the scale copy takes 16-byte unit u of the block,
  // (step i, column tile ct, unit o); the zero-point copy 4-byte units
  constexpr int SUS = PSS / 16;  // 16-byte scale units per step
  constexpr int ZUS = PSZ / 4;   // 4-byte zero-point units per step
  const bool s_on = lane < MBS * SUS, z_on = lane < MBS * ZUS;
  uint32_t s_lane, z_lane;  // from this wavefront's first column tile (clamped to the last)
  int s_step, z_step;
  const int ct_base = min(ctw, NTL - 1);
  {
    const int u = min(lane, MBS * SUS - 1);
    s_step = u / SUS;
    const int r = u - s_step * SUS, w = r / (GPC * SB), o = r - w * (GPC * SB);
    s_lane = (uint32_t)(min(ctw + w, NTL - 1) - ct_base) * (uint32_t)(Gall * 16 * SB) + (uint32_t)o * 16u;
    const int uz = min(lane, MBS * ZUS - 1);
    z_step = uz / ZUS;
    const int rz = uz - z_step * ZUS, wz = rz / (GPC * 2), oz = rz - wz * (GPC * 2);
    z_lane = (uint32_t)(min(ctw + wz, NTL - 1) - ct_base) * (uint32_t)(Gall * 8) + (uint32_t)oz * 4u;
  }
  // sources of the copies as buffer ranges (the workgroup's 64 rows; this
  // wavefront's column tiles of each metadata stream), so that the compiler
  // keeps exact waits for the weight tiles in registers while copies are in
  // flight; every offset stays below 2^31 (K <= 2^24, CT <= 2 column tiles)
  const __amdgpu_buffer_rsrc_t a_src =
      raw_rsrc(p.A + (size_t)m0 * p.K, (uint32_t)mrows * (uint32_t)p.K * 2u);
  __amdgpu_buffer_rsrc_t s_src[NW], z_src[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const size_t run = (size_t)(NTL - ct_base) * Gall;  // groups from the first column tile on
    s_src[i] = raw_rsrc(reinterpret_cast<const uint8_t *>(p.scales[i]) + (size_t)ct_base * Gall * 16 * SB,
                        (uint32_t)min(run * 16 * SB, (size_t)0xFFFFFFFFu));
    z_src[i] = has_zp ? raw_rsrc(p.zeros[i] + (size_t)ct_base * Gall * 8,
                                 (uint32_t)min(run * 8, (size_t)0xFFFFFFFFu))
                      : s_src[i];
  }

  // copies of step j: when step j opens a metadata block, that block's
  // scales and zero-points (issue_meta), then the slice's activation tile
  // into stage st, a quarter of it per column quarter, one 1 KiB copy qi at a
  // time (issue_a).  Steps past K re-read the last k tile; symmetric weights
  // copy scale bytes into the (unread) zero-point area.
  auto issue_meta = [&](int j, bool opens_block) __attribute__((always_inline)) {
    if (opens_block) {
      uint8_t *blk = mblk_of(j / MBS);
      // k tile of step j + s_step (the lane's own step in the block)
      const int kts = min(ktile(j + s_step), KC - 1), ktz = min(ktile(j + z_step), KC - 1);
      const uint32_t s_off = s_lane + (uint32_t)kts * (GPC * 16 * SB);
      const uint32_t z_off = has_zp ? z_lane + (uint32_t)ktz * (GPC * 8) : s_off;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        if (s_on) copy16_to_lds(s_src[i], s_off, 0, blk + i * BS);
        if (z_on) copy4_to_lds(z_src[i], z_off, 0, blk + NW * BS + i * BZ);
      }
    }
  };
  auto issue_a = [&](int j, int st, int qi) __attribute__((always_inline)) {
    const int kt = min(ktile(j), KC - 1);
    copy16_to_lds(a_src, aoff[qi], (uint32_t)kt * kTileK * 2, abuf_of(st) + (wc + NWC * qi) * 1024);
  };

  // weight tile (i, ct) of step j, straight into registers
  auto load_w1 = [&](int j, int i, int ct, u32x4 (&wv)[NW][CT]) __attribute__((always_inline)) {
    const int kt = min(ktile(j), KC - 1);
    const size_t tile = (size_t)min(ctw + ct, NTL - 1) * KC + kt;
    wv[i][ct] = load_weights<CT == 1>(p.w[i] + tile * kTileBytes, lane);  // CT > 1: several row blocks
  };

  f32x4 acc[NW][MT][CT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[i][mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int zshift = 4 * (c & 1);
  // (hook(b) runs before block b of 32 k, b = (i * CT + ct) * 4 + d)
  auto compute = [&](int j, int st, const u32x4 (&wreg)[NW][CT], auto &&hook) __attribute__((always_inline)) {
    // row 16mt + c, chunk 4d + kq sits at slot row * 16 + ((4d + kq) ^ c): the
    // 16 rows of one operand read land in 16 different chunk positions
    const uint8_t *abuf = abuf_of(st) + c * 256;
    const uint8_t *blk = mblk_of(j / MBS);
    const int jb = j % MBS;  // step within the metadata block
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // a step past K (its copies and loads re-read the last k tile) runs the
    // same instructions with every scale zero, so it adds exactly nothing
    const float on = ktile(j) < KC ? 1.0f : 0.0f;
    f16x8 a[4][MT];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[d][mt] = *reinterpret_cast<const f16x8 *>(abuf + mt * 4096 + ((4 * d + kq) ^ c) * 16);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const u32x4 wv = wreg[i][ct];
        const uint8_t *sp = blk + i * BS + jb * PSS + ((ct * GPC) * 16 + c) * SB;  // group 0
        const uint8_t *zp = blk + NW * BS + i * BZ + jb * PSZ + (ct * GPC) * 8 + (c >> 1);
        auto scale = [&](int g2) __attribute__((always_inline)) {
          if constexpr (SF32)
            return on * *reinterpret_cast<const float *>(sp + g2 * 16 * SB);
          else
            return on * (float)*reinterpret_cast<const f16 *>(sp + g2 * 16 * SB);
        };
        auto zconst = [&](int g2, f16x2 &zlo, f16x2 &zhi) __attribute__((always_inline)) {
          const uint32_t z = has_zp ? (uint32_t)((zp[g2 * 8] >> zshift) & 15) : 8u;
          zero_consts(z, zlo, zhi);
        };
        if constexpr (G >= 32) {
          constexpr int SPG = G / 32;  // 32-k steps per group
          f32x4 accg[MT];
          f16x2 zlo, zhi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            hook((i * CT + ct) * 4 + d);
            if (d % SPG == 0) zconst(d / SPG, zlo, zhi);
            const f16x8 b = unpack8(wv[d], zlo, zhi);
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
              if constexpr (G < 64) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) pin_acc(acc[i][mt][ct]);
              }
            }
          }
        } else {
          // group 16: k slots of lanes kq < 2 are group 2d, the others 2d + 1
          const f16x8 zero8 = {};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            hook((i * CT + ct) * 4 + d);
            f16x2 zlo, zhi;
            zconst(2 * d + (kq >> 1), zlo, zhi);
            const f16x8 b = unpack8(wv[d], zlo, zhi);
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
              pin_acc(acc[i][mt][ct]);
            }
          }
        }
      }
    }
  };

  // Pipeline: the copies of steps 0 .. ST-2 and the weights of steps
  // 0 .. D-1 are issued up front; step j waits for its copies, meets the
  // other wavefronts (which frees the stage read in step j - 1), issues the
  // copies of step j + ST - 1 into that stage and the weights of step j + D,
  // and computes.
  u32x4 wring[D + 1][NW][CT];
#pragma unroll
  for (int u = 0; u < ST - 1; ++u) {
    issue_meta(u, u % MBS == 0);
#pragma unroll
    for (int qi = 0; qi < AQ; ++qi) issue_a(u, u, qi);
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) load_w1(u, i, ct, wring[u]);
  int st = 0;
  // Step j = j0 + u (j0 a multiple of D + 1 = 4, so u, the ring slot and
  // whether a metadata block opens are known at compile time).  A step's
  // activation copies and weight loads (in that order, AQ + NW * CT of them)
  // are spread over its contraction's NW * CT * 4 blocks of 32 k instead of
  // being issued together after the barrier: the eight wavefronts' loads
  // then reach the compute unit's load path one at a time while it also
  // serves the matrix cores' operands, rather than as one burst that stalls
  // every wavefront's issue at once (measured: K=5120 N=13824 M=128 29.2 ->
  // 26.6 us).  Every step issues the same copies and loads, and every step
  // that runs its contraction runs the same one (a step past K with zero
  // scales).  Where the register file allows it (one column tile per
  // wavefront, one weight stream, groups of 64 or 128) the trip count is
  // padded to a multiple of 4 and the body has no branch at all; elsewhere
  // the contractions of the steps past the last group of 4 are skipped (the
  // compiler would otherwise interleave four contractions past what the
  // register file holds), but not their copies and loads, so that every path
  // through the loop issues the same loads in the same order and the
  // compiler's waits for the weight registers stay close to exact.
  auto step = [&](int j, auto uc, bool live) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    wait_vmcnt<AFTER>();  // this wavefront's copies of step j have landed
    lds_only_barrier();   // everyone's have, and step j - 1's reads are done
    const int jn = j + ST - 1, stn = st == 0 ? ST - 1 : st - 1;  // stage read in step j - 1
    issue_meta(jn, (u + ST - 1) % MBS == 0);
    constexpr int NB = NW * CT * 4, NL = AQ + NW * CT;
    auto hook = [&](int b) __attribute__((always_inline)) {
#pragma unroll
      for (int l = 0; l < NL; ++l)
        if (l * NB / NL == b) {
          if (l < AQ)
            issue_a(jn, stn, l);
          else
            load_w1(j + D, (l - AQ) / CT, (l - AQ) % CT, wring[(u + D) % (D + 1)]);
        }
    };
    if (live) {
      compute(j, st, wring[u], hook);
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) hook(b);
    }
    st = st == ST - 1 ? 0 : st + 1;
  };
  static_assert(D + 1 == 4 && 4 % MBS == 0, "unroll and metadata blocks");
  constexpr bool FLAT = CT == 1 && !GU && (G == 128 || (G == 64 && !SF32));
  for (int j0 = 0; j0 < nsteps; j0 += D + 1) {
    step(j0, std::integral_constant<int, 0>{}, true);
    step(j0 + 1, std::integral_constant<int, 1>{}, FLAT || j0 + 1 < nsteps);
    step(j0 + 2, std::integral_constant<int, 2>{}, FLAT || j0 + 2 < nsteps);
    step(j0 + 3, std::integral_constant<int, 3>{}, FLAT || j0 + 3 < nsteps);
  }
  // The epilogue's own inputs, loaded before the barrier so that their
  // latency overlaps it: the bias of this lane's columns and the row scales
  // (staged RMSNorm) of the rows this wavefront finishes, row tiles ks,
  // ks + NKS, ... of column quarter wc.
  static_assert(MT % NKS == 0, "row tiles per finishing wavefront");
  constexpr int MTO = MT / NKS;
  float bias_v[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    bias_v[ct] = (!GU && p.epilogue != 0 && ctw + ct < NTL) ? (float)p.bias[(ctw + ct) * kTileN + c] : 0.f;
  float rsc[MTO][4];
#pragma unroll
  for (int o = 0; o < MTO; ++o)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * (ks + NKS * o) + 4 * kq + e;
      rsc[o][e] = (p.row_ss != nullptr && row < mrows)
                      ? 1.0f / sqrtf(p.row_ss[m0 + row] / (float)p.K + p.eps)
                      : 1.0f;
    }
  __syncthreads();  // every step and every copy done: the stages become reduction scratch

  // slice partial sums -> LDS ([wave][i][mt][ct][lane], 16 bytes per lane)
  f32x4 *red = reinterpret_cast<f32x4 *>(smem);
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        red[((wave * NW + i) * MT + mt) * CT * 64 + ct * 64 + lane] = acc[i][mt][ct];
  __syncthreads();

  // Each finishing wavefront sums its tiles over the k slices in slice order
  // and applies the epilogue; the fp16 results go into a row-major tile of
  // the workgroup's 64 x WC outputs in LDS (rows padded by 16 bytes against
  // bank conflicts), after the reduction area where it fits, else over it
  // once every wavefront has read its partial sums; then each thread stores
  // whole 16-byte runs of a row (two scattered 2-byte stores per output
  // element otherwise).
  constexpr int WC = NWC * CT * kTileN;  // the workgroup's columns
  constexpr int OSTR = WC + 8;           // tile row stride, halves
  constexpr int RED_BYTES = kTileNWave * NW * MT * CT * 1024;
  constexpr bool OSEP = RED_BYTES + 64 * OSTR * 2 <= ST * STAGE;
  static_assert(64 * OSTR * 2 <= ST * STAGE, "output tile");
  f16 yv[MTO][CT][4];
#pragma unroll
  for (int o = 0; o < MTO; ++o) {
    const int mt = ks + NKS * o;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 fin[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int s2 = 0; s2 < NKS; ++s2)
          v += red[(((s2 * NWC + wc) * NW + i) * MT + mt) * CT * 64 + ct * 64 + lane];
        fin[i] = v;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y;
        if constexpr (GU) {
          y = silu(fin[0][e] * rsc[o][e]) * (fin[1][e] * rsc[o][e]);
        } else {
          y = fin[0][e] * rsc[o][e];
          if (p.epilogue != 0) y += bias_v[ct];
          if (p.epilogue == 2) y = y > 0.f ? y : 0.f;
        }
        yv[o][ct][e] = (f16)y;
      }
    }
  }
  if constexpr (!OSEP) __syncthreads();  // the partial sums are read before the tile overwrites them
  f16 *otile = reinterpret_cast<f16 *>(smem + (OSEP ? RED_BYTES : 0));
#pragma unroll
  for (int o = 0; o < MTO; ++o)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        otile[(16 * (ks + NKS * o) + 4 * kq + e) * OSTR + (wc * CT + ct) * kTileN + c] = yv[o][ct][e];
  __syncthreads();
  const int col0 = blockIdx.x * WC;
  constexpr int RUNS = WC / 8;  // 16-byte runs per row
  static_assert(64 * RUNS % (64 * kTileNWave) == 0, "whole store rounds");
#pragma unroll
  for (int q = 0; q < 64 * RUNS / (64 * kTileNWave); ++q) {
    const int idx = q * 64 * kTileNWave + tid;
    const int row = idx / RUNS, run = idx % RUNS;
    if (row < mrows && col0 + run * 8 < p.N)
      *reinterpret_cast<u32x4 *>(p.out + (size_t)(m0 + row) * p.N + col0 + run * 8) =
          *reinterpret_cast<const u32x4 *>(otile + row * OSTR + run * 8);
  }
}

template <int CT, int G, bool SF32, bool GU>
hipError_t launch_t(const GemmArgs &a, const Plan &pl, hipStream_t stream) {
  auto kern = tile_kernel<CT, G, SF32, GU>;
  static std::atomic<size_t> lds_limit[kMaxDevices];
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(kern), pl.lds_bytes, lds_limit);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.gx, pl.gy, pl.gz), dim3(64 * kTileNWave), pl.lds_bytes,
                     stream, a);
  return hipGetLastError();
}

// column tiles per wavefront: 2 when there are several 64-row blocks
// (Plan::cfg == 1), else 1, so that the grid keeps its workgroup count;
// gate_up (two weight streams) always 1
template <int G>
hipError_t launch_g(const GemmArgs &a, const Plan &pl, bool sf32, bool gu, hipStream_t st) {
  const bool wide = pl.cfg == 1;
  if (gu) return sf32 ? launch_t<1, G, true, true>(a, pl, st) : launch_t<1, G, false, true>(a, pl, st);
  if (sf32) return wide ? launch_t<2, G, true, false>(a, pl, st) : launch_t<1, G, true, false>(a, pl, st);
  return wide ? launch_t<2, G, false, false>(a, pl, st) : launch_t<1, G, false, false>(a, pl, st);
}

}  // namespace

int tile_ct(bool wide, bool gate_up) { return (wide && !gate_up) ? 2 : 1; }

size_t tile_lds_bytes(int ct, int group, int scale_bytes, bool gate_up) {
  const int nw = gate_up ? 2 : 1;
  return (size_t)tile_lds(tile_stages(ct, group, scale_bytes, nw), ct, group, scale_bytes, nw);
}

int tile_columns(int ct) { return kTileNWC * ct * kTileN; }

int tile_threads() { return 64 * kTileNWave; }

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
