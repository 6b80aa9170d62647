// Launch planning for the fused W4A16 GEMM (kernels in stream.hip for
// M <= 16, tile.hip above; oneshot.hip and ring.hip on request).
//
// The plan is a pure function of the shape: it picks the tile configuration,
// the grid and, only for grids too small to fill the chip, a k split across
// workgroups (the onnx-genai pull request "Marlin-style fused fp16xint4
// tensor-core GEMM", "P2 - widen the win: split-K": split only when the grid
// is short of waves).
#include "common.h"

namespace w4a16 {

namespace {

// Workspace layout: arrival counters first, at a fixed place and count
// (split-K only runs below kMaxSplitBlocks workgroups), so calls of any shape
// sharing one workspace never overwrite another shape's counters; then the
// partial sums of squares and the partial sums.
void plan_workspace(Plan &p, int M, int N, int base, int NW) {
  size_t off = 0;
  if (p.split > 1) {
    p.ws_cnt_off = 0;
    off = align256((size_t)kMaxSplitBlocks * 4);
    p.ws_rms_off = off;
    off = align256(off + (size_t)base * p.split * 64 * 4);
    p.ws_part_off = off;
    off = align256(off + (size_t)p.split * NW * M * N * 4);
  }
  p.ws_total = off;
}

int pow2_at_least(int v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

}  // namespace

namespace {

size_t align16(size_t v) { return (v + 15) / 16 * 16; }

// k splits across workgroups only when the grid has fewer than 512
// wavefronts; each split keeps at least `min_tiles` k tiles per slice.
int choose_split(int base, int nwave, int KC, int min_tiles, int force_split) {
  int S = 1;
  if (force_split > 0) {
    S = force_split;
  } else {
    while (base * S * nwave < 512 && KC / (S + 1) >= min_tiles) ++S;
  }
  if (S > KC) S = KC;
  if (base >= kMaxSplitBlocks) S = 1;
  return S;
}

// LDS for the staged scales ([group][16 columns]) and zero-points
// ([group][8 bytes]) of NWC column tiles per weight stream, each run rounded
// up to whole copies (1 KiB / 256 B).  Returns the next free offset.
size_t plan_meta_lds(Plan &p, size_t off, int group, int scale_bytes, int nwc, int NW) {
  p.gr = p.cps * (kTileK / group);
  const size_t scopy = ((size_t)p.gr * 16 * scale_bytes + 1023) / 1024 * 1024;
  const size_t zcopy = ((size_t)p.gr * 8 + 255) / 256 * 256;
  p.lds_s = (int)off;
  off = align16(off + (size_t)NW * nwc * scopy);
  p.lds_z = (int)off;
  off = align16(off + (size_t)NW * nwc * zcopy);
  return off;
}

// One-shot kernel plan, or false when its activation tile does not fit.
bool plan_oneshot(Plan &p, int M, int K, int N, int group, int scale_bytes, bool gate_up,
                  int force_cfg, int force_split) {
  const int NTL = N / kTileN;
  const int KC = K / kTileK;
  const int NW = gate_up ? 2 : 1;
  if (M > 16) return false;
  p.kind = kKindOneshot;
  p.cfg = (force_cfg >= 0 && force_cfg < kNumOneshotCfgs) ? force_cfg : (NTL >= 512 ? 0 : 1);
  const OneshotCfg c = kOneshotCfgs[p.cfg];
  const int nwave = c.nwc * c.nwk;
  p.gx = (NTL + c.nwc - 1) / c.nwc;
  p.gz = (M + 15) / 16;
  const int base = p.gx * p.gz;
  int S = choose_split(base, nwave, KC, c.nwk, force_split);
  // every slice must fit the wavefront's CW register tiles
  const int s_min = (KC + c.nwk * c.cw - 1) / (c.nwk * c.cw);
  if (S < s_min) S = s_min;
  if (S > KC) S = KC;
  p.cps = (KC + S - 1) / S;
  p.split = (KC + p.cps - 1) / p.cps;
  p.gy = p.split;
  p.rows_pow2 = pow2_at_least(M < 16 ? M : 16);
  const int cpw = (p.cps + c.nwk - 1) / c.nwk;
  const size_t slots = (size_t)c.nwk * cpw * 16 * p.rows_pow2;
  const size_t a_bytes = (slots + 63) / 64 * 1024;
  const size_t red = (size_t)(c.nwk - 1) * c.nwc * NW * c.mt * 4 * 64 * 4;
  size_t off = align16(a_bytes > red ? a_bytes : red);
  p.lds_g = (int)off;
  off = align16(off + ((size_t)p.cps * kTileK * 2 + 1023) / 1024 * 1024);
  off = plan_meta_lds(p, off, group, scale_bytes, c.nwc, NW);
  p.lds_r = (int)off;
  p.lds_bytes = off + (size_t)(64 * nwave + 64) * 4;
  if (p.lds_bytes > 96 * 1024 && force_cfg < 0) return false;
  plan_workspace(p, M, N, base, NW);
  return true;
}

// Stream kernel plan (M <= 16): as many column tiles per wavefront as keep
// the grid at >= 200 workgroups; k split across workgroups only when the
// k range exceeds the workgroup's NWK x KPW tiles or the grid is short of
// wavefronts.  Each wavefront has a private LDS region: its slice's scales
// and zero-points, for M <= 8 its activation rows, and at the end its
// partial sums.
bool plan_stream(Plan &p, int M, int K, int N, int group, int scale_bytes, bool gate_up,
                 int force_cfg, int force_split) {
  const int NTL = N / kTileN;
  const int KC = K / kTileK;
  const int NW = gate_up ? 2 : 1;
  if (M > 16) return false;
  p.kind = kKindStream;
  if (force_cfg >= 0 && force_cfg < kNumStreamCfgs) {
    p.cfg = force_cfg;
  } else {
    p.cfg = kNumStreamCfgs - 1;
    for (int i = 0; i < kNumStreamCfgs; ++i)
      if ((NTL + kStreamCfgs[i].cpw - 1) / kStreamCfgs[i].cpw >= 200) { p.cfg = i; break; }
  }
  const StreamCfg c = kStreamCfgs[p.cfg];
  const int per_wg = c.nwk * c.kpw;  // k tiles one workgroup covers
  p.gx = (NTL + c.cpw - 1) / c.cpw;
  p.gz = 1;
  const int base = p.gx * p.gz;
  int S = choose_split(base, c.nwk, KC, 1, force_split);
  const int s_min = (KC + per_wg - 1) / per_wg;
  if (S < s_min) S = s_min;
  if (S > KC) S = KC;
  if (S > 1 && NTL * p.gz > kMaxSplitBlocks) return false;  // one arrival counter per column tile
  p.cps = (KC + S - 1) / S;
  p.split = (KC + p.cps - 1) / p.cps;
  p.gy = p.split;
  // private region of one wavefront
  const int gpw = c.kpw * (kTileK / group);
  const size_t ms = (size_t)c.cpw * gpw * 16 * scale_bytes;
  const size_t mz = align16((size_t)c.cpw * gpw * 8);
  const size_t meta = NW * (ms + mz);
  const size_t red = (size_t)NW * c.cpw * 1024;
  p.rows_pow2 = pow2_at_least(M);
  const size_t a_lds = (size_t)c.kpw * 256 * p.rows_pow2;
  const size_t limit = 160 * 1024;
  p.alds = 0;
  size_t region = align16(meta > red ? meta : red);
  if (M <= 8) {
    const size_t with_a = align16(meta + a_lds > red ? meta + a_lds : red);
    if ((size_t)c.nwk * with_a + (size_t)c.nwk * 64 <= limit) {
      p.alds = 1;
      region = with_a;
    }
  }
  if ((size_t)c.nwk * region + (size_t)c.nwk * 64 > limit) return false;
  p.lds_s = (int)region;
  p.lds_r = (int)(c.nwk * region);
  p.lds_bytes = (size_t)p.lds_r + (size_t)c.nwk * 16 * 4;
  p.lds_g = p.lds_z = p.gr = 0;
  // workspace: arrival counters (one per column tile), row sums of squares
  // [column tile][S][16], partial sums [S][NW][M][N]
  size_t off = 0;
  if (p.split > 1) {
    p.ws_cnt_off = 0;
    off = align256((size_t)kMaxSplitBlocks * 4);
    p.ws_rms_off = off;
    off = align256(off + (size_t)NTL * p.gz * p.split * 16 * 4);
    p.ws_part_off = off;
    off = align256(off + (size_t)p.split * NW * M * N * 4);
  }
  p.ws_total = off;
  return true;
}

}  // namespace

Plan make_plan(int M, int K, int N, int group, int scale_bytes, bool gate_up, int force_kind,
               int force_cfg, int force_split) {
  Plan p{};
  if (force_kind < 0 ? M > 16 : force_kind == kKindTile) {
    // 64-row blocks x tile_columns() per workgroup over the whole K; wide
    // column blocks only when several row blocks keep the grid full
    p.kind = kKindTile;
    p.gz = (M + 63) / 64;
    p.cfg = p.gz > 1 ? 1 : 0;
    const int ct = tile_ct(p.cfg == 1, gate_up);
    p.gx = (N + tile_columns(ct) - 1) / tile_columns(ct);
    p.gy = 1;
    p.split = 1;
    p.cps = K / kTileK;
    p.lds_bytes = tile_lds_bytes(ct, group, scale_bytes, gate_up);
    p.ws_total = 0;
    return p;
  }
  if (force_kind == kKindOneshot) {
    Plan q{};
    if (plan_oneshot(q, M, K, N, group, scale_bytes, gate_up, force_cfg, force_split)) return q;
  } else if (force_kind == kKindStream || force_kind < 0) {
    Plan q{};
    if (plan_stream(q, M, K, N, group, scale_bytes, gate_up,
                    force_kind == kKindStream ? force_cfg : -1,
                    force_kind == kKindStream ? force_split : 0))
      return q;
  }
  const int NTL = N / kTileN;
  const int KC = K / kTileK;
  const int NW = gate_up ? 2 : 1;
  p.kind = kKindRing;
  if (force_kind == kKindRing && force_cfg >= 0 && force_cfg < kNumRingCfgs) {
    p.cfg = force_cfg;
  } else if (M <= 16) {
    p.cfg = NTL >= 512 ? 0 : 2;
  } else if (M <= 32) {
    p.cfg = 3;
  } else {
    p.cfg = 4;
  }
  const RingCfg c = kRingCfgs[p.cfg];
  const int MR = 16 * c.mt;
  const int nwave = c.nwc * c.nwk;
  p.gx = (NTL + c.nwc - 1) / c.nwc;
  p.gz = (M + MR - 1) / MR;
  const int base = p.gx * p.gz;
  const int S = choose_split(base, nwave, KC, c.nwk * c.da, force_split);
  p.cps = (KC + S - 1) / S;
  p.split = (KC + p.cps - 1) / p.cps;
  p.gy = p.split;
  p.rows_pow2 = pow2_at_least(M < MR ? M : MR);
  const size_t abuf = (size_t)c.nwk * c.da * 256 * p.rows_pow2;
  const size_t red = (size_t)(c.nwk - 1) * c.nwc * NW * c.mt * 4 * 64 * 4;
  const size_t region = 2 * abuf > red ? 2 * abuf : red;
  p.lds_g = 0;
  size_t off = plan_meta_lds(p, align16(region), group, scale_bytes, c.nwc, NW);
  p.lds_r = (int)off;
  p.lds_bytes = (size_t)p.lds_r + (size_t)(64 * nwave + MR) * 4;
  plan_workspace(p, M, N, base, NW);
  return p;
}

hipError_t launch_gemm(const GemmArgs &a, const Plan &pl, int group,
                       bool scale_f32, bool gate_up, hipStream_t stream) {
  switch (pl.kind) {
    case kKindStream: return launch_stream(a, pl, group, scale_f32, gate_up, stream);
    case kKindOneshot: return launch_oneshot(a, pl, group, scale_f32, gate_up, stream);
    case kKindTile: return launch_tile(a, pl, group, scale_f32, gate_up, stream);
    default: return launch_ring(a, pl, group, scale_f32, gate_up, stream);
  }
}

}  // namespace w4a16
