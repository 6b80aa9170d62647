// Launch planning for the fused W4A16 GEMM: stream.hip for M <= 16 (the
// HBM-bound decode regime), panel.hip above (tile.hip for what neither
// takes).
//
// The plan is a pure function of the shape: it picks the kernel
// configuration, the grid and, only where a workgroup's k range cannot hold
// the whole K or the grid is short of one workgroup per compute unit, a k
// split across workgroups (the onnx-genai pull request "Marlin-style fused
// fp16xint4 tensor-core GEMM", "P2 - widen the win: split-K": split only
// when the grid is short of waves).
#include "common.h"

namespace w4a16 {

namespace {

int pow2_at_least(int v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

size_t align16(size_t v) { return (v + 15) / 16 * 16; }

// Workgroups of the stream kernel resident at once: one per compute unit
// (its register use leaves room for one 8-wavefront workgroup per CU).
constexpr int kStreamSlots = 256;

// Automatic split: as many k splits as keep every workgroup of the grid
// resident at once, since a second round of workgroups costs a whole
// workgroup lifetime; a forced split is taken as given.
int choose_split(int base, int KC, int force_split) {
  int S = force_split > 0 ? force_split : kStreamSlots / base;
  if (S < 1) S = 1;
  return S > KC ? KC : S;
}

// Stream kernel plan (M <= 16): as many column tiles per wavefront as keep
// the grid at >= 200 workgroups; k split across workgroups only when the k
// range exceeds the workgroup's NWK x KPW tiles or the grid is short of
// wavefronts.  Each wavefront has a private LDS region: its slice's scales
// and zero-points, for M <= 4 its activation rows, and at the end its
// partial sums.
// One wavefront's private LDS region of the streaming kernel without staged
// activation rows: its slice's scales and zero-points per weight stream and
// its RMSNorm gamma, or (at the end) one stream's partial sums.
size_t stream_region_bytes(const StreamCfg &c, int group, int scale_bytes, int NW) {
  const int gpw = c.kpw * (kTileK / group);
  const size_t meta = NW * ((size_t)c.cpw * gpw * 16 * scale_bytes + align16((size_t)c.cpw * gpw * 8)) +
                      (size_t)c.kpw * kTileK * 2;
  const size_t red = (size_t)NW * c.cpw * 1024;
  return align16(meta > red ? meta : red);
}

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
    // the widest column block whose grid, times the k splits the shape
    // needs (deep K, or a forced split), reaches 200 workgroups and still
    // fits in one round of resident workgroups; failing that the fullest
    // single round; failing that the fewest workgroups.  A forced split
    // considers only the configurations that can run it.
    int best = -1;
    long best_total = 0;
    for (int i = 0; i < kNumStreamCfgs; ++i) {
      const StreamCfg c = kStreamCfgs[i];
      // (a configuration whose private regions exceed the LDS, e.g. group 16
      // with fp32 scales and two weight streams on 4 column tiles, is skipped
      // in favour of a narrower one)
      if (stream_region_bytes(c, group, scale_bytes, NW) * c.nwk + (size_t)c.nwk * 64 > 160 * 1024)
        continue;
      // deep slices with one column tile read the whole activation slice in
      // every workgroup: worth it against a k split only up to 8 rows
      // (K=13696 N=4096: M=8 13.7 -> 13.0 us, M=16 15.0 -> 17.3 us)
      if (c.kpw > 5 && M > 8) continue;
      const long per = (long)c.nwk * c.kpw;
      const long smin = (KC + per - 1) / per;
      if (force_split > 0 && force_split < smin) continue;
      const long total = (long)((NTL + c.cpw - 1) / c.cpw) * (force_split > 0 ? force_split : smin);
      if (total >= 200 && total <= kStreamSlots) { best = i; break; }
      const bool fits = total <= kStreamSlots;
      const bool best_fits = best >= 0 && best_total <= kStreamSlots;
      if (best < 0 || (fits && (!best_fits || total > best_total)) ||
          (!fits && !best_fits && total < best_total)) {
        best = i;
        best_total = total;
      }
    }
    if (best < 0) return false;
    p.cfg = best;
  }
  const StreamCfg c = kStreamCfgs[p.cfg];
  const int per_wg = c.nwk * c.kpw;  // k tiles one workgroup covers
  p.gx = (NTL + c.cpw - 1) / c.cpw;
  p.gz = 1;
  p.block = 64 * c.nwk;
  const int base = p.gx * p.gz;
  const int s_min = (KC + per_wg - 1) / per_wg;
  // a forced split must leave every workgroup at most its NWK x KPW tiles
  if (force_split > 0 && (force_split < s_min || force_split > KC)) return false;
  // a k range deeper than one workgroup covers takes the fewest splits that
  // cover it as long as they keep half a round of workgroups busy (every
  // extra split costs an exchange through memory: down_proj K=13696 N=4096
  // M=8 takes 13.8 us at 3 splits, 15.2 us at 4); otherwise split until
  // the grid fills one round
  int S = (force_split <= 0 && s_min > 1 && (long)base * s_min >= kStreamSlots / 2)
              ? s_min
              : choose_split(base, KC, force_split);
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
  // scales and zero-points per weight stream, then the slice's RMSNorm gamma
  // (reserved whether or not a call has one: the plan depends on the shape)
  const size_t meta = NW * (ms + mz) + (size_t)c.kpw * kTileK * 2;
  const size_t red = (size_t)NW * c.cpw * 1024;
  p.rows_pow2 = pow2_at_least(M);
  const size_t a_lds = (size_t)c.kpw * 256 * p.rows_pow2;
  const size_t limit = 160 * 1024;
  p.alds = 0;
  size_t region = align16(meta > red ? meta : red);
  // activation rows through LDS (unique rows, read back as fragments) up to 4
  // rows; above that each k tile's fragments are loaded straight into
  // registers just before its first weight tile, which measured faster
  // (M=8: 10.6 -> 9.9 us; M=3: 9.1 against 9.5 us the other way)
  if (M <= 4 && c.kpw <= 5) {
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
  // workspace: arrival counters (one per column tile), row sums of squares
  // [column tile][S][16], partial sums [S][NW][M][N]
  size_t off = 0;
  if (p.split > 1) {
    p.ws_cnt_off = 0;
    off = align256(kCounterBytes);
    p.ws_rms_off = off;
    off = align256(off + (size_t)NTL * p.gz * p.split * 16 * 4);
    p.ws_part_off = off;
    off = align256(off + (size_t)p.split * NW * M * N * 4);
  }
  p.ws_total = off;
  return true;
}

// Panel kernel plan (16 < M <= 32): one 32-row block, 4 column tiles per
// workgroup; k split across workgroups as for the stream kernel (deep K, or
// a grid short of one workgroup per compute unit).  Above 32 rows the
// activation fragments each wavefront loads from L2 grow with M while the
// weight stream does not, and the tile kernel (activations shared through
// LDS) is faster (K=5120 N=13824: M=64 28.3 vs 23.9 us).  Each
// wavefront's private LDS region holds its slice's scales and zero-points
// and, at the end, one weight stream's partial sums.
bool plan_panel(Plan &p, int M, int K, int N, int group, int scale_bytes, bool gate_up,
                int force_split) {
  const int NTL = N / kTileN;
  const int KC = K / kTileK;
  const int NW = gate_up ? 2 : 1;
  if (M <= 16 || M > 32) return false;
  const int mt = 2;
  p.kind = kKindPanel;
  p.gz = (M + 16 * mt - 1) / (16 * mt);
  p.cfg = -1;
  for (int i = 0; i < kNumPanelCfgs; ++i)
    if (kPanelCfgs[i].mt == mt) p.cfg = i;
  if (p.cfg < 0) return false;
  const PanelCfg c = kPanelCfgs[p.cfg];
  const int per_wg = c.nwk * c.kpw;  // k tiles one workgroup covers
  p.gx = (NTL + c.cpw - 1) / c.cpw;
  p.block = 64 * c.nwk;
  const int base = p.gx * p.gz;
  const int s_min = (KC + per_wg - 1) / per_wg;
  if (force_split > 0 && (force_split < s_min || force_split > KC)) return false;
  int S = choose_split(base, KC, force_split);
  if (S < s_min) S = s_min;
  if (S > KC) S = KC;
  p.cps = (KC + S - 1) / S;
  p.split = (KC + p.cps - 1) / p.cps;
  p.gy = p.split;
  const int gpw = c.kpw * (kTileK / group);
  // per wavefront: its slice's scales and zero-points per weight stream
  // then the slice's RMSNorm gamma (reserved whether or not a call has one)
  const size_t meta = NW * ((size_t)c.cpw * gpw * 16 * scale_bytes + align16((size_t)c.cpw * gpw * 8)) +
                      (size_t)c.kpw * kTileK * 2;
  const size_t red = (size_t)c.cpw * c.mt * 1024;  // one weight stream's partial sums
  const size_t region = align16(meta > red ? meta : red);
  p.lds_s = (int)region;
  p.lds_r = (int)(c.nwk * region);
  // (+ one int: the workgroup's "last to arrive" flag of the split path;
  // then the slices' row sums of squares of the RMSNorm prologue)
  p.lds_bytes = (size_t)p.lds_r + 16 + (size_t)c.nwk * 16 * c.mt * 4;
  if (p.lds_bytes > 160 * 1024) return false;
  p.rows_pow2 = 0;
  p.alds = 0;
  // workspace: arrival counters (one per output tile of a workgroup, in the
  // same fixed region as every other plan's, so that all plans leave the
  // same words at zero), partial sums [S][NW][M][N]
  size_t off = 0;
  if (p.split > 1) {
    const size_t tiles = (size_t)p.gx * p.gz;
    if (tiles > (size_t)kMaxSplitBlocks) return false;
    p.ws_cnt_off = 0;
    off = align256(kCounterBytes);
    p.ws_rms_off = 0;
    p.ws_part_off = off;
    off = align256(off + (size_t)p.split * NW * M * N * 4);
  }
  p.ws_total = off;
  return true;
}

// Tile kernel plan (M > 16 shapes the panel kernel cannot take, and M <= 16
// shapes the stream kernel cannot take): 64-row blocks x tile_columns() per workgroup over the whole K; wide
// column blocks only when several row blocks keep the grid full.
void plan_tile(Plan &p, int M, int K, int N, int group, int scale_bytes, bool gate_up) {
  p.kind = kKindTile;
  p.gz = (M + 63) / 64;
  p.cfg = p.gz > 1 ? 1 : 0;
  const int ct = tile_ct(p.cfg == 1, gate_up);
  p.gx = (N + tile_columns(ct) - 1) / tile_columns(ct);
  p.gy = 1;
  p.block = tile_threads();
  p.split = 1;
  p.cps = K / kTileK;
  p.lds_bytes = tile_lds_bytes(ct, group, scale_bytes, gate_up);
  p.ws_total = 0;
}

// Plans whose prologue may be staged: the RMSNorm staging buffers after the plan's own
// workspace (fp16 [M][K] staged rows, fp32 [M] sums of squares), and never
// inside the arrival counters at its start, which every plan shares and
// leaves at zero (a plan without split-K has no workspace of its own).
void add_staging(Plan &p, int M, int K) {
  if (!staged_prologue(p, M, true, true)) {
    p.ws_total_rms = p.ws_total;
    return;
  }
  const size_t counters = align256(kCounterBytes);
  p.ws_x_off = align256(p.ws_total > counters ? p.ws_total : counters);
  p.ws_ss_off = align256(p.ws_x_off + (size_t)M * K * 2);
  p.ws_total_rms = align256(p.ws_ss_off + (size_t)M * 4);
}

}  // namespace

Plan make_plan(int M, int K, int N, int group, int scale_bytes, bool gate_up, int force_kind,
               int force_cfg, int force_split) {
  Plan p{};
  if ((force_kind < 0 || force_kind == kKindStream) &&
      plan_stream(p, M, K, N, group, scale_bytes, gate_up,
                  force_kind == kKindStream ? force_cfg : -1, force_split)) {
    add_staging(p, M, K);
    return p;
  }
  p = Plan{};
  if ((force_kind < 0 || force_kind == kKindPanel) &&
      plan_panel(p, M, K, N, group, scale_bytes, gate_up, force_split)) {
    add_staging(p, M, K);
    return p;
  }
  p = Plan{};
  plan_tile(p, M, K, N, group, scale_bytes, gate_up);
  add_staging(p, M, K);
  return p;
}

hipError_t launch_gemm(const GemmArgs &a, const Plan &pl, int group, bool scale_f32,
                       bool gate_up, hipStream_t stream) {
  if (staged_prologue(pl, a.M, a.gamma != nullptr, a.resid != nullptr)) {
    // stage the normalized rows, then the plain product on them with the
    // row scale in the epilogue
    const hipError_t e = launch_rms_stage(a.A, a.resid, a.resid_out, a.gamma, a.M, a.K,
                                          a.ws_x, a.ws_ss, stream);
    if (e != hipSuccess) return e;
    GemmArgs b = a;
    b.A = a.ws_x;
    b.gamma = nullptr;
    b.resid = nullptr;
    b.resid_out = nullptr;
    b.row_ss = a.ws_ss;
    return launch_gemm(b, pl, group, scale_f32, gate_up, stream);
  }
  if (pl.kind == kKindStream) return launch_stream(a, pl, group, scale_f32, gate_up, stream);
  if (pl.kind == kKindPanel) return launch_panel(a, pl, group, scale_f32, gate_up, stream);
  return launch_tile(a, pl, group, scale_f32, gate_up, stream);
}

}  // namespace w4a16
