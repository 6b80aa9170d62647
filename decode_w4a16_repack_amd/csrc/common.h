// Internal declarations shared by the HIP translation units of libw4a16.so.
// Not part of the C ABI (that is include/w4a16.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kTileK = 128;      // k extent of one packed weight tile
constexpr int kTileN = 16;       // columns of one packed weight tile
constexpr int kTileBytes = 1024; // bytes of one packed tile (64 lanes x 16 B)
// Split-K arrival counters at the start of every workspace: one 32-bit word
// per column tile (stream kernel) or output tile (panel kernel), so split-K
// is possible up to this many tiles (N <= 65536 on the stream kernel).
constexpr int kMaxSplitBlocks = 4096;
constexpr int kMaxDevices = 64;  // per-device host state (LDS limits, static scratch)
constexpr size_t kCounterBytes = (size_t)kMaxSplitBlocks * 4;

// Tile configurations of the small-M stream kernel: CPW 16-column tiles per
// wavefront, KPW 128-k tiles per wavefront (its activation fragments stay in
// registers), NWK wavefronts (k slices) per workgroup, PD tiles in flight.
struct StreamCfg {
  int cpw, kpw, nwk, pd;
};
constexpr int kNumStreamCfgs = 4;
extern const StreamCfg kStreamCfgs[kNumStreamCfgs];

// Tile configurations of the panel kernel (16 < M <= 32): MT 16-row tiles
// per workgroup, and CPW, KPW, NWK, PD as for the stream kernel.
struct PanelCfg {
  int mt, cpw, kpw, nwk, pd;
};
constexpr int kNumPanelCfgs = 1;
extern const PanelCfg kPanelCfgs[kNumPanelCfgs];

inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Byte offsets of the packed regions (layout version 1).
struct PackedOffsets {
  size_t scales;
  size_t zeros;
  size_t total;
};

inline PackedOffsets packed_offsets(int K, int N, int group, int scale_bytes,
                                    bool has_zp) {
  PackedOffsets o;
  size_t G = (size_t)(K / group);
  size_t w_bytes = (size_t)K * (size_t)N / 2;
  o.scales = align256(w_bytes);
  size_t s_end = o.scales + (size_t)N * G * (size_t)scale_bytes;
  o.zeros = has_zp ? align256(s_end) : 0;
  size_t end = has_zp ? o.zeros + (size_t)N * G / 2 : s_end;
  o.total = align256(end);
  return o;
}

// Everything a GEMM launch needs; filled by the API layer.
struct GemmArgs {
  const f16 *A;
  int M, K, N;
  const uint8_t *w[2];      // packed weight tiles (gate, up); w[1] only for gate_up
  const void *scales[2];    // packed scales [N/16][G][16] inside the packed buffer
  const uint8_t *zeros[2];  // packed zero-points [N/16][G][16 nibbles], or null
  int has_zp;
  int epilogue;
  const f16 *bias;
  const f16 *gamma;  // null: no RMSNorm prologue
  const f16 *resid;  // with gamma: residual added before the norm (null: none)
  f16 *resid_out;    // with resid: the sum A + resid written here (null: not written)
  float eps;
  // panel / tile kernels: fp32 [M] sums of squares of the staged rows (the
  // RMSNorm prologue, done by the staging pass); the epilogue multiplies row
  // m by 1 / sqrt(row_ss[m] / K + eps).  Null: no row scale.
  const float *row_ss;
  f16 *out;
  f16 *ws_x;          // staging: fp16 [M][K] x * gamma (panel / tile prologue)
  float *ws_ss;       // staging: fp32 [M] row sums of squares
  float *ws_part;     // [S][2 if gate_up][M][N] fp32 partial sums
  float *ws_rms;      // [blocks][S][64] fp32 partial sums of squares
  uint32_t *ws_cnt;   // [blocks] arrival counters, zero between calls
  int split;          // number of K splits across workgroups
  int cps;            // 128-wide k tiles per split
  int rows_pow2;      // stream kernel: activation rows staged in LDS (power of two >= M)
  int lds_s;          // stream kernel: bytes of one wavefront's private LDS region
  int lds_r;          // stream kernel: byte offset of the sum-of-squares scratch in LDS
};

// Launch plan of one GEMM call, a pure function of the shape.
enum PlanKind { kKindStream = 2, kKindTile = 3, kKindPanel = 4 };

struct Plan {
  int kind;     // PlanKind: stream.hip (kStreamCfgs), panel.hip (kPanelCfgs) or tile.hip
  int cfg;      // index into the kernel's configuration table
  int gx, gy, gz;
  int block;  // threads per workgroup
  int split, cps;
  int rows_pow2;
  int lds_s, lds_r;
  int alds;  // stream kernel: activation rows staged through LDS
  size_t lds_bytes;
  size_t ws_part_off, ws_rms_off, ws_cnt_off, ws_total;
  // panel / tile plans: the RMSNorm staging buffers follow the split-K
  // region; a call with the prologue needs ws_total_rms bytes, one without
  // it ws_total (stream plans: the two are equal)
  size_t ws_x_off, ws_ss_off, ws_total_rms;
};

// k tiles per wavefront of a streaming-kernel plan (0 for other kernels)
inline int stream_kpw(const Plan &p) { return p.kind == kKindStream ? kStreamCfgs[p.cfg].kpw : 0; }

// Whether a call stages its RMSNorm prologue (stage.hip) instead of running
// it inside the product kernel: always for the tile kernel; for the panel
// kernel with the residual or a k split across workgroups; for the
// streaming kernel only with the residual, and there with more than 4 rows
// (re-reading both activation slices in every column block costs more than
// one staging pass) or a slice deeper than 5 k tiles (its registers cannot
// hold the whole slice and its residual).
inline bool staged_prologue(const Plan &p, int M, bool gamma, bool resid) {
  if (!gamma) return false;
  if (p.kind == kKindStream) return resid && (M > 4 || stream_kpw(p) > 5);
  if (p.kind == kKindPanel) return resid || p.split > 1;
  return true;
}

// force_kind: -1 automatic, else a PlanKind; force_cfg < 0 /
// force_split <= 0 select the built-in choice.
Plan make_plan(int M, int K, int N, int group, int scale_bytes, bool gate_up,
               int force_kind = -1, int force_cfg = -1, int force_split = 0);

hipError_t launch_stream(const GemmArgs &a, const Plan &p, int group, bool scale_f32,
                         bool gate_up, hipStream_t stream);
// stream_rms.hip / stream_skip.hip: the streaming kernel with the in-register
// RMSNorm / skip + RMSNorm prologue
hipError_t launch_stream_rms(const GemmArgs &a, const Plan &p, int group, bool scale_f32,
                             bool gate_up, hipStream_t stream);
hipError_t launch_stream_skip(const GemmArgs &a, const Plan &p, int group, bool scale_f32,
                              bool gate_up, hipStream_t stream);

hipError_t launch_panel(const GemmArgs &a, const Plan &p, int group, bool scale_f32,
                        bool gate_up, hipStream_t stream);

// tile.hip (M > 16): column tiles per wavefront and weight stream (wide:
// several 64-row blocks), LDS bytes, output columns per workgroup
int tile_ct(bool wide, bool gate_up);
size_t tile_lds_bytes(int ct, int group, int scale_bytes, bool gate_up);
int tile_columns(int ct);
int tile_threads();
hipError_t launch_tile(const GemmArgs &a, const Plan &p, int group, bool scale_f32,
                       bool gate_up, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs &a, const Plan &p, int group,
                       bool scale_f32, bool gate_up, hipStream_t stream);

// stage.hip: S = A (+ resid, written to resid_out when not null), x_out =
// fp16(S * gamma), ss_out[m] = sum_k S[m][k]^2 in fp32; one workgroup per row.
hipError_t launch_rms_stage(const f16 *A, const f16 *resid, f16 *resid_out, const f16 *gamma,
                            int M, int K, f16 *x_out, float *ss_out, hipStream_t stream);

hipError_t launch_repack(const uint8_t *qweight, const void *scales,
                         const uint8_t *zeros, int K, int N, int group,
                         int scale_bytes, uint8_t *packed, hipStream_t stream);

hipError_t launch_add_bias(const f16 *in, const f16 *bias, int M, int N,
                           f16 *out, hipStream_t stream);
hipError_t launch_relu(const f16 *in, int M, int N, f16 *out,
                       hipStream_t stream);
hipError_t launch_rmsnorm(const f16 *A, const f16 *gamma, float eps, int M,
                          int K, f16 *out, hipStream_t stream);
hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink,
                             hipStream_t stream);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes,
                             hipStream_t stream);
hipError_t launch_probe_lds_read(int workgroups, int iters, uint32_t *sink, hipStream_t stream);
hipError_t launch_probe_mfma_valu(int valu, int threads, int workgroups, int iters, float *sink,
                                  hipStream_t stream);
hipError_t launch_probe_lds_copy(const void *buf, size_t bytes, int workgroups, int steps,
                                 uint32_t *sink, hipStream_t stream);
unsigned probe_tiles_grid(int N, int mode, int workgroups);
hipError_t launch_probe_tiles(const void *w, int K, int N, int mode, int workgroups, uint32_t *sink,
                              hipStream_t stream);

}  // namespace w4a16
