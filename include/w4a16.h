/*
 * w4a16.h - C ABI of the MI355X (gfx950) fp16-activation x int4-weight
 * group-quantized GEMM/GEMV library (libw4a16.so).
 *
 * The operation (onnx-genai pull request "Marlin-style fused fp16xint4
 * tensor-core GEMM", section "What's landed"): activations A are fp16; the
 * weights are 4-bit codes q with one scale per (output column, group of
 * `group` consecutive k) and an optional asymmetric 4-bit zero-point zp; the
 * weight used in the product is (q - zp) * scale, with zp = 8 when the
 * weights are symmetric.  Group sizes 16, 32, 64 and 128 are supported, as on
 * that page.
 *
 *   out[m][n] = epilogue( sum_k X[m][k] * (q[k][n] - zp[n][k/group]) * s[n][k/group] )
 *
 * with X = A, or X = RMSNorm(A) when a prologue weight gamma is given
 * ("fused RMS-norm" update: x * gamma / sqrt(mean_k x^2 + eps)).  Epilogues:
 * none, + bias, or max(+ bias, 0) ("Fusion benchmark" page: matmul plus bias
 * plus relu).  w4a16_gemm_gate_up computes silu(X.Wg) * (X.Wu) ("gate_up
 * SwiGLU MLP fusion" update).
 *
 * Numerics: (q - zp) is formed exactly in fp16, products with A are exact in
 * fp32, sums are fp32, and each group's fp32 partial sum is multiplied by its
 * scale once the matrix-core contraction of that group is done (the scale
 * step of "What's landed").  The output is rounded once to fp16 (nearest
 * even).  Results
 * are run-to-run bit-identical: split-K partial sums are reduced in a fixed
 * order, never with floating-point atomics.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees, synchronizes or reads data back to the host.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  The launch grid depends only on the arguments.
 *  - Device pointers must be 16-byte aligned (W4A16_ERR_ALIGN otherwise).
 *  - Arguments are validated on the host before any HIP call; on error
 *    nothing is enqueued and a negative w4a16_status is returned.  A failed
 *    launch returns W4A16_ERR_LAUNCH.
 *  - Shapes: M >= 1, K a positive multiple of 128, N a positive multiple of
 *    16, group in {16, 32, 64, 128} (W4A16_ERR_SHAPE / W4A16_ERR_GROUP).
 *
 * Canonical (input) weight format, the ONNX MatMulNBits reading:
 *   qweight u8[N][K/2]        code k of column n is nibble (k mod 2) of byte
 *                             k/2 of row n, even k in the low nibble
 *   scales  fp16|fp32 [N][G]  G = K/group
 *   zeros   u8[N][ceil(G/2)]  zero-point of group i in nibble (i mod 2) of
 *                             byte i/2 of row n, even i low; NULL = symmetric
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_LAYOUT_VERSION 1

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_NULL = -1,      /* a required pointer is NULL */
  W4A16_ERR_SHAPE = -2,     /* M < 1, K % 128, N % 16, K % group, too large */
  W4A16_ERR_GROUP = -3,     /* group not in {16, 32, 64, 128} */
  W4A16_ERR_DTYPE = -4,     /* scale_dtype not a W4A16_SCALE_* value */
  W4A16_ERR_EPILOGUE = -5,  /* unknown epilogue, or a bias epilogue without bias */
  W4A16_ERR_WORKSPACE = -6, /* workspace NULL or smaller than required */
  W4A16_ERR_ALIGN = -7,     /* a device pointer is not 16-byte aligned */
  W4A16_ERR_LAUNCH = -8,    /* the HIP launch failed (hipGetLastError) */
  W4A16_ERR_SPLIT = -9,     /* a forced split-K factor the shape cannot use */
  W4A16_ERR_SCRATCH = -10   /* the call needs more workspace than the static
                               scratch of w4a16_gemm_noalloc holds */
} w4a16_status;

enum { W4A16_SCALE_F16 = 0, W4A16_SCALE_F32 = 1 };

enum { W4A16_EPI_NONE = 0, W4A16_EPI_BIAS = 1, W4A16_EPI_BIAS_RELU = 2 };

typedef void *w4a16_stream; /* a hipStream_t */

/*
 * Packed layout, version 1 (KC = K/128, G = K/group).  "What's landed" asks
 * for a reorder of the weights that is done once, loses nothing (a
 * bijection) and makes every load coalesced; the device repack here writes
 * the same bytes as the oracle's host repack of this layout.
 *   Weights at offset 0, K*N/2 bytes: tile (t = n/16, kc = k/128) is 1 KiB
 *     at byte (t*KC + kc)*1024; lane l (0..63) of a 64-lane wavefront owns
 *     its 16 bytes at l*16; 32-bit word d (0..3) of lane l holds the codes
 *     k = 128*kc + 32*d + 8*(l/16) + j, j = 0..7, of column n = 16*t + l%16,
 *     code j in bits 4*(j/2) (even j) or 16 + 4*(j/2) (odd j).
 *   Scales at offset align256(K*N/2), N*G elements of the scale dtype:
 *     element ((n/16)*G + i)*16 + n%16 is scales[n][i] (bytes unchanged), so
 *     the 16 scales of one column tile and group are contiguous.
 *   Zero-points (only when zeros != NULL) at offset align256(end of scales),
 *     N*G/2 bytes: nibble ((n/16)*G + i)*16 + n%16 (low nibble first) is the
 *     zero-point of column n, group i; 8 bytes per column tile and group.
 *   Total: align256(end of the last region).  Pad bytes are zero.
 */
size_t w4a16_packed_bytes(int K, int N, int group, int scale_dtype, int has_zp);

/*
 * One-time repack of canonical weights into the packed layout above.
 * qweight, scales: required; zeros: NULL for symmetric weights.  packed
 * must hold w4a16_packed_bytes(K, N, group, scale_dtype, zeros != NULL)
 * bytes and must not overlap the inputs.  The packed buffer serves every M.
 */
int w4a16_repack(const uint8_t *qweight, const void *scales,
                 const uint8_t *zeros, int K, int N, int group,
                 int scale_dtype, void *packed, w4a16_stream stream);

/*
 * Workspace bytes w4a16_gemm (gate_up = 0) or w4a16_gemm_gate_up
 * (gate_up = 1) needs for this shape: fp32 split-K partial sums and
 * arrival counters, and the RMSNorm staging rows (fp16 [M][K] x * gamma
 * activations and fp32 [M] sums of squares, written by a staging pass
 * before the product, as the "fused RMS-norm" update on the onnx-genai pull
 * request stages the normalized activation) for the calls that stage their
 * prologue: every RMSNorm call above 16 rows, and the skip + RMSNorm calls
 * above 4 rows or on deep-k shapes.  Only those calls need the staging
 * part: a call without a prologue on a shape without split-K (w4a16_plan
 * reports split 1) may pass a NULL workspace.  0 when M <= 4, the k range
 * is at most 5120 and the shape runs without split-K.  The workspace must be
 * zero-filled once after allocation; the split-K arrival counters occupy
 * its first W4A16_COUNTER_BYTES bytes for every shape (the staging rows never
 * do) and every call leaves them at zero again, so one workspace (sized for
 * the largest shape) serves calls of any shape.  Calls that share a
 * workspace must not run concurrently.
 */
#define W4A16_COUNTER_BYTES 16384
size_t w4a16_workspace_bytes(int M, int K, int N, int group, int gate_up);

/*
 * Fused GEMM.  A: fp16 [M][K] row-major.  packed: from w4a16_repack with
 * the same K, N, group, scale_dtype and has_zp (has_zp = zeros were given).
 * epilogue: W4A16_EPI_*; bias: fp16 [N], required for the bias epilogues.
 * rms_gamma: fp16 [K] enables the RMSNorm prologue with rms_eps; NULL
 * disables it.  out: fp16 [M][N] row-major; rows are written once, nothing
 * outside out[0..M-1][0..N-1] is touched.  workspace: see
 * w4a16_workspace_bytes (may be NULL when that returns 0).
 */
int w4a16_gemm(const void *A, int M, int K, int N, int group, int scale_dtype,
               int has_zp, const void *packed, int epilogue, const void *bias,
               const void *rms_gamma, float rms_eps, void *out,
               void *workspace, size_t workspace_bytes, w4a16_stream stream);

/*
 * Paired gate/up projection with the SwiGLU epilogue:
 * out = silu(X.Wg) * (X.Wu), silu(v) = v / (1 + exp(-v)), computed in fp32
 * and rounded once.  packed_gate and packed_up are two separately repacked
 * weights with the same K, N, group, scale_dtype and has_zp.  Optional
 * RMSNorm prologue as in w4a16_gemm.
 */
int w4a16_gemm_gate_up(const void *A, int M, int K, int N, int group,
                       int scale_dtype, int has_zp, const void *packed_gate,
                       const void *packed_up, const void *rms_gamma,
                       float rms_eps, void *out, void *workspace,
                       size_t workspace_bytes, w4a16_stream stream);

/*
 * Split-K control.  The "Small-M split-K retune" update on the onnx-genai
 * pull request tunes how many workgroups share one output tile's k range
 * for the small-M decode shapes (o/q 4096x4096, down 13696x4096, gate_up
 * 4096x2*13696 and 5120x2*13824 at M=8).  The automatic choice (split = 0)
 * keeps at least two wavefronts per compute unit in flight and splits
 * further only when the k range exceeds what one workgroup covers.  A
 * positive `split` forces that many k slices on the streaming kernel
 * (M <= 16) or the panel kernel (16 < M <= 32); the actual factor may round down
 * so that no slice is empty.  W4A16_ERR_SPLIT when the shape cannot run
 * with it: split larger than K/128, smaller than the k range one workgroup
 * can cover, or a shape only the tile kernel takes.
 */
enum { W4A16_KERNEL_STREAM = 1, W4A16_KERNEL_TILE = 2, W4A16_KERNEL_PANEL = 3 };

typedef struct {
  int kernel;             /* W4A16_KERNEL_STREAM (M <= 16), W4A16_KERNEL_PANEL
                             (16 < M <= 32) or W4A16_KERNEL_TILE (above, and shapes
                             the others cannot take) */
  int split;              /* workgroups along K per output tile (1 = no split-K) */
  int k_tiles_per_split;  /* 128-wide k tiles one split covers */
  int grid[3];            /* launch grid */
  int block;              /* threads per workgroup */
  int lds_bytes;          /* dynamic LDS per workgroup */
  size_t workspace_bytes; /* workspace a call with the RMSNorm prologue needs
                             (see w4a16_workspace_bytes); without it, the
                             split-K part alone */
  int col_tiles;          /* 16-column weight tiles one workgroup covers (the
                             last workgroup of a row may cover fewer) */
  int k_tiles_per_wave;   /* 128-wide k tiles one wavefront contracts per
                             column tile (the kernel configuration's depth) */
} w4a16_plan_info;

/* Host-only: fill *info with the plan a call of this shape launches.
 * Touches no device.  Returns W4A16_ERR_SPLIT as described above. */
int w4a16_plan(int M, int K, int N, int group, int scale_dtype, int gate_up,
               int split, w4a16_plan_info *info);

/* w4a16_gemm / w4a16_gemm_gate_up with a split-K factor (0 = automatic,
 * the same as the calls without it).  The workspace must hold
 * w4a16_plan(...).workspace_bytes for the same split. */
int w4a16_gemm_split(const void *A, int M, int K, int N, int group,
                     int scale_dtype, int has_zp, const void *packed,
                     int epilogue, const void *bias, const void *rms_gamma,
                     float rms_eps, void *out, void *workspace,
                     size_t workspace_bytes, int split, w4a16_stream stream);
int w4a16_gemm_gate_up_split(const void *A, int M, int K, int N, int group,
                             int scale_dtype, int has_zp,
                             const void *packed_gate, const void *packed_up,
                             const void *rms_gamma, float rms_eps, void *out,
                             void *workspace, size_t workspace_bytes,
                             int split, w4a16_stream stream);

/*
 * Skip + RMSNorm prologue (SkipSimplifiedLayerNormalization, the residual
 * step before the projections of a decoder block; named in the "Stage 2 of
 * spec-capture" update on the onnx-genai pull request, which makes it
 * capture-safe).  The normalized input is the residual sum:
 *   S = A + residual        (fp16 [M][K], each element rounded once)
 *   X = S * gamma / sqrt(mean_k S^2 + eps)
 * and the product, epilogue and gate_up pairing are those of w4a16_gemm /
 * w4a16_gemm_gate_up with X in place of RMSNorm(A).  residual: fp16 [M][K],
 * required, as is rms_gamma.  residual_out: fp16 [M][K] or NULL; when given,
 * S is written there (every element exactly once), the updated residual
 * stream for the next layer.  residual_out must not overlap A or residual.
 */
int w4a16_gemm_skip_rmsnorm(const void *A, const void *residual,
                            void *residual_out, int M, int K, int N, int group,
                            int scale_dtype, int has_zp, const void *packed,
                            int epilogue, const void *bias,
                            const void *rms_gamma, float rms_eps, void *out,
                            void *workspace, size_t workspace_bytes,
                            w4a16_stream stream);
int w4a16_gemm_gate_up_skip_rmsnorm(const void *A, const void *residual,
                                    void *residual_out, int M, int K, int N,
                                    int group, int scale_dtype, int has_zp,
                                    const void *packed_gate,
                                    const void *packed_up,
                                    const void *rms_gamma, float rms_eps,
                                    void *out, void *workspace,
                                    size_t workspace_bytes,
                                    w4a16_stream stream);

/*
 * MLP block: the paired gate/up projection followed by the down projection
 * of its output ("gate_up SwiGLU MLP fusion" update on the onnx-genai pull
 * request: the MLP carries most of the decode cost; its down projection is
 * the deep-k decode shape 13696 x 4096 of the "Small-M split-K retune"
 * update).
 *   inter = fp16( silu(X.Wg) * (X.Wu) )      fp16 [M][I]
 *   out   = fp16( inter . Wd )               fp16 [M][H]
 * with X = A, RMSNorm(A) (rms_gamma given) or RMSNorm(A + residual)
 * (residual given, as in w4a16_gemm_gate_up_skip_rmsnorm; residual_out
 * receives the sum when not NULL).  A: fp16 [M][H].  packed_gate and
 * packed_up: repacked with K = H, N = I; packed_down: repacked with K = I,
 * N = H; all three with the same group, scale_dtype and has_zp.  So I must
 * be a multiple of 128 and H a multiple of 128.  inter: caller-owned
 * device buffer of M*I fp16 that receives the intermediate (it is also the
 * down projection's input; it must not overlap A, residual, residual_out,
 * out or the workspace).  The two projections are enqueued in that order
 * on `stream` and share the workspace, which must hold
 * w4a16_mlp_workspace_bytes(M, H, I, group) bytes (zero-filled once after
 * allocation, as for w4a16_gemm).  Both calls are validated before either
 * is enqueued: on error nothing runs.
 */
size_t w4a16_mlp_workspace_bytes(int M, int H, int I, int group);
int w4a16_mlp(const void *A, const void *residual, void *residual_out, int M,
              int H, int I, int group, int scale_dtype, int has_zp,
              const void *packed_gate, const void *packed_up,
              const void *packed_down, const void *rms_gamma, float rms_eps,
              void *inter, void *out, void *workspace, size_t workspace_bytes,
              w4a16_stream stream);

/*
 * w4a16_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, results and errors are
 * those of w4a16_gemm.  The split-K partial sums, arrival counters and
 * RMSNorm staging rows that w4a16_gemm keeps in the caller's workspace are
 * kept instead in a fixed device array of the library,
 * W4A16_NOALLOC_SCRATCH_BYTES long; each GPU the library runs on holds its
 * own copy until the process ends.  A shape whose workspace need
 * (w4a16_workspace_bytes, or the split-K part alone without a prologue)
 * exceeds that size is refused with W4A16_ERR_SCRATCH before anything is
 * enqueued.  The first call on a device looks up that device's copy and
 * clears its counters with a fill kernel on `stream`; no call allocates,
 * frees or synchronizes.  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race and must not be issued; calls ordered on one
 * stream are safe, and each leaves the counters at zero.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (8u << 20)
int w4a16_gemm_noalloc(const void *A, int M, int K, int N, int group, int scale_dtype,
                       int has_zp, const void *packed, int epilogue, const void *bias,
                       const void *rms_gamma, float rms_eps, void *out,
                       w4a16_stream stream);

/* Static, human-readable text for a w4a16_status value. */
const char *w4a16_status_string(int status);

/* W4A16_LAYOUT_VERSION of the packed layout this library reads and writes. */
int w4a16_layout_version(void);

/*
 * Measurement aids.  The "Fusion benchmark" page compares a fused kernel
 * with the unfused chain built from the same source; these are the unfused
 * chain's separate passes, each one kernel reading and writing HBM.
 *   w4a16_add_bias: out[m][n] = fp16(in[m][n] + bias[n])
 *   w4a16_relu:     out[m][n] = max(in[m][n], 0)
 *   w4a16_rmsnorm:  out[m][k] = fp16(A[m][k] * gamma[k] / sqrt(mean A^2 + eps))
 * All fp16, row-major; in-place (out == in) is allowed for the first two.
 */
int w4a16_add_bias(const void *in, const void *bias, int M, int N, void *out,
                   w4a16_stream stream);
int w4a16_relu(const void *in, int M, int N, void *out, w4a16_stream stream);
int w4a16_rmsnorm(const void *A, const void *gamma, float eps, int M, int K,
                  void *out, w4a16_stream stream);

/*
 * Streaming probes for the achievable HBM rate.  w4a16_probe_read reads
 * `bytes` (a multiple of 16) and writes one 32-bit value per workgroup to
 * sink (at least 4096 * 4 bytes) so the reads cannot be elided;
 * w4a16_probe_copy copies `bytes` (a multiple of 16) from src to dst.
 */
int w4a16_probe_read(const void *buf, size_t bytes, void *sink,
                     w4a16_stream stream);
int w4a16_probe_copy(const void *src, void *dst, size_t bytes,
                     w4a16_stream stream);

/*
 * Probes of one compute unit's data paths, the limits of the MFMA-tile
 * kernel (M > 32), which moves each step's 64-row activation tile from L2
 * into LDS and reads it back from LDS once per wavefront.  Both launch
 * `workgroups` workgroups of 512 threads and write one 32-bit value per
 * thread to sink (at least workgroups * 512 * 4 bytes), so nothing is
 * elided.
 *   w4a16_probe_lds_read: 64 KiB of LDS per workgroup, then every
 *     wavefront reads iters * 16 KiB from it (16-byte conflict-free reads):
 *     workgroups * 512 * iters * 256 bytes in all.
 *   w4a16_probe_lds_copy: buf holds a 64-row fp16 matrix of bytes / 128
 *     columns (bytes a multiple of 16384, read-only, small enough to stay in
 *     L2); per step every workgroup copies one 64 x 128 k tile per pair of
 *     wavefronts (32 KiB) into LDS with direct global-to-LDS loads of whole
 *     256-byte row segments, two steps in flight, one barrier per step:
 *     workgroups * (steps + 1) * 32 KiB in all.
 * W4A16_ERR_SHAPE for workgroups outside 1..65535, iters or steps outside
 * 1..2^20, or a bad byte count.
 */
int w4a16_probe_lds_read(int workgroups, int iters, void *sink, w4a16_stream stream);
int w4a16_probe_lds_copy(const void *buf, size_t bytes, int workgroups, int steps, void *sink,
                         w4a16_stream stream);

/*
 * Issue probe: how far independent VALU work overlaps the matrix cores, the
 * limit of the MFMA-tile kernel, which unpacks every weight word and scales
 * every group's partial sums with VALU instructions next to its MFMAs.
 * `workgroups` workgroups of 256 * waves_per_simd threads (1 or 2 wavefronts
 * per SIMD when each compute unit holds one workgroup); every wavefront runs
 * iters rounds of 8 independent-accumulator v_mfma_f32_16x16x32_f16 and
 * valu_per_8_mfma (0, 8, 16, 32, 48 or 64) independent fp32 FMAs, and writes
 * one fp32 value per thread to sink (at least workgroups * threads * 4 bytes,
 * sink_bytes).  W4A16_ERR_SHAPE for another FMA count or wavefront count,
 * workgroups outside 1..65535, iters outside 1..2^20, or a sink too small.
 */
int w4a16_probe_mfma_valu(int valu_per_8_mfma, int waves_per_simd, int workgroups, int iters,
                          void *sink, size_t sink_bytes, w4a16_stream stream);


/*
 * Probe of how the streaming kernel's tiles are spread over the chip: plain
 * reads of the K*N/2-byte weight region of a packed matrix (w, as written by
 * w4a16_repack), one 16-byte load per lane per 1 KiB tile, eight tiles per
 * batch with the next batch in flight, no arithmetic, in one of two
 * decompositions over workgroups of 512 threads:
 *   mode 0: the streaming kernel's own (its widest configuration):
 *     ceil(N/64) workgroups; workgroup g reads column tiles 4g..4g+3 over
 *     all of K, its wavefront w the k tiles w*P .. w*P+P-1 of each
 *     (P = ceil(K/1024)); `workgroups` is ignored;
 *   mode 1: the (N/16)*(K/128) tiles split evenly over `workgroups`
 *     workgroups (1..65535), each taking a contiguous range of the layout
 *     and dealing it round-robin to its 8 wavefronts.
 * One 32-bit value per thread goes to sink (at least grid * 2048 bytes,
 * sink_bytes), so nothing is elided.  W4A16_ERR_SHAPE for K or N not a
 * multiple of 128 / 16, more than 2^30 tiles, another mode, workgroups
 * outside 1..65535 in mode 1, or a sink too small.
 */
int w4a16_probe_read_tiles(const void *w, int K, int N, int mode, int workgroups, void *sink,
                           size_t sink_bytes, w4a16_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
