// C ABI of libw4a16.so (declared in include/w4a16.h): host-side argument
// validation, launch planning and the kernel launches.  Validation always
// runs before any HIP call, so every error status can be produced without a
// GPU.
#include <mutex>

#include "../../include/w4a16.h"
#include "common.h"

using namespace w4a16;

namespace {

constexpr int kMaxDim = 1 << 24;  // keeps every index product inside size_t math

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool group_ok(int g) { return g == 16 || g == 32 || g == 64 || g == 128; }

int scale_bytes_of(int dtype) {
  return dtype == W4A16_SCALE_F16 ? 2 : (dtype == W4A16_SCALE_F32 ? 4 : 0);
}

int check_kn(int K, int N, int group) {
  if (K <= 0 || N <= 0 || K % kTileK != 0 || N % kTileN != 0 || K > kMaxDim ||
      N > kMaxDim)
    return W4A16_ERR_SHAPE;
  if (!group_ok(group)) return W4A16_ERR_GROUP;
  return W4A16_OK;
}

int check_gemm(const void *A, int M, int K, int N, int group, int scale_dtype,
               const void *const *packed, int npacked, const void *out) {
  if (A == nullptr || out == nullptr) return W4A16_ERR_NULL;
  for (int i = 0; i < npacked; ++i)
    if (packed[i] == nullptr) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxDim) return W4A16_ERR_SHAPE;
  const int st = check_kn(K, N, group);
  if (st != W4A16_OK) return st;
  if (scale_bytes_of(scale_dtype) == 0) return W4A16_ERR_DTYPE;
  if (!aligned16(A) || !aligned16(out)) return W4A16_ERR_ALIGN;
  for (int i = 0; i < npacked; ++i)
    if (!aligned16(packed[i])) return W4A16_ERR_ALIGN;
  return W4A16_OK;
}

// A call that stages its RMSNorm prologue needs the plan's staging buffers too.
int check_workspace(const Plan &pl, bool staged, const void *ws, size_t ws_bytes) {
  const size_t need = staged ? pl.ws_total_rms : pl.ws_total;
  if (need == 0) return W4A16_OK;
  if (ws == nullptr) return W4A16_ERR_WORKSPACE;
  if (ws_bytes < need) return W4A16_ERR_WORKSPACE;
  if (!aligned16(ws)) return W4A16_ERR_ALIGN;
  return W4A16_OK;
}

// The automatic plan (split <= 0) or the stream / panel kernel with `split`
// workgroups along K; W4A16_ERR_SPLIT when that split cannot run the shape.
int plan_for(int M, int K, int N, int group, int scale_dtype, bool gate_up, int split,
             Plan &pl) {
  const int sb = scale_bytes_of(scale_dtype);
  if (split <= 0) {
    pl = make_plan(M, K, N, group, sb, gate_up);
    return W4A16_OK;
  }
  pl = make_plan(M, K, N, group, sb, gate_up, -1, -1, split);
  return pl.kind != kKindTile ? W4A16_OK : W4A16_ERR_SPLIT;
}

void fill_packed(GemmArgs &a, int slot, const void *packed, int K, int N,
                 int group, int sbytes, bool has_zp) {
  const PackedOffsets off = packed_offsets(K, N, group, sbytes, has_zp);
  const uint8_t *base = static_cast<const uint8_t *>(packed);
  a.w[slot] = base;
  a.scales[slot] = base + off.scales;
  a.zeros[slot] = has_zp ? base + off.zeros : nullptr;
}

void fill_workspace(GemmArgs &a, const Plan &pl, void *ws) {
  uint8_t *b = static_cast<uint8_t *>(ws);
  a.split = pl.split;
  a.cps = pl.cps;
  a.rows_pow2 = pl.rows_pow2;
  a.lds_s = pl.lds_s;
  a.lds_r = pl.lds_r;
  a.ws_part = pl.ws_total ? reinterpret_cast<float *>(b + pl.ws_part_off) : nullptr;
  a.ws_rms = pl.ws_total ? reinterpret_cast<float *>(b + pl.ws_rms_off) : nullptr;
  a.ws_cnt = pl.ws_total ? reinterpret_cast<uint32_t *>(b + pl.ws_cnt_off) : nullptr;
  const bool staged = b != nullptr && pl.ws_total_rms > pl.ws_total;
  a.ws_x = staged ? reinterpret_cast<f16 *>(b + pl.ws_x_off) : nullptr;
  a.ws_ss = staged ? reinterpret_cast<float *>(b + pl.ws_ss_off) : nullptr;
}

int launched(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH; }

}  // namespace

extern "C" {

size_t w4a16_packed_bytes(int K, int N, int group, int scale_dtype, int has_zp) {
  if (check_kn(K, N, group) != W4A16_OK) return 0;
  const int sb = scale_bytes_of(scale_dtype);
  if (sb == 0) return 0;
  return packed_offsets(K, N, group, sb, has_zp != 0).total;
}

int w4a16_repack(const uint8_t *qweight, const void *scales,
                 const uint8_t *zeros, int K, int N, int group,
                 int scale_dtype, void *packed, w4a16_stream stream) {
  if (qweight == nullptr || scales == nullptr || packed == nullptr)
    return W4A16_ERR_NULL;
  const int st = check_kn(K, N, group);
  if (st != W4A16_OK) return st;
  const int sb = scale_bytes_of(scale_dtype);
  if (sb == 0) return W4A16_ERR_DTYPE;
  if (!aligned16(qweight) || !aligned16(scales) || !aligned16(packed) ||
      (zeros != nullptr && !aligned16(zeros)))
    return W4A16_ERR_ALIGN;
  return launched(launch_repack(qweight, scales, zeros, K, N, group, sb,
                                static_cast<uint8_t *>(packed),
                                static_cast<hipStream_t>(stream)));
}

size_t w4a16_workspace_bytes(int M, int K, int N, int group, int gate_up) {
  if (M < 1 || M > kMaxDim || check_kn(K, N, group) != W4A16_OK) return 0;
  // the plan (and so the workspace) may differ with the scale width: take
  // the larger of fp16 and fp32 scales
  const size_t a = make_plan(M, K, N, group, 2, gate_up != 0).ws_total_rms;
  const size_t b = make_plan(M, K, N, group, 4, gate_up != 0).ws_total_rms;
  return a > b ? a : b;
}

namespace {

// Residual (skip + RMSNorm) arguments: the residual needs the norm; both
// device buffers 16-byte aligned.
int check_residual(const void *resid, const void *resid_out, const void *gamma) {
  if (resid == nullptr) return resid_out == nullptr ? W4A16_OK : W4A16_ERR_NULL;
  if (gamma == nullptr) return W4A16_ERR_NULL;
  if (!aligned16(resid) || (resid_out != nullptr && !aligned16(resid_out))) return W4A16_ERR_ALIGN;
  return W4A16_OK;
}

// A validated launch: arguments, plan and kernel selection of one call.
struct Call {
  GemmArgs a{};
  Plan pl{};
  int group = 0;
  bool sf32 = false;
  bool gate_up = false;
};

int run(const Call &c, w4a16_stream stream) {
  return launched(launch_gemm(c.a, c.pl, c.group, c.sf32, c.gate_up,
                              static_cast<hipStream_t>(stream)));
}

// Validates a plain GEMM call and fills `c`; touches no device.
int prep_gemm(const void *A, const void *resid, void *resid_out, int M, int K, int N,
              int group, int scale_dtype, int has_zp, const void *packed, int epilogue,
              const void *bias, const void *rms_gamma, float rms_eps, void *out,
              void *workspace, size_t workspace_bytes, int split, Call &c) {
  const void *pk[1] = {packed};
  int st = check_gemm(A, M, K, N, group, scale_dtype, pk, 1, out);
  if (st != W4A16_OK) return st;
  st = check_residual(resid, resid_out, rms_gamma);
  if (st != W4A16_OK) return st;
  if (epilogue != W4A16_EPI_NONE && epilogue != W4A16_EPI_BIAS &&
      epilogue != W4A16_EPI_BIAS_RELU)
    return W4A16_ERR_EPILOGUE;
  if (epilogue != W4A16_EPI_NONE && bias == nullptr) return W4A16_ERR_EPILOGUE;
  if ((bias != nullptr && !aligned16(bias)) ||
      (rms_gamma != nullptr && !aligned16(rms_gamma)))
    return W4A16_ERR_ALIGN;
  st = plan_for(M, K, N, group, scale_dtype, false, split, c.pl);
  if (st != W4A16_OK) return st;
  st = check_workspace(c.pl, staged_prologue(c.pl, M, rms_gamma != nullptr, resid != nullptr),
                       workspace, workspace_bytes);
  if (st != W4A16_OK) return st;

  const int sb = scale_bytes_of(scale_dtype);
  GemmArgs &a = c.a;
  a = GemmArgs{};
  a.A = static_cast<const f16 *>(A);
  a.M = M;
  a.K = K;
  a.N = N;
  fill_packed(a, 0, packed, K, N, group, sb, has_zp != 0);
  a.has_zp = has_zp != 0;
  a.epilogue = epilogue;
  a.bias = static_cast<const f16 *>(bias);
  a.gamma = static_cast<const f16 *>(rms_gamma);
  a.resid = static_cast<const f16 *>(resid);
  a.resid_out = static_cast<f16 *>(resid_out);
  a.eps = rms_eps;
  a.out = static_cast<f16 *>(out);
  fill_workspace(a, c.pl, workspace);
  c.group = group;
  c.sf32 = sb == 4;
  c.gate_up = false;
  return W4A16_OK;
}

// Validates a gate_up call and fills `c`; touches no device.
int prep_gate_up(const void *A, const void *resid, void *resid_out, int M, int K, int N,
                 int group, int scale_dtype, int has_zp, const void *packed_gate,
                 const void *packed_up, const void *rms_gamma, float rms_eps, void *out,
                 void *workspace, size_t workspace_bytes, int split, Call &c) {
  const void *pk[2] = {packed_gate, packed_up};
  int st = check_gemm(A, M, K, N, group, scale_dtype, pk, 2, out);
  if (st != W4A16_OK) return st;
  st = check_residual(resid, resid_out, rms_gamma);
  if (st != W4A16_OK) return st;
  if (rms_gamma != nullptr && !aligned16(rms_gamma)) return W4A16_ERR_ALIGN;
  st = plan_for(M, K, N, group, scale_dtype, true, split, c.pl);
  if (st != W4A16_OK) return st;
  st = check_workspace(c.pl, staged_prologue(c.pl, M, rms_gamma != nullptr, resid != nullptr),
                       workspace, workspace_bytes);
  if (st != W4A16_OK) return st;

  const int sb = scale_bytes_of(scale_dtype);
  GemmArgs &a = c.a;
  a = GemmArgs{};
  a.A = static_cast<const f16 *>(A);
  a.M = M;
  a.K = K;
  a.N = N;
  fill_packed(a, 0, packed_gate, K, N, group, sb, has_zp != 0);
  fill_packed(a, 1, packed_up, K, N, group, sb, has_zp != 0);
  a.has_zp = has_zp != 0;
  a.epilogue = W4A16_EPI_NONE;
  a.gamma = static_cast<const f16 *>(rms_gamma);
  a.resid = static_cast<const f16 *>(resid);
  a.resid_out = static_cast<f16 *>(resid_out);
  a.eps = rms_eps;
  a.out = static_cast<f16 *>(out);
  fill_workspace(a, c.pl, workspace);
  c.group = group;
  c.sf32 = sb == 4;
  c.gate_up = true;
  return W4A16_OK;
}

int gemm_impl(const void *A, const void *resid, void *resid_out, int M, int K, int N,
              int group, int scale_dtype, int has_zp, const void *packed, int epilogue,
              const void *bias, const void *rms_gamma, float rms_eps, void *out,
              void *workspace, size_t workspace_bytes, int split, w4a16_stream stream) {
  Call c;
  const int st = prep_gemm(A, resid, resid_out, M, K, N, group, scale_dtype, has_zp, packed,
                           epilogue, bias, rms_gamma, rms_eps, out, workspace,
                           workspace_bytes, split, c);
  return st != W4A16_OK ? st : run(c, stream);
}

int gate_up_impl(const void *A, const void *resid, void *resid_out, int M, int K, int N,
                 int group, int scale_dtype, int has_zp, const void *packed_gate,
                 const void *packed_up, const void *rms_gamma, float rms_eps, void *out,
                 void *workspace, size_t workspace_bytes, int split, w4a16_stream stream) {
  Call c;
  const int st = prep_gate_up(A, resid, resid_out, M, K, N, group, scale_dtype, has_zp,
                              packed_gate, packed_up, rms_gamma, rms_eps, out, workspace,
                              workspace_bytes, split, c);
  return st != W4A16_OK ? st : run(c, stream);
}

}  // namespace

int w4a16_gemm_split(const void *A, int M, int K, int N, int group, int scale_dtype,
                     int has_zp, const void *packed, int epilogue, const void *bias,
                     const void *rms_gamma, float rms_eps, void *out, void *workspace,
                     size_t workspace_bytes, int split, w4a16_stream stream) {
  return gemm_impl(A, nullptr, nullptr, M, K, N, group, scale_dtype, has_zp, packed, epilogue,
                   bias, rms_gamma, rms_eps, out, workspace, workspace_bytes, split, stream);
}

int w4a16_gemm_gate_up_split(const void *A, int M, int K, int N, int group,
                             int scale_dtype, int has_zp, const void *packed_gate,
                             const void *packed_up, const void *rms_gamma,
                             float rms_eps, void *out, void *workspace,
                             size_t workspace_bytes, int split, w4a16_stream stream) {
  return gate_up_impl(A, nullptr, nullptr, M, K, N, group, scale_dtype, has_zp, packed_gate,
                      packed_up, rms_gamma, rms_eps, out, workspace, workspace_bytes, split,
                      stream);
}

int w4a16_gemm_skip_rmsnorm(const void *A, const void *residual, void *residual_out, int M,
                            int K, int N, int group, int scale_dtype, int has_zp,
                            const void *packed, int epilogue, const void *bias,
                            const void *rms_gamma, float rms_eps, void *out, void *workspace,
                            size_t workspace_bytes, w4a16_stream stream) {
  if (residual == nullptr || rms_gamma == nullptr) return W4A16_ERR_NULL;
  return gemm_impl(A, residual, residual_out, M, K, N, group, scale_dtype, has_zp, packed,
                   epilogue, bias, rms_gamma, rms_eps, out, workspace, workspace_bytes, 0,
                   stream);
}

int w4a16_gemm_gate_up_skip_rmsnorm(const void *A, const void *residual, void *residual_out,
                                    int M, int K, int N, int group, int scale_dtype,
                                    int has_zp, const void *packed_gate,
                                    const void *packed_up, const void *rms_gamma,
                                    float rms_eps, void *out, void *workspace,
                                    size_t workspace_bytes, w4a16_stream stream) {
  if (residual == nullptr || rms_gamma == nullptr) return W4A16_ERR_NULL;
  return gate_up_impl(A, residual, residual_out, M, K, N, group, scale_dtype, has_zp,
                      packed_gate, packed_up, rms_gamma, rms_eps, out, workspace,
                      workspace_bytes, 0, stream);
}

int w4a16_gemm(const void *A, int M, int K, int N, int group, int scale_dtype,
               int has_zp, const void *packed, int epilogue, const void *bias,
               const void *rms_gamma, float rms_eps, void *out,
               void *workspace, size_t workspace_bytes, w4a16_stream stream) {
  return w4a16_gemm_split(A, M, K, N, group, scale_dtype, has_zp, packed, epilogue, bias,
                          rms_gamma, rms_eps, out, workspace, workspace_bytes, 0, stream);
}

int w4a16_gemm_gate_up(const void *A, int M, int K, int N, int group,
                       int scale_dtype, int has_zp, const void *packed_gate,
                       const void *packed_up, const void *rms_gamma,
                       float rms_eps, void *out, void *workspace,
                       size_t workspace_bytes, w4a16_stream stream) {
  return w4a16_gemm_gate_up_split(A, M, K, N, group, scale_dtype, has_zp, packed_gate,
                                  packed_up, rms_gamma, rms_eps, out, workspace,
                                  workspace_bytes, 0, stream);
}

size_t w4a16_mlp_workspace_bytes(int M, int H, int I, int group) {
  const size_t a = w4a16_workspace_bytes(M, H, I, group, 1);
  const size_t b = w4a16_workspace_bytes(M, I, H, group, 0);
  return a > b ? a : b;
}

int w4a16_mlp(const void *A, const void *residual, void *residual_out, int M, int H, int I,
              int group, int scale_dtype, int has_zp, const void *packed_gate,
              const void *packed_up, const void *packed_down, const void *rms_gamma,
              float rms_eps, void *inter, void *out, void *workspace,
              size_t workspace_bytes, w4a16_stream stream) {
  // both projections are validated before either is enqueued
  Call up, down;
  int st = prep_gate_up(A, residual, residual_out, M, H, I, group, scale_dtype, has_zp,
                        packed_gate, packed_up, rms_gamma, rms_eps, inter, workspace,
                        workspace_bytes, 0, up);
  if (st != W4A16_OK) return st;
  st = prep_gemm(inter, nullptr, nullptr, M, I, H, group, scale_dtype, has_zp, packed_down,
                 W4A16_EPI_NONE, nullptr, nullptr, 0.0f, out, workspace, workspace_bytes, 0,
                 down);
  if (st != W4A16_OK) return st;
  st = run(up, stream);
  return st != W4A16_OK ? st : run(down, stream);
}

int w4a16_probe_read_tiles(const void *w, int K, int N, int mode, int workgroups, void *sink,
                           size_t sink_bytes, w4a16_stream stream) {
  if (w == nullptr || sink == nullptr) return W4A16_ERR_NULL;
  if (K < kTileK || K % kTileK != 0 || N < kTileN || N % kTileN != 0 || K > kMaxDim || N > kMaxDim ||
      (size_t)(N / kTileN) * (size_t)(K / kTileK) > ((size_t)1 << 30) || (mode != 0 && mode != 1) ||
      (mode == 1 && (workgroups < 1 || workgroups > 65535)))
    return W4A16_ERR_SHAPE;
  if ((size_t)probe_tiles_grid(N, mode, workgroups) * 512 * 4 > sink_bytes) return W4A16_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(sink)) return W4A16_ERR_ALIGN;
  return launched(launch_probe_tiles(w, K, N, mode, workgroups, static_cast<uint32_t *>(sink),
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The no-allocation entry point: w4a16_gemm with its workspace taken from a
// fixed device array of the library instead of the caller.
namespace {

constexpr size_t kScratchBytes = (size_t)W4A16_NOALLOC_SCRATCH_BYTES;

// Split-K counters (first W4A16_COUNTER_BYTES), partial sums and RMSNorm
// staging rows of w4a16_gemm_noalloc.  Each GPU the library runs on holds
// its own copy for the life of the process.  In host code `scratch` is only
// a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress (scratch_ptr below), never from the name itself.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device (with
// that device current); on the first lookup its split-K counters are
// cleared by a fill kernel on `stream` (in stream order before the GEMM
// that follows; no memset node, so the call stays capture-safe).
int scratch_ptr(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return W4A16_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return W4A16_ERR_LAUNCH;
    }
    const int words = (int)(kCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t *>(ptr), words);
    if (hipGetLastError() != hipSuccess) return W4A16_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_gemm_noalloc(const void *A, int M, int K, int N, int group, int scale_dtype,
                       int has_zp, const void *packed, int epilogue, const void *bias,
                       const void *rms_gamma, float rms_eps, void *out, w4a16_stream stream) {
  // validate and plan without a workspace first: every argument error is
  // reported before any HIP call, and a call that needs a workspace
  // stops at the workspace check with its plan filled in
  Call c;
  int st = prep_gemm(A, nullptr, nullptr, M, K, N, group, scale_dtype, has_zp, packed,
                     epilogue, bias, rms_gamma, rms_eps, out, nullptr, 0, 0, c);
  if (st != W4A16_OK && st != W4A16_ERR_WORKSPACE) return st;
  const bool staged = staged_prologue(c.pl, M, rms_gamma != nullptr, false);
  const size_t need = staged ? c.pl.ws_total_rms : c.pl.ws_total;
  if (need > kScratchBytes) return W4A16_ERR_SCRATCH;
  if (need > 0) {
    void *ws = nullptr;
    st = scratch_ptr(static_cast<hipStream_t>(stream), &ws);
    if (st != W4A16_OK) return st;
    st = prep_gemm(A, nullptr, nullptr, M, K, N, group, scale_dtype, has_zp, packed, epilogue,
                   bias, rms_gamma, rms_eps, out, ws, kScratchBytes, 0, c);
    if (st != W4A16_OK) return st;
  }
  return run(c, stream);
}

int w4a16_plan(int M, int K, int N, int group, int scale_dtype, int gate_up, int split,
               w4a16_plan_info *info) {
  if (info == nullptr) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxDim) return W4A16_ERR_SHAPE;
  int st = check_kn(K, N, group);
  if (st != W4A16_OK) return st;
  if (scale_bytes_of(scale_dtype) == 0) return W4A16_ERR_DTYPE;
  Plan pl;
  st = plan_for(M, K, N, group, scale_dtype, gate_up != 0, split, pl);
  if (st != W4A16_OK) return st;
  info->kernel = pl.kind == kKindStream  ? W4A16_KERNEL_STREAM
                 : pl.kind == kKindPanel ? W4A16_KERNEL_PANEL
                                         : W4A16_KERNEL_TILE;
  info->split = pl.split;
  info->k_tiles_per_split = pl.cps;
  info->grid[0] = pl.gx;
  info->grid[1] = pl.gy;
  info->grid[2] = pl.gz;
  info->block = pl.block;
  info->lds_bytes = (int)pl.lds_bytes;
  info->workspace_bytes = pl.ws_total_rms;
  if (pl.kind == kKindStream) {
    info->col_tiles = kStreamCfgs[pl.cfg].cpw;
    info->k_tiles_per_wave = kStreamCfgs[pl.cfg].kpw;
  } else if (pl.kind == kKindPanel) {
    info->col_tiles = kPanelCfgs[pl.cfg].cpw;
    info->k_tiles_per_wave = kPanelCfgs[pl.cfg].kpw;
  } else {
    // the tile kernel's two k slices take every other k tile
    info->col_tiles = tile_columns(tile_ct(pl.cfg == 1, gate_up != 0)) / kTileN;
    info->k_tiles_per_wave = (pl.cps + 1) / 2;
  }
  return W4A16_OK;
}

const char *w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL: return "a required pointer is NULL";
    case W4A16_ERR_SHAPE: return "bad shape (need M >= 1, K % 128 == 0, N % 16 == 0)";
    case W4A16_ERR_GROUP: return "group must be 16, 32, 64 or 128";
    case W4A16_ERR_DTYPE: return "unknown scale dtype";
    case W4A16_ERR_EPILOGUE: return "unknown epilogue, or bias missing for a bias epilogue";
    case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
    case W4A16_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case W4A16_ERR_LAUNCH: return "kernel launch failed";
    case W4A16_ERR_SPLIT: return "forced split-K factor not possible for this shape";
    case W4A16_ERR_SCRATCH:
      return "shape needs more workspace than the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

int w4a16_layout_version(void) { return W4A16_LAYOUT_VERSION; }

int w4a16_add_bias(const void *in, const void *bias, int M, int N, void *out,
                   w4a16_stream stream) {
  if (in == nullptr || bias == nullptr || out == nullptr) return W4A16_ERR_NULL;
  if (M < 1 || N < 1 || N % 16 != 0 || M > kMaxDim || N > kMaxDim) return W4A16_ERR_SHAPE;
  if (!aligned16(in) || !aligned16(bias) || !aligned16(out)) return W4A16_ERR_ALIGN;
  return launched(launch_add_bias(static_cast<const f16 *>(in), static_cast<const f16 *>(bias),
                                  M, N, static_cast<f16 *>(out),
                                  static_cast<hipStream_t>(stream)));
}

int w4a16_relu(const void *in, int M, int N, void *out, w4a16_stream stream) {
  if (in == nullptr || out == nullptr) return W4A16_ERR_NULL;
  if (M < 1 || N < 1 || N % 16 != 0 || M > kMaxDim || N > kMaxDim) return W4A16_ERR_SHAPE;
  if (!aligned16(in) || !aligned16(out)) return W4A16_ERR_ALIGN;
  return launched(launch_relu(static_cast<const f16 *>(in), M, N, static_cast<f16 *>(out),
                              static_cast<hipStream_t>(stream)));
}

int w4a16_rmsnorm(const void *A, const void *gamma, float eps, int M, int K,
                  void *out, w4a16_stream stream) {
  if (A == nullptr || gamma == nullptr || out == nullptr) return W4A16_ERR_NULL;
  if (M < 1 || K < 1 || K % 128 != 0 || M > kMaxDim || K > kMaxDim) return W4A16_ERR_SHAPE;
  if (!aligned16(A) || !aligned16(gamma) || !aligned16(out)) return W4A16_ERR_ALIGN;
  return launched(launch_rmsnorm(static_cast<const f16 *>(A), static_cast<const f16 *>(gamma),
                                 eps, M, K, static_cast<f16 *>(out),
                                 static_cast<hipStream_t>(stream)));
}

int w4a16_probe_read(const void *buf, size_t bytes, void *sink, w4a16_stream stream) {
  if (buf == nullptr || sink == nullptr) return W4A16_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return W4A16_ERR_SHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return W4A16_ERR_ALIGN;
  return launched(launch_probe_read(buf, bytes, static_cast<uint32_t *>(sink),
                                    static_cast<hipStream_t>(stream)));
}

int w4a16_probe_copy(const void *src, void *dst, size_t bytes, w4a16_stream stream) {
  if (src == nullptr || dst == nullptr) return W4A16_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return W4A16_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return W4A16_ERR_ALIGN;
  return launched(launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int w4a16_probe_lds_read(int workgroups, int iters, void *sink, w4a16_stream stream) {
  if (sink == nullptr) return W4A16_ERR_NULL;
  if (workgroups < 1 || workgroups > 65535 || iters < 1 || iters > (1 << 20)) return W4A16_ERR_SHAPE;
  if (!aligned16(sink)) return W4A16_ERR_ALIGN;
  return launched(launch_probe_lds_read(workgroups, iters, static_cast<uint32_t *>(sink),
                                        static_cast<hipStream_t>(stream)));
}

int w4a16_probe_mfma_valu(int valu_per_8_mfma, int waves_per_simd, int workgroups, int iters,
                          void *sink, size_t sink_bytes, w4a16_stream stream) {
  if (sink == nullptr) return W4A16_ERR_NULL;
  const int v = valu_per_8_mfma;
  if ((v != 0 && v != 8 && v != 16 && v != 32 && v != 48 && v != 64) ||
      (waves_per_simd != 1 && waves_per_simd != 2) || workgroups < 1 || workgroups > 65535 ||
      iters < 1 || iters > (1 << 20))
    return W4A16_ERR_SHAPE;
  const int threads = 256 * waves_per_simd;
  if ((size_t)workgroups * threads * 4 > sink_bytes) return W4A16_ERR_SHAPE;
  if (!aligned16(sink)) return W4A16_ERR_ALIGN;
  return launched(launch_probe_mfma_valu(v, threads, workgroups, iters, static_cast<float *>(sink),
                                         static_cast<hipStream_t>(stream)));
}

int w4a16_probe_lds_copy(const void *buf, size_t bytes, int workgroups, int steps, void *sink,
                         w4a16_stream stream) {
  if (buf == nullptr || sink == nullptr) return W4A16_ERR_NULL;
  if (bytes < 16384 || bytes % 16384 != 0 || bytes / 16384 > (size_t)kMaxDim || workgroups < 1 ||
      workgroups > 65535 || steps < 1 || steps > (1 << 20))
    return W4A16_ERR_SHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return W4A16_ERR_ALIGN;
  return launched(launch_probe_lds_copy(buf, bytes, workgroups, steps, static_cast<uint32_t *>(sink),
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
