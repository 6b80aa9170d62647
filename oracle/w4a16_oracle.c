/*
 * CPU oracle for the fp16-activation x int4-weight group-quantized GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header or constant with the GPU library and must never be on the
 * product path.
 *
 * Source of the method: the onnx-genai pull request "Marlin-style fused
 * fp16xint4 tensor-core GEMM" (page section "What's landed": weights are
 * stored in the ONNX-native nibble format with an asymmetric zero-point and a
 * per-(column, group) scale; the dequantized weight is (q - zp) * scale; group
 * sizes 16/32/64/128), its "Validation" section (an f64 dequant -> GEMM oracle),
 * the "fused RMS-norm prologue" update, and the "gate_up SwiGLU" update
 * (paired gate/up GEMMs followed by SiLU(gate) * up).  The bias + ReLU
 * epilogue follows the "Fusion benchmark" page (matmul plus bias plus relu).
 *
 * All arithmetic is IEEE double.  Inputs arrive already widened to double by
 * the caller (fp16 and fp32 values are exact in double), so this file never
 * touches a 16-bit float encoding.  Loops are written in the order of the
 * definition; the only parallelism is an OpenMP loop over independent output
 * columns, which does not change any sum's order.
 *
 * Canonical storage read here (the reading of the ONNX MatMulNBits format):
 *   qweight u8[N][K/2]   nibble k of column n is nibble (k mod 2) of byte
 *                        qweight[n*(K/2) + k/2]; even k in bits 0-3.
 *   scales  f64[N][G]    G = K / group, scale of column n, group i.
 *   zeros   u8[N][ceil(G/2)] nibble i of row n; even i in bits 0-3;
 *                        NULL means the symmetric case, zero-point 8.
 */
#include <math.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR (-1)

enum { ORACLE_EPI_NONE = 0, ORACLE_EPI_BIAS = 1, ORACLE_EPI_BIAS_RELU = 2 };

/* Nibble number idx of a byte array, low nibble first. */
static int nibble_at(const uint8_t *bytes, long idx) {
  uint8_t b = bytes[idx / 2];
  return (idx % 2 == 0) ? (b & 0x0F) : (b >> 4);
}

/* Quantized code q[k][n] of the canonical weights. */
static int q_at(const uint8_t *qweight, int K, int k, int n) {
  return nibble_at(qweight + (long)n * (K / 2), k);
}

/* Zero-point z[n][i]; 8 when the weights are symmetric. */
static int z_at(const uint8_t *zeros, int G, int n, int i) {
  if (zeros == NULL) return 8;
  long row_bytes = (G + 1) / 2;
  return nibble_at(zeros + (long)n * row_bytes, i);
}

static int check_shape(int M, int K, int N, int group) {
  if (M < 0 || K <= 0 || N <= 0 || group <= 0) return ORACLE_ERR;
  if (K % 2 != 0 || K % group != 0) return ORACLE_ERR;
  return ORACLE_OK;
}

/*
 * Dequantized weight w[k][n] = (q[k][n] - z[n][k/g]) * s[n][k/g], written to
 * W as a dense [K][N] row-major matrix.
 */
int oracle_dequant(const uint8_t *qweight, const double *scales,
                   const uint8_t *zeros, int K, int N, int group, double *W) {
  if (check_shape(0, K, N, group) != ORACLE_OK) return ORACLE_ERR;
  int G = K / group;
  for (int k = 0; k < K; ++k) {
    int i = k / group;
    for (int n = 0; n < N; ++n) {
      int q = q_at(qweight, K, k, n);
      int z = z_at(zeros, G, n, i);
      W[(long)k * N + n] = (double)(q - z) * scales[(long)n * G + i];
    }
  }
  return ORACLE_OK;
}

/*
 * RMSNorm of one activation row (the prologue of the "fused RMS-norm" update):
 *   x[k] = a[k] * gamma[k] / sqrt( (1/K) * sum_k a[k]^2 + eps )
 * eps sits inside the root and the mean runs over the whole row of K.
 */
static void rmsnorm_row(const double *a, const double *gamma, double eps,
                        int K, double *x) {
  double ss = 0.0;
  for (int k = 0; k < K; ++k) ss += a[k] * a[k];
  double inv = 1.0 / sqrt(ss / (double)K + eps);
  for (int k = 0; k < K; ++k) x[k] = a[k] * gamma[k] * inv;
}

/*
 * The RMSNorm prologue alone (the same rmsnorm_row per row):
 *   A f64[M][K], gamma f64[K], x f64[M][K] out.  Also returns, when r is not
 *   NULL, the row factor r[m] = 1 / sqrt((1/K) * sum_k A[m][k]^2 + eps).
 * The staged readings of the prologue (the normalized row, or A * gamma,
 * kept as fp16 between the norm and the product) are built from these.
 */
int oracle_rmsnorm(const double *A, int M, int K, const double *gamma, double eps,
                   double *x, double *r) {
  if (A == NULL || gamma == NULL || x == NULL || M < 1 || K < 1) return ORACLE_ERR;
  for (int m = 0; m < M; ++m) {
    rmsnorm_row(A + (long)m * K, gamma, eps, K, x + (long)m * K);
    if (r != NULL) {
      double ss = 0.0;
      for (int k = 0; k < K; ++k) ss += A[(long)m * K + k] * A[(long)m * K + k];
      r[m] = 1.0 / sqrt(ss / (double)K + eps);
    }
  }
  return ORACLE_OK;
}

/* y = sum_k x[k] * w[k][n] for one column, dequantizing as it goes. */
static double dot_column(const double *x, const uint8_t *qweight,
                         const double *scales, const uint8_t *zeros, int K,
                         int group, int n) {
  int G = K / group;
  double y = 0.0;
  for (int k = 0; k < K; ++k) {
    int i = k / group;
    double w = (double)(q_at(qweight, K, k, n) - z_at(zeros, G, n, i)) *
               scales[(long)n * G + i];
    y += x[k] * w;
  }
  return y;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* Sets the threads the OpenMP loops over output columns use (no effect
 * without OpenMP). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Threads the OpenMP loops over output columns use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Fused GEMM with optional RMSNorm prologue and bias / bias+ReLU epilogue.
 *
 *   A       f64[M][K]        activations
 *   gamma   f64[K] or NULL   RMSNorm weight; NULL = no prologue
 *   bias    f64[N] or NULL   required for the bias epilogues
 *   cols    int[ncols]       output columns to compute; NULL = all N, in order
 *   xwork   f64[M][K]        caller-provided scratch for the normalized rows
 *   out     f64[M][ncols]
 */
int oracle_gemm(const double *A, int M, int K, int N, const uint8_t *qweight,
                const double *scales, const uint8_t *zeros, int group,
                const double *gamma, double eps, int epilogue,
                const double *bias, const int *cols, int ncols, double *xwork,
                double *out) {
  if (check_shape(M, K, N, group) != ORACLE_OK) return ORACLE_ERR;
  if (epilogue != ORACLE_EPI_NONE && bias == NULL) return ORACLE_ERR;
  if (epilogue < ORACLE_EPI_NONE || epilogue > ORACLE_EPI_BIAS_RELU)
    return ORACLE_ERR;
  if (cols == NULL) ncols = N;
  for (int j = 0; j < ncols; ++j) {
    int n = cols ? cols[j] : j;
    if (n < 0 || n >= N) return ORACLE_ERR;
  }

  const double *X = A;
  if (gamma != NULL) {
    for (int m = 0; m < M; ++m)
      rmsnorm_row(A + (long)m * K, gamma, eps, K, xwork + (long)m * K);
    X = xwork;
  }

#pragma omp parallel for schedule(dynamic, 16)
  for (int j = 0; j < ncols; ++j) {
    int n = cols ? cols[j] : j;
    for (int m = 0; m < M; ++m) {
      double y = dot_column(X + (long)m * K, qweight, scales, zeros, K, group, n);
      if (epilogue == ORACLE_EPI_BIAS || epilogue == ORACLE_EPI_BIAS_RELU)
        y = y + bias[n];
      if (epilogue == ORACLE_EPI_BIAS_RELU) y = (y > 0.0) ? y : 0.0;
      out[(long)m * ncols + j] = y;
    }
  }
  return ORACLE_OK;
}

/*
 * Paired gate/up projection with the SwiGLU epilogue (the "gate_up SwiGLU
 * MLP fusion" update): out = silu(X . Wg) * (X . Wu), silu(v) = v/(1+e^-v).
 * Gate and up carry their own codes, scales and zero-points; both share K, N
 * and the group size.  No intermediate rounding.
 */
int oracle_gate_up(const double *A, int M, int K, int N,
                   const uint8_t *q_gate, const double *s_gate,
                   const uint8_t *z_gate, const uint8_t *q_up,
                   const double *s_up, const uint8_t *z_up, int group,
                   const double *gamma, double eps, const int *cols,
                   int ncols, double *xwork, double *out) {
  if (check_shape(M, K, N, group) != ORACLE_OK) return ORACLE_ERR;
  if (cols == NULL) ncols = N;
  for (int j = 0; j < ncols; ++j) {
    int n = cols ? cols[j] : j;
    if (n < 0 || n >= N) return ORACLE_ERR;
  }

  const double *X = A;
  if (gamma != NULL) {
    for (int m = 0; m < M; ++m)
      rmsnorm_row(A + (long)m * K, gamma, eps, K, xwork + (long)m * K);
    X = xwork;
  }

#pragma omp parallel for schedule(dynamic, 16)
  for (int j = 0; j < ncols; ++j) {
    int n = cols ? cols[j] : j;
    for (int m = 0; m < M; ++m) {
      const double *x = X + (long)m * K;
      double yg = dot_column(x, q_gate, s_gate, z_gate, K, group, n);
      double yu = dot_column(x, q_up, s_up, z_up, K, group, n);
      out[(long)m * ncols + j] = silu(yg) * yu;
    }
  }
  return ORACLE_OK;
}
