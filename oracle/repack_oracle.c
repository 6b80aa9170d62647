/*
 * CPU oracle for the one-time weight repack.
 *
 * TEST INFRASTRUCTURE ONLY (see w4a16_oracle.c).  Written from the documented
 * packed layout below, not from the GPU kernel.
 *
 * In the onnx-genai pull request "Marlin-style fused fp16xint4 tensor-core
 * GEMM" ("What's landed") the int4 weights are reordered once, losslessly,
 * for coalesced loads, and the GPU's repack is checked against a host
 * repack byte for byte.  The reorder here is this library's
 * own (one 16-byte load per lane, 1 KiB per 64-lane wavefront); only the
 * properties (a bijection of nibbles, bit-preserving for scales and
 * zero-points) come from the page.
 *
 * Packed layout, version 1.  KC = K/128, G = K/group, NT = N/16.
 *   Region W (offset 0, K*N/2 bytes).  Canonical nibble (k, n) goes to packed
 *   nibble index
 *       ((((n/16) * KC + k/128) * 64 + lane) * 4 + d) * 8 + pos
 *   with kk = k mod 128, d = kk/32, kq = (kk mod 32)/8, j = kk mod 8,
 *   lane = (n mod 16) + 16*kq, pos = 4*(j mod 2) + j/2.
 *   Packed nibble index p is nibble (p mod 2) of byte p/2, low nibble first.
 *   So lane `lane` of tile (n/16, k/128) owns 16 contiguous bytes; 32-bit
 *   word d of them holds the 8 codes k = 128*kc + 32*d + 8*kq + j of column n,
 *   even j in bits 4*(j/2).., odd j in bits 16 + 4*(j/2)...
 *   Region S (offset align256(K*N/2), N*G*esize bytes).  Element
 *   ((n/16) * G + i) * 16 + (n mod 16) holds scales[n][i], bytes unchanged:
 *   the 16 scales of one column tile and group are contiguous.
 *   Region Z (only with zero-points; offset align256(end of S), N*G/2
 *   bytes).  Nibble ((n/16) * G + i) * 16 + (n mod 16), low nibble first,
 *   holds z[n][i]: 8 bytes per column tile and group.
 *   Total size: align256(end of the last region); pad bytes are zero.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR (-1)

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

static int layout_ok(int K, int N, int group) {
  if (K <= 0 || N <= 0 || group <= 0) return 0;
  if (K % 128 != 0 || N % 16 != 0 || K % group != 0) return 0;
  return 1;
}

/* Byte offsets of the three regions and the total size. */
int oracle_packed_layout(int K, int N, int group, int esize, int has_zp,
                         size_t *s_off, size_t *z_off, size_t *total) {
  if (!layout_ok(K, N, group) || (esize != 2 && esize != 4)) return ORACLE_ERR;
  size_t G = (size_t)(K / group);
  size_t w_bytes = (size_t)K * (size_t)N / 2;
  size_t so = align256(w_bytes);
  size_t s_end = so + (size_t)N * G * (size_t)esize;
  size_t zo = align256(s_end);
  size_t end = has_zp ? zo + (size_t)N * G / 2 : s_end;
  *s_off = so;
  *z_off = has_zp ? zo : 0;
  *total = align256(end);
  return ORACLE_OK;
}

/* Packed nibble index of canonical weight nibble (k, n). */
long oracle_weight_nibble_index(int K, int k, int n) {
  long KC = K / 128;
  int kk = k % 128;
  int d = kk / 32, kq = (kk % 32) / 8, j = kk % 8;
  int lane = (n % 16) + 16 * kq;
  int pos = 4 * (j % 2) + j / 2;
  long tile = (long)(n / 16) * KC + k / 128;
  return (((tile * 64 + lane) * 4 + d) * 8) + pos;
}

static int get_nibble(const uint8_t *b, long idx) {
  return (idx % 2 == 0) ? (b[idx / 2] & 0x0F) : (b[idx / 2] >> 4);
}

static void put_nibble(uint8_t *b, long idx, int v) {
  if (idx % 2 == 0)
    b[idx / 2] = (uint8_t)((b[idx / 2] & 0xF0) | (v & 0x0F));
  else
    b[idx / 2] = (uint8_t)((b[idx / 2] & 0x0F) | ((v & 0x0F) << 4));
}

/*
 * Canonical (qweight u8[N][K/2], scales [N][G] raw bytes of esize each,
 * zeros u8[N][ceil(G/2)] or NULL) -> packed buffer of oracle_packed_layout's
 * total size.  Pad bytes between regions are written as zero.
 */
int oracle_repack(const uint8_t *qweight, const uint8_t *scales,
                  const uint8_t *zeros, int K, int N, int group, int esize,
                  uint8_t *packed) {
  size_t so, zo, total;
  if (oracle_packed_layout(K, N, group, esize, zeros != NULL, &so, &zo,
                           &total) != ORACLE_OK)
    return ORACLE_ERR;
  int G = K / group;
  memset(packed, 0, total);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) {
      int q = get_nibble(qweight + (long)n * (K / 2), k);
      put_nibble(packed, oracle_weight_nibble_index(K, k, n), q);
    }
  for (int n = 0; n < N; ++n)
    for (int i = 0; i < G; ++i) {
      long e = ((long)(n / 16) * G + i) * 16 + (n % 16);
      memcpy(packed + so + (size_t)e * esize,
             scales + ((size_t)n * G + i) * esize, (size_t)esize);
    }
  if (zeros != NULL) {
    long zrow = (G + 1) / 2;
    for (int n = 0; n < N; ++n)
      for (int i = 0; i < G; ++i) {
        long e = ((long)(n / 16) * G + i) * 16 + (n % 16);
        put_nibble(packed + zo, e, get_nibble(zeros + (long)n * zrow, i));
      }
  }
  return ORACLE_OK;
}

/* Inverse of oracle_repack.  zeros may be NULL when has_zp is 0. */
int oracle_unrepack(const uint8_t *packed, int K, int N, int group, int esize,
                    int has_zp, uint8_t *qweight, uint8_t *scales,
                    uint8_t *zeros) {
  size_t so, zo, total;
  if (oracle_packed_layout(K, N, group, esize, has_zp, &so, &zo, &total) !=
      ORACLE_OK)
    return ORACLE_ERR;
  int G = K / group;
  memset(qweight, 0, (size_t)N * (size_t)K / 2);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k)
      put_nibble(qweight + (long)n * (K / 2), k,
                 get_nibble(packed, oracle_weight_nibble_index(K, k, n)));
  for (int n = 0; n < N; ++n)
    for (int i = 0; i < G; ++i) {
      long e = ((long)(n / 16) * G + i) * 16 + (n % 16);
      memcpy(scales + ((size_t)n * G + i) * esize,
             packed + so + (size_t)e * esize, (size_t)esize);
    }
  if (has_zp && zeros != NULL) {
    long zrow = (G + 1) / 2;
    memset(zeros, 0, (size_t)N * (size_t)zrow);
    for (int n = 0; n < N; ++n)
      for (int i = 0; i < G; ++i) {
        long e = ((long)(n / 16) * G + i) * 16 + (n % 16);
        put_nibble(zeros + (long)n * zrow, i, get_nibble(packed + zo, e));
      }
  }
  return ORACLE_OK;
}
