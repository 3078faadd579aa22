/*
 * tern_oracle.c -- plain, slow, obviously-correct CPU oracle for the ternary
 * packed-bit linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; both are written from the same statement of the method.
 *
 * What it computes (sources are the Neutrino-1 pages):
 *  - every projection weight is one of three states, minus, zero or plus
 *    (article "Neutrino-1: quantization is a training decision, not a
 *    deployment one", intro and section "What's actually ternary");
 *  - a weight's value is its state times a higher-precision scale, and signed
 *    accumulation replaces multiplies (same article, "What's actually
 *    ternary" and "The take");
 *  - weights stay bit-packed at rest, with per-row metadata holding row
 *    dimensions, scales and row sums (Neutrino-1 8B model card, "Overview"
 *    and "Where the bytes live").  The pages call their own packing
 *    proprietary (wiki entry "Neutrino-1", "What is actually new here"), so
 *    the 2-bit layout below is this project's own.
 *
 *  The row sum has exactly one arithmetic use: an activation given as
 *  x_j = s_act * (q_j - z) (int8 q, fp32 scale s_act, int32 zero point z)
 *  gives  sum_j w_ij * (q_j - z) = sum_j w_ij * q_j - z * rowsum_i.  So for
 *  M tokens m and N rows i:
 *
 *     acc[m][i] = sum_j w_ij * q[m][j]  -  z[m] * rowsum[i]         (exact)
 *     y[m][i]   = (s_row[i] * acc[m][i]) * s_act[m]
 *
 *  The sum is taken in int64 and must fit in +-2^24 (then the int32 result
 *  and its conversion to float are exact).  y is returned twice: in fp64
 *  (the reference value) and in fp32 with the two products rounded in the
 *  order written above (round-to-nearest-even, no fused multiply-add; build
 *  with -ffp-contract=off).
 *
 * 2-bit layout (this project's own):
 *  - code(w) = w + 1:  -1 -> 00, 0 -> 01, +1 -> 10;  11 is invalid;
 *  - a row occupies row_bytes(K) = 16 * ceil(K / 64) bytes, so every row
 *    starts 16-byte aligned;
 *  - weight j of a row lives in the little-endian 32-bit word j / 16, at bit
 *    8 * (j % 4) + 2 * ((j % 16) / 4) of that word, i.e. in byte
 *    4 * (j / 16) + j % 4 of the row, at bit 2 * ((j % 16) / 4) of that byte;
 *  - columns j >= K are padding and hold code 01 (weight 0), so a byte made
 *    only of padding reads 0x55.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_OVERFLOW 1     /* |acc| >= 2^24 */
#define ORACLE_INVALID_CODE 2 /* a 11 field among the real columns */

int64_t oracle_row_bytes(int64_t K) { return 16 * ((K + 63) / 64); }

/* Byte of the row that holds weight j, and the shift of its 2-bit field. */
static int64_t field_byte(int64_t j) { return 4 * (j / 16) + j % 4; }
static int field_shift(int64_t j) { return 2 * (int)((j % 16) / 4); }

static unsigned read_code(const uint8_t* row, int64_t j) {
  return (row[field_byte(j)] >> field_shift(j)) & 3u;
}

static void write_code(uint8_t* row, int64_t j, unsigned code) {
  uint8_t* b = &row[field_byte(j)];
  int s = field_shift(j);
  *b = (uint8_t)((*b & ~(3u << s)) | (code << s));
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Pack an N x K int8 matrix (row stride ldw elements) whose entries are in
 * {-1, 0, +1}.  Writes N rows of row_bytes(K) bytes and rowsum[i] = sum_j w_ij.
 * Returns the number of entries outside {-1, 0, +1}; such an entry is stored
 * as weight 0 and left out of the row sum.
 */
int64_t oracle_pack(const int8_t* w, int64_t N, int64_t K, int64_t ldw,
                    uint8_t* packed, int32_t* rowsum) {
  const int64_t ld = oracle_row_bytes(K);
  int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t i = 0; i < N; ++i) {
    uint8_t* row = packed + i * ld;
    memset(row, 0x55, (size_t)ld); /* every field 01: weight 0 */
    int64_t sum = 0;
    for (int64_t j = 0; j < K; ++j) {
      int v = w[i * ldw + j];
      if (v < -1 || v > 1) {
        ++bad;
        continue;
      }
      write_code(row, j, (unsigned)(v + 1));
      sum += v;
    }
    rowsum[i] = (int32_t)sum;
  }
  return bad;
}

/*
 * Unpack N rows back to int8 weights (row stride ldw elements).  A field
 * holding the invalid code 11 is written as 0 and counted; the count is
 * returned.
 */
int64_t oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w,
                      int64_t ldw) {
  const int64_t ld = oracle_row_bytes(K);
  int64_t invalid = 0;
#pragma omp parallel for schedule(static) reduction(+ : invalid)
  for (int64_t i = 0; i < N; ++i) {
    const uint8_t* row = packed + i * ld;
    for (int64_t j = 0; j < K; ++j) {
      unsigned c = read_code(row, j);
      if (c == 3u) {
        ++invalid;
        w[i * ldw + j] = 0;
      } else {
        w[i * ldw + j] = (int8_t)((int)c - 1);
      }
    }
  }
  return invalid;
}

/*
 * Check packed rows: counts[0] = fields with code 11 among columns j < K,
 * counts[1] = padding fields (K <= j < 4 * row_bytes) that are not 01.
 */
void oracle_validate(const uint8_t* packed, int64_t N, int64_t K,
                     int64_t counts[2]) {
  const int64_t ld = oracle_row_bytes(K);
  int64_t invalid = 0, padding = 0;
#pragma omp parallel for schedule(static) reduction(+ : invalid, padding)
  for (int64_t i = 0; i < N; ++i) {
    const uint8_t* row = packed + i * ld;
    for (int64_t j = 0; j < 4 * ld; ++j) {
      unsigned c = read_code(row, j);
      if (j < K) {
        if (c == 3u) ++invalid;
      } else if (c != 1u) {
        ++padding;
      }
    }
  }
  counts[0] = invalid;
  counts[1] = padding;
}

/*
 * The linear layer on packed weights.  q is M x K int8 (row stride ldq),
 * s_act and z hold one value per token, s_row and rowsum one per row.
 * Outputs are M x N with row stride ldy: acc (int32), y32 (fp32) and y64
 * (fp64); any of them may be NULL.  Returns ORACLE_OK, or the first error
 * met (outputs of the failing entries are then unspecified).
 */
int oracle_linear(const uint8_t* packed, const float* s_row,
                  const int32_t* rowsum, int64_t N, int64_t K, int64_t M,
                  const int8_t* q, int64_t ldq, const float* s_act,
                  const int32_t* z, int32_t* acc, float* y32, double* y64,
                  int64_t ldy) {
  const int64_t ld = oracle_row_bytes(K);
  const int64_t limit = (int64_t)1 << 24;
  int status = ORACLE_OK;
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t i = 0; i < N; ++i) {
      const uint8_t* row = packed + i * ld;
      int64_t sum = 0;
      int bad_code = 0;
      for (int64_t j = 0; j < K; ++j) {
        unsigned c = read_code(row, j);
        if (c == 3u) {
          bad_code = 1;
          continue;
        }
        int wv = (int)c - 1;
        /* add for +1, subtract for -1, skip for 0 */
        if (wv > 0) sum += q[m * ldq + j];
        else if (wv < 0) sum -= q[m * ldq + j];
      }
      int64_t a = sum - (int64_t)z[m] * (int64_t)rowsum[i];
      int err = bad_code ? ORACLE_INVALID_CODE
                         : ((a >= limit || a <= -limit) ? ORACLE_OVERFLOW : 0);
      if (err) {
#pragma omp critical
        if (status == ORACLE_OK) status = err;
      }
      if (acc) acc[m * ldy + i] = (int32_t)a;
      if (y64) y64[m * ldy + i] = (double)s_row[i] * (double)a * (double)s_act[m];
      if (y32) {
        float fa = (float)a;           /* exact: |a| < 2^24 */
        float t = s_row[i] * fa;       /* first rounding  */
        y32[m * ldy + i] = t * s_act[m]; /* second rounding */
      }
    }
  }
  return status;
}

/*
 * The same layer from the unpacked int8 weights (row stride ldw), by the
 * second formula  acc = sum_j w_ij * (q[m][j] - z[m]),  which uses neither
 * the packing nor the stored row sum.  Writes acc (int64) and y64.
 */
int oracle_linear_direct(const int8_t* w, int64_t ldw, const float* s_row,
                         int64_t N, int64_t K, int64_t M, const int8_t* q,
                         int64_t ldq, const float* s_act, const int32_t* z,
                         int64_t* acc, double* y64, int64_t ldy) {
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t i = 0; i < N; ++i) {
      int64_t sum = 0;
      for (int64_t j = 0; j < K; ++j)
        sum += (int64_t)w[i * ldw + j] * ((int64_t)q[m * ldq + j] - (int64_t)z[m]);
      if (acc) acc[m * ldy + i] = sum;
      if (y64) y64[m * ldy + i] = (double)s_row[i] * (double)sum * (double)s_act[m];
    }
  }
  return ORACLE_OK;
}
