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
#include <math.h>
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

/* Threads the parallel loops use from now on (the CPU baseline is timed
 * single-threaded and on every core); no effect on any result. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
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

/* ====================== neighbours of the ternary linear ======================
 *
 * Output head.  The token embedding and the output head stay int8 with one
 * scale per row; they are not ternary because no long sum hides their
 * rounding (Neutrino-1 8B model card, "Where the bytes live"; article,
 * "What's actually ternary").  Against the same per-token activations
 * (q, s_act, z) the head's logits are
 *
 *     rowsum_i  = sum_j W_ij
 *     acc[m][i] = sum_j W_ij * q[m][j]  -  z[m] * rowsum_i          (exact)
 *     y[m][i]   = (s_row[i] * (float)acc[m][i]) * s_act[m]
 *
 * Here |acc| can pass 2^24, so the conversion to float is itself rounded
 * (to nearest even): y32 is three roundings in that order.  The sum is
 * taken in int64 and must fit in int32 (else ORACLE_OVERFLOW).
 */
void oracle_head_rowsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw,
                        int32_t* rowsum) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    int64_t s = 0;
    for (int64_t j = 0; j < K; ++j) s += W[i * ldw + j];
    rowsum[i] = (int32_t)s;
  }
}

int oracle_head(const int8_t* W, int64_t ldw, const float* s_row,
                const int32_t* rowsum, int64_t N, int64_t K, int64_t M,
                const int8_t* q, int64_t ldq, const float* s_act,
                const int32_t* z, int32_t* acc, float* y32, double* y64,
                int64_t ldy) {
  int status = ORACLE_OK;
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t i = 0; i < N; ++i) {
      int64_t sum = 0;
      for (int64_t j = 0; j < K; ++j)
        sum += (int64_t)W[i * ldw + j] * (int64_t)q[m * ldq + j];
      const int64_t a = sum - (int64_t)rowsum[i] * (int64_t)z[m];
      if (a > INT32_MAX || a < INT32_MIN) {
#pragma omp critical
        if (status == ORACLE_OK) status = ORACLE_OVERFLOW;
      }
      if (acc) acc[m * ldy + i] = (int32_t)a;
      if (y64) y64[m * ldy + i] = (double)s_row[i] * (double)a * (double)s_act[m];
      if (y32) {
        float fa = (float)(int32_t)a;    /* rounded when |a| > 2^24 */
        float t = s_row[i] * fa;
        y32[m * ldy + i] = t * s_act[m];
      }
    }
  }
  return status;
}

/*
 * Activation quantiser.  The pages use int8 activations with a per-token
 * scale and zero point but never say how they are made, so this is the
 * plainest reading: asymmetric int8 over the token's range widened to
 * contain zero (so that zero is exact and |z| <= 128):
 *
 *     lo  = min(0, min_j x_j),   hi = max(0, max_j x_j)
 *     s   = (hi - lo) / 255          (fp32; s = 1 when hi == lo: all zeros)
 *     z   = -128 - rint(lo / s)
 *     q_j = clamp(rint(x_j / s) + z, -128, 127)
 *
 * Each division is one correctly rounded fp32 division; rint rounds half to
 * even.  Then s * (q_j - z) is within s / 2 of x_j.  x holds M rows of K
 * finite floats (row stride ldx); q is written with row stride ldq.
 */
void oracle_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx,
                         int8_t* q, int64_t ldq, float* s_act, int32_t* z) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const float* r = x + m * ldx;
    float lo = 0.0f, hi = 0.0f;
    for (int64_t j = 0; j < K; ++j) {
      if (r[j] < lo) lo = r[j];
      if (r[j] > hi) hi = r[j];
    }
    float s = (hi - lo) / 255.0f;
    if (s == 0.0f) s = 1.0f;
    const int32_t zm = -128 - (int32_t)rintf(lo / s);
    for (int64_t j = 0; j < K; ++j) {
      int32_t v = (int32_t)rintf(r[j] / s) + zm;
      if (v < -128) v = -128;
      if (v > 127) v = 127;
      q[m * ldq + j] = (int8_t)v;
    }
    s_act[m] = s;
    z[m] = zm;
  }
}

/*
 * Block-wise scales along K.  The article ("What's actually ternary") groups
 * a row's weights into fixed-size blocks along the input dimension, each with
 * its own higher-precision scale ("state times scale"); one scale per row is
 * the coarsest case.  With block size B, block b of a row holds columns
 * [b*B, min((b+1)*B, K)), nb = ceil(K / B) blocks, and
 *
 *     rowsum_b[i][b] = sum_{j in b} w_ij
 *     acc_b          = sum_{j in b} w_ij * q[m][j]  -  z[m] * rowsum_b[i][b]  (exact)
 *     y[m][i]        = (sum_{b = 0 .. nb-1} s_b[i][b] * acc_b) * s_act[m]
 *
 * y32 evaluates that in fp32 in the order written (each product rounded, a
 * running sum from b = 0 up, then the product with s_act); y64 in fp64; and
 * yabs = s_act * sum_b |s_b * acc_b| (fp64), which bounds the rounding of any
 * fp32 evaluation order: |y_fp32 - y| <= (nb + 1) * 2^-24 * yabs to first
 * order.  Metadata rows have stride nb.
 */
void oracle_block_rowsum(const int8_t* w, int64_t N, int64_t K, int64_t ldw,
                         int64_t B, int32_t* rowsum_b) {
  const int64_t nb = (K + B - 1) / B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    for (int64_t b = 0; b < nb; ++b) {
      int64_t s = 0;
      for (int64_t j = b * B; j < K && j < (b + 1) * B; ++j) s += w[i * ldw + j];
      rowsum_b[i * nb + b] = (int32_t)s;
    }
  }
}

int oracle_linear_blocked(const uint8_t* packed, const float* s_b,
                          const int32_t* rowsum_b, int64_t N, int64_t K,
                          int64_t B, int64_t M, const int8_t* q, int64_t ldq,
                          const float* s_act, const int32_t* z, float* y32,
                          double* y64, double* yabs, int64_t ldy) {
  const int64_t ld = oracle_row_bytes(K);
  const int64_t nb = (K + B - 1) / B;
  const int64_t limit = (int64_t)1 << 24;
  int status = ORACLE_OK;
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t i = 0; i < N; ++i) {
      const uint8_t* row = packed + i * ld;
      float run = 0.0f;
      double exact = 0.0, mag = 0.0;
      int err = 0;
      for (int64_t b = 0; b < nb; ++b) {
        int64_t sum = 0;
        for (int64_t j = b * B; j < K && j < (b + 1) * B; ++j) {
          unsigned c = read_code(row, j);
          if (c == 3u) {
            err = ORACLE_INVALID_CODE;
            continue;
          }
          sum += (int64_t)((int)c - 1) * q[m * ldq + j]; /* add, subtract or skip */
        }
        const int64_t a = sum - (int64_t)z[m] * (int64_t)rowsum_b[i * nb + b];
        if (!err && (a >= limit || a <= -limit)) err = ORACLE_OVERFLOW;
        const float sb = s_b[i * nb + b];
        run = run + sb * (float)a; /* one rounding for the product, one for the sum */
        exact += (double)sb * (double)a;
        mag += fabs((double)sb * (double)a);
      }
      if (err) {
#pragma omp critical
        if (status == ORACLE_OK) status = err;
      }
      if (y32) y32[m * ldy + i] = run * s_act[m];
      if (y64) y64[m * ldy + i] = exact * (double)s_act[m];
      if (yabs) yabs[m * ldy + i] = mag * fabs((double)s_act[m]);
    }
  }
  return status;
}

/* ====================== 1.6-bit rows: five weights per byte ======================
 *
 * Three states hold log2(3), about 1.58 bits, per weight (article
 * "Neutrino-1: quantization is a training decision, not a deployment one",
 * "Where the bytes go"), so 2-bit fields leave a fifth of every row unused.
 * This second layout (this project's own, like the 2-bit one) stores five
 * weights per byte:
 *  - a byte's five weights, as digits d = w + 1 in {0, 1, 2}, form the
 *    base-3 number v = 81 d0 + 27 d1 + 9 d2 + 3 d3 + d4  (0 <= v <= 242);
 *  - the byte stored is b = ceil(256 v / 243); it is read back as
 *    v = floor(243 b / 256), which every byte value decodes to, so no byte
 *    is invalid (13 values are simply never written);
 *  - a row takes row_bytes5(K) = 16 * ceil(K / 80) bytes (80 weights per
 *    16-byte chunk), so rows start 16-byte aligned;
 *  - weight j of a row is digit (j % 20) / 4 of byte 4 * (j / 20) + j % 4:
 *    a 4-byte word holds 20 weights, its digit i of bytes 0..3 being
 *    weights 4i..4i+3 of the word;
 *  - columns j >= K are padding and hold weight 0, so a byte made only of
 *    padding holds v = 121 and reads 0x80.
 * The layer itself is the one above: the same acc, y32 and y64.
 */
int64_t oracle_row_bytes5(int64_t K) { return 16 * ((K + 79) / 80); }

static const unsigned kPlace5[5] = {81u, 27u, 9u, 3u, 1u}; /* value of digit i */

static int64_t byte5_of(int64_t j) { return 4 * (j / 20) + j % 4; }
static int digit5_of(int64_t j) { return (int)((j % 20) / 4); }

/* The weight in column j of a 1.6-bit row. */
static int read_weight5(const uint8_t* row, int64_t j) {
  unsigned v = (243u * row[byte5_of(j)]) / 256u;
  return (int)((v / kPlace5[digit5_of(j)]) % 3u) - 1;
}

/*
 * Pack an N x K int8 matrix (row stride ldw elements) with entries in
 * {-1, 0, +1} into 1.6-bit rows; rowsum[i] = sum_j w_ij.  Entries outside
 * {-1, 0, +1} are counted (the return value), stored as 0 and left out of
 * the row sum.
 */
int64_t oracle_pack5(const int8_t* w, int64_t N, int64_t K, int64_t ldw,
                     uint8_t* packed, int32_t* rowsum) {
  const int64_t ld = oracle_row_bytes5(K);
  int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t i = 0; i < N; ++i) {
    uint8_t* row = packed + i * ld;
    int64_t sum = 0;
    for (int64_t p = 0; p < ld; ++p) {
      unsigned v = 0;
      for (int d = 0; d < 5; ++d) {
        /* the column whose weight is digit d of byte p */
        int64_t j = 20 * (p / 4) + 4 * d + p % 4;
        int wv = 0;
        if (j < K) {
          wv = w[i * ldw + j];
          if (wv < -1 || wv > 1) {
            ++bad;
            wv = 0;
          }
          sum += wv;
        }
        v += (unsigned)(wv + 1) * kPlace5[d];
      }
      row[p] = (uint8_t)((256u * v + 242u) / 243u); /* ceil(256 v / 243) */
    }
    rowsum[i] = (int32_t)sum;
  }
  return bad;
}

/* 1.6-bit rows back to int8 weights (row stride ldw elements). */
void oracle_unpack5(const uint8_t* packed, int64_t N, int64_t K, int8_t* w,
                    int64_t ldw) {
  const int64_t ld = oracle_row_bytes5(K);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i)
    for (int64_t j = 0; j < K; ++j) w[i * ldw + j] = (int8_t)read_weight5(packed + i * ld, j);
}

/*
 * The linear layer on 1.6-bit rows: the same outputs, status and rounding
 * as oracle_linear (acc exact in int64 and within +-2^24; y32 two rounded
 * products (s_row * acc) * s_act).
 */
int oracle_linear5(const uint8_t* packed, const float* s_row,
                   const int32_t* rowsum, int64_t N, int64_t K, int64_t M,
                   const int8_t* q, int64_t ldq, const float* s_act,
                   const int32_t* z, int32_t* acc, float* y32, double* y64,
                   int64_t ldy) {
  const int64_t ld = oracle_row_bytes5(K);
  const int64_t limit = (int64_t)1 << 24;
  int status = ORACLE_OK;
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t i = 0; i < N; ++i) {
      const uint8_t* row = packed + i * ld;
      int64_t dot = 0;
      for (int64_t j = 0; j < K; ++j)
        dot += (int64_t)read_weight5(row, j) * (int64_t)q[m * ldq + j];
      const int64_t a = dot - (int64_t)rowsum[i] * (int64_t)z[m];
      if (a >= limit || a <= -limit) {
#pragma omp critical
        if (status == ORACLE_OK) status = ORACLE_OVERFLOW;
      }
      if (acc) acc[m * ldy + i] = (int32_t)a;
      if (y64) y64[m * ldy + i] = (double)s_row[i] * (double)a * (double)s_act[m];
      if (y32) {
        float prod = s_row[i] * (float)a; /* exact conversion, then round */
        y32[m * ldy + i] = prod * s_act[m];
      }
    }
  }
  return status;
}

/* ====================== weight quantiser ======================
 *
 * The article ("What's actually ternary") states how a weight becomes a
 * state: weights are grouped into fixed-size blocks along the input
 * dimension, the block's scale is the mean absolute value of its weights,
 * and each weight's state is the rounded, clamped ratio w / scale; one block
 * for the whole row is the coarsest case.  The pages fix no precision or
 * order for the mean, so it is defined here:
 *
 *     sum  = |w_0| + |w_1| + ... + |w_(n-1)|   in fp64, in column order
 *     s_b  = fp32(sum / n)                     (n = the block's columns; the
 *                                               last block may be shorter)
 *     state_j = rint(clamp(w_j / s_b, -1, 1))  (fp32 division; rint rounds
 *                                               half to even)
 *
 * A block of zeros has s_b = 0 and all states 0.  W holds N rows of K finite
 * floats (row stride ldw); the states go to t (row stride ldt) and the
 * scales to s_b (N x nb, nb = ceil(K / B)).
 */
void oracle_quantize_weights(const float* W, int64_t N, int64_t K, int64_t ldw, int64_t B,
                             int8_t* t, int64_t ldt, float* s_b) {
  const int64_t nb = (K + B - 1) / B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    const float* row = W + i * ldw;
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t j0 = b * B, j1 = (j0 + B < K) ? j0 + B : K;
      double total = 0.0;
      for (int64_t j = j0; j < j1; ++j) total += fabs((double)row[j]);
      const float scale = (float)(total / (double)(j1 - j0));
      s_b[i * nb + b] = scale;
      for (int64_t j = j0; j < j1; ++j) {
        float state = 0.0f;
        if (scale > 0.0f) {
          float ratio = row[j] / scale;
          if (ratio > 1.0f) ratio = 1.0f;
          if (ratio < -1.0f) ratio = -1.0f;
          state = rintf(ratio);
        }
        t[i * ldt + j] = (int8_t)state;
      }
    }
  }
}

/*
 * The gated feed-forward activation.  The model card ("Neutrino-1 8B",
 * "Architecture") gives each layer a gated SwiGLU feed-forward of three
 * linears; the pages do not write the gate out, so this takes the plainest
 * reading, the SiLU-gated product of the gate and up projections' outputs:
 *
 *     h_j = silu(g_j) * u_j,      silu(x) = x / (1 + e^(-x))
 *
 * h is the down projection's input, quantised per token like any other
 * activation.  A correctly rounded exp is not available on both sides, so
 * the fp32 evaluation is fixed step by step (round to nearest even, no
 * fused multiply-add) and the GPU follows the same steps:
 *
 *   e = exp32(min(max(-g, -87), 100))     (e^-87 is still a normal float, and
 *                                          below it 1 + e rounds to 1 anyway;
 *                                          past 88.7 exp32 overflows to +inf
 *                                          and s below is -0)
 *   s = g / (1 + e)                       (one correctly rounded division)
 *   h = s * u
 *
 * exp32(x): Cody and Waite's argument reduction x = k ln2 + r with
 *   k = rint(x * log2(e)),  r = (x - k * L1) - k * L2,
 * L1 = 0.693145751953125 (ln 2 to 15 significant bits, so k * L1 is exact
 * for |k| <= 256) and L2 = ln 2 - L1 rounded to fp32, then the
 * Taylor series of e^r through r^7 by Horner's rule with coefficients
 * 1/n! rounded to fp32, scaled by 2^k.  |r| <= ln 2 / 2 makes the truncation
 * below 6e-9 relative; oracle_exp32_ulp tests bound the whole error.
 */
static float exp32(float x) {
  const double ln2 = 0.69314718055994530942;
  const float kLog2e = (float)(1.0 / ln2);
  const float kL1 = 0.693145751953125f;
  const float kL2 = (float)(ln2 - 0.693145751953125);
  const float k = rintf(x * kLog2e);
  const float r = (x - k * kL1) - k * kL2;
  /* 1/n! for n = 7 .. 2, then 1, 1 */
  const float c7 = (float)(1.0 / 5040.0), c6 = (float)(1.0 / 720.0), c5 = (float)(1.0 / 120.0);
  const float c4 = (float)(1.0 / 24.0), c3 = (float)(1.0 / 6.0), c2 = 0.5f;
  float p = c7;
  p = p * r + c6;
  p = p * r + c5;
  p = p * r + c4;
  p = p * r + c3;
  p = p * r + c2;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return ldexpf(p, (int)k);
}

void oracle_exp32(const float* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = exp32(x[i]);
}

/* h = silu(g) * u, element by element (M x K with row strides ldg = ldu). */
void oracle_swiglu(const float* g, const float* u, int64_t M, int64_t K, int64_t ld, float* h) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t j = 0; j < K; ++j) {
      const float gv = g[m * ld + j];
      float t = -gv;
      if (t < -87.0f) t = -87.0f;
      if (t > 100.0f) t = 100.0f;
      const float e = exp32(t);
      const float s = gv / (1.0f + e);
      h[m * K + j] = s * u[m * ld + j];
    }
  }
}
