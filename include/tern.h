/*
 * tern.h -- C ABI of the ternary packed-bit GEMV / small-M GEMM library for
 * AMD MI355X (gfx950).
 *
 * The operation.  Every transformer linear holds weights in three states,
 * minus, zero and plus (article "Neutrino-1: quantization is a training
 * decision, not a deployment one", intro and "What's actually ternary").
 * The weights stay bit-packed at rest and are decoded inside the matrix
 * kernels, with nothing in the decode path stored as fp16 or fp32 weight
 * material (Neutrino-1 8B model card, "Overview"; wpnews item "Neutrino-1 8B:
 * 763 tok/s ...", "Not Quantization -- Trained Ternary").  A weight is a
 * state times a higher-precision scale, and signed accumulation replaces
 * multiplies (article, "What's actually ternary" and "The take").  Per-row
 * metadata holds the row's scale and row sum (model card, "Where the bytes
 * live").  With activations given per token as int8 q, an fp32 scale s_act
 * and an int32 zero point z (x_j = s_act * (q_j - z)), every entry point
 * computes, for token m and output row i,
 *
 *     acc[m][i] = sum_j w_ij * q[m][j]  -  z[m] * rowsum[i]      (int32, exact)
 *     y[m][i]   = (s_row[i] * (float)acc[m][i]) * s_act[m]       (fp32, RNE, in
 *                                                                  this order)
 *
 * which is sum_j (s_row[i] w_ij) * (s_act[m] (q[m][j] - z[m])) up to the two
 * fp32 roundings.  The stored row sum turns the zero point into one
 * multiply-subtract per output.
 *
 * Packed layout (the pages call their own format proprietary and
 * unpublished -- wiki entry "Neutrino-1", "What is actually new here" -- so
 * this one is the library's own):
 *   - code(w) = w + 1: -1 -> 00, 0 -> 01, +1 -> 10; 11 is invalid;
 *   - row i starts at packed + i * tern_row_bytes(K); a row is
 *     16 * ceil(K / 64) bytes, so every row is 16-byte aligned;
 *   - weight j sits in the little-endian 32-bit word j / 16 of its row, at
 *     bit 8 * (j % 4) + 2 * ((j % 16) / 4); hence (word >> 2k) & 0x03030303
 *     holds the codes of weights 4k .. 4k+3 of that word in byte order;
 *   - columns K <= j < 4 * row_bytes are padding with code 01 (weight 0).
 *   - metadata are separate arrays: float s_row[N], int32 rowsum[N].
 *
 * Conventions common to every call:
 *   - Pointers marked "device" are device memory of the current HIP device;
 *     the caller allocates and owns every buffer (including the stack
 *     workspace).  The library allocates no device memory and keeps no global
 *     state; calls are reentrant.
 *   - Every call enqueues on `stream` and returns without synchronising
 *     (tern_linear_stack_prepare is the one exception, see there).  Argument
 *     errors are returned before anything is enqueued.  A failed launch
 *     returns TERN_ERR_HIP (the HIP code is kept per thread, see
 *     tern_last_hip_error); faults during execution surface at the caller's
 *     next synchronisation.
 *   - Sizes are int64.  N == 0 or M == 0 is an empty problem: nothing is
 *     enqueued and TERN_OK is returned.  K must be >= 1.
 *   - Alignment: `packed`, `q` and each q row (ldq) must be 16-byte aligned;
 *     y and acc 4-byte aligned; otherwise TERN_ERR_ALIGNMENT.
 *   - Outputs must not overlap inputs.
 *   - Range: |z| <= 255 is a precondition (z is not read on the host).  Then
 *     |acc| <= K * 383, and K > TERN_MAX_K is rejected with TERN_ERR_RANGE so
 *     that no int32 intermediate can wrap.  The fp32 conversion of acc is
 *     exact while |acc| < 2^24 (always so for K <= 43,804).
 *   - Packed input holding the invalid code 11 gives unspecified outputs
 *     (no fault); tern_validate finds such data.
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TERN_OK = 0,
  TERN_ERR_INVALID_ARG = 1, /* null pointer, K < 1, negative size, bad stride */
  TERN_ERR_ALIGNMENT = 2,   /* see "Alignment" above */
  TERN_ERR_RANGE = 3,       /* K > TERN_MAX_K, or a size beyond int32 rows */
  TERN_ERR_UNSUPPORTED = 4, /* a path hint the shape cannot take */
  TERN_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned */
  TERN_ERR_HIP = 6,         /* a HIP runtime call failed */
  TERN_ERR_TIMEOUT = 7      /* see tern_linear_stack_status */
} tern_status;

/* Path hints for tern_gemm_smallM and tern_linear_stack_prepare. */
enum {
  TERN_PATH_AUTO = 0, /* M == 1: VALU GEMV; M >= 2: MFMA int8 */
  TERN_PATH_VALU = 1, /* VALU dot4 path (M <= TERN_VALU_MAX_M) */
  TERN_PATH_MFMA = 2  /* MFMA int8 path (any M) */
};

#define TERN_MAX_K 5600000
#define TERN_VALU_MAX_M 8
/* Rows tern_pack, tern_unpack and tern_validate take in one call (one
 * 64-lane wave per row, and a launch counts at most 2^32 - 1 lanes). */
#define TERN_MAX_ROWS_PACK 67108860

/* Bytes of one packed row: 16 * ceil(K / 64); 0 for K < 1. */
int64_t tern_row_bytes(int64_t K);

/*
 * tern_pack -- load-time packing of an int8 ternary matrix (the weights are
 * packed once and stay packed at rest; no decode pass at load: Fermion
 * Research models page, "Neutrino-1 0.6B").
 *   w         device, N x K int8, row stride ldw >= K elements, values in
 *             {-1, 0, +1};
 *   packed    device, N * tern_row_bytes(K) bytes, 16-byte aligned (written);
 *   rowsum    device, N int32 (written): sum_j w_ij;
 *   bad_count device, one int32 or NULL; when given it is set to the number
 *             of entries outside {-1, 0, +1} (each is stored as weight 0 and
 *             left out of the row sum).
 */
int tern_pack(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
              int32_t* rowsum, int32_t* bad_count, hipStream_t stream);

/*
 * tern_unpack -- packed rows back to int8 weights (a test aid).
 *   w  device, N x K int8 with row stride ldw >= K (written); a field with the
 *      invalid code 11 is written as 0.
 */
int tern_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, int64_t ldw,
                hipStream_t stream);

/*
 * tern_validate -- checks packed rows.
 *   counts  device, two int32 (written): counts[0] = fields with code 11 among
 *           the real columns, counts[1] = padding fields that are not 01.
 */
int tern_validate(const uint8_t* packed, int64_t N, int64_t K, int32_t* counts,
                  hipStream_t stream);

/*
 * tern_gemv -- one token (M = 1).
 *   packed, s_row, rowsum  device: the packed N x K matrix and its metadata;
 *   q                      device, K int8 (16-byte aligned);
 *   s_act, z               device, one float / one int32;
 *   y                      device, N floats (written);
 *   acc                    device, N int32 (written) or NULL.
 */
int tern_gemv(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
              int64_t K, const int8_t* q, const float* s_act, const int32_t* z, float* y,
              int32_t* acc, hipStream_t stream);

/*
 * tern_gemm_smallM -- M tokens against the same packed weights (the batched
 * verify pass of drafted decoding and prefill-sized batches: wiki entry
 * "Neutrino-1", "What is actually new here"; models page "Neutrino-1 0.6B").
 *   q      device, M x K int8, row stride ldq >= K (multiple of 16 when M > 1);
 *   s_act  device, M floats;  z  device, M int32;
 *   y      device, M x N floats, row stride ldy >= N (written);
 *   acc    device, M x N int32 with the same stride ldy (written) or NULL;
 *   path   TERN_PATH_AUTO, _VALU (M <= TERN_VALU_MAX_M) or _MFMA;
 *          TERN_ERR_UNSUPPORTED for a hint the shape cannot take.
 */
int tern_gemm_smallM(const uint8_t* packed, const float* s_row, const int32_t* rowsum,
                     int64_t N, int64_t K, int64_t M, const int8_t* q, int64_t ldq,
                     const float* s_act, const int32_t* z, float* y, int64_t ldy,
                     int32_t* acc, int path, hipStream_t stream);

/*
 * A stack of L independent linears evaluated by one kernel launch over a
 * schedule made once by tern_linear_stack_prepare (the
 * 8B carries 252 such linears, seven per decoder layer, and the 0.6B 196:
 * article "What's actually ternary"; models page "The family").  Every linear
 * sees the same token count M; each has its own shapes and buffers (all
 * pointers device, same meaning and rules as in tern_gemm_smallM).
 */
typedef struct {
  const uint8_t* packed;
  const float* s_row;
  const int32_t* rowsum;
  int64_t N, K;
  const int8_t* q;
  int64_t ldq;
  const float* s_act;
  const int32_t* z;
  float* y;
  int64_t ldy;
  int32_t* acc; /* may be NULL */
  /* Block-wise scales along K (see "Block-wise scales" below): block = 0
   * keeps one scale per row (s_row, rowsum).  block = B > 0 (a power of two
   * in [64, 4096]; a multiple of 512 on the MFMA path) gives row i
   * the scale s_block[i * nb + b] and row sum rowsum_block[i * nb + b] of
   * each block b of B columns (nb = ceil(K / B); from tern_block_rowsum);
   * s_row and rowsum are then not read and may be NULL.  acc, when given,
   * receives sum_b acc_b. */
  int64_t block;
  const float* s_block;
  const int32_t* rowsum_block;
  /* fp32 input quantised by the launch itself (NULL: q, s_act and z are
   * the caller's, ready before the launch).  x holds M rows of K finite
   * floats (row stride ldx >= K, 4-byte aligned); the launch writes q (row
   * stride ldq; columns < K), s_act and z from it exactly as
   * tern_quantize_act does, before any linear of the launch reads them.
   * Each distinct q buffer is quantised once: linears naming the same q
   * must name the same x, ldx, K, ldq, s_act and z (and every linear
   * naming such a q reads the quantised values, with or without x);
   * otherwise TERN_ERR_INVALID_ARG.  q, s_act and z are outputs of the
   * launch, complete when it is; x (and x_up) must not overlap them. */
  const float* x;
  int64_t ldx;
  /* With x_up (NULL: the input is x itself) the input the launch quantises
   * is the gated feed-forward activation of the model card's SwiGLU layers
   * ("Neutrino-1 8B", "Architecture"), h = silu(x) * x_up element by element
   * (x the gate projection's output, x_up the up projection's, both M x K
   * with row stride ldx, 4-byte aligned), in these fp32 steps (round to
   * nearest even, no fused multiply-add):
   *     t = min(max(-x_j, -87), 100)
   *     e = exp32(t): k = rint(t * fp32(1/ln 2)), r = (t - k * 0.693145751953125)
   *                   - k * fp32(ln 2 - 0.693145751953125), then the Taylor
   *                   series of e^r through r^7 (coefficients 1/n! rounded to
   *                   fp32) by Horner's rule, times 2^k (+inf past 88.7)
   *     h_j = (x_j / (1 + e)) * x_up_j   (one correctly rounded division)
   * so a down projection reads its input straight from the gate and up
   * outputs of an earlier launch, with the gate and the quantisation done in
   * its own launch.  Linears naming the same q must name the same x_up. */
  const float* x_up;
} tern_linear_desc;

/* Host-side handle filled by tern_linear_stack_prepare (plain data; copy it
 * freely; it stays valid while the workspace and the buffers live). */
typedef struct {
  void* workspace;
  int64_t workspace_bytes;
  int32_t L, M;
  int32_t path;      /* the path chosen */
  int32_t grid;      /* workgroups launched */
  int32_t block;     /* threads per workgroup */
  int32_t workers;   /* waves with a schedule entry */
  int32_t segments;  /* schedule entries */
  int32_t kernel;    /* internal kernel selector */
  int64_t bytes;     /* algorithmic bytes one launch moves (see below) */
  int32_t splits;    /* linears split along K (then tern_linear_stack enqueues
                        a fill kernel and a finishing kernel around the main
                        one; see tern_linear_stack_prepare) */
  int32_t restages;  /* activation windows (4,096 columns of the M tokens)
                        the workgroups of one launch load into LDS (the
                        M = 2..16 window kernels; 0 otherwise): linears that
                        read the same activation buffers and follow each other
                        in a workgroup's run share one load */
} tern_stack_plan;

/* Upper bound of the workspace tern_linear_stack_prepare needs for L linears
 * at M tokens on the current device; 0 on bad arguments. */
int64_t tern_linear_stack_workspace_bytes(int64_t L, int64_t M);

/*
 * tern_linear_stack_prepare -- validates every descriptor, builds the static
 * schedule (contiguous row ranges balanced by packed bytes over all waves of
 * the launch) and copies descriptors and schedule into `workspace`
 * (device, >= tern_linear_stack_workspace_bytes(L, M) bytes, 256-byte
 * aligned).  Enqueues the copy on `stream` and synchronises that stream
 * before returning (a one-time set-up step).  Fills *plan.
 * plan->bytes = sum over linears of N*row_bytes(K) + 8*N + M*K + 8*M + 4*M*N.
 * On the MFMA path (M >= 2), a stack too small to spread its longest units
 * (their cost over 3x a worker's share: e.g. one 8B layer, whose K = 12,288
 * projection walks three 4,096-column windows per unit) has such linears
 * (K a multiple of 64, at most 4 windows) split along K: their windows run
 * as separate work, the exact int32 partial sums are added into y (used as
 * int32 scratch), and a finishing kernel writes y and acc -- the results
 * are the same bits.  plan->splits counts them.  At 9..16 tokens such a
 * small stack takes the prefill GEMM's kernel instead (the same test on the
 * units of the kernel it would otherwise take); the results are the same
 * bits either way.
 * Outputs of linears that return y only (acc NULL) may be held on chip by
 * the kernel and written when its work ends: as always, y is complete once
 * the launch has completed on the stream, and no other work may read or
 * write it in between.
 * A block-scaled linear (block > 0) needs K a multiple of 64; on the VALU
 * path (M <= TERN_VALU_MAX_M) K <= 16,384, on the MFMA path (M <= 16) B a
 * multiple of 512: otherwise TERN_ERR_UNSUPPORTED.  On the automatic path a
 * stack of 2..TERN_VALU_MAX_M tokens holding a linear whose B is not a
 * multiple of 512 takes the VALU path, which runs every linear of it token
 * by token through the one-token kernels (each token's y the bits of the
 * one-token result; the rows are re-read from the L2, at M times the vector
 * ALU work of one token).  plan->bytes counts 8 bytes of block metadata per
 * row and block in place of the 8 per row.
 */
int tern_linear_stack_prepare(const tern_linear_desc* descs, int64_t L, int64_t M, int path,
                              void* workspace, int64_t workspace_bytes,
                              tern_stack_plan* plan, hipStream_t stream);

/* tern_linear_stack -- one launch over the prepared stack (three when
 * plan->splits > 0: clear, main, finish).  Launches on one plan (or on
 * plans sharing a workspace) must not overlap: enqueue them on one stream,
 * or order them. */
int tern_linear_stack(const tern_stack_plan* plan, hipStream_t stream);

/*
 * Fused activation quantisation (descriptors with x): inside the launch,
 * before the linears, the launch's workgroups claim token rows of the
 * distinct inputs from a counter in the workspace, quantise them and flag
 * each one finished; a wave about to read a quantised input waits for its
 * rows' flags.  Every row is claimed by a workgroup already running, so the
 * waits end; they are bounded all the same (about a second), and a wait
 * that gives up is recorded in the workspace.  plan->bytes adds, per
 * distinct input, 4*M*K bytes read, M*K + 8*M written.
 * tern_linear_stack_status -- synchronises `stream` and returns
 * TERN_ERR_TIMEOUT if any launch of the plan since its prepare gave up such
 * a wait (its outputs are then not to be used), else TERN_OK.
 */
int tern_linear_stack_status(const tern_stack_plan* plan, hipStream_t stream);

/*
 * tern_linear_stack_prepare_static -- tern_linear_stack_prepare for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The schedule goes to a
 * workspace the library holds instead of a caller's: a file-scope device
 * array of TERN_STATIC_WORKSPACE_BYTES, one on each device the library runs
 * on, held until the process ends.  Arguments, plan and results are those of
 * tern_linear_stack_prepare without the workspace pair; TERN_ERR_RANGE when
 * the stack's schedule needs more than TERN_STATIC_WORKSPACE_BYTES (the
 * full 8B-shaped stack of 252 linears needs about 1.2 MB at M = 1).  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine): like the other prepare it copies the schedule in and
 * synchronises `stream`.  Every static plan of a device shares that
 * device's array, which keeps the last prepare's schedule: preparing another
 * static plan replaces it (an earlier static plan must not be launched
 * again), and a prepare that overlaps a launch of a static plan on the same
 * device races with it.
 */
#define TERN_STATIC_WORKSPACE_BYTES 4194304
int tern_linear_stack_prepare_static(const tern_linear_desc* descs, int64_t L, int64_t M, int path,
                                     tern_stack_plan* plan, hipStream_t stream);

/*
 * Block-wise scales along K.  The article ("What's actually ternary")
 * groups each row's weights into fixed-size blocks along the input
 * dimension, each block with its own higher-precision scale; one scale per
 * row (the calls above) is the coarsest case.  With block size B, block b of
 * a row holds columns [b*B, min((b+1)*B, K)), nb = ceil(K / B), and for one
 * token
 *     acc_b = sum_{j in b} w_ij q_j - z * rowsum_b[i][b]          (int32, exact)
 *     y_i   = (sum_b s_b[i][b] * acc_b) * s_act                    (fp32)
 * The fp32 sum over blocks is taken in block order from +0, each product
 * s_b * (float)acc_b and each partial sum rounded to nearest (the order the
 * definition is written in), so y has the bits of that left-to-right
 * evaluation.
 * Weights use the packed layout above; B is a power of two in [64, 4096]
 * and K <= TERN_BLOCK_MAX_K.  Metadata rows have stride nb.
 */
#define TERN_BLOCK_MAX_K 16384

/*
 * tern_block_rowsum -- load-time block row sums from packed weights.
 *   rowsum_b  device, N x nb int32 (written).
 */
int tern_block_rowsum(const uint8_t* packed, int64_t N, int64_t K, int64_t B, int32_t* rowsum_b,
                      hipStream_t stream);

/*
 * tern_gemv_blocked -- one token against block-scaled packed weights.
 *   packed    device, N rows of tern_row_bytes(K) bytes, 16-byte aligned;
 *   s_b       device, N x nb floats;  rowsum_b  device, N x nb int32;
 *   q         device, K int8 (16-byte aligned);  s_act, z  device, one each;
 *   y         device, N floats (written).
 */
int tern_gemv_blocked(const uint8_t* packed, const float* s_b, const int32_t* rowsum_b, int64_t N,
                      int64_t K, int64_t B, const int8_t* q, const float* s_act, const int32_t* z,
                      float* y, hipStream_t stream);

/*
 * tern_quantize_act -- per-token asymmetric int8 activations for the calls
 * above (they take x_j = s_act * (q_j - z)).  The pages do not describe the
 * activation quantiser; this is the plainest reading, the token's range
 * widened to contain zero, in 255 steps:
 *     lo = min(0, min_j x_j),  hi = max(0, max_j x_j)
 *     s_act = (hi - lo) / 255   (1 for an all-zero token)
 *     z = -128 - rint(lo / s_act),  q_j = clamp(rint(x_j / s_act) + z, -128, 127)
 * with correctly rounded fp32 divisions and rint rounding half to even, so
 * zero is exact, |z| <= 128 and s_act * (q_j - z) is within s_act / 2 of x_j.
 *   x      device, M x K finite floats, row stride ldx >= K;
 *   q      device, M x K int8, row stride ldq >= K (columns < K written);
 *   s_act  device, M floats (written);  z  device, M int32 (written).
 */
int tern_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                      float* s_act, int32_t* z, hipStream_t stream);

/*
 * tern_quantize_weights -- load-time ternarisation of fp32 weights with one
 * scale per block of B columns along K (article "What's actually ternary":
 * the block's scale is its mean absolute weight, the state of a weight its
 * rounded, clamped ratio to that scale; B >= K gives one scale per row):
 *     s_b[i][b] = fp32( (sum of |W_ij| over the block, in fp64, in column
 *                       order) / (the block's column count) )
 *     w_ij      = rint(clamp(W_ij / s_b[i][b], -1, 1))   (fp32 division,
 *                                                          half to even)
 * A block of zeros gets scale 0 and states 0.  The states pack with
 * tern_pack (and tern_block_rowsum) for tern_gemv_blocked.
 *   W    device, N x K finite floats, row stride ldw >= K, 4-byte aligned;
 *   w    device, N x K int8 states, row stride ldt >= K (written);
 *   s_b  device, N x ceil(K / B) floats, row stride ceil(K / B) (written).
 */
int tern_quantize_weights(const float* W, int64_t N, int64_t K, int64_t ldw, int64_t B, int8_t* w,
                          int64_t ldt, float* s_b, hipStream_t stream);

/*
 * The int8 output head.  The token embedding and the output head are not
 * ternary: they stay int8 with one scale per row (Neutrino-1 8B model card,
 * "Where the bytes live"), because nothing sums their rounding errors away
 * and the head decides tokens by small logit margins (article, "What's
 * actually ternary").  Against the same per-token activations as the
 * ternary calls the logits are
 *
 *     acc[m][i] = sum_j W_ij * q[m][j]  -  z[m] * rowsum[i]        (int32, exact)
 *     y[m][i]   = (s_row[i] * (float)acc[m][i]) * s_act[m]         (fp32, RNE, in
 *                                                                   this order)
 *
 * with rowsum[i] = sum_j W_ij from tern_head_rowsum.  |acc| may pass 2^24,
 * so the conversion to float rounds too.  K <= TERN_HEAD_MAX_K keeps every
 * intermediate inside int32 for |z| <= 255.
 */
#define TERN_HEAD_MAX_M 8
#define TERN_HEAD_MAX_K 43803

/*
 * tern_head_rowsum -- load-time row sums of an int8 matrix.
 *   W       device, N x K int8, row stride ldw >= K elements;
 *   rowsum  device, N int32 (written).
 */
int tern_head_rowsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw, int32_t* rowsum,
                     hipStream_t stream);

/*
 * tern_head_gemv -- logits of M <= TERN_HEAD_MAX_M tokens (M = 1 for plain
 * decode, up to 8 for a drafted-and-verified step).
 *   W       device, N x K int8, 16-byte aligned, row stride ldw >= K a
 *           multiple of 16 (at most 2^28);
 *   s_row   device, N floats;  rowsum  device, N int32 (tern_head_rowsum);
 *   q       device, M x K int8, 16-byte aligned, row stride ldq >= K (a
 *           multiple of 16 when M > 1);  s_act, z  device, M each;
 *   y       device, M x N floats, row stride ldy >= N (written);
 *   acc     device, M x N int32 with stride ldy (written) or NULL.
 * M > TERN_HEAD_MAX_M gives TERN_ERR_UNSUPPORTED; a K whose activations do
 * not fit the kernel's 64 KB of staging (about 7,900 columns at M > 4,
 * 15,900 at M = 3..4) gives TERN_ERR_RANGE.
 */
int tern_head_gemv(const int8_t* W, const float* s_row, const int32_t* rowsum, int64_t N, int64_t K,
                   int64_t ldw, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                   const int32_t* z, float* y, int64_t ldy, int32_t* acc, hipStream_t stream);

/*
 * The 1.6-bit layout.  Three states carry about 1.58 bits per weight
 * (article "Neutrino-1: quantization is a training decision, not a
 * deployment one", "Where the bytes go"), so this second layout (also the
 * library's own) packs five weights per byte, 20 % fewer bytes per row:
 *   - a byte's five weights, as digits d = w + 1 (most significant first),
 *     form v = 81 d0 + 27 d1 + 9 d2 + 3 d3 + d4, stored as
 *     b = ceil(256 v / 243) (read back as v = floor(243 b / 256); every byte
 *     value decodes, 13 of them are never written);
 *   - row i starts at packed5 + i * tern_row_bytes5(K); a row is
 *     16 * ceil(K / 80) bytes (80 weights per 16-byte chunk);
 *   - weight j is digit (j % 20) / 4 of byte 4 * (j / 20) + j % 4 of its row;
 *   - columns j >= K are padding with weight 0 (a padding-only byte is 0x80);
 *   - metadata as for the 2-bit layout: float s_row[N], int32 rowsum[N].
 * The layer computed is the one at the top of this file.  Decoding costs
 * about 1.3 VALU operations per weight here against 0.5 for 2-bit rows.
 */
#define TERN5_MAX_K 65520

/* Bytes of one 1.6-bit row: 16 * ceil(K / 80); 0 for K < 1. */
int64_t tern_row_bytes5(int64_t K);

/*
 * tern_pack5 -- load-time packing of an int8 ternary matrix into 1.6-bit
 * rows; arguments as tern_pack, with rows of tern_row_bytes5(K) bytes and
 * K <= TERN5_MAX_K.
 */
int tern_pack5(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed5,
               int32_t* rowsum, int32_t* bad_count, hipStream_t stream);

/*
 * tern_gemv5 -- one token (M = 1) against 1.6-bit rows; arguments as
 * tern_gemv, with packed5 (16-byte aligned) holding N rows of
 * tern_row_bytes5(K) bytes and 1 <= K <= TERN5_MAX_K.  rowsum must be the
 * row sums of the packed weights (tern_pack5 writes them): the kernel takes
 * the zero-point and bias terms from it.
 */
int tern_gemv5(const uint8_t* packed5, const float* s_row, const int32_t* rowsum, int64_t N,
               int64_t K, const int8_t* q, const float* s_act, const int32_t* z, float* y,
               int32_t* acc, hipStream_t stream);

/*
 * tern_read_probe -- a measurement aid, not part of the method: reads `bytes`
 * bytes of `buf` (device, 16-byte aligned, bytes a multiple of 16) with the
 * same 16-byte loads and workgroup shape as the GEMV kernels and does nothing
 * else, so its rate is the achievable read-bandwidth ceiling.
 *   sink           device, one uint32; written only when the XOR of all data
 *                  happens to equal a fixed constant (it keeps the loads live)
 *   blocks_per_cu  1..8 workgroups of 256 threads per compute unit
 *   unroll         4, 8 or 16 loads in flight per lane
 *   nontemporal    nonzero: streaming (non-temporal) loads, as the kernels use
 */
int tern_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int blocks_per_cu, int unroll,
                    int nontemporal, hipStream_t stream);

/* Static text for a status code. */
const char* tern_status_string(int status);

/* The hipError_t of the last TERN_ERR_HIP returned on this thread. */
int tern_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TERN_H */
