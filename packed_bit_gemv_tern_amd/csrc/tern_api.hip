// tern_api.hip -- the C ABI declared in include/tern.h: argument checks,
// path dispatch and the static schedule of the persistent stack launch.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "tern.h"
#include "tern_internal.h"

using namespace tern;

// The workspace of tern_linear_stack_prepare_static: each device holds its
// own copy of this array, at its own address.  Host code never uses the
// name itself (a host-side stand-in) but the device address looked up below.
static __device__ __align__(256) uint8_t scratch[TERN_STATIC_WORKSPACE_BYTES];

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return TERN_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kI32Max = 2147483647;

int64_t row_bytes(int64_t K) { return K < 1 ? 0 : 16 * ((K + 63) / 64); }

// Shape and pointer checks shared by every compute entry point.
int check_linear(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
                 int64_t K, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                 const int32_t* z, const float* y, int64_t ldy, const int32_t* acc) {
  if (N < 0 || M < 0 || K < 1) return TERN_ERR_INVALID_ARG;
  if (K > TERN_MAX_K) return TERN_ERR_RANGE;
  if (N > kI32Max || M > kI32Max) return TERN_ERR_RANGE;
  if (N == 0 || M == 0) return TERN_OK;
  if (!packed || !s_row || !rowsum || !q || !s_act || !z || !y) return TERN_ERR_INVALID_ARG;
  if (M > 1 && ldq < K) return TERN_ERR_INVALID_ARG;
  if (M > 1 && ldy < N) return TERN_ERR_INVALID_ARG;
  if (ldq > kI32Max || ldy > kI32Max) return TERN_ERR_RANGE;
  if (!aligned(packed, 16) || !aligned(q, 16)) return TERN_ERR_ALIGNMENT;
  if (M > 1 && (ldq % 16) != 0) return TERN_ERR_ALIGNMENT;
  if (!aligned(y, 4) || !aligned(s_row, 4) || !aligned(rowsum, 4) || !aligned(s_act, 4) ||
      !aligned(z, 4) || (acc && !aligned(acc, 4)))
    return TERN_ERR_ALIGNMENT;
  return TERN_OK;
}

LinearArgs make_args(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
                     int64_t K, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                     const int32_t* z, float* y, int64_t ldy, int32_t* acc) {
  LinearArgs a;
  memset(&a, 0, sizeof(a));
  a.packed = packed;
  a.s_row = s_row;
  a.rowsum = rowsum;
  a.q = q;
  a.s_act = s_act;
  a.z = z;
  a.y = y;
  a.acc = acc;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.ld = (int32_t)row_bytes(K);
  a.nch = a.ld / 16;
  a.ldq = (int32_t)(M > 1 ? ldq : 0);
  a.ldy = (int32_t)(M > 1 ? ldy : 0);
  a.M = (int32_t)M;
  a.variant = valu_variant_for(K);
  a.qjob = -1;
  return a;
}

// Path the call takes, or -1 when the hint cannot be honoured.
int resolve_path(int path, int64_t M) {
  switch (path) {
    case TERN_PATH_AUTO: return M == 1 ? TERN_PATH_VALU : TERN_PATH_MFMA;
    case TERN_PATH_VALU: return M <= TERN_VALU_MAX_M ? TERN_PATH_VALU : -1;
    case TERN_PATH_MFMA: return TERN_PATH_MFMA;
    default: return -1;
  }
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

constexpr int kStackBlock = 256;
constexpr int kWavesPerBlock = kStackBlock / 64;
constexpr int kMaxWavesPerCu = 32;  // 8 waves per SIMD x 4 SIMDs
// The VALU stack kernels launch up to this many times the workgroups that
// fit on the chip at once, each with a matching fraction of a resident
// workgroup's share: the dispatcher then starts a new workgroup wherever one
// finishes, which evens out compute units and dispatch ranks that stream at
// different speeds (8B stack at M = 1: 280 us with one workgroup per slot,
// 267 at 8x, 261 at 16x, 270 at 32x).  The factor stops growing where a
// wave's share would fall below kValuWaveBytes (the 8B stack's share at 16x):
// small stacks lose more to per-workgroup set-up than they gain (one 8B
// layer: 14.4 us at 1x, 19.8 at 16x).  The MFMA window kernel gained nothing
// from it.
constexpr int kValuOversubscribe = 16;
// A stack is split along K when its longest unit costs more than this many
// times a worker's even share.  Measured on 8B layers: one layer (about 4x
// at M = 17..64, 9x at M <= 8) gains 23-26 %; four layers at M <= 8 (2.3x)
// lose 30 %, and at about 1x (four layers at M = 64, one at M = 512) the
// partial sums' atomics cost more than the shorter tail saves.
constexpr double kSplitRatio = 3.0;
// The 9..16-token stacks go to the prefill GEMM when their longest unit
// outlasts this many even shares of a workgroup.  One 8B layer (the down
// projection's unit is ~4.2 shares) runs faster on the window kernel: 39.4 ->
// 30.3 us at M = 9, 40.1 -> 30.9 us at M = 16 (at 3 shares it went to the
// GEMM); two and four layers (2.1 and 1.05 shares) measured the same either
// way; single linears and small stacks (tens of shares) keep the GEMM.
constexpr double kGemmRouteRatio = 6.0;
constexpr int64_t kValuWaveBytes = 24 << 10;
// Tokens up to which the MFMA path takes block-scaled linears (the
// activation-window kernels).
constexpr int64_t kMfmaBlockedMaxM = 16;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Device address of `scratch` on the current device, looked up (with that
// device current) the first time a device asks and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return TERN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return hip_fail(hipErrorInvalidSymbol);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TERN_OK;
}

int stack_prepare(const tern_linear_desc* descs, int64_t L, int64_t M, int path, void* workspace,
                  int64_t workspace_bytes, bool static_ws, tern_stack_plan* plan, hipStream_t stream);

// Schedule cost of one activation-window restage, in streamed bytes: a
// restage stalls its workgroup about 2 us (the barriers wait for its
// slowest wave), about what a workgroup streams in 50 KB at M = 8.
constexpr double kRestageCost = 40000.0;
// A window-major unit is charged its windows' restages divided by this many
// units (each window is staged once per group; its restages stall longer
// than unit-by-unit ones, the waves having drifted apart over a whole pass):
// the 8B stack at M = 8 took 277.8 / 277.8 / 274.3 / 279.4 us at 8 / 4 /
// 2.4 / 1.6 on one box.
constexpr double kWindowMajorGroup = 2.4;

struct Layout {
  int64_t off_lin, off_seg_start, off_seg, off_split, off_job, off_sync, off_flag, off_part, total;
};

// nlin LinearArgs entries, `workers` schedule heads, nseg segments, nsplit
// split linears, njobs quantisation jobs with nitems rows, npart words of
// claiming-workgroup bits
Layout layout_for(int64_t nlin, int64_t workers, int64_t nseg, int64_t nsplit, int64_t njobs,
                  int64_t nitems, int64_t npart) {
  Layout l;
  l.off_sync = kStackSyncOffset;
  l.off_flag = l.off_sync + (int64_t)sizeof(StackSync);
  l.off_lin = align_up(l.off_flag + nitems * 4, 64);
  l.off_seg_start = align_up(l.off_lin + nlin * (int64_t)sizeof(LinearArgs), 16);
  l.off_seg = align_up(l.off_seg_start + (workers + 1) * 4, 16);
  l.off_split = align_up(l.off_seg + nseg * (int64_t)sizeof(Segment), 16);
  l.off_job = align_up(l.off_split + nsplit * 4, 64);
  l.off_part = l.off_job + njobs * (int64_t)sizeof(QuantJob);
  l.total = l.off_part + npart * 4;
  return l;
}

}  // namespace

extern "C" {

int64_t tern_row_bytes(int64_t K) { return row_bytes(K); }

const char* tern_status_string(int status) {
  switch (status) {
    case TERN_OK: return "ok";
    case TERN_ERR_INVALID_ARG: return "invalid argument";
    case TERN_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case TERN_ERR_RANGE: return "size out of range";
    case TERN_ERR_UNSUPPORTED: return "unsupported path for this shape";
    case TERN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case TERN_ERR_HIP: return "HIP runtime error";
    case TERN_ERR_TIMEOUT: return "a stack launch gave up waiting for a quantised input";
    default: return "unknown status";
  }
}

int tern_last_hip_error(void) { return g_last_hip; }

int tern_pack(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
              int32_t* rowsum, int32_t* bad_count, hipStream_t stream) {
  if (N < 0 || K < 1 || ldw < K) return TERN_ERR_INVALID_ARG;
  if (K > TERN_MAX_K || N > TERN_MAX_ROWS_PACK) return TERN_ERR_RANGE;
  if (bad_count && !aligned(bad_count, 4)) return TERN_ERR_ALIGNMENT;
  if (bad_count) {
    hipError_t e = launch_zero_i32(bad_count, 1, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (N == 0) return TERN_OK;
  if (!w || !packed || !rowsum) return TERN_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(rowsum, 4)) return TERN_ERR_ALIGNMENT;
  hipError_t e = launch_pack(w, N, K, ldw, packed, rowsum, bad_count, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, int64_t ldw,
                hipStream_t stream) {
  if (N < 0 || K < 1 || ldw < K) return TERN_ERR_INVALID_ARG;
  if (K > TERN_MAX_K || N > TERN_MAX_ROWS_PACK) return TERN_ERR_RANGE;
  if (N == 0) return TERN_OK;
  if (!packed || !w) return TERN_ERR_INVALID_ARG;
  if (!aligned(packed, 16)) return TERN_ERR_ALIGNMENT;
  hipError_t e = launch_unpack(packed, N, K, w, ldw, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_validate(const uint8_t* packed, int64_t N, int64_t K, int32_t* counts,
                  hipStream_t stream) {
  if (N < 0 || K < 1 || !counts) return TERN_ERR_INVALID_ARG;
  if (K > TERN_MAX_K || N > TERN_MAX_ROWS_PACK) return TERN_ERR_RANGE;
  if (!aligned(counts, 4)) return TERN_ERR_ALIGNMENT;
  if (N > 0 && !packed) return TERN_ERR_INVALID_ARG;
  if (N > 0 && !aligned(packed, 16)) return TERN_ERR_ALIGNMENT;
  hipError_t e = launch_zero_i32(counts, 2, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (N == 0) return TERN_OK;
  e = launch_validate(packed, N, K, counts, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_gemm_smallM(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
                     int64_t K, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                     const int32_t* z, float* y, int64_t ldy, int32_t* acc, int path,
                     hipStream_t stream) {
  int st = check_linear(packed, s_row, rowsum, N, K, M, q, ldq, s_act, z, y, ldy, acc);
  if (st != TERN_OK) return st;
  const int p = resolve_path(path, M < 1 ? 1 : M);
  if (p < 0) return TERN_ERR_UNSUPPORTED;
  if (N == 0 || M == 0) return TERN_OK;
  const LinearArgs a = make_args(packed, s_row, rowsum, N, K, M, q, ldq, s_act, z, y, ldy, acc);
  const hipError_t e = p == TERN_PATH_VALU ? launch_valu_linear(a, stream)
                                           : launch_mfma_linear(a, device_cus(), stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_gemv(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
              int64_t K, const int8_t* q, const float* s_act, const int32_t* z, float* y,
              int32_t* acc, hipStream_t stream) {
  return tern_gemm_smallM(packed, s_row, rowsum, N, K, 1, q, K, s_act, z, y, N, acc,
                          TERN_PATH_AUTO, stream);
}

static bool block_size_ok(int64_t B) {
  return B >= 64 && B <= 4096 && (B & (B - 1)) == 0;
}

int tern_block_rowsum(const uint8_t* packed, int64_t N, int64_t K, int64_t B, int32_t* rowsum_b,
                      hipStream_t stream) {
  if (N < 0 || K < 1 || !block_size_ok(B)) return TERN_ERR_INVALID_ARG;
  if (K > TERN_BLOCK_MAX_K || N > kI32Max) return TERN_ERR_RANGE;
  if (block_rowsum_work_items(N, K, B) > kMaxDispatchItems) return TERN_ERR_RANGE;
  if (N == 0) return TERN_OK;
  if (!packed || !rowsum_b) return TERN_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(rowsum_b, 4)) return TERN_ERR_ALIGNMENT;
  const hipError_t e = launch_block_rowsum(packed, N, K, B, rowsum_b, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_gemv_blocked(const uint8_t* packed, const float* s_b, const int32_t* rowsum_b, int64_t N,
                      int64_t K, int64_t B, const int8_t* q, const float* s_act, const int32_t* z,
                      float* y, hipStream_t stream) {
  if (N < 0 || K < 1 || !block_size_ok(B)) return TERN_ERR_INVALID_ARG;
  if (K > TERN_BLOCK_MAX_K || N > kI32Max) return TERN_ERR_RANGE;
  if (N == 0) return TERN_OK;
  if (!packed || !s_b || !rowsum_b || !q || !s_act || !z || !y) return TERN_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(q, 16)) return TERN_ERR_ALIGNMENT;
  if (!aligned(s_b, 4) || !aligned(rowsum_b, 4) || !aligned(s_act, 4) || !aligned(z, 4) || !aligned(y, 4))
    return TERN_ERR_ALIGNMENT;
  const int cus = device_cus();
  if (cus <= 0) return hip_fail(hipErrorNoDevice);
  const int64_t waves = (N + blocked_rows_per_wave(K) - 1) / blocked_rows_per_wave(K);
  const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 4 * (int64_t)cus);
  const hipError_t e = launch_blocked_gemv(packed, s_b, rowsum_b, N, K, B, q, s_act, z, y, (int)blocks, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                      float* s_act, int32_t* z, hipStream_t stream) {
  if (M < 0 || K < 1 || ldx < K || ldq < K) return TERN_ERR_INVALID_ARG;
  if (M > kI32Max || quantize_act_work_items(M) > kMaxDispatchItems) return TERN_ERR_RANGE;
  if (M == 0) return TERN_OK;
  if (!x || !q || !s_act || !z) return TERN_ERR_INVALID_ARG;
  if (!aligned(x, 4) || !aligned(s_act, 4) || !aligned(z, 4)) return TERN_ERR_ALIGNMENT;
  const hipError_t e = launch_quantize_act(x, M, K, ldx, q, ldq, s_act, z, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int64_t tern_row_bytes5(int64_t K) { return K < 1 ? 0 : 16 * ((K + 79) / 80); }

int tern_pack5(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed5,
               int32_t* rowsum, int32_t* bad_count, hipStream_t stream) {
  if (N < 0 || K < 1 || ldw < K) return TERN_ERR_INVALID_ARG;
  if (K > TERN5_MAX_K || N > kI32Max || pack5_work_items(N) > kMaxDispatchItems) return TERN_ERR_RANGE;
  if (bad_count && !aligned(bad_count, 4)) return TERN_ERR_ALIGNMENT;
  if (bad_count) {
    hipError_t e = launch_zero_i32(bad_count, 1, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (N == 0) return TERN_OK;
  if (!w || !packed5 || !rowsum) return TERN_ERR_INVALID_ARG;
  if (!aligned(packed5, 16) || !aligned(rowsum, 4)) return TERN_ERR_ALIGNMENT;
  const hipError_t e = launch_pack5(w, N, K, ldw, packed5, rowsum, bad_count, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_gemv5(const uint8_t* packed5, const float* s_row, const int32_t* rowsum, int64_t N,
               int64_t K, const int8_t* q, const float* s_act, const int32_t* z, float* y,
               int32_t* acc, hipStream_t stream) {
  if (K > TERN5_MAX_K) return TERN_ERR_RANGE;
  const int st = check_linear(packed5, s_row, rowsum, N, K, 1, q, K, s_act, z, y, N, acc);
  if (st == TERN_OK && gemv5_work_items(N, K) > kMaxDispatchItems) return TERN_ERR_RANGE;
  if (st != TERN_OK || N == 0) return st;
  const hipError_t e = launch_gemv5(packed5, s_row, rowsum, N, K, q, s_act, z, y, acc, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_quantize_weights(const float* W, int64_t N, int64_t K, int64_t ldw, int64_t B, int8_t* w,
                          int64_t ldt, float* s_b, hipStream_t stream) {
  if (N < 0 || K < 1 || B < 1 || ldw < K || ldt < K) return TERN_ERR_INVALID_ARG;
  // one thread per (row, block), all in one 32-bit dispatch
  if (N > kI32Max || K > kI32Max || quantize_weights_work_items(N, K, B) > kMaxDispatchItems)
    return TERN_ERR_RANGE;
  if (N == 0) return TERN_OK;
  if (!W || !w || !s_b) return TERN_ERR_INVALID_ARG;
  if (!aligned(W, 4) || !aligned(s_b, 4)) return TERN_ERR_ALIGNMENT;
  const hipError_t e = launch_quantize_weights(W, N, K, ldw, B, w, ldt, s_b, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_head_rowsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw, int32_t* rowsum,
                     hipStream_t stream) {
  if (N < 0 || K < 1 || ldw < K) return TERN_ERR_INVALID_ARG;
  if (K > TERN_HEAD_MAX_K || N > kI32Max || head_rowsum_work_items(N) > kMaxDispatchItems)
    return TERN_ERR_RANGE;
  if (N == 0) return TERN_OK;
  if (!W || !rowsum) return TERN_ERR_INVALID_ARG;
  if (!aligned(rowsum, 4)) return TERN_ERR_ALIGNMENT;
  const hipError_t e = launch_head_rowsum(W, N, K, ldw, rowsum, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_head_gemv(const int8_t* W, const float* s_row, const int32_t* rowsum, int64_t N, int64_t K,
                   int64_t ldw, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                   const int32_t* z, float* y, int64_t ldy, int32_t* acc, hipStream_t stream) {
  if (N < 0 || M < 0 || K < 1 || ldw < K) return TERN_ERR_INVALID_ARG;
  if (M > TERN_HEAD_MAX_M) return TERN_ERR_UNSUPPORTED;
  if (K > TERN_HEAD_MAX_K || N > kI32Max || ldw > (1 << 28)) return TERN_ERR_RANGE;
  if (N == 0 || M == 0) return TERN_OK;
  if (!W || !s_row || !rowsum || !q || !s_act || !z || !y) return TERN_ERR_INVALID_ARG;
  if (M > 1 && (ldq < K || ldy < N)) return TERN_ERR_INVALID_ARG;
  if (ldq > kI32Max || ldy > kI32Max) return TERN_ERR_RANGE;
  if (!aligned(W, 16) || (ldw % 16) != 0 || !aligned(q, 16) || (M > 1 && (ldq % 16) != 0))
    return TERN_ERR_ALIGNMENT;
  if (!aligned(y, 4) || !aligned(s_row, 4) || !aligned(rowsum, 4) || !aligned(s_act, 4) ||
      !aligned(z, 4) || (acc && !aligned(acc, 4)))
    return TERN_ERR_ALIGNMENT;
  // head_wg_per_cu() workgroups per CU, each with a whole number of units
  const int cus = device_cus();
  if (cus <= 0) return hip_fail(hipErrorNoDevice);
  const int64_t unit = head_rows_per_unit(M);
  const int64_t wgc = (int64_t)head_wg_per_cu() * cus;
  const int64_t per = (N + wgc - 1) / wgc;
  const int64_t rows = (per + unit - 1) / unit * unit;
  if (head_lds_bytes(M, K, rows) > 65536) return TERN_ERR_RANGE;
  const hipError_t e = launch_head(W, s_row, rowsum, N, K, ldw, M, q, M > 1 ? ldq : K, s_act, z, y,
                                   M > 1 ? ldy : N, acc, rows, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int64_t tern_linear_stack_workspace_bytes(int64_t L, int64_t M) {
  if (L < 0 || M < 0 || L > kI32Max) return 0;
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  const int64_t workers = (int64_t)cus * kMaxWavesPerCu * kValuOversubscribe;
  // every linear may be split into kMaxSplitWindows windows, each with its
  // own LinearArgs entry and segments
  const int64_t nlin = L * (1 + kMaxSplitWindows);
  // every linear may carry its own fp32 input: L jobs of M rows (at most
  // kMaxQuantItems rows in all)
  const int64_t items = M > 0 && L > kMaxQuantItems / M ? kMaxQuantItems : std::min(kMaxQuantItems, L * M);
  return layout_for(nlin, workers, workers + nlin, L, L, items, workers / 32 + 1).total;
}

int tern_linear_stack_prepare(const tern_linear_desc* descs, int64_t L, int64_t M, int path,
                              void* workspace, int64_t workspace_bytes, tern_stack_plan* plan,
                              hipStream_t stream) {
  return stack_prepare(descs, L, M, path, workspace, workspace_bytes, false, plan, stream);
}

int tern_linear_stack_prepare_static(const tern_linear_desc* descs, int64_t L, int64_t M, int path,
                                     tern_stack_plan* plan, hipStream_t stream) {
  if (!plan || L < 0 || M < 0) return TERN_ERR_INVALID_ARG;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != TERN_OK) return st;
  return stack_prepare(descs, L, M, path, ws, TERN_STATIC_WORKSPACE_BYTES, true, plan, stream);
}

}  // extern "C"

namespace {

// The schedule of tern_linear_stack_prepare into `workspace` (with
// static_ws, the library's own: a schedule too large for it is a range
// error rather than a workspace error).
int stack_prepare(const tern_linear_desc* descs, int64_t L, int64_t M, int path, void* workspace,
                  int64_t workspace_bytes, bool static_ws, tern_stack_plan* plan, hipStream_t stream) {
  if (!plan || L < 0 || M < 0) return TERN_ERR_INVALID_ARG;
  if (L > kI32Max || M > kI32Max) return TERN_ERR_RANGE;
  if (L > 0 && !descs) return TERN_ERR_INVALID_ARG;
  int p = resolve_path(path, M < 1 ? 1 : M);
  if (p < 0) return TERN_ERR_UNSUPPORTED;
  // block sizes the activation-window kernels cannot take (below 512
  // columns, or not a multiple of it) send a stack of 2..8 tokens on the
  // automatic path to the vector ALU, which runs it token by token
  if (path == TERN_PATH_AUTO && M > 1 && M <= TERN_VALU_MAX_M) {
    for (int64_t i = 0; i < L; ++i)
      if (descs[i].block != 0 && descs[i].block % mfma_step_k() != 0) p = TERN_PATH_VALU;
  }
  // every descriptor is checked before anything is written
  int64_t bytes = 0;
  bool any_blocked = false;
  // fp32 inputs the launch quantises: one job per distinct q buffer, named
  // by the linears that give x (and read by every linear naming that q)
  std::vector<QuantJob> jobs;
  std::vector<int32_t> qjob((size_t)L, -1);
  std::map<const void*, int32_t> job_of_q;
  for (int64_t i = 0; i < L; ++i) {
    const tern_linear_desc& d = descs[i];
    if (!d.x) {
      if (d.x_up) return TERN_ERR_INVALID_ARG;  // the gate without its input
      continue;
    }
    // (checked here as well as below: a linear with no rows still has its
    // input quantised)
    if (d.K < 1 || d.ldx < d.K || !d.q || !d.s_act || !d.z) return TERN_ERR_INVALID_ARG;
    if (d.K > TERN_MAX_K || d.ldx > kI32Max || d.ldq > kI32Max) return TERN_ERR_RANGE;
    if (M > 1 && d.ldq < d.K) return TERN_ERR_INVALID_ARG;
    if (!aligned(d.x, 4) || !aligned(d.x_up, 4) || !aligned(d.q, 16) || !aligned(d.s_act, 4) ||
        !aligned(d.z, 4) || (M > 1 && d.ldq % 16 != 0))
      return TERN_ERR_ALIGNMENT;
    const int64_t ldq = M > 1 ? d.ldq : d.K;
    auto it = job_of_q.find(d.q);
    if (it == job_of_q.end()) {
      QuantJob j;
      memset(&j, 0, sizeof(j));
      j.x = d.x;
      j.x_up = d.x_up;
      j.q = const_cast<int8_t*>(d.q);
      j.s_act = const_cast<float*>(d.s_act);
      j.z = const_cast<int32_t*>(d.z);
      j.ldx = d.ldx;
      j.ldq = ldq;
      j.K = (int32_t)std::min<int64_t>(d.K, kI32Max);
      job_of_q[d.q] = (int32_t)jobs.size();
      jobs.push_back(j);
      continue;
    }
    const QuantJob& j = jobs[(size_t)it->second];
    if (j.x != d.x || j.x_up != d.x_up || j.ldx != d.ldx || j.K != d.K || j.ldq != ldq ||
        j.s_act != d.s_act || j.z != d.z)
      return TERN_ERR_INVALID_ARG;
  }
  if (!jobs.empty()) {
    for (int64_t i = 0; i < L; ++i) {
      const tern_linear_desc& d = descs[i];
      auto it = job_of_q.find(d.q);
      if (it == job_of_q.end()) continue;
      // a linear reading a buffer the launch writes reads all of it, as
      // written: the same activations, scales and zero points
      const QuantJob& j = jobs[(size_t)it->second];
      if (j.K != d.K || j.ldq != (M > 1 ? d.ldq : d.K) || j.s_act != d.s_act || j.z != d.z)
        return TERN_ERR_INVALID_ARG;
      qjob[(size_t)i] = it->second;
    }
    if (M > 0 && (int64_t)jobs.size() > kMaxQuantItems / M) return TERN_ERR_RANGE;
    for (const QuantJob& j : jobs) bytes += 5 * M * (int64_t)j.K + 8 * M;  // fp32 in, int8 out, s_act and z
  }
  const int64_t nitems = (int64_t)jobs.size() * M;
  for (int64_t i = 0; i < L; ++i) {
    const tern_linear_desc& d = descs[i];
    const bool blk = d.block != 0;
    if (blk && !block_size_ok(d.block)) return TERN_ERR_INVALID_ARG;
    // a block-scaled linear's metadata arrays stand in for s_row / rowsum
    const int st = check_linear(d.packed, blk ? d.s_block : d.s_row, blk ? d.rowsum_block : d.rowsum, d.N,
                                d.K, M, d.q, d.ldq, d.s_act, d.z, d.y, d.ldy, d.acc);
    if (st != TERN_OK) return st;
    if (d.N == 0 || M == 0) continue;
    const int64_t nb = blk ? (d.K + d.block - 1) / d.block : 1;
    if (blk) {
      any_blocked = true;
      if (d.K % 64 != 0) return TERN_ERR_UNSUPPORTED;
      if (p == TERN_PATH_VALU && valu_blocked_variant(d.K, d.block) < 0) return TERN_ERR_UNSUPPORTED;
      if (p == TERN_PATH_MFMA && (M > kMfmaBlockedMaxM || d.block % mfma_step_k() != 0))
        return TERN_ERR_UNSUPPORTED;
      if (d.N * nb > kI32Max) return TERN_ERR_RANGE;
    }
    bytes += d.N * row_bytes(d.K) + 8 * d.N * nb + M * d.K + 8 * M + 4 * M * d.N;
  }
  memset(plan, 0, sizeof(*plan));
  plan->workspace = workspace;
  plan->workspace_bytes = workspace_bytes;
  plan->L = (int32_t)L;
  plan->M = (int32_t)M;
  plan->path = p;
  plan->bytes = bytes;
  plan->block = kStackBlock;
  if (L == 0 || M == 0) return TERN_OK;  // empty stack: launches nothing
  if (!workspace) return TERN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return TERN_ERR_WORKSPACE;

  // the VALU variant of each linear (block-scaled ones: a variant whose
  // lanes per row hold whole blocks)
  auto variant_of = [&](const tern_linear_desc& d) -> int32_t {
    if (d.block != 0 && p == TERN_PATH_VALU) return valu_blocked_variant(d.K, d.block);
    return d.K % 64 ? (int32_t)VGEN : valu_variant_for(d.K);
  };
  uint32_t used = 0;
  bool big = false;
  for (int64_t i = 0; i < L; ++i) {
    if (descs[i].N == 0) continue;
    used |= 1u << variant_of(descs[i]);
    big = big || !mfma_win_offsets_fit(descs[i].N, row_bytes(descs[i].K), M, descs[i].ldy);
  }
  const bool ragged = (used >> VGEN) & 1u;
  int32_t kernel = p == TERN_PATH_VALU ? valu_stack_kernel_for((int32_t)M, used, any_blocked)
                                       : (int32_t)SK_MFMA + mfma_stack_variant((int32_t)M, ragged, big, any_blocked);
  // block-scaled linears on the MFMA path: the activation-window kernels
  if (p == TERN_PATH_MFMA && any_blocked && !mfma_is_window(kernel - SK_MFMA)) return TERN_ERR_UNSUPPORTED;
  const int cus = device_cus();
  if (cus <= 0) return hip_fail(hipErrorNoDevice);
  auto mfma_per_cu = [&](int32_t v) {
    return std::min(mfma_stack_blocks_per_cu(v), kMaxWavesPerCu / kWavesPerBlock);
  };
  // The kernels at 9..16 tokens keep a workgroup on one unit of rows for
  // the linear's whole K.  When the longest unit outlasts kGemmRouteRatio
  // even shares of a workgroup (a single linear, a small stack), the prefill
  // GEMM, whose tiles end sooner and which may split long K, takes the stack
  // instead; deeper stacks keep their kernel, which streams them faster.
  if (p == TERN_PATH_MFMA && M > 8 && !any_blocked &&
      (mfma_is_lockstep(kernel - SK_MFMA) || mfma_is_window(kernel - SK_MFMA))) {
    const int32_t v = kernel - SK_MFMA;
    const int unit = mfma_unit_rows(v);
    const double workers_v = (double)std::max(8, cus * mfma_per_cu(v) / 8 * 8);
    double tot = 0.0, gm = 0.0;
    for (int64_t i = 0; i < L; ++i) {
      const tern_linear_desc& d = descs[i];
      if (d.N == 0) continue;
      const double ld = (double)row_bytes(d.K);
      tot += (double)d.N * ld + 256.0 * (double)((d.N + unit - 1) / unit);
      gm = std::max(gm, (double)std::min<int64_t>(unit, d.N) * ld + 256.0);
    }
    if (gm > kGemmRouteRatio * tot / workers_v) kernel = (int32_t)SK_MFMA + mfma_gemm_variant((int32_t)M);
  }
  // the prefill GEMM's row tile: 512 rows for stacks of a few such tiles per
  // CU or more, else 256
  if (p == TERN_PATH_MFMA) {
    int64_t tiles512 = 0;
    for (int64_t i = 0; i < L; ++i)
      if (descs[i].N > 0) tiles512 += (descs[i].N + 511) / 512 * ((M + 127) / 128);
    kernel = (int32_t)SK_MFMA + mfma_gemm_refine(kernel - SK_MFMA, (int32_t)M, tiles512, cus);
  }
  int per_cu = p == TERN_PATH_VALU ? valu_stack_blocks_per_cu(kernel) : mfma_per_cu(kernel - SK_MFMA);
  per_cu = std::min(per_cu, kMaxWavesPerCu / kWavesPerBlock);
  int over = 1;
  if (p == TERN_PATH_VALU) {
    const int64_t resident_waves = (int64_t)cus * per_cu * kWavesPerBlock;
    over = (int)std::min<int64_t>(kValuOversubscribe, std::max<int64_t>(1, bytes / (resident_waves * kValuWaveBytes)));
  }
  int grid = cus * per_cu * over;
  grid = std::max(8, grid / 8 * 8);  // a multiple of 8 for the XCD-aware numbering
  // schedule entries belong to waves, or to whole workgroups for the
  // lockstep MFMA kernel
  const bool per_wg = p == TERN_PATH_MFMA && mfma_per_workgroup(kernel - SK_MFMA);
  const int64_t workers = (int64_t)grid * (per_wg ? 1 : kWavesPerBlock);

  // Granules: units of each linear's rows, cost = packed bytes + a fixed
  // per-unit overhead; contiguous granule runs balanced over the workers.
  std::vector<LinearArgs> lin((size_t)L);
  for (int64_t i = 0; i < L; ++i) {
    const tern_linear_desc& d = descs[i];
    LinearArgs& a = lin[(size_t)i];
    a = make_args(d.packed, d.s_row, d.rowsum, d.N, d.K, M, d.q, d.ldq, d.s_act, d.z, d.y, d.ldy, d.acc);
    a.qjob = qjob[(size_t)i];
    if (d.block != 0 && d.N > 0) {
      a.s_b = d.s_block;
      a.rowsum_b = d.rowsum_block;
      a.nb = (int32_t)((d.K + d.block - 1) / d.block);
      int lg = 0;
      while ((64ll << lg) < d.block) ++lg;
      a.blg = lg;
      if (p == TERN_PATH_VALU) a.variant = variant_of(d);
    }
  }
  struct Gran {
    int32_t lin, r0, r1, flags;
    double cost;
  };
  std::vector<Gran> gran;
  std::vector<int32_t> split;  // linears split along K
  double total = 0.0, gmax = 0.0;
  // 0: segments hold rows; else the prefill GEMM's token tiles per row unit
  // (its segments hold tile indices)
  const int32_t ntok = p == TERN_PATH_VALU ? 0 : mfma_token_tiles(kernel - SK_MFMA, (int32_t)M);
  // (block-scaled linears are never split)
  const bool splittable = p == TERN_PATH_MFMA && mfma_can_split(kernel - SK_MFMA) && !any_blocked;
  const int64_t wk_k = mfma_window_k();
  auto add_units = [&](int32_t li, int32_t flags) {
    const LinearArgs& a = lin[(size_t)li];
    // (the token-by-token kernel takes one-token units)
    const int32_t mu = any_blocked ? 1 : (int32_t)M;
    const int unit = p == TERN_PATH_VALU ? (a.s_b ? valu_blocked_unit_rows(a.variant) : valu_unit_rows(a.variant, mu))
                                         : mfma_unit_rows(kernel - SK_MFMA);
    // bytes of a row the unit reads: packed weights (and block metadata)
    const double ld = 16.0 * a.nch + (a.s_b ? 8.0 * a.nb : 0.0);
    // a unit that restages the activation window stalls its workgroup for
    // about as long as streaming kRestageCost bytes takes
    // (a 16-token window, M > 8, is twice the activation bytes to restage:
    // 80 KB measured best for it, 40 KB for the 8-token one)
    const double restage = kRestageCost * (M > 8 ? 2.0 : 1.0);
    const int32_t mv = kernel - SK_MFMA;
    const double restages = p == TERN_PATH_VALU ? 0.0
                            : mfma_window_major(mv, a.K, a.acc == nullptr && !(flags & kSegPartial))
                                ? mfma_unit_restages(mv, a.K) / kWindowMajorGroup
                                : (double)mfma_unit_restages(mv, a.K);
    const double fixed = 256.0 + restage * restages;
    for (int64_t r0 = 0; r0 < a.N; r0 += unit) {
      const int64_t r1 = std::min<int64_t>(a.N, r0 + unit);
      const double c = (double)(r1 - r0) * ld + fixed;
      if (ntok == 0) {
        gran.push_back({li, (int32_t)r0, (int32_t)r1, flags, c});
      } else {
        // prefill GEMM: one granule per (row tile, token tile), numbered
        // row tile first, so a run keeps reusing one weight tile
        const int32_t t0 = (int32_t)(r0 / unit) * ntok;
        for (int32_t tt = 0; tt < ntok; ++tt) gran.push_back({li, t0 + tt, t0 + tt + 1, flags, c});
      }
      total += c * (ntok == 0 ? 1 : ntok);
      gmax = std::max(gmax, c);
    }
  };
  for (int64_t i = 0; i < L; ++i)
    if (descs[i].N > 0) add_units((int32_t)i, 0);
  // A small stack whose longest unit outlasts the even share of a worker
  // (one layer: a K = 12,288 unit restages its window three times, or walks
  // 192 GEMM K-steps, while most workgroups idle) splits such linears along
  // K: one entry per 4,096-column window, each window's units scheduled on
  // their own, their int32 partial sums added into the output buffer, which
  // a fill kernel clears before and a finishing kernel turns into y (and
  // acc) after.
  // (the fill and finishing kernels take one workgroup per split linear and
  // token: all of them must fit one dispatch)
  if (splittable && gmax > kSplitRatio * total / (double)workers &&
      L * M * (int64_t)kSplitBlock <= kMaxDispatchItems) {
    // only K a multiple of 64: every window's reads then lie inside the
    // linear's K columns (the kernels clamp activation addresses to the row)
    auto splits_k = [&](const LinearArgs& a) {
      const int64_t nwin = (a.K + wk_k - 1) / wk_k;
      return a.N > 0 && a.K % 64 == 0 && nwin > 1 && nwin <= kMaxSplitWindows;
    };
    bool any = false;
    for (int64_t i = 0; i < L && !any; ++i) any = splits_k(lin[(size_t)i]);
    if (any) {
      gran.clear();
      total = gmax = 0.0;
      for (int64_t i = 0; i < L; ++i) {
        const LinearArgs a = lin[(size_t)i];
        if (a.N == 0) continue;
        const int64_t nwin = (a.K + wk_k - 1) / wk_k;
        if (!splits_k(a)) {
          add_units((int32_t)i, 0);
          continue;
        }
        split.push_back((int32_t)i);
        for (int64_t w = 0; w < nwin; ++w) {
          LinearArgs v = a;
          v.packed = a.packed + w * (wk_k / 4);  // 2-bit codes: K / 4 bytes
          v.q = a.q + w * wk_k;
          v.K = (int32_t)std::min<int64_t>(wk_k, a.K - w * wk_k);
          v.nch = (v.K + 63) / 64;
          v.acc = nullptr;
          lin.push_back(v);
          add_units((int32_t)lin.size() - 1, kSegPartial | (w == 0 ? kSegZeroPoint : 0));
        }
      }
    }
  }
  // Contiguous runs of granules, the largest run as small as it can be: the
  // smallest cap C for which runs of total cost <= C need at most `workers`
  // runs (bisection on C, each probe a greedy fill over the prefix sums).
  // When fewer runs suffice, the idle workers are spread evenly over the
  // worker numbering (and so over the XCDs).
  const size_t G = gran.size();
  std::vector<double> pre(G + 1, 0.0);
  for (size_t i = 0; i < G; ++i) pre[i + 1] = pre[i] + gran[i].cost;
  auto runs_for = [&](double cap, std::vector<size_t>* ends) {
    int64_t n = 0;
    size_t i = 0;
    while (i < G) {
      // last j with pre[j] - pre[i] <= cap; at least one granule per run
      size_t j = (size_t)(std::upper_bound(pre.begin() + (ptrdiff_t)i + 1, pre.end(), pre[i] + cap) -
                          pre.begin()) - 1;
      if (j <= i) j = i + 1;
      if (ends) ends->push_back(j);
      ++n;
      i = j;
    }
    return n;
  };
  double lo = std::max(total / (double)workers, gmax), hi = lo + gmax;
  if (runs_for(lo, nullptr) <= workers) hi = lo;
  for (int it = 0; it < 60 && hi - lo > 1e-6 * hi; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (runs_for(mid, nullptr) <= workers)
      hi = mid;
    else
      lo = mid;
  }
  std::vector<size_t> ends;
  ends.reserve((size_t)workers);
  const int64_t nruns = runs_for(hi, &ends);
  std::vector<int32_t> seg_start((size_t)workers + 1, 0);
  std::vector<Segment> segs;
  segs.reserve(G / 4 + (size_t)workers + (size_t)L);
  size_t gi = 0;
  int64_t wk = 0;
  for (int64_t k = 0; k < nruns; ++k) {
    // run k goes to worker floor(k * workers / nruns); the workers skipped
    // over get empty ranges
    const int64_t target = k * workers / nruns;
    while (wk <= target) seg_start[(size_t)wk++] = (int32_t)segs.size();
    for (; gi < ends[(size_t)k]; ++gi) {
      const Gran& g = gran[gi];
      if (gi > 0 && gi != (k == 0 ? 0 : ends[(size_t)k - 1]) && segs.back().lin == g.lin &&
          segs.back().row_end == g.r0) {
        segs.back().row_end = g.r1;
        continue;
      }
      segs.push_back({g.lin, g.r0, g.r1, g.flags});
    }
  }
  while (wk <= workers) seg_start[(size_t)wk++] = (int32_t)segs.size();

  // Workgroups that claim rows to quantise (launches with jobs): the first
  // few of the grid (one per row, at least 8: spread over the XCDs, and
  // dispatched first), and every workgroup whose run reads a quantised input
  // (its waves wait for that input only after their own claims have run
  // out).  The others skip the prologue.
  std::vector<uint32_t> part;
  int32_t claimers = 0;
  if (nitems > 0) {
    part.assign((size_t)(grid + 31) / 32, 0u);
    auto set = [&](int64_t b) { part[(size_t)(b >> 5)] |= 1u << (b & 31); };
    const int64_t first = std::min<int64_t>(grid, std::max<int64_t>(8, nitems));
    for (int64_t b = 0; b < first; ++b) set(b);
    const int64_t per = grid / 8;  // (the grid is a multiple of 8: XCD-aware numbering)
    for (int64_t wr = 0; wr < workers; ++wr) {
      bool reads = false;
      for (int32_t sx = seg_start[(size_t)wr]; sx < seg_start[(size_t)wr + 1] && !reads; ++sx)
        reads = lin[(size_t)segs[(size_t)sx].lin].qjob >= 0;
      if (!reads) continue;
      // the worker's logical workgroup, and the workgroup index it runs as
      const int64_t lb = per_wg ? wr : wr / kWavesPerBlock;
      set((lb % per) * 8 + lb / per);
    }
    for (uint32_t wd : part) claimers += __builtin_popcount(wd);
  }
  const Layout lay = layout_for((int64_t)lin.size(), workers, (int64_t)segs.size(), (int64_t)split.size(),
                               (int64_t)jobs.size(), nitems, (int64_t)part.size());
  if (workspace_bytes < lay.total) return static_ws ? TERN_ERR_RANGE : TERN_ERR_WORKSPACE;
  std::vector<char> host((size_t)lay.total, 0);
  StackHeader h;
  memset(&h, 0, sizeof(h));
  h.magic = kStackMagic;
  h.L = (int32_t)L;
  h.M = (int32_t)M;
  h.workers = (int32_t)workers;
  h.nseg = (int32_t)segs.size();
  h.kernel = kernel;
  h.nlin = (int32_t)lin.size();
  h.nsplit = (int32_t)split.size();
  h.off_lin = lay.off_lin;
  h.off_seg_start = lay.off_seg_start;
  h.off_seg = lay.off_seg;
  h.off_split = lay.off_split;
  h.njobs = (int32_t)jobs.size();
  h.nitems = (int32_t)nitems;
  h.off_job = lay.off_job;
  h.off_sync = lay.off_sync;
  h.off_flag = lay.off_flag;
  h.claimers = claimers;
  h.off_part = lay.off_part;
  memcpy(host.data(), &h, sizeof(h));
  if (!part.empty()) memcpy(host.data() + lay.off_part, part.data(), part.size() * 4);
  // (the claim counter, the error word and the flags start at zero)
  if (!jobs.empty()) memcpy(host.data() + lay.off_job, jobs.data(), jobs.size() * sizeof(QuantJob));
  memcpy(host.data() + lay.off_lin, lin.data(), lin.size() * sizeof(LinearArgs));
  memcpy(host.data() + lay.off_seg_start, seg_start.data(), seg_start.size() * 4);
  if (!segs.empty()) memcpy(host.data() + lay.off_seg, segs.data(), segs.size() * sizeof(Segment));
  if (!split.empty()) memcpy(host.data() + lay.off_split, split.data(), split.size() * 4);
  hipError_t e = hipMemcpyAsync(workspace, host.data(), (size_t)lay.total, hipMemcpyHostToDevice,
                                stream);
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);

  plan->grid = grid;
  plan->workers = (int32_t)workers;
  plan->segments = (int32_t)segs.size();
  plan->kernel = kernel;
  plan->splits = (int32_t)split.size();
  // activation-window loads of one launch (window kernels): a segment of a
  // single-window linear loads its window unless the workgroup's segment
  // before it read the same activations; a longer K loads every window of
  // every unit
  // (the kernel's own walk: units in order, all windows of each; a
  // window-major linear in groups of held units, each window once per group)
  if (p == TERN_PATH_MFMA && mfma_is_window(kernel - SK_MFMA)) {
    const int32_t mv = kernel - SK_MFMA;
    const int unit = mfma_unit_rows(mv);
    const int64_t hmax = mfma_held_units(mv);
    int64_t restages = 0;
    for (int64_t wr = 0; wr < workers; ++wr) {
      const LinearArgs* prev = nullptr;  // staged window: window `pwin` of prev's activations
      int64_t pwin = 0, nheld = 0;
      for (int32_t sx = seg_start[(size_t)wr]; sx < seg_start[(size_t)wr + 1]; ++sx) {
        const Segment& sg = segs[(size_t)sx];
        const LinearArgs& a = lin[(size_t)sg.lin];
        const int64_t nwin = (a.K + wk_k - 1) / wk_k;
        const int64_t units = (sg.row_end - sg.row_begin + unit - 1) / unit;
        const bool y_only = a.acc == nullptr && !(sg.flags & kSegPartial);
        auto stage = [&](int64_t w) {
          const bool same = prev && prev->q == a.q && prev->z == a.z && prev->s_act == a.s_act &&
                            prev->K == a.K && prev->ldq == a.ldq && pwin == w;
          if (!same) ++restages;
          prev = &a;
          pwin = w;
        };
        if (hmax > 0 && mfma_window_major(mv, a.K, y_only)) {
          for (int64_t rem = units; rem > 0;) {
            const int64_t need = std::min(rem, hmax);
            if (hmax - nheld < need) nheld = 0;
            const int64_t gn = std::min(rem, hmax - nheld);
            for (int64_t w = 0; w < nwin; ++w) stage(w);
            nheld += gn;
            rem -= gn;
          }
          continue;
        }
        for (int64_t k = 0; k < units; ++k) {
          for (int64_t w = 0; w < nwin; ++w) stage(w);
          if (hmax > 0 && y_only) nheld = nheld == hmax ? 1 : nheld + 1;
        }
      }
    }
    plan->restages = (int32_t)std::min<int64_t>(restages, kI32Max);
  }
  return TERN_OK;
}

}  // namespace

extern "C" {

int tern_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int blocks_per_cu, int unroll,
                    int nontemporal, hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return TERN_ERR_INVALID_ARG;
  if (blocks_per_cu < 1 || blocks_per_cu > kMaxWavesPerCu / kWavesPerBlock) return TERN_ERR_INVALID_ARG;
  if (unroll != 4 && unroll != 8 && unroll != 16) return TERN_ERR_UNSUPPORTED;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return TERN_ERR_ALIGNMENT;
  const int cus = device_cus();
  if (cus <= 0) return hip_fail(hipErrorNoDevice);
  const hipError_t e =
      launch_read_probe(buf, bytes, sink, cus * blocks_per_cu, unroll, nontemporal != 0, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

int tern_linear_stack_status(const tern_stack_plan* plan, hipStream_t stream) {
  if (!plan) return TERN_ERR_INVALID_ARG;
  if (plan->L == 0 || plan->M == 0) return TERN_OK;
  if (!plan->workspace || !aligned(plan->workspace, 256)) return TERN_ERR_WORKSPACE;
  StackHeader h;
  hipError_t e = hipMemcpyAsync(&h, plan->workspace, sizeof(h), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  if (h.magic != kStackMagic) return TERN_ERR_WORKSPACE;
  StackSync sy;
  e = hipMemcpyAsync(&sy, static_cast<const char*>(plan->workspace) + h.off_sync, sizeof(sy),
                     hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  return sy.err ? TERN_ERR_TIMEOUT : TERN_OK;
}

int tern_linear_stack(const tern_stack_plan* plan, hipStream_t stream) {
  if (!plan) return TERN_ERR_INVALID_ARG;
  if (plan->L == 0 || plan->M == 0 || plan->workers == 0) return TERN_OK;
  if (!plan->workspace || !aligned(plan->workspace, 256)) return TERN_ERR_WORKSPACE;
  LaunchShape shp;
  shp.grid = plan->grid;
  shp.block = plan->block;
  shp.waves_per_block = plan->block / 64;
  shp.M = plan->M;
  shp.splits = plan->splits;
  if (shp.grid <= 0 || shp.block != kStackBlock || shp.splits < 0) return TERN_ERR_INVALID_ARG;
  const hipError_t e = plan->kernel >= SK_MFMA
                           ? launch_mfma_stack(plan->kernel - SK_MFMA, plan->workspace, shp, stream)
                           : launch_valu_stack(plan->kernel, plan->workspace, shp, stream);
  return e == hipSuccess ? TERN_OK : hip_fail(e);
}

}  // extern "C"
