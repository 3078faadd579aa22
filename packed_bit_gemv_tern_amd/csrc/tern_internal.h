// tern_internal.h -- shared between the host API (tern_api.cpp) and the HIP
// kernels: the device-side descriptor of one linear, the stack workspace
// layout and the kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

// Kernel variants of the VALU path.  LPR = lanes per row (a row is split
// over LPR lanes, 64 / LPR rows per wave-wide load), CPL = 16-byte chunks of
// a row per lane (one chunk = 64 weights), so a row holds up to LPR*CPL
// chunks.  The generic variant streams q from memory and takes any K.
enum ValuVariant : int32_t {
  V8x1 = 0,   // K <= 512
  V16x1 = 1,  // K <= 1024
  V32x1 = 2,  // K <= 2048
  V16x3 = 3,  // K <= 3072
  V64x1 = 4,  // K <= 4096
  V64x2 = 5,  // K <= 8192
  V64x3 = 6,  // K <= 12288
  V64x4 = 7,  // K <= 16384
  VGEN = 8,   // any K
  kNumValuVariants = 9
};

// Device-side view of one linear layer; 128 bytes, read by the kernels from
// kernel arguments (single-linear calls) or from the stack workspace.
struct alignas(16) LinearArgs {
  const uint8_t* packed;  // N rows of ld bytes
  const float* s_row;     // N (null with block scales)
  const int32_t* rowsum;  // N (null with block scales)
  const int8_t* q;        // M rows of ldq bytes
  const float* s_act;     // M
  const int32_t* z;       // M
  float* y;               // M rows of ldy floats
  int32_t* acc;           // M rows of ldy int32, or null
  int32_t N, K, ld, nch;  // rows, columns, row bytes, 16-byte chunks per row
  int32_t ldq, ldy, M, variant;
  // block-wise scales along K: null for one scale per row; else row i's
  // block b (columns [64 * 2^blg * b, 64 * 2^blg * (b + 1)) inside K) has
  // scale s_b[i * nb + b] and row sum rowsum_b[i * nb + b]
  const float* s_b;
  const int32_t* rowsum_b;
  int32_t blg, nb;  // log2(block / 64), blocks per row
  // the launch's quantisation job that writes q, s_act and z (-1: the
  // caller's activations, ready before the launch)
  int32_t qjob;
  int32_t pad;
};
static_assert(sizeof(LinearArgs) == 128, "LinearArgs layout");

// One schedule entry: rows [row_begin, row_end) of linear `lin` (all
// tokens); for the prefill GEMM instead its tiles [row_begin, row_end) in
// (row tile, token tile) order, tile = row_tile * token_tiles + token_tile.
// `flags` marks entries of a linear split along K (activation-window kernel).
struct Segment {
  int32_t lin, row_begin, row_end, flags;
};
// The entry covers one K-window of a split linear: its int32 partial sums
// are added into the output buffer (viewed as int32) instead of stored; the
// zero-point term is part of exactly one window's sums.
constexpr int32_t kSegPartial = 1, kSegZeroPoint = 2;
// Windows a linear may be split into (each K-window is 4,096 columns).
constexpr int kMaxSplitWindows = 4;

// Stack workspace layout (device memory, 256-byte aligned):
//   StackHeader | StackSync | uint32 flag[njobs * M] | LinearArgs[nlin] |
//   int32 seg_start[workers + 1] | Segment[nseg] | int32 split[nsplit] |
//   QuantJob[njobs] | uint32 part[ceil(grid / 32)]
// The first L entries of LinearArgs are the caller's linears; a linear split
// along K adds one entry per window after them, and split[] lists the split
// linears (their outputs are cleared before and finished after the main
// kernel).  QuantJob lists the fp32 inputs the launch quantises itself
// (each distinct q buffer once); its items are (job, token) rows, item
// i = job * M + m, and flag[i] says which launch has finished item i.
struct alignas(256) StackHeader {
  int32_t magic, L, M, workers, nseg, kernel, nlin, nsplit;
  int64_t off_lin, off_seg_start, off_seg, off_split;
  int32_t njobs, nitems;  // quantisation jobs, and their rows (njobs * M)
  int64_t off_job, off_sync, off_flag;
  // workgroups that claim rows: their number, and one bit per workgroup of
  // the grid (uint32 words at off_part)
  int32_t claimers, pad0;
  int64_t off_part;
};
static_assert(sizeof(StackHeader) == 256, "StackHeader layout");

// One fp32 input quantised inside the launch: M rows of K floats (stride
// ldx) into M rows of int8 codes (stride ldq), a scale and a zero point per
// row -- the arithmetic of tern_quantize_act.
struct alignas(16) QuantJob {
  const float* x;
  int8_t* q;
  float* s_act;
  int32_t* z;
  int64_t ldx, ldq;
  int32_t K;
  int32_t pad;
  const float* x_up;  // non-null: quantise silu(x) * x_up (the SwiGLU gate)
};
static_assert(sizeof(QuantJob) == 64, "QuantJob layout");

// Words the launch updates: claim counts the rows claimed by workgroups over
// every launch of the plan (each launch advances it by a fixed amount, which
// numbers the launches); err is set when a wait for a quantised input gave
// up.  They sit at a fixed offset after the header, with the flags right
// after them, and reach the kernels as an argument of their own: everything
// the kernels read through the header pointer stays read-only for the whole
// launch, so the compiler keeps those reads in scalar loads (written through
// the same pointer, they would become vector loads whose waits also wait for
// the weight tiles in flight).
struct alignas(64) StackSync {
  unsigned long long claim;
  uint32_t err;
  uint32_t pad[13];
};
static_assert(sizeof(StackSync) == 64, "StackSync layout");
constexpr int64_t kStackSyncOffset = sizeof(StackHeader);
inline StackSync* stack_sync(const void* ws) {
  return reinterpret_cast<StackSync*>(static_cast<char*>(const_cast<void*>(ws)) + kStackSyncOffset);
}
// Rows of quantisation jobs one plan may hold.
constexpr int64_t kMaxQuantItems = 1ll << 22;
constexpr int32_t kStackMagic = 0x7e54a11;

// Kernel selectors of a prepared stack.
// SK_VALU_M1 .. SK_VALU_M1 + 3 are the M = 1 kernel compiled for growing
// variant sets (8B shapes, 0.6B shapes, every register variant, all).
// SK_VALU_M1_BLK .. + 3: the same sets for stacks holding block-scaled
// linears; SK_VALU_TOK_BLK .. + 3: such stacks at 2..8 tokens, run token by
// token through the M = 1 paths.
enum StackKernel : int32_t {
  SK_VALU_M1 = 0,
  SK_VALU_M2 = 4,
  SK_VALU_M4 = 5,
  SK_VALU_M8 = 6,
  SK_VALU_M1_BLK = 8,
  SK_VALU_TOK_BLK = 12,
  SK_MFMA = 16  // SK_MFMA + mfma_stack_variant(M, ragged)
};

// Launch parameters chosen by the launchers below.
struct LaunchShape {
  int grid, block, waves_per_block;
  int M, splits;  // tokens; linears split along K (0: no extra kernels)
};

// A launch counts its work-items (workgroups x threads per workgroup) in 32
// bits; the entry points refuse sizes whose launch would need more.
constexpr int64_t kMaxDispatchItems = 0xFFFFFFFFll;
// Work-items of the launches whose grid grows with the problem size.
int64_t pack_work_items(int64_t N);  // tern_pack, tern_unpack, tern_validate
int64_t pack5_work_items(int64_t N);
int64_t gemv5_work_items(int64_t N, int64_t K);
int64_t head_rowsum_work_items(int64_t N);
int64_t block_rowsum_work_items(int64_t N, int64_t K, int64_t B);
int64_t quantize_weights_work_items(int64_t N, int64_t K, int64_t B);
int64_t quantize_act_work_items(int64_t M);
// threads of one workgroup of the split clear / finish kernels (one per
// split linear and token)
constexpr int kSplitBlock = 256;

// ---- launchers (defined in the .hip files) ----
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_pack(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                       int32_t* rowsum, int32_t* bad, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, int64_t ldw,
                         hipStream_t s);
hipError_t launch_validate(const uint8_t* packed, int64_t N, int64_t K, int32_t* counts,
                           hipStream_t s);

// VALU path for one linear, M in {1, 2, 4} token registers (M <= 4).
hipError_t launch_valu_linear(const LinearArgs& a, hipStream_t s);
// MFMA path for one linear, any M (cus: compute units of the device, for
// the prefill GEMM's choice of tile).
hipError_t launch_mfma_linear(const LinearArgs& a, int cus, hipStream_t s);

// Rows handled per work unit (schedule granularity) of each path.
int valu_unit_rows(int32_t variant, int32_t M);
int mfma_unit_rows(int32_t variant);
// activation-window restages per unit of a linear with K columns (the
// window kernel restages once per 4096 columns when K exceeds one window)
int mfma_unit_restages(int32_t variant, int64_t K);
// y-only outputs a wave of the window stack kernel holds (0: none held), and
// whether a linear of K columns is walked window-major (its units in groups,
// window by window: each window staged once per group)
int mfma_held_units(int32_t variant);
bool mfma_window_major(int32_t variant, int64_t K, bool y_only);
bool mfma_per_workgroup(int32_t variant);
int32_t valu_variant_for(int64_t K);

// Persistent stack launches over a prepared workspace.
int32_t valu_stack_kernel_for(int32_t M, uint32_t used_variants, bool blocked);
// block-scaled linears at M = 1: the register variant (-1: none takes K) and
// its rows per unit
int32_t valu_blocked_variant(int64_t K, int64_t B);
int valu_blocked_unit_rows(int32_t variant);
hipError_t launch_valu_stack(int32_t kernel, const void* ws, const LaunchShape& shp,
                             hipStream_t s);
int valu_stack_blocks_per_cu(int32_t kernel);
// big: some linear's weight or output offsets do not fit the 32-bit offsets
// of the activation-window kernel (see mfma_win_offsets_fit)
int32_t mfma_stack_variant(int32_t M, bool ragged, bool big, bool blocked);
bool mfma_win_offsets_fit(int64_t N, int64_t ld, int64_t M, int64_t ldy);
// the prefill GEMM's variant for M tokens (any M >= 1, any K), and whether
// `variant` is the lockstep kernel (a workgroup takes whole rows over all K)
int32_t mfma_gemm_variant(int32_t M);
// the prefill GEMM variant for a stack of tiles512 512 x 128 tiles (variant
// unchanged if it is not the prefill GEMM's)
int32_t mfma_gemm_refine(int32_t variant, int32_t M, int64_t tiles512, int cus);
bool mfma_is_lockstep(int32_t variant);
// the activation-window kernel: is `variant` it, and its window width in K
bool mfma_is_window(int32_t variant);
int mfma_window_k();
// K columns of one step of the window kernels (block scales there come in
// whole steps)
int mfma_step_k();
// kernels that take linears split along K (window kernel, prefill GEMM), and
// the fill and finishing kernels of split linears
bool mfma_can_split(int32_t variant);
hipError_t launch_split_clear(const void* ws, const LaunchShape& shp, hipStream_t s);
hipError_t launch_split_finish(const void* ws, const LaunchShape& shp, hipStream_t s);

// Prefill GEMM (M > 16; tern_gemm.hip): one workgroup per tile of
// gemm_kind_rows(kind) rows x gemm_kind_tokens(kind) tokens.  Kind 0: 128 x
// 64 (M <= 64); 1: 256 x 128; 2: 512 x 128, for work of at least a few of
// its tiles per CU (tiles512: the work's tile count at 512 x 128).
int gemm_tile_tokens(int32_t M);
int gemm_kind(int32_t M, int64_t tiles512, int cus);
int gemm_kind_rows(int kind);
int gemm_kind_tokens(int kind);
hipError_t launch_gemm_linear(const LinearArgs& a, int cus, hipStream_t s);
hipError_t launch_gemm_stack(int kind, const void* ws, const LaunchShape& shp, hipStream_t s);
int gemm_stack_blocks_per_cu(int kind);
// token tiles of the prefill GEMM per row unit (its schedule counts tiles);
// 0 for every other kernel (its schedule counts rows)
int32_t mfma_token_tiles(int32_t variant, int32_t M);
hipError_t launch_mfma_stack(int32_t variant, const void* ws, const LaunchShape& shp,
                             hipStream_t s);
// int8 output head (tern_head.hip): M <= 8 tokens, workgroups of contiguous rows
int head_tokens(int64_t M);
int head_wg_per_cu();
int head_rows_per_unit(int64_t M);  // rows a workgroup takes per pass of its waves
int64_t head_lds_bytes(int64_t M, int64_t K, int64_t rows);
hipError_t launch_head(const int8_t* W, const float* s_row, const int32_t* rowsum, int64_t N, int64_t K,
                       int64_t ldw, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                       const int32_t* z, float* y, int64_t ldy, int32_t* acc, int64_t rows_per_wg,
                       hipStream_t s);
hipError_t launch_head_rowsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw, int32_t* rowsum,
                              hipStream_t s);
// one token against block-scaled ternary weights (tern_block.hip)
int blocked_rows_per_wave(int64_t K);
hipError_t launch_blocked_gemv(const uint8_t* packed, const float* s_b, const int32_t* rowsum_b, int64_t N,
                               int64_t K, int64_t B, const int8_t* q, const float* s_act, const int32_t* z,
                               float* y, int grid_blocks, hipStream_t s);
hipError_t launch_block_rowsum(const uint8_t* packed, int64_t N, int64_t K, int64_t B, int32_t* rowsum_b,
                               hipStream_t s);
// per-token asymmetric int8 quantisation of activations (tern_quant.hip)
int packed5_lanes_per_row(int64_t K);
hipError_t launch_pack5(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                        int32_t* rowsum, int32_t* bad, hipStream_t s);
hipError_t launch_gemv5(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
                        int64_t K, const int8_t* q, const float* s_act, const int32_t* z, float* y,
                        int32_t* acc, hipStream_t s);
hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, int64_t ldw, int64_t B,
                                   int8_t* t, int64_t ldt, float* s_b, hipStream_t s);
hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               int64_t ldq, float* s_act, int32_t* z, hipStream_t s);
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int grid, int unroll,
                             bool nontemporal, hipStream_t s);
int mfma_stack_blocks_per_cu(int32_t variant);

}  // namespace tern
