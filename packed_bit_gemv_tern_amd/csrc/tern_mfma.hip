// tern_mfma.hip -- MFMA int8 path of the ternary linear, for M >= 2 tokens
// (the batched verify pass of drafted decoding, and prefill-sized batches).
//
// The same packed weights serve M tokens (wiki entry "Neutrino-1", "What is
// actually new here": the 8B scores up to seven drafted tokens in one batched
// pass).  At M = 8 the VALU dot4 path would need 2.3 operations per weight,
// about twice what the VALU can issue at full HBM rate, so the contraction
// goes to the matrix cores with v_mfma_i32_16x16x64_i8:
//
//  * A operand: 16 tokens x 64 activations (int8 q as given; tokens past M
//    and activations past K are zero);
//  * B operand: 64 weights x 16 rows, decoded in registers from the packed
//    words: (w >> 2k) & 0x03030303 gives the codes c of weights 4k..4k+3, and
//    one v_perm_b32 per code word maps c = 0, 1, 2 to the signed bytes
//    -1, 0, +1 (a 4-entry byte table), so the MFMA sums w * q directly and
//    only z * rowsum remains for the epilogue;
//  * lane l of a wave holds row / token l % 16 and K-group l / 16; both
//    operands are filled with the same K positions per (lane, byte), so the
//    sum is over all of K whatever order the hardware pairs them in;
//  * result: lane l, register v holds token 4*(l/16)+v of row l%16.
//
// A wave computes R blocks of 16 rows for T blocks of 16 tokens; weights are
// loaded once per (R-unit, token group) with coalesced 16-byte non-temporal
// loads.
#include "tern_device.h"

namespace tern {

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kR = 4;  // row blocks of 16 per wave

// Code byte c in {0, 1, 2} -> weight byte {-1, 0, +1}: v_perm_b32 picks byte
// c of the table 0x000100FF (both halves hold the table, so the operand
// order of the builtin does not matter).
constexpr uint32_t kCodeTable = 0x000100FFu;

__device__ __forceinline__ i32x4 decode_word(uint32_t x) {
  i32x4 b;
  b[0] = (int32_t)__builtin_amdgcn_perm(kCodeTable, kCodeTable, x & 0x03030303u);
  b[1] = (int32_t)__builtin_amdgcn_perm(kCodeTable, kCodeTable, (x >> 2) & 0x03030303u);
  b[2] = (int32_t)__builtin_amdgcn_perm(kCodeTable, kCodeTable, (x >> 4) & 0x03030303u);
  b[3] = (int32_t)__builtin_amdgcn_perm(kCodeTable, kCodeTable, (x >> 6) & 0x03030303u);
  return b;
}

// 16 activations of token row `qrow` starting at column j0, zero past K.
__device__ __forceinline__ i32x4 load_q16(const int8_t* qrow, int K, int j0) {
  if (j0 + 16 <= K) {
    const u32x4 t = load16(qrow + j0);
    return i32x4{(int32_t)t.x, (int32_t)t.y, (int32_t)t.z, (int32_t)t.w};
  }
  i32x4 v = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t d = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + 4 * i + b;
      if (j < K) d |= (uint32_t)(uint8_t)load_g(qrow + j) << (8 * b);
    }
    v[i] = (int32_t)d;
  }
  return v;
}

// Units of 16*R rows, unit0 + k*ustride, inside [row_lo, row_hi); every
// token group of T*16 tokens for each unit.
template <int R, int T>
__device__ __forceinline__ void mfma_range(const LinearArgs& a, int row_lo, int row_hi, int unit0,
                                           int ustride, int lane) {
  constexpr int UNIT = 16 * R;
  const int r = lane & 15, g = lane >> 4;
  const int nch = a.nch, K = a.K, M = a.M;
  const int nks = (nch + 3) / 4;  // K-steps of 4 chunks (256 weights)

  for (int unit = unit0;; unit += ustride) {
    const int base = row_lo + unit * UNIT;
    if (base >= row_hi) break;
    for (int tok0 = 0; tok0 < M; tok0 += 16 * T) {
      i32x4 acc[R][T];
#pragma unroll
      for (int b = 0; b < R; ++b)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[b][t] = i32x4{0, 0, 0, 0};

      for (int ks = 0; ks < nks; ++ks) {
        const int ch = 4 * ks + g;
        const bool ch_ok = ch < nch;
        u32x4 w[R];
#pragma unroll
        for (int b = 0; b < R; ++b) {
          const int row = base + 16 * b + r;
          w[b] = (ch_ok && row < row_hi) ? load_weights16(a.packed + (int64_t)row * a.ld + 16 * ch)
                                         : u32x4{0, 0, 0, 0};
        }
        i32x4 qa[T][4];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int m = tok0 + 16 * t + r;
          const int8_t* qrow = a.q + (int64_t)m * a.ldq;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            qa[t][j] = (ch_ok && m < M) ? load_q16(qrow, K, 64 * ch + 16 * j) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int b = 0; b < R; ++b) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i32x4 wb = decode_word(w[b][j]);
#pragma unroll
            for (int t = 0; t < T; ++t)
              acc[b][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[t][j], wb, acc[b][t], 0, 0, 0);
          }
        }
      }

      // epilogue: lane holds tokens tok0 + 16t + 4g + v of row base + 16b + r
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int row = base + 16 * b + r;
        if (row >= row_hi) continue;
        const int32_t rs = load_g(a.rowsum + row);
        const float sr = load_g(a.s_row + row);
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = tok0 + 16 * t + 4 * g + v;
            if (m < M) {
              const int32_t accv =
                  (int32_t)((uint32_t)acc[b][t][v] - (uint32_t)load_g(a.z + m) * (uint32_t)rs);
              const int64_t o = (int64_t)m * a.ldy + row;
              store_g(a.y + o, epilogue(sr, accv, load_g(a.s_act + m)));
              if (a.acc) store_g(a.acc + o, accv);
            }
          }
        }
      }
    }
  }
}

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ int xcd_logical_block() {
  const int n = gridDim.x, b = blockIdx.x;
  return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

}  // namespace

template <int T>
__global__ __launch_bounds__(kBlock) void mfma_linear_kernel(LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesPerBlock + wave_id_uniform();
  const int nw = gridDim.x * kWavesPerBlock;
  mfma_range<kR, T>(a, 0, a.N, wave, nw, lane);
}

template <int T>
__global__ __launch_bounds__(kBlock) void mfma_stack_kernel(const StackHeader* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const int worker = xcd_logical_block() * kWavesPerBlock + wave_id_uniform();
  if (worker >= h->workers) return;
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(base + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(base + h->off_seg);
  const int s1 = seg_start[worker + 1];
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    mfma_range<kR, T>(a, sg.row_begin, sg.row_end, 0, 1, lane);
  }
}

int mfma_unit_rows(int32_t /*M*/) { return 16 * kR; }

static int mfma_t(int32_t M) { return M <= 16 ? 1 : 4; }

hipError_t launch_mfma_linear(const LinearArgs& a, hipStream_t s) {
  const int64_t units = (a.N + 16 * kR - 1) / (16 * kR);
  int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(kBlock);
  if (mfma_t(a.M) == 1)
    hipLaunchKernelGGL(mfma_linear_kernel<1>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(mfma_linear_kernel<4>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mfma_stack(int32_t M, const void* ws, const LaunchShape& shp, hipStream_t s) {
  const StackHeader* h = static_cast<const StackHeader*>(ws);
  const dim3 grid(shp.grid), block(shp.block);
  if (mfma_t(M) == 1)
    hipLaunchKernelGGL(mfma_stack_kernel<1>, grid, block, 0, s, h);
  else
    hipLaunchKernelGGL(mfma_stack_kernel<4>, grid, block, 0, s, h);
  return hipGetLastError();
}

int mfma_stack_blocks_per_cu(int32_t M) {
  int n = 0;
  hipError_t e = mfma_t(M) == 1
                     ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mfma_stack_kernel<1>, kBlock, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mfma_stack_kernel<4>, kBlock, 0);
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace tern
