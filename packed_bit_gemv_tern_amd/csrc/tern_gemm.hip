// tern_gemm.hip -- prefill-sized batches (M > 16 tokens): a tiled int8 GEMM
// on the matrix cores with the ternary weights decoded in registers.
//
// At prefill M the same packed weights meet hundreds of tokens (wiki entry
// "Neutrino-1", model card "Overview": the weights stay packed and are
// decoded inside the matrix kernels), so the work is a dense contraction and
// the tile below is the usual one: a workgroup owns ROWS output rows x BM
// tokens (256 x 128 with eight waves, or 128 x 64 with four) and walks K in
// steps of 64.
//
//  * Each K-step's operands go HBM/L2 -> LDS by DMA (global_load_lds): the
//    BM x 64 activation tile and the ROWS x 16-byte packed weight tile, in a
//    ring of STAGES buffers, so that later steps are in flight while the
//    current ones are used (the loads take several steps of MFMA work to
//    arrive).  One barrier per SS steps (after each wave's own DMA for them
//    has landed) publishes those buffers and frees the SS the next DMAs
//    overwrite.  It is a bare s_barrier: the usual workgroup barrier also
//    waits for every load in flight, which would drain the ring.
//  * The tile's row operands (rowsum, s_row) and token operands (z, s_act)
//    come in with the first step by 4-byte DMA into LDS, so the epilogue has
//    no dependent global loads.
//  * v_mfma_i32_16x16x64_i8: A = 16 tokens x 64 activations (lane (r, g):
//    token r, K positions 16g..16g+15 of the step), B = 64 weights x 16 rows
//    (lane (r, g): the packed dword g of row r, i.e. the same 16 K
//    positions, decoded to signed bytes by one v_perm_b32 per 4 codes).  The
//    MFMA then sums w * q directly and the epilogue only subtracts
//    z * rowsum.  Result: lane l, register v holds token 4 (l / 16) + v of
//    row l % 16.
//  * Activation tile layout: token t's 16-byte chunk c of the step sits at
//    t * 64 + 16 (c ^ f(t)), f(t) = t.bit2 | (t.bit1 ^ t.bit3) << 1, so that
//    a 128-bit LDS read of 16 tokens (one chunk each) touches every bank
//    once per 128 bytes whether the hardware serves it 8 or 16 lanes at a
//    time.
//  * K not a multiple of 64: activation bytes at K positions >= K are zeroed
//    in registers on the last step (packed padding columns decode to 0 as
//    well); tokens past M and rows past N are read at clamped addresses and
//    never stored.
#include <algorithm>

#include "tern_device.h"

namespace tern {

namespace {

constexpr uint32_t kGCodeTable = 0x000100FFu;  // code byte 0, 1, 2 -> -1, 0, +1

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Tile shapes.  BM = 128: 256 rows x 128 tokens, eight waves in a 4 x 2 grid
// of 64 rows x 64 tokens each.  BM = 64: 128 rows x 64 tokens, four waves of
// 32 rows x 64 tokens.  Every wave brings 32 weight rows and BM / 16 / WAVES
// activation instructions per step, so all waves issue the same count.
template <int BM>
struct GemmShape {
  static constexpr int ROWS = BM == 128 ? 256 : 128;
  static constexpr int WAVES = BM == 128 ? 8 : 4;
  static constexpr int RGROUPS = BM == 128 ? 4 : 4;  // row groups of the wave grid
  static constexpr int WT = 4;                       // token blocks of 16 per wave
  static constexpr int WR = ROWS / RGROUPS / 16;     // row blocks of 16 per wave
  static constexpr int QLD = BM / 16 / WAVES;        // activation DMA instructions per wave
  static constexpr int PER = QLD + 1;                // DMA instructions per wave per step
  // LDS ring depth and K-steps per barrier.  The 64-token tile waits and
  // synchronises once per 6 steps (a barrier per step kept its four waves in
  // the same phase, LDS reads and MFMAs never overlapping: 133 -> 84 us per
  // four 8B layers at M = 64); the eight-wave 128-token tile, which is bound
  // by LDS bandwidth, was slower that way and keeps one barrier per step.
  static constexpr int STAGES = BM == 128 ? 6 : 12;
  static constexpr int SS = BM == 128 ? 1 : 6;
  static constexpr int META = (2 * ROWS + 2 * BM) / 64;  // operand DMA instructions per tile
  static_assert(WAVES * 32 == ROWS && QLD * WAVES * 16 == BM, "tile shape");
  static_assert(PER * (STAGES - 2 * SS) < 64 && STAGES % SS == 0, "vmcnt field");
};

template <int BM>
struct GemmTiles {
  using S = GemmShape<BM>;
  uint8_t q[S::STAGES][BM * 64];
  uint8_t w[S::STAGES][S::ROWS * 16];
  int32_t rowsum[S::ROWS];
  float s_row[S::ROWS];
  int32_t z[BM];
  float s_act[BM];
};

__device__ __forceinline__ i32x4 gemm_decode(uint32_t x) {
  i32x4 b;
  b[0] = (int32_t)__builtin_amdgcn_perm(kGCodeTable, kGCodeTable, x & 0x03030303u);
  b[1] = (int32_t)__builtin_amdgcn_perm(kGCodeTable, kGCodeTable, (x >> 2) & 0x03030303u);
  b[2] = (int32_t)__builtin_amdgcn_perm(kGCodeTable, kGCodeTable, (x >> 4) & 0x03030303u);
  b[3] = (int32_t)__builtin_amdgcn_perm(kGCodeTable, kGCodeTable, (x >> 6) & 0x03030303u);
  return b;
}

template <int N>
__device__ __forceinline__ void gemm_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which waits
// for all of the wave's loads in flight); the clobber keeps the compiler from
// moving memory accesses across it.  LDS written by DMA is complete once the
// writing wave's vmcnt says so, and each wave waits for its own before this.
__device__ __forceinline__ void gemm_barrier() { asm volatile("s_barrier" ::: "memory"); }

// swizzle of 16-byte activation chunks within a token's 64 bytes
__device__ __forceinline__ int gemm_qswz(int t) { return ((t >> 2) & 1) | ((((t >> 1) ^ (t >> 3)) & 1) << 1); }

__device__ __forceinline__ int gemm_wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Zero the bytes of a 16-byte activation fragment whose K position (first
// byte at j0) is >= K.
__device__ __forceinline__ i32x4 gemm_mask_tail(i32x4 v, int j0, int K) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int n = K - (j0 + 4 * d);  // bytes of this dword still inside K
    const uint32_t keep = n >= 4 ? 0xFFFFFFFFu : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
    v[d] = (int32_t)((uint32_t)v[d] & keep);
  }
  return v;
}

// One ROWS x BM tile over all of K: rows row0.., tokens tok0..  With SPLIT,
// `flags` may mark the tile as one K-window of a linear split along K: its
// exact int32 sums are then added into y viewed as int32 (cleared before the
// launch and finished after it), the zero-point term in one window only.
template <int BM, bool SPLIT>
__device__ __forceinline__ void gemm_tile(const LinearArgs& a, int row0, int tok0, int lane, int w,
                                          GemmTiles<BM>& L, int flags) {
  using S = GemmShape<BM>;
  const int r = lane & 15, g = lane >> 4;
  const int K = a.K, M = a.M, N = a.N;
  const int nks = a.nch;  // K-steps: one 16-byte packed chunk (64 weights) per row each
  // this wave's place in the tile
  const int wr = w % S::RGROUPS, wt = w / S::RGROUPS;
  const int rbase = wr * 16 * S::WR, tbase = wt * 64;

  // DMA sources: activation rows for this wave's QLD instructions, and the
  // weight row of lane l < 32 (rows 32w + l of the tile)
  const int8_t* qsrc[S::QLD];
  int qchunk[S::QLD];
#pragma unroll
  for (int j = 0; j < S::QLD; ++j) {
    const int i = w * S::QLD + j;                 // instruction: tokens 16i .. 16i+15
    const int t = 16 * i + (lane >> 2);           // token within the tile
    qchunk[j] = (lane & 3) ^ gemm_qswz(t);        // source chunk of this LDS slot
    qsrc[j] = a.q + (int64_t)min(tok0 + t, M - 1) * a.ldq;
  }
  const uint8_t* wsrc = a.packed + (int64_t)min(row0 + 32 * w + (lane & 31), N - 1) * a.ld;
  const int qmax = a.ldq - 16;  // last in-row 16-byte activation chunk

  // row and token operands of the tile, 64 values (4 bytes per lane) per
  // DMA instruction: rowsum, then s_row (ROWS each), then z, s_act (BM each);
  // instruction j goes to wave j % WAVES
  auto issue_meta = [&]() {
    for (int j = w; j < S::META; j += S::WAVES) {
      const void* src;
      void* dst;
      int k = j;
      if (k < S::ROWS / 64) {
        src = a.rowsum + min(row0 + 64 * k + lane, N - 1), dst = &L.rowsum[64 * k];
      } else if ((k -= S::ROWS / 64) < S::ROWS / 64) {
        src = a.s_row + min(row0 + 64 * k + lane, N - 1), dst = &L.s_row[64 * k];
      } else if ((k -= S::ROWS / 64) < BM / 64) {
        src = a.z + min(tok0 + 64 * k + lane, M - 1), dst = &L.z[64 * k];
      } else {
        k -= BM / 64;
        src = a.s_act + min(tok0 + 64 * k + lane, M - 1), dst = &L.s_act[64 * k];
      }
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 4, 0, 0);
    }
  };

  auto issue = [&](int k) {
    const int s = k % S::STAGES;
#pragma unroll
    for (int j = 0; j < S::QLD; ++j) {
      const int off = min(64 * k + 16 * qchunk[j], qmax);
      __builtin_amdgcn_global_load_lds((const void*)(qsrc[j] + off),
                                       (lds_ptr_t)(&L.q[s][1024 * (w * S::QLD + j)]), 16, 0, 0);
    }
    if (lane < 32)
      __builtin_amdgcn_global_load_lds((const void*)(wsrc + 16 * k), (lds_ptr_t)(&L.w[s][512 * w]),
                                       16, 0, 0);
  };

  i32x4 acc[S::WR][S::WT];
#pragma unroll
  for (int b = 0; b < S::WR; ++b)
#pragma unroll
    for (int t = 0; t < S::WT; ++t) acc[b][t] = i32x4{0, 0, 0, 0};

  // a step's operands in registers: packed weight dwords and activation
  // fragments (the tail of K zeroed)
  struct Ops {
    uint32_t wd[S::WR];
    i32x4 qa[S::WT];
  };
  auto load_ops = [&](int k, Ops& o) {
    const int s = k % S::STAGES;
#pragma unroll
    for (int b = 0; b < S::WR; ++b)
      o.wd[b] = *reinterpret_cast<const uint32_t*>(&L.w[s][16 * (rbase + 16 * b + r) + 4 * g]);
#pragma unroll
    for (int t = 0; t < S::WT; ++t) {
      const int tt = tbase + 16 * t + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&L.q[s][64 * tt + 16 * (g ^ gemm_qswz(tt))]);
      o.qa[t] = i32x4{(int32_t)v.x, (int32_t)v.y, (int32_t)v.z, (int32_t)v.w};
    }
    if (64 * k + 64 > K) {
#pragma unroll
      for (int t = 0; t < S::WT; ++t) o.qa[t] = gemm_mask_tail(o.qa[t], 64 * k + 16 * g, K);
    }
  };
  auto compute = [&](const Ops& o) {
#pragma unroll
    for (int b = 0; b < S::WR; ++b) {
      const i32x4 wb = gemm_decode(o.wd[b]);
#pragma unroll
      for (int t = 0; t < S::WT; ++t)
        acc[b][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.qa[t], wb, acc[b][t], 0, 0, 0);
    }
  };
  issue_meta();  // older than every step's loads, so step 0's wait covers it
#pragma unroll
  for (int s = 0; s < S::STAGES - S::SS; ++s)
    if (s < nks) issue(s);
  // step k: my loads landed (later steps may still fly), then everybody's;
  // the barrier also frees the buffer the next issue reuses
  // steps k0 .. k0 + SS - 1 landed (mine, then everybody's); the barrier
  // also frees the SS buffers the next issues reuse, read in the previous
  // round
  for (int k0 = 0; k0 < nks; k0 += S::SS) {
    if (nks - k0 - S::SS >= S::STAGES - 2 * S::SS)
      gemm_wait_vm<S::PER * (S::STAGES - 2 * S::SS)>();
    else
      gemm_wait_vm<0>();
    gemm_barrier();
#pragma unroll
    for (int i = 0; i < S::SS; ++i)
      if (k0 + S::STAGES - S::SS + i < nks) issue(k0 + S::STAGES - S::SS + i);
#pragma unroll
    for (int i = 0; i < S::SS; ++i) {
      if (k0 + i < nks) {
        Ops o;
        load_ops(k0 + i, o);
        compute(o);
      }
    }
  }

  // epilogue: lane holds tokens tok0 + tbase + 16t + 4g + v of row row0 + rbase + 16b + r
  const bool partial = SPLIT && (flags & kSegPartial) != 0;
  const bool zpoint = !partial || (flags & kSegZeroPoint) != 0;
#pragma unroll
  for (int b = 0; b < S::WR; ++b) {
    const int rl = rbase + 16 * b + r;
    const int row = row0 + rl;
    if (row >= N) continue;
    const int32_t rs = L.rowsum[rl];
    const float sr = L.s_row[rl];
#pragma unroll
    for (int t = 0; t < S::WT; ++t) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ml = tbase + 16 * t + 4 * g + v;
        const int m = tok0 + ml;
        if (m < M) {
          const int32_t zz = zpoint ? L.z[ml] : 0;
          const int32_t accv = (int32_t)((uint32_t)acc[b][t][v] - (uint32_t)zz * (uint32_t)rs);
          const int64_t o = (int64_t)m * a.ldy + row;
          if (partial) {
            __hip_atomic_fetch_add((int32_t __attribute__((address_space(1)))*)(reinterpret_cast<int32_t*>(a.y) + o),
                                   accv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            store_g(a.y + o, epilogue(sr, accv, L.s_act[ml]));
            if (a.acc) store_g(a.acc + o, accv);
          }
        }
      }
    }
  }
  // every wave is done with the ring and the operands before the next
  // tile's prologue overwrites them
  gemm_barrier();
}

// Tiles tile0, tile0 + tstride, ... below tile1 of a linear, numbered in
// (row tile, token tile) order: tile = row_tile * token_tiles + token_tile,
// so the token tiles of one row tile are adjacent.
template <int BM, bool SPLIT>
__device__ __forceinline__ void gemm_range(const LinearArgs& a, int tile0, int tile1, int tstride,
                                           int lane, int w, GemmTiles<BM>& L, int flags) {
  const int ntok = (int)(((int64_t)a.M + BM - 1) / BM);
  for (int tile = tile0; tile < tile1; tile += tstride) {
    const int rt = tile / ntok, tt = tile - rt * ntok;
    gemm_tile<BM, SPLIT>(a, rt * GemmShape<BM>::ROWS, tt * BM, lane, w, L, flags);
  }
}

__device__ __forceinline__ int gemm_xcd_block() {
  const int n = gridDim.x, b = blockIdx.x;
  return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

template <int BM>
__global__ __launch_bounds__(64 * GemmShape<BM>::WAVES) __attribute__((amdgpu_waves_per_eu(BM == 128 ? 2 : 4)))
void gemm_linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) GemmTiles<BM> L;
  constexpr int ROWS = GemmShape<BM>::ROWS;
  const int ntiles = (int)((((int64_t)a.N + ROWS - 1) / ROWS) * (((int64_t)a.M + BM - 1) / BM));
  gemm_range<BM, false>(a, gemm_xcd_block(), ntiles, gridDim.x, threadIdx.x & 63, gemm_wave_id(), L, 0);
}

template <int BM, bool SPLIT>
__global__ __launch_bounds__(64 * GemmShape<BM>::WAVES) __attribute__((amdgpu_waves_per_eu(BM == 128 ? 2 : 4)))
void gemm_stack_kernel(const StackHeader* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) GemmTiles<BM> L;
  const int worker = gemm_xcd_block();
  if (worker >= h->workers) return;  // the same for the whole workgroup
  const int lane = threadIdx.x & 63;
  const int w = gemm_wave_id();
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(base + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(base + h->off_seg);
  const int s1 = seg_start[worker + 1];
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    gemm_range<BM, SPLIT>(a, sg.row_begin, sg.row_end, 1, lane, w, L, SPLIT ? sg.flags : 0);
  }
}

template <typename F>
static hipError_t with_gemm_stack_kernel(int bm, bool split, F&& f) {
  if (split) return bm == 128 ? f(gemm_stack_kernel<128, true>) : f(gemm_stack_kernel<64, true>);
  return bm == 128 ? f(gemm_stack_kernel<128, false>) : f(gemm_stack_kernel<64, false>);
}

}  // namespace

int gemm_tile_tokens(int32_t M) { return M > 64 ? 128 : 64; }

int gemm_unit_rows(int bm) { return bm == 128 ? GemmShape<128>::ROWS : GemmShape<64>::ROWS; }

static int gemm_block(int bm) { return 64 * (bm == 128 ? GemmShape<128>::WAVES : GemmShape<64>::WAVES); }

hipError_t launch_gemm_linear(const LinearArgs& a, hipStream_t s) {
  const int bm = gemm_tile_tokens(a.M);
  const int rows = gemm_unit_rows(bm);
  const int64_t tiles = (((int64_t)a.N + rows - 1) / rows) * (((int64_t)a.M + bm - 1) / bm);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(tiles, 65535));
  const dim3 grid((unsigned)blocks), block(gemm_block(bm));
  if (bm == 128)
    hipLaunchKernelGGL(gemm_linear_kernel<128>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(gemm_linear_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_stack(int bm, const void* ws, const LaunchShape& shp, hipStream_t s) {
  const StackHeader* h = static_cast<const StackHeader*>(ws);
  const bool split = shp.splits > 0;
  if (split) {
    const hipError_t e = launch_split_clear(ws, shp, s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = with_gemm_stack_kernel(bm, split, [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(shp.grid), dim3(gemm_block(bm)), 0, s, h);
    return hipGetLastError();
  });
  if (e != hipSuccess || !split) return e;
  return launch_split_finish(ws, shp, s);
}

int gemm_stack_blocks_per_cu(int bm) {
  int n = 0;
  const hipError_t e = with_gemm_stack_kernel(bm, false, [&](auto kern) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, gemm_block(bm), 0);
  });
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace tern
