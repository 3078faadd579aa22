// tern_gemm.hip -- prefill-sized batches (M > 16 tokens): a tiled int8 GEMM
// on the matrix cores with the ternary weights decoded in registers.
//
// At prefill M the same packed weights meet hundreds of tokens (wiki entry
// "Neutrino-1", model card "Overview": the weights stay packed and are
// decoded inside the matrix kernels), so the work is a dense contraction and
// the tile below is the usual one: a workgroup owns ROWS output rows x BM
// tokens (512 x 128 with eight waves, or 128 x 64 with four) and walks K in
// steps of 64.  The two tiles stage their operands differently (below).
//
//  * 64-token tile: each K-step's operands go HBM/L2 -> LDS by DMA (global_load_lds): the
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
#include <type_traits>

#include "tern_prologue.h"

namespace tern {

namespace {

constexpr uint32_t kGCodeTable = 0x000100FFu;  // code byte 0, 1, 2 -> -1, 0, +1

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The 64-token tile: 128 rows x 64 tokens, four waves of 32 rows x 64 tokens.
// Every wave brings ROWS / WAVES weight rows and BM / 16 / WAVES activation
// instructions per step, so all waves issue the same count.
template <int BM>
struct GemmShape {
  static_assert(BM == 64, "the 128-token tile is LineShape");
  static constexpr int ROWS = 128;
  static constexpr int WAVES = 4;
  static constexpr int RGROUPS = 4;                  // row groups of the wave grid
  static constexpr int WT = 4;                       // token blocks of 16 per wave
  static constexpr int WR = ROWS / RGROUPS / 16;     // row blocks of 16 per wave
  static constexpr int RPW = ROWS / WAVES;           // weight rows each wave brings (one lane each)
  static constexpr int QLD = BM / 16 / WAVES;        // activation DMA instructions per wave
  static constexpr int PER = QLD + 1;                // DMA instructions per wave per step
  // LDS ring depth and K-steps per barrier: the tile waits and synchronises
  // once per 6 steps (a barrier per step kept its four waves in the same
  // phase, LDS reads and MFMAs never overlapping: 133 -> 84 us per four 8B
  // layers at M = 64)
  static constexpr int STAGES = 12;
  static constexpr int SS = 6;
  static constexpr int META = (2 * ROWS + 2 * BM) / 64;  // operand DMA instructions per tile
  static_assert(RPW <= 64 && RGROUPS * WR * 16 == ROWS && (WAVES / RGROUPS) * WT * 16 == BM &&
                QLD * WAVES * 16 == BM, "tile shape");
  static_assert(PER * (STAGES - 2 * SS) < 64 && STAGES % SS == 0, "vmcnt field");
};

// The 128-token tiles: ROWS = 512 or 256 rows x 128 tokens, eight waves of
// ROWS / 8 rows x 128 tokens (two waves per SIMD; the decode of one weight
// dword serves eight MFMAs).  512-row tiles read each activation tile half
// as often; 256-row tiles give a stack twice as many, for stacks too small
// to fill the chip evenly with the larger ones (one 8B layer at M = 512:
// 304 of them for 256 workgroups).  Their operands are staged in runs of whole cache lines: a weight
// stage holds WS = 4 K-steps of every row (64 contiguous bytes), an
// activation stage AS = 2 K-steps of every token (128 bytes), each in a ring
// of RING stages.  Staged one K-step at a time, every row's 16 bytes and
// every token's 64 were an L2 request of their own (640 per step for four 8B
// layers at M = 512), and the requests in flight per CU, not bytes or MFMAs,
// set the pace.  Their MFMAs take the decoded weights as A and the
// activations as B, so that a lane's four results are four adjacent rows of
// one token (16 contiguous bytes of y) rather than four tokens of one row:
// the epilogue stores 16 bytes per instruction instead of 4 (four 8B layers
// at M = 512: 415.6 -> 389.3 us).
template <int ROWS_>
struct LineShape {
  static constexpr int ROWS = ROWS_, BM = 128, WAVES = 8;
  static constexpr int RGROUPS = 8, WR = ROWS / 128, WT = 8;  // wave grid 8 x 1
  static constexpr int WS = 4, AS = 2, RING = 3;
  static constexpr int WPW = ROWS * 16 * WS / 1024 / WAVES;  // weight DMA instructions per wave per stage
  static constexpr int APW = BM * 64 * AS / 1024 / WAVES;    // activation DMA instructions per wave per stage
  static constexpr int META = (2 * ROWS + 2 * BM) / 64;
  static_assert(WPW * WAVES * 1024 == ROWS * 16 * WS && APW * WAVES * 1024 == BM * 64 * AS, "stage split");
  static_assert(RGROUPS * WR * 16 == ROWS && (WAVES / RGROUPS) * WT * 16 == BM, "wave grid");
  static_assert(WS == 2 * AS && AS == 2 && RING == 3, "the boundary logic below assumes these");
  static_assert(WPW + APW < 64, "vmcnt field");
};

template <int ROWS>
struct LineTiles {
  using S = LineShape<ROWS>;
  uint8_t q[S::RING][S::BM * 64 * S::AS];    // [stage][token][8 pieces of 16 B], swizzled
  uint8_t w[S::RING][S::ROWS * 16 * S::WS];  // [stage][row][4 chunks of 16 B], swizzled
  int32_t rowsum[S::ROWS];
  float s_row[S::ROWS];
  int32_t z[S::BM];
  float s_act[S::BM];
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
  const int rbase = wr * 16 * S::WR, tbase = wt * 16 * S::WT;

  // DMA sources: activation rows for this wave's QLD instructions, and the
  // weight row of lane l < RPW (rows RPW w + l of the tile)
  const int8_t* qsrc[S::QLD];
  int qchunk[S::QLD];
#pragma unroll
  for (int j = 0; j < S::QLD; ++j) {
    const int i = w * S::QLD + j;                 // instruction: tokens 16i .. 16i+15
    const int t = 16 * i + (lane >> 2);           // token within the tile
    qchunk[j] = (lane & 3) ^ gemm_qswz(t);        // source chunk of this LDS slot
    qsrc[j] = a.q + (int64_t)min(tok0 + t, M - 1) * a.ldq;
  }
  const uint8_t* wsrc = a.packed + (int64_t)min(row0 + S::RPW * w + (lane & (S::RPW - 1)), N - 1) * a.ld;
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
    if (lane < S::RPW)
      __builtin_amdgcn_global_load_lds((const void*)(wsrc + 16 * k), (lds_ptr_t)(&L.w[s][16 * S::RPW * w]),
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

  // epilogue: lane holds tokens tok0 + tbase + 16t + 4g + v of row row0 +
  // rbase + 16b + r; token by token (its zero point and scale read once),
  // the rows' operands read from LDS where used
  const bool partial = SPLIT && (flags & kSegPartial) != 0;
  const bool zpoint = !partial || (flags & kSegZeroPoint) != 0;
#pragma unroll
  for (int t = 0; t < S::WT; ++t) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ml = tbase + 16 * t + 4 * g + v;
      const int m = tok0 + ml;
      if (m >= M) continue;
      const int32_t zz = zpoint ? L.z[ml] : 0;
      const float sa = L.s_act[ml];
      const int64_t o0 = (int64_t)m * a.ldy + row0 + rbase + r;
#pragma unroll
      for (int b = 0; b < S::WR; ++b) {
        const int rl = rbase + 16 * b + r;
        if (row0 + rl >= N) continue;
        const int32_t accv = (int32_t)((uint32_t)acc[b][t][v] - mul_zr(zz, L.rowsum[rl]));
        const int64_t o = o0 + 16 * b;
        if (partial) {
          __hip_atomic_fetch_add((int32_t __attribute__((address_space(1)))*)(reinterpret_cast<int32_t*>(a.y) + o),
                                 accv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          store_g(a.y + o, epilogue(L.s_row[rl], accv, sa));
          if (a.acc) store_g(a.acc + o, accv);
        }
      }
    }
  }
  // every wave is done with the ring and the operands before the next
  // tile's prologue overwrites them
  gemm_barrier();
}

// swizzles of 16-byte pieces in the line-staged rings: activation piece p of
// token t (8 per token) sits at position p ^ line_fa(t), weight chunk c of row
// rho (4 per row) at c ^ line_fw(rho).  A 128-bit activation read of 16 tokens
// (t % 16 = 0..15, one piece each) and a 32-bit weight read of 16 rows x 4
// dwords then touch every bank once per 128 bytes, whether the LDS serves
// 8 or 16 lanes (128 or 256 bytes) per cycle.
__device__ __forceinline__ int line_fa(int t) { return ((t >> 1) & 7) ^ ((t & 1) << 2); }
__device__ __forceinline__ int line_fw(int rho) { return ((rho >> 1) & 3) ^ ((rho >> 2) & 3); }

// One ROWS x 128 tile over all of K (see LineShape): rows row0.., tokens
// tok0..; SPLIT and flags as for gemm_tile.
//  * Weight stage J (K-steps 4J .. 4J+3) and activation stage j (K-steps 2j,
//    2j+1) live in ring slots J % 3 and j % 3.  At the boundary of K-step
//    k = 2j the wave waits for activation stage j (and, with it, weight stage
//    k / 4, issued earlier), then a barrier publishes them and frees the slots
//    of weight stage k / 4 - 1 and activation stage j - 1, which take weight
//    stage k / 4 + 2 (when k % 4 == 0) and activation stage j + 2: weights
//    arrive 8 K-steps ahead, activations 4.
//  * A weight DMA instruction brings 16 rows x 64 B (lane l: row l / 4, its
//    chunk (l % 4) ^ line_fw(row)), an activation one 8 tokens x 128 B (lane
//    l: token l / 8, piece (l % 8) ^ line_fa(token)); lane l lands at byte
//    16 l of the instruction's 1 KB block, so the pieces arrive swizzled.
//    Chunks past the row's last are read at the last (never used), pieces
//    past ldq at the row's last 16 bytes (they meet zero weights or are
//    masked), rows past N and tokens past M at the last one (never stored).
template <int ROWS, bool SPLIT>
__device__ __forceinline__ void gemm_tile_lines(const LinearArgs& a, int row0, int tok0, int lane, int w,
                                                LineTiles<ROWS>& L, int flags) {
  using S = LineShape<ROWS>;
  const int r = lane & 15, g = lane >> 4;
  const int K = a.K, M = a.M, N = a.N;
  const int nks = a.nch;
  const int nas = (nks + S::AS - 1) / S::AS, nws = (nks + S::WS - 1) / S::WS;
  const int wr = w % S::RGROUPS, wt = w / S::RGROUPS;
  const int rbase = wr * 16 * S::WR, tbase = wt * 16 * S::WT;

  // DMA sources: each issue derives its lanes' row / token index and swizzled
  // piece from the lane number afresh (an opaque copy, so that the compiler
  // cannot hoist them and hold twelve registers through the loop: the kernel
  // then spilled them and reloaded them at the issues, whose wait for the
  // reload also waited for every DMA in flight)
  const int qmax = a.ldq - 16;

  auto issue_meta = [&]() {
    for (int j = w; j < S::META; j += S::WAVES) {
      const void* src;
      void* dst;
      int k = j;
      if (k < S::ROWS / 64) {
        src = a.rowsum + min(row0 + 64 * k + lane, N - 1), dst = &L.rowsum[64 * k];
      } else if ((k -= S::ROWS / 64) < S::ROWS / 64) {
        src = a.s_row + min(row0 + 64 * k + lane, N - 1), dst = &L.s_row[64 * k];
      } else if ((k -= S::ROWS / 64) < S::BM / 64) {
        src = a.z + min(tok0 + 64 * k + lane, M - 1), dst = &L.z[64 * k];
      } else {
        k -= S::BM / 64;
        src = a.s_act + min(tok0 + 64 * k + lane, M - 1), dst = &L.s_act[64 * k];
      }
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 4, 0, 0);
    }
  };
  auto issue_w = [&](int J) {
    uint8_t* dst = L.w[J % S::RING];
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int i = 0; i < S::WPW; ++i) {
      const int rho = 16 * (w * S::WPW + i) + (l >> 2);
      const int row = min(row0 + rho, N - 1);
      const int ch = min(S::WS * J + ((l & 3) ^ line_fw(rho)), nks - 1);
      __builtin_amdgcn_global_load_lds((const void*)(a.packed + (int64_t)row * a.ld + 16 * ch),
                                       (lds_ptr_t)(dst + 1024 * (w * S::WPW + i)), 16, 0, 0);
    }
  };
  auto issue_a = [&](int j) {
    uint8_t* dst = L.q[j % S::RING];
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int i = 0; i < S::APW; ++i) {
      const int t = 8 * (w * S::APW + i) + (l >> 3);
      const int tok = min(tok0 + t, M - 1);
      const int off = min(64 * S::AS * j + 16 * ((l & 7) ^ line_fa(t)), qmax);
      __builtin_amdgcn_global_load_lds((const void*)(a.q + (int64_t)tok * a.ldq + off),
                                       (lds_ptr_t)(dst + 1024 * (w * S::APW + i)), 16, 0, 0);
    }
  };

  i32x4 acc[S::WR][S::WT];
#pragma unroll
  for (int b = 0; b < S::WR; ++b)
#pragma unroll
    for (int t = 0; t < S::WT; ++t) acc[b][t] = i32x4{0, 0, 0, 0};

  // this lane's read offsets within a stage: weight chunk c of row block b at
  // wofs[b] + 16 (c ^ fw), activation piece p of token block t at qofs[t] +
  // 16 (p ^ fa); fw and fa depend on the row / token only through r
  const int fw = line_fw(r), fa = line_fa(r);
  auto step = [&](const uint8_t* qs, const uint8_t* ws, int k, auto last) {
    uint32_t wd[S::WR];
    i32x4 qa[S::WT];
#pragma unroll
    for (int b = 0; b < S::WR; ++b)
      wd[b] = *reinterpret_cast<const uint32_t*>(ws + 64 * (rbase + 16 * b + r) + 16 * ((k & 3) ^ fw) + 4 * g);
#pragma unroll
    for (int t = 0; t < S::WT; ++t) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qs + 128 * (tbase + 16 * t + r) +
                                                      16 * ((4 * (k & 1) + g) ^ fa));
      qa[t] = i32x4{(int32_t)v.x, (int32_t)v.y, (int32_t)v.z, (int32_t)v.w};
    }
    if constexpr (decltype(last)::value) {  // the tail of K lies in the last stage
#pragma unroll
      for (int t = 0; t < S::WT; ++t) qa[t] = gemm_mask_tail(qa[t], 64 * k + 16 * g, K);
    }
#pragma unroll
    for (int b = 0; b < S::WR; ++b) {
      const i32x4 wb = gemm_decode(wd[b]);
#pragma unroll
      for (int t = 0; t < S::WT; ++t)
        acc[b][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wb, qa[t], acc[b][t], 0, 0, 0);
    }
    // issue order: the LDS reads, the first row block's decode, then each
    // MFMA followed by a share of the next row block's decode, so that the
    // VALU works while the matrix core does (in program order the decode of
    // block b + 1 waited for block b's MFMAs to release its registers)
    constexpr int kDecode = 11;                               // VALU per decoded dword
    constexpr int kShare = (kDecode + S::WT - 1) / S::WT + 1;  // VALU after each MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, S::WR / 2 + S::WT, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x002, kDecode + 1, 0);       // VALU
#pragma unroll
    for (int i = 0; i < S::WR * S::WT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, kShare, 0);
    }
  };

  issue_meta();  // older than every stage's loads, so the first wait covers it
  issue_w(0);
  issue_a(0);
  if (nws > 1) issue_w(1);
  if (nas > 1) issue_a(1);
  auto stage = [&](int j, auto last) {
    const int k = S::AS * j;
    // loads issued after activation stage j: those of the previous boundary
    // (or, for j = 0, of the prologue), weights before activations
    const bool w_after = j == 0 ? nws > 1 : ((k - 2) & 3) == 0 && (k - 2) / 4 + 2 < nws;
    const bool a_after = j + 1 < nas;
    if (w_after) {
      if (a_after)
        gemm_wait_vm<S::WPW + S::APW>();
      else
        gemm_wait_vm<S::WPW>();
    } else {
      if (a_after)
        gemm_wait_vm<S::APW>();
      else
        gemm_wait_vm<0>();
    }
    gemm_barrier();
    if ((k & 3) == 0 && k / 4 + 2 < nws) issue_w(k / 4 + 2);
    if (j + 2 < nas) issue_a(j + 2);
    const uint8_t* qs = L.q[j % S::RING];
    const uint8_t* ws = L.w[(k / 4) % S::RING];
    step(qs, ws, k, last);
    __builtin_amdgcn_sched_barrier(0);  // one step's operands in registers at a time
    if (k + 1 < nks) step(qs, ws, k + 1, last);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int j = 0; j + 1 < nas; ++j) stage(j, std::false_type{});
  stage(nas - 1, std::true_type{});

  // epilogue: lane (r, g) holds rows row0 + rbase + 16b + 4g + v (v = 0..3)
  // of token tok0 + tbase + 16t + r, i.e. 16 contiguous bytes of y's token
  // row: one 16-byte store per (b, t) where y's rows allow it.  (The lane's
  // row and token offsets are taken here, where the compiler cannot lift the
  // addresses derived from them above the loop and hold them through it.)
  const bool partial = SPLIT && (flags & kSegPartial) != 0;
  const bool zpoint = !partial || (flags & kSegZeroPoint) != 0;
  const bool vec = (a.ldy & 3) == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.acc) & 15) == 0;
  int rl0 = rbase + 4 * g, ml0 = tbase + r;
  asm volatile("" : "+v"(rl0), "+v"(ml0));
  int32_t zz[S::WT];
  float sa[S::WT];
#pragma unroll
  for (int t = 0; t < S::WT; ++t) {
    zz[t] = zpoint ? L.z[ml0 + 16 * t] : 0;
    sa[t] = L.s_act[ml0 + 16 * t];
  }
#pragma unroll
  for (int b = 0; b < S::WR; ++b) {
    const int row = row0 + rl0 + 16 * b;  // the first of the lane's four
    const i32x4 rsum = *reinterpret_cast<const i32x4*>(&L.rowsum[rl0 + 16 * b]);
    const f32x4 srow = *reinterpret_cast<const f32x4*>(&L.s_row[rl0 + 16 * b]);
#pragma unroll
    for (int t = 0; t < S::WT; ++t) {
      const int m = tok0 + ml0 + 16 * t;
      if (m >= M) continue;
      i32x4 av;
      f32x4 yv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        av[v] = (int32_t)((uint32_t)acc[b][t][v] - mul_zr(zz[t], rsum[v]));
        yv[v] = epilogue(srow[v], av[v], sa[t]);
      }
      const int64_t o = (int64_t)m * a.ldy + row;
      if (partial) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (row + v < N)
            __hip_atomic_fetch_add(
                (int32_t __attribute__((address_space(1)))*)(reinterpret_cast<int32_t*>(a.y) + o + v), av[v],
                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (vec && row + 3 < N) {
        store_g(reinterpret_cast<f32x4*>(a.y + o), yv);
        if (a.acc) store_g(reinterpret_cast<i32x4*>(a.acc + o), av);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (row + v >= N) continue;
          store_g(a.y + o + v, yv[v]);
          if (a.acc) store_g(a.acc + o + v, av[v]);
        }
      }
    }
  }
  gemm_barrier();
}

// Tile kinds: BM = 64 with 128 rows (gemm_tile), BM = 128 with 256 or 512
// rows (gemm_tile_lines).
template <int BM, int ROWS>
struct GemmTile;
template <>
struct GemmTile<64, 128> {
  using Shape = GemmShape<64>;
  using Tiles = GemmTiles<64>;
};
template <int ROWS>
struct GemmTile<128, ROWS> {
  using Shape = LineShape<ROWS>;
  using Tiles = LineTiles<ROWS>;
};

// Tiles tile0, tile0 + tstride, ... below tile1 of a linear, numbered in
// (row tile, token tile) order: tile = row_tile * token_tiles + token_tile,
// so the token tiles of one row tile are adjacent.
template <int BM, int ROWS, bool SPLIT>
__device__ __forceinline__ void gemm_range(const LinearArgs& a, int tile0, int tile1, int tstride,
                                           int lane, int w, typename GemmTile<BM, ROWS>::Tiles& L, int flags) {
  const int ntok = (int)(((int64_t)a.M + BM - 1) / BM);
  for (int tile = tile0; tile < tile1; tile += tstride) {
    const int rt = tile / ntok, tt = tile - rt * ntok;
    if constexpr (BM == 128)
      gemm_tile_lines<ROWS, SPLIT>(a, rt * ROWS, tt * BM, lane, w, L, flags);
    else
      gemm_tile<BM, SPLIT>(a, rt * ROWS, tt * BM, lane, w, L, flags);
  }
}

__device__ __forceinline__ int gemm_xcd_block() {
  const int n = gridDim.x, b = blockIdx.x;
  return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

template <int BM, int ROWS>
__global__ __launch_bounds__((64 * GemmTile<BM, ROWS>::Shape::WAVES)) __attribute__((amdgpu_waves_per_eu(BM == 128 ? 2 : 4)))
void gemm_linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) typename GemmTile<BM, ROWS>::Tiles L;
  const int ntiles = (int)((((int64_t)a.N + ROWS - 1) / ROWS) * (((int64_t)a.M + BM - 1) / BM));
  gemm_range<BM, ROWS, false>(a, gemm_xcd_block(), ntiles, gridDim.x, threadIdx.x & 63, gemm_wave_id(), L, 0);
}

template <int BM, int ROWS, bool SPLIT>
__global__ __launch_bounds__((64 * GemmTile<BM, ROWS>::Shape::WAVES)) __attribute__((amdgpu_waves_per_eu(BM == 128 ? 2 : 4)))
void gemm_stack_kernel(const StackHeader* __restrict__ h,
                                  StackSync* __restrict__ sy) {
  // one LDS object: with two, the compiler tags every LDS access with its
  // object's alias scope and then makes the first LDS read after a tile DMA
  // wait for that DMA (the tag says "may alias"), which drained the rings
  struct Lds {
    typename GemmTile<BM, ROWS>::Tiles tiles;
    PrologueLds prol;
  };
  __shared__ __attribute__((aligned(16))) Lds lds;
  auto& L = lds.tiles;
  const uint32_t launch1 = stack_prologue(h, sy, lds.prol);
  const int worker = gemm_xcd_block();
  if (worker >= h->workers) return;  // the same for the whole workgroup
  const int lane = threadIdx.x & 63;
  const int w = gemm_wave_id();
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(base + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(base + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    gemm_range<BM, ROWS, SPLIT>(a, sg.row_begin, sg.row_end, 1, lane, w, L, SPLIT ? sg.flags : 0);
  }
}

// kind 0: 128 rows x 64 tokens; 1: 256 x 128; 2: 512 x 128
template <typename F>
static hipError_t with_gemm_stack_kernel(int kind, bool split, F&& f) {
  if (split) {
    if (kind == 2) return f(gemm_stack_kernel<128, 512, true>);
    if (kind == 1) return f(gemm_stack_kernel<128, 256, true>);
    return f(gemm_stack_kernel<64, 128, true>);
  }
  if (kind == 2) return f(gemm_stack_kernel<128, 512, false>);
  if (kind == 1) return f(gemm_stack_kernel<128, 256, false>);
  return f(gemm_stack_kernel<64, 128, false>);
}

template <typename F>
static hipError_t with_gemm_linear_kernel(int kind, F&& f) {
  if (kind == 2) return f(gemm_linear_kernel<128, 512>);
  if (kind == 1) return f(gemm_linear_kernel<128, 256>);
  return f(gemm_linear_kernel<64, 128>);
}

// A stack (or one linear) with fewer than this many 512-row tiles per CU
// takes 256-row tiles: with the larger ones its last tiles leave most of
// the chip idle (one 8B layer at M = 512: 166 -> 116 us; four layers, 1,216
// tiles: 447 -> 417 us the other way).
constexpr int64_t kBigTilesPerCu = 3;

}  // namespace

int gemm_tile_tokens(int32_t M) { return M > 64 ? 128 : 64; }

int gemm_kind(int32_t M, int64_t tiles512, int cus) {
  if (gemm_tile_tokens(M) == 64) return 0;
  return tiles512 >= kBigTilesPerCu * (int64_t)cus ? 2 : 1;
}

int gemm_kind_rows(int kind) { return kind == 2 ? 512 : kind == 1 ? 256 : GemmShape<64>::ROWS; }

int gemm_kind_tokens(int kind) { return kind == 0 ? 64 : 128; }

static int gemm_block(int kind) { return 64 * (kind == 0 ? GemmShape<64>::WAVES : LineShape<512>::WAVES); }

hipError_t launch_gemm_linear(const LinearArgs& a, int cus, hipStream_t s) {
  const int64_t ntok = ((int64_t)a.M + 127) / 128;
  const int kind = gemm_kind(a.M, (((int64_t)a.N + 511) / 512) * ntok, cus);
  const int rows = gemm_kind_rows(kind), bm = gemm_kind_tokens(kind);
  const int64_t tiles = (((int64_t)a.N + rows - 1) / rows) * (((int64_t)a.M + bm - 1) / bm);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(tiles, 65535));
  return with_gemm_linear_kernel(kind, [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(gemm_block(kind)), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_gemm_stack(int kind, const void* ws, const LaunchShape& shp, hipStream_t s) {
  const StackHeader* h = static_cast<const StackHeader*>(ws);
  const bool split = shp.splits > 0;
  if (split) {
    const hipError_t e = launch_split_clear(ws, shp, s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = with_gemm_stack_kernel(kind, split, [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(shp.grid), dim3(gemm_block(kind)), 0, s, h, stack_sync(ws));
    return hipGetLastError();
  });
  if (e != hipSuccess || !split) return e;
  return launch_split_finish(ws, shp, s);
}

int gemm_stack_blocks_per_cu(int kind) {
  int n = 0;
  const hipError_t e = with_gemm_stack_kernel(kind, false, [&](auto kern) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, gemm_block(kind), 0);
  });
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace tern
