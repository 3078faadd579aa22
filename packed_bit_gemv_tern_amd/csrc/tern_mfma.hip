// tern_mfma.hip -- MFMA int8 path of the ternary linear for 2 <= M <= 16
// tokens (the batched verify pass of drafted decoding), and the MFMA path's
// kernel selection (M > 16 goes to the prefill GEMM in tern_gemm.hip).
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
// Two kernels: the lockstep workgroup kernel (9 <= M <= 16, or any K) and
// the activation-window kernel (M <= 8, K a multiple of 64).
#include "tern_prologue.h"

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

// 16 activations of token row `qrow` starting at column j0, zero past K
// (the ragged tail of K; K a multiple of 64 never takes this path).
__device__ __forceinline__ i32x4 load_q16_tail(const int8_t* qrow, int K, int j0) {
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

__device__ __forceinline__ i32x4 as_i32x4(u32x4 t) {
  return i32x4{(int32_t)t.x, (int32_t)t.y, (int32_t)t.z, (int32_t)t.w};
}

// LDS tile of one wave: 16*R rows of one K-step (128 packed bytes = 512
// weights per row), rows 144 bytes apart so that the 16 lanes reading 16
// rows at the same offset hit 16 disjoint groups of 4 banks.
constexpr int kStepBytes = 128;
constexpr int kRowPitch = 144;

// ---------------------------------------------------------------------------
// M <= 16: the four waves of a workgroup take the four 64-row quarters of a
// 256-row unit of one linear and walk K in lockstep.  Each K-step's
// activations (MQ tokens x 512 bytes) are loaded once per workgroup with
// whole-line loads -- wave w brings tokens 2*(QLD*w + i) and 2*(QLD*w + i) + 1
// -- into a double-buffered LDS tile that every wave then reads its MFMA
// operands from; weights go through a per-wave LDS tile (rows kRowPitch apart,
// whole 128-byte lines per global load instruction).  Reading the
// activations straight from memory in MFMA layout touched 32 cache lines per
// load instruction and stalled the address unit.  One barrier per K-step:
// it publishes step ks+1's activations, and it also guarantees every wave
// has finished with the buffer that step ks+2 will overwrite.
constexpr int kQPitch = 528;  // 512 activation bytes of a step + 16 of padding
constexpr int kWgRows = kWavesPerBlock * 16 * kR;

template <int MQ>
struct WgTiles {
  uint8_t w[kWavesPerBlock][16 * kR * kRowPitch];
  uint8_t q[2][MQ][kQPitch];
  uint8_t zero[kQPitch];  // operand row of the MFMA token rows MQ..15
};

template <int MQ, bool RAGGED>
__device__ __forceinline__ void mfma_wg_range(const LinearArgs& a, int row_lo, int row_hi, int unit0,
                                              int ustride, int lane, int w, WgTiles<MQ>& L) {
  constexpr int R = kR;
  constexpr int NLD = 16 * R / 8;               // weight loads per wave per K-step
  constexpr int QLD = MQ / (2 * kWavesPerBlock);  // activation loads per wave per K-step
  static_assert(QLD >= 1, "MQ");
  const int r = lane & 15, g = lane >> 4;
  const int lrow = lane >> 3, lchunk = lane & 7;
  const int nch = a.nch, K = a.K, M = a.M;
  const int nks = (nch + 7) / 8;
  uint8_t* tile = L.w[w];
  const int qoff = 16 * (lane & 31);  // step byte this lane stages

  auto load_q = [&](int ks, u32x4 (&qv)[QLD]) {
#pragma unroll
    for (int i = 0; i < QLD; ++i) {
      const int tq = 2 * (QLD * w + i) + (lane >> 5);
      const int ch = 8 * ks + qoff / 64;
      const int8_t* qr = a.q + (int64_t)min(tq, M - 1) * a.ldq;
      const int j0 = 64 * min(ch, nch - 1) + qoff % 64;
      u32x4 v;
      if (RAGGED && j0 + 16 > K) {
        const i32x4 t = load_q16_tail(qr, K, j0);
        v = u32x4{(uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w};
      } else {
        v = load16(qr + j0);
      }
      qv[i] = (tq < M && ch < nch) ? v : u32x4{0, 0, 0, 0};
    }
  };
  auto store_q = [&](int buf, const u32x4 (&qv)[QLD]) {
#pragma unroll
    for (int i = 0; i < QLD; ++i) {
      const int tq = 2 * (QLD * w + i) + (lane >> 5);
      *reinterpret_cast<u32x4*>(&L.q[buf][tq][qoff]) = qv[i];
    }
  };

#pragma unroll 1
  for (int unit = unit0;; unit += ustride) {
    const int ubase = row_lo + unit * kWgRows;
    if (ubase >= row_hi) break;  // the same for every wave of the workgroup
    const int base = ubase + 16 * R * w;
    const uint8_t* src[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      src[i] = a.packed + (int64_t)min(base + 8 * i + lrow, row_hi - 1) * a.ld;
    i32x4 acc[R];
#pragma unroll
    for (int b = 0; b < R; ++b) acc[b] = i32x4{0, 0, 0, 0};

    u32x4 st[NLD];
    u32x4 qv[QLD];
    {
      const int ch = min(lchunk, nch - 1);
#pragma unroll
      for (int i = 0; i < NLD; ++i) st[i] = load_weights16(src[i] + 16 * ch);
      load_q(0, qv);
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        *reinterpret_cast<u32x4*>(tile + (8 * i + lrow) * kRowPitch + 16 * lchunk) = st[i];
      store_q(0, qv);
    }
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      const bool more = ks + 1 < nks;
      if (more) {
        const int ch = min(8 * (ks + 1) + lchunk, nch - 1);
#pragma unroll
        for (int i = 0; i < NLD; ++i) st[i] = load_weights16(src[i] + 16 * ch);
        load_q(ks + 1, qv);
      }
      const uint8_t* qrow = r < MQ ? &L.q[ks & 1][r][0] : L.zero;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        i32x4 qa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qa[j] = as_i32x4(*reinterpret_cast<const u32x4*>(qrow + 128 * g + 64 * half + 16 * j));
#pragma unroll
        for (int b = 0; b < R; ++b) {
          const u32x4 wv = *reinterpret_cast<const u32x4*>(
              tile + (16 * b + r) * kRowPitch + 32 * g + 16 * half);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[j], decode_word(wv[j]), acc[b], 0, 0, 0);
        }
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          *reinterpret_cast<u32x4*>(tile + (8 * i + lrow) * kRowPitch + 16 * lchunk) = st[i];
        store_q((ks + 1) & 1, qv);
      }
      __syncthreads();
    }

    // epilogue: lane holds tokens 4g + v of row base + 16b + r
#pragma unroll
    for (int b = 0; b < R; ++b) {
      const int row = base + 16 * b + r;
      if (row >= row_hi) continue;
      const int32_t rs = load_g(a.rowsum + row);
      const float sr = load_g(a.s_row + row);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) {
          const int32_t accv =
              (int32_t)((uint32_t)acc[b][v] - mul_zr(load_g(a.z + m), rs));
          const int64_t o = (int64_t)m * a.ldy + row;
          store_g(a.y + o, epilogue(sr, accv, load_g(a.s_act + m)));
          if (a.acc) store_g(a.acc + o, accv);
        }
      }
    }
  }
}

template <int MQ>
__device__ __forceinline__ void clear_zero_row(WgTiles<MQ>& L) {
  for (int i = threadIdx.x; i < kQPitch / 4; i += blockDim.x)
    reinterpret_cast<uint32_t*>(L.zero)[i] = 0;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// M <= 8, K a multiple of 64: the activation window.  A workgroup keeps the
// activations of 8 tokens x 4096 K positions in LDS and restages them only
// when its (linear, window) changes -- once per segment for K <= 4096 and
// once per window per unit beyond -- so the K loop itself has no barrier and
// no activation traffic.  Weights go from HBM straight into a per-wave LDS
// tile (global_load_lds_dwordx4, 16 bytes per lane at tile + 1 KB*i +
// 16*lane): load i brings rows 8i..8i+7 of the wave's 32 rows, lane l chunk
// (l%8) ^ (row%8) of row 8i + l/8 of the K-step -- whole 128-byte lines per
// instruction, and the XOR spreads the 16 lanes that later read one chunk of
// 16 rows over the banks.  Two tiles per wave are in flight: a step's tile is
// read into registers and the tile two steps ahead is issued into its slot.
// The stack kernel holds its fp32 outputs in registers and stores them when
// its run of work ends: output stores trickled into the saturated weight
// stream slow it by about 1 us per MB, one burst at the end far less.  That
// takes 2 waves per SIMD (256 VGPRs): one 8-wave workgroup per CU keeps the
// same 64 KB of weights in flight as four waves per SIMD with one tile each,
// with 256-row units (a window restage serves twice the rows of a 4-wave
// unit, and 24 held units cover a whole run of the 8B stack).
// Decode by code planes: word & (0x03030303 << 2k) holds the codes c = w + 1
// of weights 4k..4k+3 of the word scaled by 4^k (the top plane is shifted
// down instead), so plane k of four words is one MFMA operand for four ANDs.
// MFMA k of a chunk pairs plane k of its four words with the activations at
// 16j + 4k + {0..3}, j = 0..3 -- 16 contiguous bytes once every 64-byte
// chunk of the staged window is stored as a transposed 4x4 block of dwords.
// Planes 0 and 3 accumulate into one register set, planes 1 and 2 into two
// more; sum(c*q) = acc1 + acc4/4 + acc16/16 exactly, and sum(w*q) =
// sum(c*q) - sum(q).
constexpr int kWinK = 4096;    // activation window (K positions)
constexpr int kWinPitch = kWinK + 16;
constexpr int kWinTokens = 8;
constexpr int kWinR = 2;       // row blocks of 16 per wave
constexpr int kWinDepth8 = 2;  // weight tiles per wave (K-steps in flight), 8 tokens
constexpr int kWinWaves = 8;   // waves per workgroup
constexpr int kWinBlock = 64 * kWinWaves;
constexpr int kWinRows = kWinWaves * 16 * kWinR;
// Geometry per staged token count (both run one 8-wave workgroup per CU).
template <int T>
struct WinGeo {
  static_assert(T == 8 || T == 16, "window tokens");
  static constexpr int WAVES = kWinWaves;
  static constexpr int BLOCK = 64 * WAVES;
  static constexpr int ROWS = WAVES * 16 * kWinR;
  // weight tiles in flight per wave (the 16-token window leaves LDS for two)
  static constexpr int DEPTH = T == 8 ? kWinDepth8 : 2;
};
constexpr int kWinTile = 16 * kWinR * kStepBytes;

// Block-wise scales (BLK): the block scales and row sums of a wave's 32 rows
// for a group of up to kBlkGroup consecutive blocks of one window, by four
// 4-byte DMA instructions (scales of rows 0..15, of rows 16..31, then the
// row sums likewise; lane l: row l / 4, block l % 4 of the group, so four
// lanes read 16 contiguous bytes of a row: one instruction touches 16 cache
// lines where one block per instruction touched 64), in a ring of kBlkSlots
// groups per wave: slot word 128 a + 4 row + block (a = 0 scale, 1 row sum).
// A step issues the DMA of the tile D = 2 steps ahead before it finishes its
// own block, so with one-step groups three are live at once;
// and each staged token's activation sums over the window's 512-column
// pieces (an exclusive prefix: qpre[m][k] sums pieces 0 .. k - 1).
constexpr int kBlkGroup = 4;
constexpr int kBlkDma = 4;  // DMA instructions per group
constexpr int kBlkSlots = 3;
template <int T, bool BLK>
struct WinBlk {
  uint32_t meta[WinGeo<T>::WAVES][kBlkSlots][kBlkDma * 64];
  int32_t qpre[T][9];
};
template <int T>
struct WinBlk<T, false> {};

template <int T, bool BLK = false>
struct WinTiles {
  uint8_t w[WinGeo<T>::WAVES][WinGeo<T>::DEPTH][kWinTile];
  uint8_t q[T][kWinPitch];  // each 64-byte chunk stored dword-transposed
  int32_t qsum[T];          // sum of the token's activations over all of K
  int32_t z[T];             // zero points and scales of the staged tokens
  float s_act[T];
  WinBlk<T, BLK> blk;
};

// s_waitcnt on this wave's global loads (LDS DMA included): at most N still
// outstanding; or on its LDS reads (lgkmcnt 0)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A register copy the compiler cannot look through.  Placed right after an
// explicit wait for all of the wave's loads, it hands on a loaded value as
// one the compiler knows is present: otherwise a value loaded inside the
// K-step loop and used after it makes the compiler wait for every load and
// store in flight (the next unit's tile, earlier outputs) at each use.
__device__ __forceinline__ int32_t settled(int32_t x) {
  int32_t y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}
__device__ __forceinline__ float settled(float x) {
  return __int_as_float(settled(__float_as_int(x)));
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier for the activation window: the wave's LDS accesses are
// complete and no memory access moves across it.  Unlike __syncthreads it
// does not wait for the wave's global loads: the weight tiles in flight,
// which land in the wave's own tile slots, never in the window.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// What the workgroup's window holds: window `win` of the activations (with
// their zero points and scales) at q, reused by the next unit or segment that
// needs the same window of the same buffers (q == nullptr: nothing staged).
struct WinStaged {
  const int8_t* q = nullptr;
  const int32_t* z = nullptr;
  const float* s_act = nullptr;
  int K = 0, ldq = 0, win = 0;
  __device__ bool holds(const LinearArgs& a, int w) const {
    return q && q == a.q && z == a.z && s_act == a.s_act && K == a.K && ldq == a.ldq && win == w;
  }
};

// Outputs held in registers until the worker's run ends (or the buffer is
// full).  The 16 x 16 MFMA result of a row block holds tokens 0..7 twice
// (activation rows 8..15 repeat 0..7), so lane (r, g) keeps row block g >> 1
// of a unit, tokens 4 (g & 1) + v, v = 0..3: four registers per unit.
// NV values per unit and lane: 4 with 8 tokens staged, 8 (both row blocks)
// with 16.
template <int MAXU, int NV = 4>
struct OutBuf {
  float v[MAXU > 0 ? MAXU : 1][NV];
  int n = 0;
};
// where a held unit goes (one entry per wave and held unit, in LDS)
struct OutMeta {
  float* y;
  int32_t ldy, M, base, row_hi;
  int32_t pad[2];
};
static_assert(sizeof(OutMeta) == 32, "OutMeta");
// units a wave holds: what each kernel leaves free at 256 VGPRs (96 and
// 112 registers)
constexpr int kOutUnits = 24, kOut16Units = 14;
// the same for the kernels of stacks with block scales (their running sums
// take registers)
constexpr int kOutUnitsBlk = 12, kOut16UnitsBlk = 6;

// value j of a held unit: with 8 tokens row block g >> 1, token
// 4 (g & 1) + j; with 16, row block j >> 2, token 4 g + (j & 3)
template <int MAXU, int NV>
__device__ __forceinline__ void flush_out(OutBuf<MAXU, NV>& ob, const OutMeta* meta, int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < MAXU; ++i) {
    if (i < ob.n) {
      const OutMeta mt = meta[i];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int row = mt.base + 16 * (NV == 4 ? g >> 1 : j >> 2) + r;
        const int m = NV == 4 ? 4 * (g & 1) + j : 4 * g + (j & 3);
        if (m < mt.M && row < mt.row_hi) {
          const uint32_t off = ((uint32_t)m * (uint32_t)mt.ldy + (uint32_t)row) * 4u;
          store_g(reinterpret_cast<float*>(reinterpret_cast<char*>(mt.y) + off), ob.v[i][j]);
        }
      }
    }
  }
  ob.n = 0;
}

// SPLIT: segments may be windows of linears split along K (their flags say
// so); compiled apart so that the kernel for unsplit stacks carries none of it.
// T: tokens staged (8: activation rows 8..15 of the MFMA repeat 0..7; 16).
// BLK: linears may carry block-wise scales along K (blocks of whole K-steps,
// B a multiple of 512): each block's exact sum is finished and scaled at the
// block's last step and added to a running fp32 sum per output value, in
// block order from +0 -- the order of the definition.  Compiled apart so
// that kernels for stacks without block scales carry none of it.
template <bool SPLIT, int MAXU, int T, bool BLK = false>
__device__ __forceinline__ void mfma_win_range(const LinearArgs& a, int row_lo, int row_hi, int unit0,
                                               int ustride, int lane, int w, WinTiles<T, BLK>& L,
                                               WinStaged& staged, int flags, OutBuf<MAXU, T / 2>& ob,
                                               OutMeta* meta) {
  constexpr int R = kWinR;
  constexpr int NLD = 16 * R / 8;  // 1 KB wave loads per K-step
  constexpr int ROWS = WinGeo<T>::ROWS, BLOCK = WinGeo<T>::BLOCK, WAVES = WinGeo<T>::WAVES;
  constexpr int D = WinGeo<T>::DEPTH;
  static_assert(!BLK || kBlkSlots >= D + 1, "block metadata groups live at once");
  constexpr int NV = T / 2;  // held values per unit and lane
  static_assert(D >= 1 && D <= 3, "tile depth");
  static_assert(!BLK || D == 2, "block metadata counts assume two tiles in flight");
  static_assert(kWinR == 2, "one row block per half-wave");
  const int r = lane & 15, g = lane >> 4;
  const int lrow = lane >> 3, lpos = lane & 7;
  const int nch = a.nch, K = a.K, M = a.M;
  const int nks = (nch + 7) / 8;
  const int nwin = (K + kWinK - 1) / kWinK;
  // block scales: K-steps per block
  const bool blk = BLK && a.s_b != nullptr;
  // K-steps per block, a power of two (B = 512 << lbks)
  const int lbks = blk ? a.blg - 3 : 0, bks = 1 << lbks, bmask = bks - 1;
  const int nb = a.nb;
  int mb_issue = 0, mb_use = 0;  // block-metadata ring slots: next to fill, block being summed
  const bool partial = SPLIT && (flags & kSegPartial) != 0;
  const bool zpoint = !partial || (flags & kSegZeroPoint) != 0;
  // y-only outputs are held in registers until the worker's run ends (a
  // split window's partial sums and linears that also return acc are
  // stored at once)
  const bool held = MAXU > 0 && !partial && !a.acc;
  // Window-major order: a held linear of several whole windows takes its
  // units in groups (as many as the held slots take) and walks each group
  // window by window -- window 0 of every unit of the group, then window 1,
  // ... -- so the group stages each window once, where unit by unit every
  // unit would stage all of them (restaging stalls the workgroup at a
  // barrier until its slowest wave arrives).  The exact int32 sums of the
  // earlier windows wait in the units' held slots.
  const bool wmajor = held && nwin > 1 && (K % kWinK) == 0 && ustride == 1;
  const int ufirst = row_lo + unit0 * ROWS;
  const int uend = ufirst < row_hi ? unit0 + (row_hi - ufirst + ROWS - 1) / ROWS : unit0;
  // byte offsets (below 2^32: checked by the host) of the wave's weight rows
  // within a unit, and the chunk each lane brings
  auto unit_src = [&](int unit, uint32_t (&src)[NLD]) {
    const int base = row_lo + unit * ROWS + 16 * R * w;
#pragma unroll
    for (int i = 0; i < NLD; ++i) src[i] = (uint32_t)min(base + 8 * i + lrow, row_hi - 1) * (uint32_t)a.ld;
  };
  // K-step ks of unit `unit` into the slot of tile number t (tiles are
  // numbered in the order the wave consumes them, across units); with block
  // scales the block's scales and row sums go first when ks starts a block
  // (one DMA instruction, counted by the waits below)
  // (block scales: the lane's rows l / 4 and 16 + l / 4 of the wave, times
  // nb (below 2^31: checked by the host); groups of gsz = min(4, blocks per
  // window) blocks, aligned within the window, so a group never spans two
  // passes of the window-major walk)
  const int gmask = BLK && blk ? min(kBlkGroup, (kWinK / 512) >> lbks) - 1 : 0;
  auto unit_meta = [&](int unit) -> uint2 {
    if (!(BLK && blk)) return uint2{0u, 0u};
    const int b0 = row_lo + unit * ROWS + 16 * R * w + (lane >> 2);
    return uint2{(uint32_t)min(b0, row_hi - 1) * (uint32_t)nb, (uint32_t)min(b0 + 16, row_hi - 1) * (uint32_t)nb};
  };
  auto issue = [&](const uint32_t (&src)[NLD], uint2 mo, int ks, int t) {
    if constexpr (BLK) {
      const int bk = ks >> lbks;
      if (blk && (ks & bmask) == 0 && (bk & gmask) == 0) {
        const uint32_t bi = (uint32_t)min(bk + (lane & 3), nb - 1);
        uint32_t* dst = &L.blk.meta[w][mb_issue][0];
#pragma unroll
        for (int i = 0; i < kBlkDma; ++i) {
          const char* base = i < 2 ? reinterpret_cast<const char*>(a.s_b) : reinterpret_cast<const char*>(a.rowsum_b);
          const void* msrc = base + 4 * (uint64_t)(((i & 1) ? mo.y : mo.x) + bi);
          __builtin_amdgcn_global_load_lds(msrc, (lds_ptr)(dst + 64 * i), 4, 0, 0);
        }
        mb_issue = mb_issue + 1 == kBlkSlots ? 0 : mb_issue + 1;
      }
    }
    uint8_t* tile = L.w[w][t % D];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = min(8 * ks + (lpos ^ ((8 * i + lrow) & 7)), nch - 1);
      __builtin_amdgcn_global_load_lds((const void*)(a.packed + src[i] + 16 * ch),
                                       (lds_ptr)(tile + 1024 * i), 16, 0, 2 /* nt */);
    }
  };
  // rowsum and s_row of a unit's rows, loaded one unit ahead (a block-scaled
  // linear has neither: its pointers may be null)
  auto load_rowops = [&](int unit, int32_t (&rs)[R], float (&sr)[R]) {
    if (blk) return;
    const int base = row_lo + unit * ROWS + 16 * R * w;
#pragma unroll
    for (int b = 0; b < R; ++b) {
      const int row = min(base + 16 * b + r, row_hi - 1);
      rs[b] = load_g(a.rowsum + row);
      sr[b] = load_g(a.s_row + row);
    }
  };
  uint32_t src[NLD];
  int32_t nrs[R];
  float nsr[R];
#pragma unroll
  for (int b = 0; b < R; ++b) nrs[b] = 0, nsr[b] = 0.0f;
  // tiles in flight ahead of the one being consumed: never more than a
  // unit's (a window's, window-major) K-steps, so a lookahead reaches at
  // most into the next unit
  const int depth = min(D, nks);
  uint2 mo{0u, 0u};
  if (ufirst < row_hi) {
    unit_src(unit0, src);
    mo = unit_meta(unit0);
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < depth) issue(src, mo, d, d);
    load_rowops(unit0, nrs, nsr);
  }

  // (unit u, window pass p): one pass over K-steps [kb, ke) of a unit --
  // all of K, or window p of it window-major; g0 .. g0 + gn - 1: the
  // window-major group; tb: number of the pass's first tile
  int u = unit0, p = 0, g0 = unit0, gn = 0;
#pragma unroll 1
  for (int tb = 0; u < uend;) {
    if (wmajor && p == 0 && u == g0 + gn) {
      // a new group: empty the held slots first when fewer are free than
      // it would take
      const int need = min(uend - u, MAXU);
      if (MAXU - ob.n < need) flush_out(ob, meta, lane);
      g0 = u;
      gn = min(uend - u, MAXU - ob.n);
    }
    const int base = row_lo + u * ROWS + 16 * R * w;
    const int kb = wmajor ? 8 * p : 0, ke = wmajor ? 8 * p + 8 : nks;
    const bool last_pass = !wmajor || p == nwin - 1;
    // the pass after this one
    int nu = -1, np = 0;
    if (wmajor) {
      if (u + 1 < g0 + gn)
        nu = u + 1, np = p;
      else if (p + 1 < nwin)
        nu = g0, np = p + 1;
      else if (g0 + gn < uend)
        nu = g0 + gn, np = 0;
    } else if (u + ustride < uend) {
      nu = u + ustride;
    }
    const bool has_next = nu >= 0;
    const int nkb = wmajor ? 8 * np : 0;
    uint32_t nsrc[NLD];
    uint2 nmo{0u, 0u};
    if (has_next) unit_src(nu, nsrc), nmo = unit_meta(nu);
    int32_t rs[R];
    float sr[R];
    i32x4 acc1[R], acc4[R], acc16[R];
#pragma unroll
    for (int b = 0; b < R; ++b) acc1[b] = acc4[b] = acc16[b] = i32x4{0, 0, 0, 0};
    // block scales: the lane's values (as held: with 8 tokens row block
    // g >> 1, tokens 4 (g & 1) + v; with 16 both row blocks, tokens 4g + v)
    // as running fp32 sums over the blocks so far, and their int32 totals;
    // window-major, a later pass resumes from the sum held in the unit's slot
    float bsum[BLK ? NV : 1];
    int32_t bint[BLK ? NV : 1];
    // (the plane accumulators run on over the blocks of the pass: each block's
    // sum(c*q) is the difference of their combined value from the previous
    // block's end, exact in int32)
    int32_t cprev[BLK ? NV : 1];
    if constexpr (BLK) {
#pragma unroll
      for (int j = 0; j < NV; ++j) bsum[j] = 0.0f, bint[j] = 0, cprev[j] = 0;
      if (blk && wmajor && p > 0) {
        const int slot = ob.n + (u - g0);
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
          if (i == slot) {
#pragma unroll
            for (int j = 0; j < NV; ++j) bsum[j] = ob.v[i][j];
          }
      }
    }
    for (int ks = kb; ks < ke; ++ks) {
      const uint8_t* tile = L.w[w][(tb + ks - kb) % D];
      if ((ks & 7) == 0) {
        const int win = ks >> 3;
        if (win > 0 && !wmajor) {
          // fold the scaled planes into the exact sum once per window: a
          // plane-2 sum is 16 * sum(c*q), which over all of a long K
          // (beyond 2^21 columns) would pass 2^31
#pragma unroll
          for (int b = 0; b < R; ++b) {
            acc1[b] += (acc4[b] >> 2) + (acc16[b] >> 4);
            acc4[b] = acc16[b] = i32x4{0, 0, 0, 0};
          }
        }
        // a window already staged (the previous unit's, or the previous
        // segment's when it reads the same activations) is used as it is
        if (!staged.holds(a, win)) {
          // every wave is done with the previous window before it is replaced
          lds_barrier();
          {
            // all of a thread's window loads first, then the LDS writes
            constexpr int NE = T * (kWinK / 16) / BLOCK;
            static_assert(NE * BLOCK == T * (kWinK / 16), "window split");
            u32x4 rv[NE];
#pragma unroll
            for (int i = 0; i < NE; ++i) {
              const int e = threadIdx.x + i * BLOCK;
              const int tq = e / (kWinK / 16), off = 16 * (e % (kWinK / 16));
              const int pos = win * kWinK + off;  // K position
              rv[i] = u32x4{0, 0, 0, 0};
              if (tq < M && pos < K) rv[i] = load16(a.q + (int64_t)tq * a.ldq + pos);
            }
#pragma unroll
            for (int i = 0; i < NE; ++i) {
              const int e = threadIdx.x + i * BLOCK;
              const int tq = e / (kWinK / 16), off = 16 * (e % (kWinK / 16));
              // word j = (off % 64) / 16 of its chunk: dword k goes to 16k + 4j
              uint32_t* dst = reinterpret_cast<uint32_t*>(&L.q[tq][off & ~63]) + ((off % 64) / 16);
#pragma unroll
              for (int k = 0; k < 4; ++k) dst[4 * k] = rv[i][k];
            }
          }
          lds_barrier();
          // per-token activation sums of this window, added to the earlier
          // windows' (windows are staged in order); wave w owns tokens w,
          // w + WAVES, ... so no two waves write one entry
          for (int tq = w; tq < T; tq += WAVES) {
            uint32_t part = 0, run = 0;
            if constexpr (BLK) {
              if (lane == 0) L.blk.qpre[tq][0] = 0;
            }
#pragma unroll
            for (int i = 0; i < kWinK / 1024; ++i) {
              const u32x4 v = *reinterpret_cast<const u32x4*>(&L.q[tq][16 * lane + 1024 * i]);
              uint32_t pi = 0;
#pragma unroll
              for (int k = 0; k < 4; ++k) pi = (uint32_t)__builtin_amdgcn_sdot4((int)v[k], 0x01010101, (int)pi, false);
              part += pi;
              if constexpr (BLK) {
                // the window's 512-column pieces 2i and 2i + 1 (half-wave
                // sums), kept as an exclusive prefix: qpre[k] = the sum of
                // pieces 0 .. k - 1
                const uint32_t ph = group_sum<32>(pi);
                const uint32_t p0 = __builtin_amdgcn_readlane(ph, 0), p1 = __builtin_amdgcn_readlane(ph, 32);
                if (lane == 0) {
                  L.blk.qpre[tq][2 * i + 1] = (int32_t)(run + p0);
                  L.blk.qpre[tq][2 * i + 2] = (int32_t)(run + p0 + p1);
                }
                run += p0 + p1;
              }
            }
            const int32_t tot = (int32_t)group_sum<64>(part);
            if (lane == 0) L.qsum[tq] = (win == 0 ? 0 : L.qsum[tq]) + tot;
          }
          if (win == 0 && threadIdx.x < T) {
            const int tq = threadIdx.x;
            L.z[tq] = tq < M ? load_g(a.z + tq) : 0;
            L.s_act[tq] = tq < M ? load_g(a.s_act + tq) : 0.0f;
          }
          lds_barrier();
          staged.q = a.q;
          staged.z = a.z;
          staged.s_act = a.s_act;
          staged.K = K;
          staged.ldq = a.ldq;
          staged.win = win;
        }
      }
      // this step's weight tile has landed once no more loads are in flight
      // than the tiles issued after it (NLD each; loads complete in order,
      // and other loads and stores in between only add to the count)
      {
        const int after = has_next ? depth - 1 : min(depth - 1, ke - 1 - ks);
        // (the tile after this one carries a block group's metadata DMA
        // first when it starts a group)
        const int kn = ks + 1 < ke ? ks + 1 : nkb;
        const bool meta_after = BLK && blk && after == 1 && (kn & bmask) == 0 && ((kn >> lbks) & gmask) == 0;
        if (after >= 2)
          wait_vm<2 * NLD>();
        else if (meta_after)
          wait_vm<NLD + kBlkDma>();
        else if (after == 1)
          wait_vm<NLD>();
        else
          wait_vm<0>();
      }
      if (ks == kb) {
        // this pass's row operands arrived with (or before) its first tile
        // (the wait above covers them); those of the next unit to finish
        // are loaded now, a whole pass ahead of their use
        if (last_pass) {
#pragma unroll
          for (int b = 0; b < R; ++b) rs[b] = settled(nrs[b]), sr[b] = settled(nsr[b]);
        }
        if (has_next && (!wmajor || np == nwin - 1)) load_rowops(nu, nrs, nsr);
      }
      u32x4 wv[R][2];
#pragma unroll
      for (int b = 0; b < R; ++b)
#pragma unroll
        for (int half = 0; half < 2; ++half)
          wv[b][half] = *reinterpret_cast<const u32x4*>(
              tile + (16 * b + r) * kStepBytes + 16 * ((2 * g + half) ^ (r & 7)));
      wait_lgkm();  // tile read: it may be overwritten
      if (ks + depth < ke)
        issue(src, mo, ks + depth, tb + ks - kb + depth);
      else if (has_next)
        issue(nsrc, nmo, nkb + ks + depth - ke, tb + ks - kb + depth);  // the next pass's first tiles
      // activations come from the window, which the loads never overwrite
      const uint8_t* qrow = &L.q[r & (T - 1)][64 * (8 * (ks & 7) + 2 * g)];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 qv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qv[j] = *reinterpret_cast<const u32x4*>(qrow + 64 * half + 16 * j);
#pragma unroll
        for (int b = 0; b < R; ++b) {
          const u32x4 x = wv[b][half];
          const i32x4 p0 = as_i32x4(x & 0x03030303u), p1 = as_i32x4(x & 0x0C0C0C0Cu);
          const i32x4 p2 = as_i32x4(x & 0x30303030u), p3 = as_i32x4((x >> 6) & 0x03030303u);
          acc1[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(qv[0]), p0, acc1[b], 0, 0, 0);
          acc4[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(qv[1]), p1, acc4[b], 0, 0, 0);
          acc16[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(qv[2]), p2, acc16[b], 0, 0, 0);
          acc1[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(qv[3]), p3, acc1[b], 0, 0, 0);
        }
      }
      if constexpr (BLK) {
        if (blk && (((ks + 1) & bmask) == 0 || ks + 1 == nks)) {
          // the block ends: acc_b = sum(c*q) - sum(q) - z * rowsum_b, exact;
          // then one rounding for s_b * acc_b and one for the running sum.
          // Its metadata landed with the tile of its first step.
          const uint32_t* ms = L.blk.meta[w][mb_use];
          const int bi = (ks >> lbks) & gmask;  // block within its group
          if (bi == gmask || ks + 1 == nks) mb_use = mb_use + 1 == kBlkSlots ? 0 : mb_use + 1;
          const int kw = (ks & 7) >> lbks;  // block within the window (blocks never span windows)
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            const int b = T == 8 ? (g >> 1) : (j >> 2);
            const int v = j & 3;
            const int m = T == 8 ? 4 * (g & 1) + v : 4 * g + v;
            const int32_t c1 = b ? acc1[1][v] : acc1[0][v];
            const int32_t c4 = b ? acc4[1][v] : acc4[0][v];
            const int32_t c16 = b ? acc16[1][v] : acc16[0][v];
            const int32_t qb = L.blk.qpre[m][(kw + 1) << lbks] - L.blk.qpre[m][kw << lbks];
            const int32_t cq = c1 + (c4 >> 2) + (c16 >> 4);
            const int32_t accb = (int32_t)((uint32_t)cq - (uint32_t)cprev[j] - (uint32_t)qb -
                                           mul_zr(L.z[m], (int32_t)ms[128 + 4 * (16 * b + r) + bi]));
            cprev[j] = cq;
            bsum[j] = add_product_rn(bsum[j], __uint_as_float(ms[4 * (16 * b + r) + bi]), (float)accb);
            bint[j] += accb;
          }
        }
      }
    }

    // epilogue: lane holds tokens 4g + v of row base + 16b + r.  A window of
    // a linear split along K adds its exact partial sums into y, viewed as
    // int32 (cleared before the launch, finished after it); the zero-point
    // term belongs to one window only.
    if (BLK && blk && held) {
      // block scales, y only: the running sums (window-major, an earlier
      // pass's sum stays in the slot until the last pass scales it)
      if (!wmajor && ob.n == MAXU) flush_out(ob, meta, lane);
      const int slot = wmajor ? ob.n + (u - g0) : ob.n;
      float vals[NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int m = T == 8 ? 4 * (g & 1) + (j & 3) : (4 * g + (j & 3)) & (T - 1);
        vals[j] = last_pass ? __fmul_rn(bsum[j], L.s_act[m]) : bsum[j];
      }
#pragma unroll
      for (int i = 0; i < MAXU; ++i)
        if (i == slot) {
#pragma unroll
          for (int j = 0; j < NV; ++j) ob.v[i][j] = vals[j];
        }
      if (last_pass) {
        OutMeta mt;
        mt.y = a.y;
        mt.ldy = a.ldy;
        mt.M = M;
        mt.base = row_lo + u * ROWS + 16 * R * w;
        mt.row_hi = row_hi;
        mt.pad[0] = mt.pad[1] = 0;
        meta[slot] = mt;
        if (!wmajor)
          ob.n = ob.n + 1;
        else if (u == g0 + gn - 1)
          ob.n = ob.n + gn;
      }
    } else if (BLK && blk) {
      // block scales, y and acc stored at once: the lane's values
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int b = T == 8 ? (g >> 1) : (j >> 2);
        const int m = T == 8 ? 4 * (g & 1) + (j & 3) : 4 * g + (j & 3);
        const int row = base + 16 * b + r;
        if (m < M && row < row_hi) {
          const uint32_t off = ((uint32_t)m * (uint32_t)a.ldy + (uint32_t)row) * 4u;
          store_g(reinterpret_cast<float*>(reinterpret_cast<char*>(a.y) + off), __fmul_rn(bsum[j], L.s_act[m]));
          if (a.acc) store_g(reinterpret_cast<int32_t*>(reinterpret_cast<char*>(a.acc) + off), bint[j]);
        }
      }
    } else if (held) {
      // the lane's held values: with 8 tokens row block g >> 1, tokens
      // 4 (g & 1) + v (the MFMA result holds tokens 0..7 twice); with 16
      // both row blocks, tokens 4g + v
      int32_t cq[NV];  // sum(c*q) of this pass, exact
      if (T == 8) {
        const int bs = g >> 1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int32_t c1 = bs ? acc1[1][v] : acc1[0][v];
          const int32_t c4 = bs ? acc4[1][v] : acc4[0][v];
          const int32_t c16 = bs ? acc16[1][v] : acc16[0][v];
          cq[v] = c1 + (c4 >> 2) + (c16 >> 4);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int b = j >> 2, v = j & 3;
          cq[j] = acc1[b][v] + (acc4[b][v] >> 2) + (acc16[b][v] >> 4);
        }
      }
      if (!wmajor && ob.n == MAXU) flush_out(ob, meta, lane);
      const int slot = wmajor ? ob.n + (u - g0) : ob.n;
      if (wmajor && p > 0) {
        // the earlier windows' sums, held in the slot as int32 bits
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
          if (i == slot) {
#pragma unroll
            for (int j = 0; j < NV; ++j) cq[j] += __float_as_int(ob.v[i][j]);
          }
      }
      float vals[NV];
      if (last_pass) {
        if (T == 8) {
          const int bs = g >> 1;
          const int32_t rsel = bs ? rs[1] : rs[0];
          const float ssel = bs ? sr[1] : sr[0];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = 4 * (g & 1) + v;
            const int32_t accv = (int32_t)((uint32_t)cq[v] - (uint32_t)L.qsum[m] - mul_zr(L.z[m], rsel));
            vals[v] = epilogue(ssel, accv, L.s_act[m]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            const int b = j >> 2, m = (4 * g + (j & 3)) & (T - 1);
            const int32_t accv = (int32_t)((uint32_t)cq[j] - (uint32_t)L.qsum[m] - mul_zr(L.z[m], rs[b]));
            vals[j] = epilogue(sr[b], accv, L.s_act[m]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) vals[j] = __int_as_float(cq[j]);
      }
#pragma unroll
      for (int i = 0; i < MAXU; ++i)
        if (i == slot) {
#pragma unroll
          for (int j = 0; j < NV; ++j) ob.v[i][j] = vals[j];
        }
      if (last_pass) {
        OutMeta mt;
        mt.y = a.y;
        mt.ldy = a.ldy;
        mt.M = M;
        mt.base = row_lo + u * ROWS + 16 * R * w;
        mt.row_hi = row_hi;
        mt.pad[0] = mt.pad[1] = 0;
        meta[slot] = mt;  // every lane writes the same entry
        if (!wmajor)
          ob.n = ob.n + 1;
        else if (u == g0 + gn - 1)
          ob.n = ob.n + gn;
      }
    } else {
      int32_t zt[4];
      float sa[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        zt[v] = zpoint ? L.z[(4 * g + v) & (T - 1)] : 0;
        sa[v] = L.s_act[(4 * g + v) & (T - 1)];
      }
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int row = base + 16 * b + r;
        if (row >= row_hi) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * g + v;
          if (m < M) {
            const int32_t cq = acc1[b][v] + (acc4[b][v] >> 2) + (acc16[b][v] >> 4);  // sum(c*q)
            const int32_t accv = (int32_t)((uint32_t)cq - (uint32_t)L.qsum[m] -
                                           mul_zr(zt[v], rs[b]));
            // byte offset of (m, row) in y and acc: below 2^32 (checked by the host)
            const uint32_t off = ((uint32_t)m * (uint32_t)a.ldy + (uint32_t)row) * 4u;
            if (partial) {
              __hip_atomic_fetch_add((int32_t __attribute__((address_space(1)))*)(
                                         reinterpret_cast<char*>(a.y) + off),
                                     accv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
              store_g(reinterpret_cast<float*>(reinterpret_cast<char*>(a.y) + off),
                      epilogue(sr[b], accv, sa[v]));
              if (a.acc) store_g(reinterpret_cast<int32_t*>(reinterpret_cast<char*>(a.acc) + off), accv);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) src[i] = nsrc[i];
    mo = nmo;
    tb += ke - kb;
    if (!has_next) break;
    u = nu;
    p = np;
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

// M <= 16: workgroups of four lockstep waves (per-workgroup schedule).
template <int MQ, bool RAGGED>
__global__ __launch_bounds__(kBlock) void mfma_wg_linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) WgTiles<MQ> L;
  clear_zero_row(L);
  const int lane = threadIdx.x & 63;
  mfma_wg_range<MQ, RAGGED>(a, 0, a.N, blockIdx.x, gridDim.x, lane, wave_id_uniform(), L);
}

template <int MQ, bool RAGGED>
__global__ __launch_bounds__(kBlock) void mfma_wg_stack_kernel(const StackHeader* __restrict__ h,
                                  StackSync* __restrict__ sy) {
  __shared__ __attribute__((aligned(16))) WgTiles<MQ> L;
  __shared__ PrologueLds prol;
  const uint32_t launch1 = stack_prologue(h, sy, prol);
  const int worker = xcd_logical_block();
  if (worker >= h->workers) return;  // the same for the whole workgroup
  clear_zero_row(L);
  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(base + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(base + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    if (RAGGED && (a.K & 63) != 0)
      mfma_wg_range<MQ, RAGGED>(a, sg.row_begin, sg.row_end, 0, 1, lane, w, L);
    else
      mfma_wg_range<MQ, false>(a, sg.row_begin, sg.row_end, 0, 1, lane, w, L);
  }
}

// M <= 8, every K a multiple of 64: the activation-window kernel.
__global__ __launch_bounds__(kWinBlock) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_win_linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) WinTiles<8> L;
  WinStaged staged;
  OutBuf<0, 4> ob;
  mfma_win_range<false, 0, 8>(a, 0, a.N, blockIdx.x, gridDim.x, threadIdx.x & 63, wave_id_uniform(), L, staged, 0,
                           ob, nullptr);
}

// The stack kernel: a worker's segments in order, y-only outputs held in
// registers (kOutUnits units per wave, kOutUnitsBlk in the kernel for stacks
// with block scales) and stored at the end of the run.
template <bool SPLIT, bool BLK = false>
__global__ __launch_bounds__(kWinBlock) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_win_stack_kernel(const StackHeader* __restrict__ h,
                                  StackSync* __restrict__ sy) {
  constexpr int MAXU = BLK ? kOutUnitsBlk : kOutUnits;
  __shared__ __attribute__((aligned(16))) WinTiles<8, BLK> L;
  __shared__ OutMeta meta[kWinWaves][MAXU];
  __shared__ PrologueLds prol;
  const uint32_t launch1 = stack_prologue(h, sy, prol);
  const int worker = xcd_logical_block();
  if (worker >= h->workers) return;  // the same for the whole workgroup
  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(base + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(base + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  WinStaged staged;
  OutBuf<MAXU, 4> ob;
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    mfma_win_range<SPLIT, MAXU, 8, BLK>(a, sg.row_begin, sg.row_end, 0, 1, lane, w, L, staged,
                                        SPLIT ? sg.flags : 0, ob, meta[w]);
  }
  flush_out(ob, meta[w], lane);
}

// 9 <= M <= 16 tokens, every K a multiple of 64: the same window kernel with
// all 16 activation rows staged, one 8-wave workgroup per CU, y-only outputs
// held (kOut16Units units per wave, kOut16UnitsBlk with block scales).
// (Only SPLIT = false is launched.)
template <bool SPLIT, bool BLK = false>
__global__ __launch_bounds__(WinGeo<16>::BLOCK) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_win16_stack_kernel(
    const StackHeader* __restrict__ h, StackSync* __restrict__ sy) {
  constexpr int MAXU = BLK ? kOut16UnitsBlk : kOut16Units;
  __shared__ __attribute__((aligned(16))) WinTiles<16, BLK> L;
  __shared__ OutMeta meta[WinGeo<16>::WAVES][MAXU];
  __shared__ PrologueLds prol;
  const uint32_t launch1 = stack_prologue(h, sy, prol);
  const int worker = xcd_logical_block();
  if (worker >= h->workers) return;  // the same for the whole workgroup
  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(base + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(base + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  WinStaged staged;
  OutBuf<MAXU, 8> ob;
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    mfma_win_range<SPLIT, MAXU, 16, BLK>(lin[sg.lin], sg.row_begin, sg.row_end, 0, 1, lane, w, L, staged,
                                         SPLIT ? sg.flags : 0, ob, meta[w]);
  }
  flush_out(ob, meta[w], lane);
}

// Linears split along K: before the main kernel their outputs are cleared
// (the windows add int32 partial sums into them), after it each sum becomes
// y = (s_row * acc) * s_act, and acc when asked for.  One workgroup per
// (split linear, token).
__global__ __launch_bounds__(kSplitBlock) void split_clear_kernel(const StackHeader* __restrict__ h) {
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* split = reinterpret_cast<const int32_t*>(base + h->off_split);
  const int M = h->M;
  const LinearArgs& a = lin[split[blockIdx.x / M]];
  const int m = blockIdx.x % M;
  int32_t* y = reinterpret_cast<int32_t*>(a.y) + (int64_t)m * a.ldy;
  for (int row = threadIdx.x; row < a.N; row += blockDim.x) store_g(y + row, 0);
}

__global__ __launch_bounds__(kSplitBlock) void split_finish_kernel(const StackHeader* __restrict__ h) {
  const char* base = reinterpret_cast<const char*>(h);
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(base + h->off_lin);
  const int32_t* split = reinterpret_cast<const int32_t*>(base + h->off_split);
  const int M = h->M;
  const LinearArgs& a = lin[split[blockIdx.x / M]];
  const int m = blockIdx.x % M;
  const int64_t o0 = (int64_t)m * a.ldy;
  const float sa = load_g(a.s_act + m);
  for (int row = threadIdx.x; row < a.N; row += blockDim.x) {
    const int32_t acc = load_g(reinterpret_cast<const int32_t*>(a.y) + o0 + row);
    store_g(a.y + o0 + row, epilogue(load_g(a.s_row + row), acc, sa));
    if (a.acc) store_g(a.acc + o0 + row, acc);
  }
}

// Kernel selector of the MFMA path: bit 1 = ragged K compiled in, bit 2 =
// 9 <= M <= 16 (16 activation rows) for the lockstep workgroup kernel;
// 8 = the activation-window kernel (M <= 8, no ragged K); 9, 14 and 10 = the
// prefill GEMM (M > 16) with tiles of 128 x 64, 256 x 128 and 512 x 128.
constexpr int32_t kWinVariant = 8;
constexpr int32_t kGemm64Variant = 9;
constexpr int32_t kGemm128Variant = 10;
constexpr int32_t kGemm128sVariant = 14;
constexpr int32_t kWin16Variant = 11;  // the window kernel for 9 <= M <= 16
// the window kernels compiled for stacks with block scales
constexpr int32_t kWinBlkVariant = 12;
constexpr int32_t kWin16BlkVariant = 13;

static bool is_gemm(int32_t v) { return v == kGemm64Variant || v == kGemm128Variant || v == kGemm128sVariant; }

// tile kind of a prefill GEMM variant (gemm_kind_rows)
static int gemm_kind_of(int32_t v) { return v == kGemm128Variant ? 2 : v == kGemm128sVariant ? 1 : 0; }

bool mfma_win_offsets_fit(int64_t N, int64_t ld, int64_t M, int64_t ldy) {
  // weight row offsets and output byte offsets are 32-bit in that kernel
  return N * ld < (1ll << 32) && M * ldy * 4 < (1ll << 32);
}

bool mfma_is_window(int32_t variant) {
  return variant == kWinVariant || variant == kWin16Variant || variant == kWinBlkVariant ||
         variant == kWin16BlkVariant;
}

// (the 16-token window kernel never splits: stacks small enough to want it
// take the prefill GEMM at 9..16 tokens)
bool mfma_can_split(int32_t variant) {
  return variant == kWinVariant || is_gemm(variant);
}

hipError_t launch_split_clear(const void* ws, const LaunchShape& shp, hipStream_t s) {
  hipLaunchKernelGGL(split_clear_kernel, dim3((unsigned)(shp.splits * shp.M)), dim3(kSplitBlock), 0, s,
                     static_cast<const StackHeader*>(ws));
  return hipGetLastError();
}

hipError_t launch_split_finish(const void* ws, const LaunchShape& shp, hipStream_t s) {
  hipLaunchKernelGGL(split_finish_kernel, dim3((unsigned)(shp.splits * shp.M)), dim3(kSplitBlock), 0, s,
                     static_cast<const StackHeader*>(ws));
  return hipGetLastError();
}

int mfma_window_k() { return kWinK; }

int mfma_step_k() { return 8 * 64; }

int32_t mfma_gemm_variant(int32_t M) {
  return gemm_tile_tokens(M) == 128 ? kGemm128Variant : kGemm64Variant;
}

int32_t mfma_gemm_refine(int32_t variant, int32_t M, int64_t tiles512, int cus) {
  if (variant != kGemm128Variant && variant != kGemm128sVariant) return variant;
  return gemm_kind(M, tiles512, cus) == 2 ? kGemm128Variant : kGemm128sVariant;
}

bool mfma_is_lockstep(int32_t variant) { return variant >= 0 && variant < kWinVariant; }

int32_t mfma_stack_variant(int32_t M, bool ragged, bool big, bool blocked) {
  if (M > 16) return mfma_gemm_variant(M);
  if (M <= kWinTokens && !ragged && !big) return blocked ? kWinBlkVariant : kWinVariant;
  if (M <= 16 && !ragged && !big) return blocked ? kWin16BlkVariant : kWin16Variant;
  return (ragged ? 2 : 0) | (M > 8 ? 4 : 0);
}

int32_t mfma_token_tiles(int32_t variant, int32_t M) {
  if (!is_gemm(variant)) return 0;
  const int bm = gemm_kind_tokens(gemm_kind_of(variant));
  return (int32_t)(((int64_t)M + bm - 1) / bm);
}

bool mfma_per_workgroup(int32_t) { return true; }

int mfma_unit_rows(int32_t variant) {
  if (variant == kWinVariant || variant == kWinBlkVariant) return kWinRows;
  if (variant == kWin16Variant || variant == kWin16BlkVariant) return WinGeo<16>::ROWS;
  if (is_gemm(variant)) return gemm_kind_rows(gemm_kind_of(variant));
  return kWgRows;
}

int mfma_unit_restages(int32_t variant, int64_t K) {
  return mfma_is_window(variant) && K > kWinK ? (int)((K + kWinK - 1) / kWinK) : 0;
}

int mfma_held_units(int32_t variant) {
  switch (variant) {
    case kWinVariant: return kOutUnits;
    case kWin16Variant: return kOut16Units;
    case kWinBlkVariant: return kOutUnitsBlk;
    case kWin16BlkVariant: return kOut16UnitsBlk;
    default: return 0;
  }
}

bool mfma_window_major(int32_t variant, int64_t K, bool y_only) {
  return mfma_is_window(variant) && y_only && K > kWinK && K % kWinK == 0;
}

template <typename F>
static hipError_t with_mfma_stack_kernel(int32_t variant, F&& f) {
  switch (variant) {
    case 0: return f(mfma_wg_stack_kernel<8, false>);
    case 2: return f(mfma_wg_stack_kernel<8, true>);
    case 4: return f(mfma_wg_stack_kernel<16, false>);
    case 6: return f(mfma_wg_stack_kernel<16, true>);
    case kWinVariant: return f(mfma_win_stack_kernel<false>);
    case kWin16Variant: return f(mfma_win16_stack_kernel<false>);
    case kWinBlkVariant: return f(mfma_win_stack_kernel<false, true>);
    case kWin16BlkVariant: return f(mfma_win16_stack_kernel<false, true>);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mfma_linear(const LinearArgs& a, int cus, hipStream_t s) {
  int32_t v = mfma_stack_variant(a.M, (a.K & 63) != 0, !mfma_win_offsets_fit(a.N, a.ld, a.M, a.ldy), false);
  if (is_gemm(v)) return launch_gemm_linear(a, cus, s);
  if (v == kWin16Variant) v = 4;  // one linear at 9..16 tokens: the lockstep kernel
  const int64_t units = (a.N + mfma_unit_rows(v) - 1) / mfma_unit_rows(v);
  int64_t blocks = units;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(kBlock);
  switch (v) {
    case kWinVariant: hipLaunchKernelGGL(mfma_win_linear_kernel, grid, dim3(kWinBlock), 0, s, a); break;
    case 0: hipLaunchKernelGGL((mfma_wg_linear_kernel<8, false>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((mfma_wg_linear_kernel<8, true>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((mfma_wg_linear_kernel<16, false>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((mfma_wg_linear_kernel<16, true>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mfma_stack(int32_t variant, const void* ws, const LaunchShape& shp, hipStream_t s) {
  if (is_gemm(variant)) return launch_gemm_stack(gemm_kind_of(variant), ws, shp, s);
  const StackHeader* h = static_cast<const StackHeader*>(ws);
  const dim3 grid(shp.grid), block(variant == kWinVariant || variant == kWinBlkVariant       ? kWinBlock
                                    : variant == kWin16Variant || variant == kWin16BlkVariant ? WinGeo<16>::BLOCK
                                                                                            : shp.block);
  const bool split = variant == kWinVariant && shp.splits > 0;
  if (split) {
    const hipError_t e = launch_split_clear(ws, shp, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  if (split) {
    hipLaunchKernelGGL(mfma_win_stack_kernel<true>, grid, block, 0, s, h, stack_sync(ws));
    e = hipGetLastError();
  } else {
    e = with_mfma_stack_kernel(variant, [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, s, h, stack_sync(ws));
      return hipGetLastError();
    });
  }
  if (e != hipSuccess || !split) return e;
  return launch_split_finish(ws, shp, s);
}

int mfma_stack_blocks_per_cu(int32_t variant) {
  if (is_gemm(variant)) return gemm_stack_blocks_per_cu(gemm_kind_of(variant));
  int n = 0;
  const int block = variant == kWinVariant || variant == kWinBlkVariant       ? kWinBlock
                    : variant == kWin16Variant || variant == kWin16BlkVariant ? WinGeo<16>::BLOCK
                                                                            : kBlock;
  const hipError_t e = with_mfma_stack_kernel(variant, [&](auto kern) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, block, 0);
  });
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace tern
