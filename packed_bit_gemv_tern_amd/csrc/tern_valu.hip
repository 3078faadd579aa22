// tern_valu.hip -- VALU path of the ternary linear: in-register 2-bit decode
// with add / subtract / skip accumulation through v_dot4_u32_u8.
//
// The article "Neutrino-1: quantization is a training decision, not a
// deployment one" ("The take") says signed accumulation replaces multiplies;
// the model card ("Overview") says packed weights are decoded inside the
// matrix kernels.  Single-stream decode reads every weight once per token and
// is bound by bytes moved (article, "Serving it: the Neutrino Engine"), so
// this path is built around one coalesced 16-byte non-temporal load per lane
// per 64 weights and as few VALU operations per weight as possible:
//
//  * activations are biased to unsigned once, qb = q + 128 (q ^ 0x80), and
//    zero past K;
//  * a packed 32-bit word w holds 16 weights; (w & 0x03030303 << 2k) keeps
//    the codes c = w+1 of weights 4k..4k+3 scaled by 4^k, one per byte, so
//    four ANDs and four unsigned dot4s against the matching qb bytes give
//    4^k-scaled partial sums of c * qb -- 0.5 VALU operations per weight;
//  * with S = sum_j c_j qb_j and QB = sum_{j<K} qb_j (padding has qb = 0):
//      sum_j w_j q_j - z * rowsum = S - QB - (z + 128) * rowsum,
//    all in wrapping 32-bit arithmetic, exact whenever the result fits in
//    int32 (guaranteed by the host's K bound and |z| <= 255).
//
// A row is split over LPR lanes; each wave reduces U rows at once with a
// transposed butterfly (v_permlane32/16_swap and DPP), so the cross-lane cost
// is about two operations per row instead of six.
#include "tern_prologue.h"

namespace tern {

namespace {

constexpr uint32_t kPlane0 = 0x03030303u, kPlane1 = 0x0C0C0C0Cu, kPlane2 = 0x30303030u,
                   kPlane3 = 0xC0C0C0C0u;
constexpr uint32_t kBias = 0x80808080u, kOnes = 0x01010101u;

__device__ __forceinline__ uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_udot4(a, b, c, false);
}

// 64 biased activations of one token, [64*ch, 64*ch + 64), zero past K.
// Without RAGGED the caller guarantees 64*ch + 64 <= K.
template <bool RAGGED>
__device__ __forceinline__ void load_q_chunk(const int8_t* q, int K, int ch, uint32_t (&out)[16]) {
  const int j0 = ch * 64;
  if (!RAGGED || j0 + 64 <= K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 t = load16(q + j0 + 16 * i);
      out[4 * i + 0] = t.x ^ kBias;
      out[4 * i + 1] = t.y ^ kBias;
      out[4 * i + 2] = t.z ^ kBias;
      out[4 * i + 3] = t.w ^ kBias;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = j0 + 4 * i + b;
        if (j < K) v |= (uint32_t)((uint8_t)load_g(q + j) ^ 0x80u) << (8 * b);
      }
      out[i] = v;
    }
  }
}

// Accumulate the four 4^k-scaled planes of one 16-byte weight chunk against
// the matching 64 biased activations.
__device__ __forceinline__ void dot_chunk(const u32x4 w, const uint32_t (&qc)[16], uint32_t (&p)[4]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = w[d];
    p[0] = udot4(x & kPlane0, qc[4 * d + 0], p[0]);
    p[1] = udot4(x & kPlane1, qc[4 * d + 1], p[1]);
    p[2] = udot4(x & kPlane2, qc[4 * d + 2], p[2]);
    p[3] = udot4(x & kPlane3, qc[4 * d + 3], p[3]);
  }
}

// 64 * sum(c * qb) from the four plane sums (plane k is 4^k-scaled).
__device__ __forceinline__ uint32_t combine_scaled(const uint32_t (&p)[4]) {
  return ((((p[0] << 2) + p[1]) << 2) + p[2]) * 4u + p[3];
}

// sum(c * qb) exactly, without the 64x headroom (any K).
__device__ __forceinline__ uint32_t combine_exact(const uint32_t (&p)[4]) {
  return p[0] + (p[1] >> 2) + (p[2] >> 4) + (p[3] >> 6);
}

template <int N>
__device__ __forceinline__ uint32_t pick(const uint32_t (&v)[N], int i) {
  uint32_t r = v[0];
#pragma unroll
  for (int k = 1; k < N; ++k) r = (i == k) ? v[k] : r;
  return r;
}

__device__ __forceinline__ void store_out(const LinearArgs& a, int m, int row, uint32_t s,
                                          uint32_t qb_sum, int32_t zb, int32_t rs, float sr,
                                          float sa) {
  const int32_t acc = (int32_t)(s - qb_sum - (uint32_t)zb * (uint32_t)rs);
  const int64_t o = (int64_t)m * a.ldy + row;
  store_g(a.y + o, epilogue(sr, acc, sa));
  if (a.acc) store_g(a.acc + o, acc);
}

// ---------------------------------------------------------------------------
// One token, activations held in registers: lane (sub, r) of the wave owns
// chunks r, r + LPR, ..., r + LPR*(CPL-1) of rows  base + u*RPW + sub.
// Units of U*RPW rows are taken as unit0, unit0 + ustride, ... inside
// [row_lo, row_hi).
template <int LPR, int CPL, int U, bool RAGGED>
__device__ __forceinline__ void valu_range_reg(const LinearArgs& a, int row_lo, int row_hi,
                                               int unit0, int ustride, int lane) {
  constexpr int RPW = 64 / LPR;
  constexpr int UNIT = U * RPW;
  static_assert(U <= LPR, "U");
  static_assert(64.0 * 510.0 * 64.0 * LPR * CPL < 2147483648.0, "scaled sum headroom");
  const int sub = lane / LPR, r = lane % LPR;
  const int nch = a.nch;

  uint32_t qc[CPL][16];
  uint32_t qsum = 0;
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int ch = r + LPR * t;
    if (ch < nch) {
      load_q_chunk<RAGGED>(a.q, a.K, ch, qc[t]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) qc[t][i] = 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) qsum = udot4(qc[t][i], kOnes, qsum);
  }
  const uint32_t qb_sum = group_sum<LPR>(qsum);

  const int my_u = split_index<LPR, U>(lane);
  const bool writer = (r % (LPR / U)) == 0;
  const float sa = load_g(a.s_act);
  const int32_t zb = load_g(a.z) + 128;

  // One unit's loads: U*CPL 16-byte weight chunks per lane plus the row sum
  // and scale of the row this lane may store, all range-checked buffer
  // loads over the unit's rows: rows past row_hi read as zero and are never
  // stored, and a unit with live == false (there is no next unit) reads
  // nothing at all -- the loads are still issued, so the wait counts are the
  // same on every iteration.  Chunks past the row (K < 64 * LPR * CPL) are
  // clamped to the row's last chunk; they meet zero activations.  All
  // offsets below are fixed per lane.
  struct Unit {
    u32x4 w[U][CPL];
    int32_t rs;
    float sr;
  };
  uint32_t woff[U][CPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < CPL; ++t)
      woff[u][t] = (uint32_t)(u * RPW + sub) * (uint32_t)a.ld + 16u * (uint32_t)min(r + LPR * t, nch - 1);
  const uint32_t roff = (uint32_t)(my_u * RPW + sub) * 4u;
  auto issue = [&](int base, bool live, Unit& b) {
    const uint32_t n = live ? (uint32_t)min(UNIT, row_hi - base) : 0u;
    const auto rw = buffer_rsrc(const_cast<uint8_t*>(a.packed) + (int64_t)base * a.ld, n * (uint32_t)a.ld);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < CPL; ++t) b.w[u][t] = buffer_load_weights16(rw, woff[u][t]);
    b.rs = (int32_t)buffer_load_u32(buffer_rsrc(const_cast<int32_t*>(a.rowsum) + base, 4u * n), roff);
    b.sr = __uint_as_float(buffer_load_u32(buffer_rsrc(const_cast<float*>(a.s_row) + base, 4u * n), roff));
  };

  // Two units in flight: the next unit's loads are issued before the
  // current one is reduced, so each wave keeps its memory queue busy while
  // it computes.  The loop alternates two buffers (no copy between them,
  // which would wait for the loads in flight).  Outputs go out through
  // range-checked buffer stores (rows of the unit past row_hi and
  // non-writer lanes are dropped).
  auto finish = [&](const Unit& c, int base) {
    uint32_t part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t p[4] = {0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < CPL; ++t) dot_chunk(c.w[u][t], qc[t], p);
      part[u] = combine_scaled(p);
    }
    const uint32_t tot = reduce_split<LPR, U>(part, lane);
    const int32_t acc = (int32_t)((tot >> 6) - qb_sum - (uint32_t)zb * (uint32_t)c.rs);
    const uint32_t rows = (uint32_t)min(UNIT, row_hi - base) * 4u;
    const uint32_t off = writer ? roff : kDropOffset;
    buffer_store_u32(__float_as_uint(epilogue(c.sr, acc, sa)), buffer_rsrc(a.y + base, rows), off);
    buffer_store_u32((uint32_t)acc, buffer_rsrc(a.acc ? a.acc + base : nullptr, a.acc ? rows : 0u), off);
  };
  const int step = ustride * UNIT;
  if ((int64_t)row_lo + (int64_t)unit0 * UNIT >= row_hi) return;
  int base = row_lo + unit0 * UNIT;
  Unit ua, ub;
  issue(base, true, ua);
#pragma unroll 1
  for (;;) {
    // (64-bit compare: base + step may pass INT_MAX for N near it)
    bool more = (int64_t)base + step < row_hi;
    issue(more ? base + step : base, more, ub);
    __builtin_amdgcn_sched_barrier(0);  // the next unit's loads go out first
    finish(ua, base);
    if (!more) break;
    base += step;
    more = (int64_t)base + step < row_hi;
    issue(more ? base + step : base, more, ua);
    __builtin_amdgcn_sched_barrier(0);
    finish(ub, base);
    if (!more) break;
    base += step;
  }
}

// ---------------------------------------------------------------------------
// Block-wise scales along K, one token (article "Neutrino-1: quantization is
// a training decision, not a deployment one", "What's actually ternary": a
// scale per fixed-size block of the input dimension).  Blocks of
// B = 64 * 2^blg columns; lane (sub, r) holds chunk r + LPR t of its rows,
// so a block is an aligned group of G = 2^blg lanes of one slice t (G <= LPR).
// The group sums its lanes' exact sum(c * qb) into S_b and forms
//     acc_b = S_b - QB_b - (z + 128) * rowsum_b        (exact, wrapping int32)
// (QB_b: the block's biased activations); the first lane of the group puts
// s_b * (float)acc_b (one rounding) into the wave's LDS row, and lane j then
// adds row j's products in block order b = 0, 1, ... (one rounding each,
// from +0) and multiplies by s_act: the order of the definition, so y has
// the bits of its left-to-right evaluation.  acc, when asked for, is
// sum_b acc_b.
constexpr int kBlkLdsWave = 8192;  // LDS bytes per wave for the row products

// sum over aligned groups of 2^lg lanes (lg <= 6), in every lane
__device__ __forceinline__ uint32_t group_sum_lg(uint32_t x, int lg) {
  if (lg >= 1) x = pair_sum<1>(x);
  if (lg >= 2) x = pair_sum<2>(x);
  if (lg >= 3) x = pair_sum<4>(x);
  if (lg >= 4) x = pair_sum<8>(x);
  if (lg >= 5) x = pair_sum<16>(x);
  if (lg >= 6) x = pair_sum<32>(x);
  return x;
}

template <int LPR, int CPL, int U>
__device__ __forceinline__ void valu_range_blk(const LinearArgs& a, int row_lo, int row_hi, int unit0,
                                               int ustride, int lane, float* prow, int pitch) {
  constexpr int RPW = 64 / LPR;
  constexpr int UNIT = U * RPW;
  const int sub = lane / LPR, r = lane % LPR;
  const int nch = a.nch, lg = a.blg, nb = a.nb;
  int32_t* arow = reinterpret_cast<int32_t*>(prow + UNIT * pitch);  // block accs, when acc is asked for

  // activations in registers (as the per-row path), and per slice the
  // block's biased activation sum
  uint32_t qc[CPL][16];
  uint32_t qbb[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int ch = r + LPR * t;
    if (ch < nch) {
      load_q_chunk<false>(a.q, a.K, ch, qc[t]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) qc[t][i] = 0;
    }
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = udot4(qc[t][i], kOnes, s);
    qbb[t] = group_sum_lg(s, lg);
  }
  const float sa = load_g(a.s_act);
  const uint32_t zb = (uint32_t)(load_g(a.z) + 128);
  const bool first = (r & ((1 << lg) - 1)) == 0;

  // one unit's loads: weight chunks, and the scale and row sum of the block
  // of each (row, slice), through range-checked buffer loads over the
  // unit's rows (rows past row_hi read as zero and are never stored; a
  // unit with live == false reads nothing)
  struct Unit {
    u32x4 w[U][CPL];
    int32_t rs[U][CPL];
    float sb[U][CPL];
  };
  uint32_t woff[U][CPL], boff[U][CPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int ch = r + LPR * t;
      woff[u][t] = (uint32_t)(u * RPW + sub) * (uint32_t)a.ld + 16u * (uint32_t)min(ch, nch - 1);
      boff[u][t] = ((uint32_t)(u * RPW + sub) * (uint32_t)nb + (uint32_t)min(ch >> lg, nb - 1)) * 4u;
    }
  auto issue = [&](int base, bool live, Unit& b) {
    const uint32_t n = live ? (uint32_t)min(UNIT, row_hi - base) : 0u;
    const auto rw = buffer_rsrc(const_cast<uint8_t*>(a.packed) + (int64_t)base * a.ld, n * (uint32_t)a.ld);
    const auto rr = buffer_rsrc(const_cast<int32_t*>(a.rowsum_b) + (int64_t)base * nb, n * (uint32_t)nb * 4u);
    const auto rsb = buffer_rsrc(const_cast<float*>(a.s_b) + (int64_t)base * nb, n * (uint32_t)nb * 4u);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        b.w[u][t] = buffer_load_weights16(rw, woff[u][t]);
        b.rs[u][t] = (int32_t)buffer_load_u32(rr, boff[u][t]);
        b.sb[u][t] = __uint_as_float(buffer_load_u32(rsb, boff[u][t]));
      }
  };
  auto finish = [&](const Unit& c, int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        uint32_t p[4] = {0, 0, 0, 0};
        dot_chunk(c.w[u][t], qc[t], p);
        const uint32_t sbk = group_sum_lg(combine_exact(p), lg);
        const int32_t accb = (int32_t)(sbk - qbb[t] - mul_zr((int32_t)zb, c.rs[u][t]));
        const int ch = r + LPR * t;
        if (first && ch < nch) {
          const int o = (u * RPW + sub) * pitch + (ch >> lg);
          prow[o] = __fmul_rn(c.sb[u][t], (float)accb);
          if (a.acc) arow[o] = accb;
        }
      }
    }
    wait_lds();  // the wave's products are in LDS (its own accesses complete in order)
    // lane j < UNIT: row j of the unit, its blocks in order
    const int j = lane;
    const int row = base + j;
    float tot = 0.0f;
    int32_t isum = 0;
    if (j < UNIT && row < row_hi) {
      const float* pr = prow + j * pitch;
      int b = 0;
      for (; b + 4 <= nb; b += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pr + b);
        tot = __fadd_rn(tot, v.x);
        tot = __fadd_rn(tot, v.y);
        tot = __fadd_rn(tot, v.z);
        tot = __fadd_rn(tot, v.w);
      }
      for (; b < nb; ++b) tot = __fadd_rn(tot, pr[b]);
      if (a.acc) {
        const int32_t* ar = arow + j * pitch;
        for (int k = 0; k < nb; ++k) isum += ar[k];
      }
    }
    const uint32_t rows = (uint32_t)min(UNIT, row_hi - base) * 4u;
    const uint32_t off = j < UNIT ? 4u * (uint32_t)j : kDropOffset;
    buffer_store_u32(__float_as_uint(__fmul_rn(tot, sa)), buffer_rsrc(a.y + base, rows), off);
    buffer_store_u32((uint32_t)isum, buffer_rsrc(a.acc ? a.acc + base : nullptr, a.acc ? rows : 0u), off);
    wait_lds();  // every lane has read its row before the next unit's products go in
  };
  const int step = ustride * UNIT;
  if ((int64_t)row_lo + (int64_t)unit0 * UNIT >= row_hi) return;
  int base = row_lo + unit0 * UNIT;
  Unit ua, ub;
  issue(base, true, ua);
#pragma unroll 1
  for (;;) {
    bool more = (int64_t)base + step < row_hi;
    issue(more ? base + step : base, more, ub);
    __builtin_amdgcn_sched_barrier(0);  // the next unit's loads go out first
    finish(ua, base);
    if (!more) break;
    base += step;
    more = (int64_t)base + step < row_hi;
    issue(more ? base + step : base, more, ua);
    __builtin_amdgcn_sched_barrier(0);
    finish(ub, base);
    if (!more) break;
    base += step;
  }
}

// ---------------------------------------------------------------------------
// Any K, MT tokens (rows of q streamed through registers one 64-weight chunk
// at a time).  One row per 64 lanes, U rows per unit.
template <int U, int MT>
__device__ __forceinline__ void valu_range_stream(const LinearArgs& a, int row_lo, int row_hi,
                                                  int unit0, int ustride, int lane) {
  constexpr int NV = U * MT;
  static_assert(NV <= 64, "NV");
  const int nch = a.nch;
  const int M = a.M;

  // biased activation sums per token
  uint32_t qb_sums[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t s = 0;
    if (m < M) {
      for (int ch = lane; ch < nch; ch += 64) {
        uint32_t qc[16];
        load_q_chunk<true>(a.q + (int64_t)m * a.ldq, a.K, ch, qc);
#pragma unroll
        for (int i = 0; i < 16; ++i) s = udot4(qc[i], kOnes, s);
      }
    }
    qb_sums[m] = group_sum<64>(s);
  }

  const int vidx = split_index<64, NV>(lane);
  const int my_u = vidx / MT, my_m = vidx % MT;
  const bool writer = (lane % (64 / NV)) == 0;
  const uint32_t my_qb = pick<MT>(qb_sums, my_m);
  const bool tok_ok = my_m < M;
  const float sa = tok_ok ? load_g(a.s_act + my_m) : 0.f;
  const int32_t zb = tok_ok ? load_g(a.z + my_m) + 128 : 0;

#pragma unroll 1
  for (int unit = unit0;; unit += ustride) {
    if ((int64_t)row_lo + (int64_t)unit * U >= row_hi) break;
    const int base = row_lo + unit * U;
    uint32_t part[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) part[v] = 0;
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const int ch = c0 + lane;
      const int ch_c = min(ch, nch - 1);  // past the row: activations are zero
      u32x4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = min(base + u, row_hi - 1);
        w[u] = load_weights16(a.packed + (int64_t)row * a.ld + 16 * ch_c);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint32_t qc[16];
        if (m < M && ch < nch) {
          load_q_chunk<true>(a.q + (int64_t)m * a.ldq, a.K, ch, qc);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) qc[i] = 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint32_t p[4] = {0, 0, 0, 0};
          dot_chunk(w[u], qc, p);
          part[u * MT + m] += combine_exact(p);
        }
      }
    }
    const int my_row = base + my_u;
    const bool do_store = writer && tok_ok && my_row < row_hi;
    const uint32_t tot = reduce_split<64, NV>(part, lane);
    if (do_store) {
      store_out(a, my_m, my_row, tot, my_qb, zb, load_g(a.rowsum + my_row),
                load_g(a.s_row + my_row), sa);
    }
  }
}

// Rows per unit and dispatch of the register variants.
template <int V>
struct ValuCfg;
template <> struct ValuCfg<V8x1>  { static constexpr int LPR = 8,  CPL = 1, U = 8; };
template <> struct ValuCfg<V16x1> { static constexpr int LPR = 16, CPL = 1, U = 8; };
template <> struct ValuCfg<V32x1> { static constexpr int LPR = 32, CPL = 1, U = 8; };
template <> struct ValuCfg<V16x3> { static constexpr int LPR = 16, CPL = 3, U = 2; };
template <> struct ValuCfg<V64x1> { static constexpr int LPR = 64, CPL = 1, U = 8; };
template <> struct ValuCfg<V64x2> { static constexpr int LPR = 64, CPL = 2, U = 4; };
template <> struct ValuCfg<V64x3> { static constexpr int LPR = 64, CPL = 3, U = 2; };
template <> struct ValuCfg<V64x4> { static constexpr int LPR = 64, CPL = 4, U = 2; };
constexpr int kStreamU = 8;

template <int V, bool RAGGED>
__device__ __forceinline__ void run_reg(const LinearArgs& a, int lo, int hi, int u0, int us, int lane) {
  using C = ValuCfg<V>;
  valu_range_reg<C::LPR, C::CPL, C::U, RAGGED>(a, lo, hi, u0, us, lane);
}

// Units of the block-scaled path: fewer rows than the per-row path (each
// (row, slice) also loads its block's scale and row sum).
template <int V> struct BlkU;
template <> struct BlkU<V8x1>  { static constexpr int U = 2; };
template <> struct BlkU<V16x1> { static constexpr int U = 2; };
template <> struct BlkU<V32x1> { static constexpr int U = 2; };
template <> struct BlkU<V16x3> { static constexpr int U = 1; };
template <> struct BlkU<V64x1> { static constexpr int U = 4; };
template <> struct BlkU<V64x2> { static constexpr int U = 2; };
template <> struct BlkU<V64x3> { static constexpr int U = 2; };
template <> struct BlkU<V64x4> { static constexpr int U = 1; };

template <int V>
__device__ __forceinline__ void run_blk(const LinearArgs& a, int lo, int hi, int u0, int us, int lane,
                                        float* prow) {
  using C = ValuCfg<V>;
  // a row pitch of the products that is a multiple of 4 floats and 4 more
  // than needed, so that lanes reading rows side by side use other banks
  const int pitch = (a.nb + 3) / 4 * 4 + 4;
  valu_range_blk<C::LPR, C::CPL, BlkU<V>::U>(a, lo, hi, u0, us, lane, prow, pitch);
}

// A block-scaled linear of the M = 1 stack (register variants in VSET; the
// host picks one whose lanes per row hold whole blocks).
template <uint32_t VSET>
__device__ __forceinline__ void valu_m1_segment_blk(const LinearArgs& a, int lo, int hi, int lane, float* prow) {
#define TERN_BLK_CASE(V)                                                 \
  case V:                                                                \
    if constexpr ((VSET >> V) & 1u) run_blk<V>(a, lo, hi, 0, 1, lane, prow); \
    break;
  switch (a.variant) {
    TERN_BLK_CASE(V8x1)
    TERN_BLK_CASE(V16x1)
    TERN_BLK_CASE(V32x1)
    TERN_BLK_CASE(V16x3)
    TERN_BLK_CASE(V64x1)
    TERN_BLK_CASE(V64x2)
    TERN_BLK_CASE(V64x3)
    TERN_BLK_CASE(V64x4)
    default: break;
  }
#undef TERN_BLK_CASE
}

// M = 1, one segment of a prepared stack.  VSET is the set of variants the
// kernel is compiled for (bit V for register variant V, bit VGEN for the
// streaming one, which also takes K not a multiple of 64): each extra
// variant in the switch can raise the register budget of the whole kernel,
// so the host picks the smallest set that covers the stack.
template <uint32_t VSET>
__device__ __forceinline__ void valu_m1_segment(const LinearArgs& a, int lo, int hi, int lane) {
  if constexpr ((VSET >> VGEN) & 1u) {
    if ((a.K & 63) != 0 || a.variant == VGEN) {
      valu_range_stream<kStreamU, 1>(a, lo, hi, 0, 1, lane);
      return;
    }
  }
#define TERN_SEG_CASE(V)                                  \
  case V:                                                 \
    if constexpr ((VSET >> V) & 1u) run_reg<V, false>(a, lo, hi, 0, 1, lane); \
    break;
  switch (a.variant) {
    TERN_SEG_CASE(V8x1)
    TERN_SEG_CASE(V16x1)
    TERN_SEG_CASE(V32x1)
    TERN_SEG_CASE(V16x3)
    TERN_SEG_CASE(V64x1)
    TERN_SEG_CASE(V64x2)
    TERN_SEG_CASE(V64x3)
    TERN_SEG_CASE(V64x4)
    default: break;
  }
#undef TERN_SEG_CASE
}

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that consecutive schedule ranges land on the same XCD (and its L2).
__device__ __forceinline__ int xcd_logical_block() {
  const int n = gridDim.x, b = blockIdx.x;
  return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

// Variant sets the persistent M = 1 kernel is compiled for.
constexpr uint32_t bit(int v) { return 1u << v; }
constexpr uint32_t kSet8B = bit(V64x1) | bit(V64x3);
constexpr uint32_t kSet06B = bit(V16x1) | bit(V32x1) | bit(V16x3);
constexpr uint32_t kSetReg = bit(V8x1) | bit(V16x1) | bit(V32x1) | bit(V16x3) | bit(V64x1) |
                             bit(V64x2) | bit(V64x3) | bit(V64x4);
constexpr uint32_t kSetAll = kSetReg | bit(VGEN);
constexpr uint32_t kSets[] = {kSet8B, kSet06B, kSetReg, kSetAll};
constexpr uint32_t kNone = 0;

}  // namespace

template <int V, bool RAGGED>
__global__ __launch_bounds__(kBlock) void valu_linear_kernel(LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesPerBlock + wave_id_uniform();
  const int nw = gridDim.x * kWavesPerBlock;
  run_reg<V, RAGGED>(a, 0, a.N, wave, nw, lane);
}

template <int MT>
__global__ __launch_bounds__(kBlock) void valu_stream_kernel(LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesPerBlock + wave_id_uniform();
  const int nw = gridDim.x * kWavesPerBlock;
  valu_range_stream<(MT >= 8 ? 4 : kStreamU), MT>(a, 0, a.N, wave, nw, lane);
}

template <int MT, uint32_t VSET>
__global__ __launch_bounds__(kBlock) void valu_stack_kernel(const StackHeader* __restrict__ h,
                                  StackSync* __restrict__ sy) {
  __shared__ PrologueLds prol;
  const uint32_t launch1 = stack_prologue(h, sy, prol);
  const int lane = threadIdx.x & 63;
  const int worker = xcd_logical_block() * kWavesPerBlock + wave_id_uniform();
  if (worker >= h->workers) return;
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(
      reinterpret_cast<const char*>(h) + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(
      reinterpret_cast<const char*>(h) + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(
      reinterpret_cast<const char*>(h) + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    if constexpr (MT == 1)
      valu_m1_segment<VSET>(a, sg.row_begin, sg.row_end, lane);
    else
      valu_range_stream<(MT >= 8 ? 4 : kStreamU), MT>(a, sg.row_begin, sg.row_end, 0, 1, lane);
  }
}

// M = 1 stacks holding block-scaled linears: those take the block path,
// the others the per-row path (both compiled for the variant set VSET).
template <uint32_t VSET>
__global__ __launch_bounds__(kBlock) void valu_stack_blk_kernel(const StackHeader* __restrict__ h,
                                  StackSync* __restrict__ sy) {
  __shared__ __attribute__((aligned(16))) float prods[kWavesPerBlock][kBlkLdsWave / 4];
  __shared__ PrologueLds prol;
  const uint32_t launch1 = stack_prologue(h, sy, prol);
  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const int worker = xcd_logical_block() * kWavesPerBlock + w;
  if (worker >= h->workers) return;
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(
      reinterpret_cast<const char*>(h) + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(
      reinterpret_cast<const char*>(h) + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(
      reinterpret_cast<const char*>(h) + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    if (a.s_b)
      valu_m1_segment_blk<VSET>(a, sg.row_begin, sg.row_end, lane, prods[w]);
    else
      valu_m1_segment<VSET>(a, sg.row_begin, sg.row_end, lane);
  }
}

// Stacks of 2..8 tokens holding block-scaled linears: every segment is run
// token by token through the M = 1 paths above (block-scaled linears the
// block path, the others the per-row one), token m reading q row m, s_act[m]
// and z[m] and writing y (and acc) row m.  A segment's rows are re-read for
// each token from the L2 (a segment is a few hundred KB at most), and each
// token's y has the bits of the one-token evaluation, the blocks summed in
// order.  It takes block sizes the activation-window kernels cannot (below
// 512 columns), at the M = 1 path's vector-ALU cost per token.
template <uint32_t VSET>
__global__ __launch_bounds__(kBlock) void valu_stack_tok_kernel(const StackHeader* __restrict__ h,
                                  StackSync* __restrict__ sy) {
  __shared__ __attribute__((aligned(16))) float prods[kWavesPerBlock][kBlkLdsWave / 4];
  __shared__ PrologueLds prol;
  const uint32_t launch1 = stack_prologue(h, sy, prol);
  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const int worker = xcd_logical_block() * kWavesPerBlock + w;
  if (worker >= h->workers) return;
  const LinearArgs* lin = reinterpret_cast<const LinearArgs*>(
      reinterpret_cast<const char*>(h) + h->off_lin);
  const int32_t* seg_start = reinterpret_cast<const int32_t*>(
      reinterpret_cast<const char*>(h) + h->off_seg_start);
  const Segment* seg = reinterpret_cast<const Segment*>(
      reinterpret_cast<const char*>(h) + h->off_seg);
  const int s1 = seg_start[worker + 1];
  wait_segment_inputs(h, sy, lin, seg, seg_start[worker], s1, launch1);
  for (int s = seg_start[worker]; s < s1; ++s) {
    const Segment sg = seg[s];
    const LinearArgs a = lin[sg.lin];
    for (int m = 0; m < a.M; ++m) {
      LinearArgs t = a;
      t.M = 1;
      t.q = a.q + (int64_t)m * a.ldq;
      t.s_act = a.s_act + m;
      t.z = a.z + m;
      t.y = a.y + (int64_t)m * a.ldy;
      if (a.acc) t.acc = a.acc + (int64_t)m * a.ldy;
      if (t.s_b)
        valu_m1_segment_blk<VSET>(t, sg.row_begin, sg.row_end, lane, prods[w]);
      else
        valu_m1_segment<VSET>(t, sg.row_begin, sg.row_end, lane);
    }
  }
}

// ------------------------------------------------------------- launchers --

// The register variant of a block-scaled linear: the per-row one when its
// lanes per row hold whole blocks (B <= 64 * LPR), else the 64-lane one for
// K; -1 when no register variant takes K (K > 16,384 or not a multiple of 64).
int32_t valu_blocked_variant(int64_t K, int64_t B) {
  if (K % 64 != 0 || K > 16384) return -1;
  const int32_t v = valu_variant_for(K);
  int lpr = 64;
  switch (v) {
    case V8x1: lpr = ValuCfg<V8x1>::LPR; break;
    case V16x1: lpr = ValuCfg<V16x1>::LPR; break;
    case V32x1: lpr = ValuCfg<V32x1>::LPR; break;
    case V16x3: lpr = ValuCfg<V16x3>::LPR; break;
    default: break;
  }
  if (B <= 64 * lpr) return v;
  return K <= 4096 ? V64x1 : K <= 8192 ? V64x2 : K <= 12288 ? V64x3 : V64x4;
}

int valu_blocked_unit_rows(int32_t variant) {
  switch (variant) {
    case V8x1: return BlkU<V8x1>::U * 64 / ValuCfg<V8x1>::LPR;
    case V16x1: return BlkU<V16x1>::U * 64 / ValuCfg<V16x1>::LPR;
    case V32x1: return BlkU<V32x1>::U * 64 / ValuCfg<V32x1>::LPR;
    case V16x3: return BlkU<V16x3>::U * 64 / ValuCfg<V16x3>::LPR;
    case V64x1: return BlkU<V64x1>::U;
    case V64x2: return BlkU<V64x2>::U;
    case V64x3: return BlkU<V64x3>::U;
    default: return BlkU<V64x4>::U;
  }
}

int32_t valu_variant_for(int64_t K) {
  if (K <= 512) return V8x1;
  if (K <= 1024) return V16x1;
  if (K <= 2048) return V32x1;
  if (K <= 3072) return V16x3;
  if (K <= 4096) return V64x1;
  if (K <= 8192) return V64x2;
  if (K <= 12288) return V64x3;
  if (K <= 16384) return V64x4;
  return VGEN;
}

static int stream_u(int32_t M) { return M > 4 ? 4 : kStreamU; }

int valu_unit_rows(int32_t variant, int32_t M) {
  if (M > 1) return stream_u(M);
  switch (variant) {
    case V8x1: return ValuCfg<V8x1>::U * 64 / ValuCfg<V8x1>::LPR;
    case V16x1: return ValuCfg<V16x1>::U * 64 / ValuCfg<V16x1>::LPR;
    case V32x1: return ValuCfg<V32x1>::U * 64 / ValuCfg<V32x1>::LPR;
    case V16x3: return ValuCfg<V16x3>::U * 64 / ValuCfg<V16x3>::LPR;
    case V64x1: return ValuCfg<V64x1>::U;
    case V64x2: return ValuCfg<V64x2>::U;
    case V64x3: return ValuCfg<V64x3>::U;
    case V64x4: return ValuCfg<V64x4>::U;
    default: return kStreamU;
  }
}

static int blocks_for_units(int64_t units) {
  // enough waves to cover the units, capped at 64 workgroups per CU-sized
  // slice; each wave loops over its units
  int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

hipError_t launch_valu_linear(const LinearArgs& a, hipStream_t s) {
  const int64_t units = (a.N + valu_unit_rows(a.variant, a.M) - 1) / valu_unit_rows(a.variant, a.M);
  const dim3 grid(blocks_for_units(units)), block(kBlock);
  if (a.M == 1) {
    const bool ragged = (a.K & 63) != 0;
#define TERN_REG_CASE(V)                                                              \
  case V:                                                                             \
    if (ragged)                                                                       \
      hipLaunchKernelGGL((valu_linear_kernel<V, true>), grid, block, 0, s, a);        \
    else                                                                              \
      hipLaunchKernelGGL((valu_linear_kernel<V, false>), grid, block, 0, s, a);       \
    break;
    switch (a.variant) {
      TERN_REG_CASE(V8x1)
      TERN_REG_CASE(V16x1)
      TERN_REG_CASE(V32x1)
      TERN_REG_CASE(V16x3)
      TERN_REG_CASE(V64x1)
      TERN_REG_CASE(V64x2)
      TERN_REG_CASE(V64x3)
      TERN_REG_CASE(V64x4)
      default: hipLaunchKernelGGL(valu_stream_kernel<1>, grid, block, 0, s, a); break;
    }
#undef TERN_REG_CASE
  } else if (a.M == 2) {
    hipLaunchKernelGGL(valu_stream_kernel<2>, grid, block, 0, s, a);
  } else if (a.M <= 4) {
    hipLaunchKernelGGL(valu_stream_kernel<4>, grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL(valu_stream_kernel<8>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}


int32_t valu_stack_kernel_for(int32_t M, uint32_t used_variants, bool blocked) {
  if (M == 1 || blocked) {
    const int32_t k0 = blocked ? (M == 1 ? SK_VALU_M1_BLK : SK_VALU_TOK_BLK) : SK_VALU_M1;
    for (int i = 0; i < 4; ++i)
      if ((used_variants & ~kSets[i]) == 0) return k0 + i;
    return k0 + 3;
  }
  if (M == 2) return SK_VALU_M2;
  if (M <= 4) return SK_VALU_M4;
  return SK_VALU_M8;
}

template <typename F>
static hipError_t with_valu_stack_kernel(int32_t kernel, F&& f) {
  switch (kernel) {
    case SK_VALU_M1 + 0: return f(valu_stack_kernel<1, kSets[0]>);
    case SK_VALU_M1 + 1: return f(valu_stack_kernel<1, kSets[1]>);
    case SK_VALU_M1 + 2: return f(valu_stack_kernel<1, kSets[2]>);
    case SK_VALU_M1 + 3: return f(valu_stack_kernel<1, kSets[3]>);
    case SK_VALU_M2: return f(valu_stack_kernel<2, kNone>);
    case SK_VALU_M4: return f(valu_stack_kernel<4, kNone>);
    case SK_VALU_M8: return f(valu_stack_kernel<8, kNone>);
    case SK_VALU_M1_BLK + 0: return f(valu_stack_blk_kernel<kSets[0]>);
    case SK_VALU_M1_BLK + 1: return f(valu_stack_blk_kernel<kSets[1]>);
    case SK_VALU_M1_BLK + 2: return f(valu_stack_blk_kernel<kSets[2]>);
    case SK_VALU_M1_BLK + 3: return f(valu_stack_blk_kernel<kSets[3]>);
    case SK_VALU_TOK_BLK + 0: return f(valu_stack_tok_kernel<kSets[0]>);
    case SK_VALU_TOK_BLK + 1: return f(valu_stack_tok_kernel<kSets[1]>);
    case SK_VALU_TOK_BLK + 2: return f(valu_stack_tok_kernel<kSets[2]>);
    case SK_VALU_TOK_BLK + 3: return f(valu_stack_tok_kernel<kSets[3]>);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_valu_stack(int32_t kernel, const void* ws, const LaunchShape& shp, hipStream_t s) {
  const StackHeader* h = static_cast<const StackHeader*>(ws);
  const dim3 grid(shp.grid), block(shp.block);
  return with_valu_stack_kernel(kernel, [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, h, stack_sync(ws));
    return hipGetLastError();
  });
}

int valu_stack_blocks_per_cu(int32_t kernel) {
  int n = 0;
  const hipError_t e = with_valu_stack_kernel(kernel, [&](auto kern) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kBlock, 0);
  });
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace tern
