// tern_packed5.hip -- the 1.6-bit layout: five ternary weights per byte.
//
// Three states hold about 1.58 bits of information per weight (article
// "Neutrino-1: quantization is a training decision, not a deployment one",
// "Where the bytes go"); 2-bit fields spend a fifth of every row on nothing.
// This layout (the project's own, as is the 2-bit one) packs five weights
// per byte, 20 % fewer bytes per row than the 2-bit layout:
//
//   digits d = w + 1 of a byte's five weights, most significant first:
//     v = 81 d0 + 27 d1 + 9 d2 + 3 d3 + d4           (0 <= v <= 242)
//   stored byte b = ceil(256 v / 243), i.e. v / 243 as an 8-bit fraction
//   row stride 16 * ceil(K / 80) bytes (a 16-byte chunk holds 80 weights)
//   weight j: digit (j % 20) / 4 of byte 4 * (j / 20) + j % 4, so digit i of
//     the four bytes of a word holds weights 4i .. 4i+3 of that word
//   padding columns hold weight 0 (a padding-only byte reads 0x80)
//
// Decode.  Tripling b pushes the next digit above bit 8:  H_i =
// floor(3^i b / 256) = 3 H_(i-1) + d_i, and H_5 = v.  Each byte sits in its
// own 16-bit lane of a register (bytes 0 and 2 in one, 1 and 3 in another;
// 3^i b < 2^16 for i <= 5), so H_i of all four bytes is one 24-bit multiply
// per register and one v_perm_b32 that gathers the four high bytes.  The
// digits themselves are never formed: with the biased activations u (q + 128)
// of digit i's four weights in U_i,
//     sum_i dot(d_i, U_i) = sum_i dot(H_i, U_i) - 3 sum_(i<5) dot(H_i, U_(i+1))
// (d_i = H_i - 3 H_(i-1), H_0 = 0), which is 26 VALU operations per 20
// weights (two splits, ten multiplies, five perms, nine dot4s), against 0.5
// per weight for the 2-bit layout.
//
// The rest is the 2-bit path's arithmetic: with S = sum_j d_j u_j (padding
// has u = 0) and QB = sum_(j<K) u_j,
//     sum_j w_j q_j - z * rowsum = S - QB - (z + 128) * rowsum     (wrapping).
#include "tern_device.h"

namespace tern {

namespace {

constexpr int kP5Block = 256;
constexpr int kP5Waves = kP5Block / 64;

__device__ __forceinline__ uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_udot4(a, b, c, false);
}

// ---- load-time packing: one wave per row, one lane per 4-byte word ----
__global__ __launch_bounds__(kP5Block) void pack5_kernel(const int8_t* __restrict__ w, int64_t N,
                                                         int K, int64_t ldw, int words,
                                                         uint8_t* __restrict__ packed,
                                                         int32_t* __restrict__ rowsum,
                                                         int32_t* __restrict__ bad) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kP5Waves + (threadIdx.x >> 6);
  if (row >= N) return;
  const int8_t* wr = w + row * ldw;
  uint32_t* out = reinterpret_cast<uint32_t*>(packed + row * (int64_t)words * 4);
  int32_t sum = 0, nbad = 0;
  for (int wi = lane; wi < words; wi += 64) {
    const int j0 = 20 * wi;
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      uint32_t v = 0;  // Horner over the byte's digits, most significant first
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int j = j0 + 4 * i + n;
        uint32_t d = 1u;  // weight 0: padding and values outside {-1, 0, 1}
        if (j < K) {
          const int x = wr[j];
          if (x >= -1 && x <= 1) {
            d = (uint32_t)(x + 1);
            sum += x;
          } else {
            ++nbad;
          }
        }
        v = 3u * v + d;
      }
      word |= ((256u * v + 242u) / 243u) << (8 * n);
    }
    out[wi] = word;
  }
  sum = (int32_t)group_sum<64>((uint32_t)sum);
  nbad = (int32_t)group_sum<64>((uint32_t)nbad);
  if (lane == 0) {
    rowsum[row] = sum;
    if (bad && nbad) atomicAdd(bad, nbad);
  }
}

// ---- M = 1 linear ----
struct Gemv5Args {
  const uint8_t* packed;
  const float* s_row;
  const int32_t* rowsum;
  const int8_t* q;
  const float* s_act;
  const int32_t* z;
  float* y;
  int32_t* acc;
  int32_t N, K, ld, nch;  // ld = 16 * nch bytes per row
};

// One packed word (20 weights) against its activations u[0..4] (u[i]: the
// biased activations of digit i of bytes 0..3): a += sum_i dot(H_i, u[i]),
// b += sum_(i<4) dot(H_i, u[i + 1]).
__device__ __forceinline__ void word5(uint32_t x, const uint32_t* u, uint32_t& a, uint32_t& b) {
  const uint32_t lo = x & 0x00FF00FFu;                           // bytes 0, 2
  const uint32_t hi = __builtin_amdgcn_perm(0u, x, 0x0C030C01u);  // bytes 1, 3
  constexpr uint32_t kPow3[5] = {3u, 9u, 27u, 81u, 243u};
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t yl = lo * kPow3[i];
    const uint32_t yh = hi * kPow3[i];
    // (24-bit operands: v_mul_u32_u24) bytes 1 and 3 of each: H_i of bytes
    // 0, 1, 2, 3 in byte order
    const uint32_t h = __builtin_amdgcn_perm(yh, yl, 0x07030501u);
    a = udot4(h, u[i], a);
    if (i < 4) b = udot4(h, u[i + 1], b);
  }
}

// A workgroup stages the biased activations (zero past K) in LDS once, then
// its waves take units of UR = (64 / LPR) * U rows: lane group g = lane / LPR
// owns rows g*U .. g*U + U-1 of the unit, lane r = lane % LPR its 16-byte
// chunks r, r + LPR, ...  The next step's chunks are loaded (range-checked:
// rows past N and chunks past the row read as zero, and zero bytes add
// nothing) before the current step is computed.
template <int LPR, int U>
__global__ __launch_bounds__(kP5Block) void gemv5_kernel(Gemv5Args a) {
  constexpr int UR = (64 / LPR) * U;
  extern __shared__ __attribute__((aligned(16))) uint32_t qs[];  // 20 * nch words
  __shared__ uint32_t red[kP5Waves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nwords = 20 * a.nch;

  uint32_t part = 0;
  for (int e = threadIdx.x; e < nwords; e += kP5Block) {
    const int j0 = 4 * e;
    uint32_t v = 0;
    if (j0 + 4 <= a.K) {
      v = load_g(reinterpret_cast<const uint32_t*>(a.q + j0)) ^ 0x80808080u;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (j0 + b < a.K) v |= ((uint32_t)(uint8_t)load_g(a.q + j0 + b) ^ 0x80u) << (8 * b);
    }
    qs[e] = v;
    part = udot4(v, 0x01010101u, part);
  }
  part = group_sum<64>(part);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  uint32_t qb = 0;
#pragma unroll
  for (int i = 0; i < kP5Waves; ++i) qb += red[i];
  const float sa = load_g(a.s_act);
  const uint32_t zb = (uint32_t)(load_g(a.z) + 128);

  const int g = lane / LPR, r = lane % LPR;
  const int steps = (a.nch + LPR - 1) / LPR;
  const int units = (int)(((int64_t)a.N + UR - 1) / UR);
  const int wstride = (int)gridDim.x * kP5Waves;
  int unit = (int)blockIdx.x * kP5Waves + wave;
  if (unit >= units) return;

  auto issue = [&](int un, int t, bool live, u32x4 (&w)[U]) {
    const int r0 = un * UR;
    const uint32_t rows = live ? (uint32_t)min(UR, a.N - r0) : 0u;
    const auto rs = buffer_rsrc(const_cast<uint8_t*>(a.packed) + (int64_t)r0 * a.ld, rows * (uint32_t)a.ld);
    const int c = r + LPR * t;
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = buffer_load_weights16(
          rs, c < a.nch ? (uint32_t)(g * U + u) * (uint32_t)a.ld + 16u * (uint32_t)c : kDropOffset);
  };
  uint32_t sa_[U], sb_[U];
#pragma unroll
  for (int u = 0; u < U; ++u) sa_[u] = sb_[u] = 0;
  auto compute = [&](int t, const u32x4 (&w)[U]) {
    const int c = min(r + LPR * t, a.nch - 1);  // its weights are zero when clamped
    uint32_t uq[20];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&qs[20 * c + 4 * k]);
      uq[4 * k] = v.x, uq[4 * k + 1] = v.y, uq[4 * k + 2] = v.z, uq[4 * k + 3] = v.w;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) word5(w[u][k], &uq[5 * k], sa_[u], sb_[u]);
  };
  auto finish = [&](int un) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = sa_[u] - 3u * sb_[u];
      sa_[u] = sb_[u] = 0;
    }
    const uint32_t tot = reduce_split<LPR, U>(v, lane);
    const int row = un * UR + g * U + split_index<LPR, U>(lane);
    if ((r % (LPR / U)) == 0 && row < a.N) {
      const int32_t rs = load_g(a.rowsum + row);
      const int32_t accv = (int32_t)(tot - qb - zb * (uint32_t)rs);
      store_g(a.y + row, epilogue(load_g(a.s_row + row), accv, sa));
      if (a.acc) store_g(a.acc + row, accv);
    }
  };
  auto next = [&](int& un, int& t) {
    if (++t == steps) {
      t = 0;
      un += wstride;
    }
    return un < units;
  };

  u32x4 wa[U], wb[U];
  int t = 0;
  issue(unit, 0, true, wa);
#pragma unroll 1
  for (;;) {
    int nu = unit, nt = t;
    bool more = next(nu, nt);
    issue(more ? nu : unit, nt, more, wb);
    __builtin_amdgcn_sched_barrier(0);  // the next step's loads go out first
    compute(t, wa);
    if (t == steps - 1) finish(unit);
    if (!more) break;
    unit = nu, t = nt;
    nu = unit, nt = t;
    more = next(nu, nt);
    issue(more ? nu : unit, nt, more, wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(t, wb);
    if (t == steps - 1) finish(unit);
    if (!more) break;
    unit = nu, t = nt;
  }
}

// One unit per wave: the dispatcher hands out workgroups as earlier ones
// finish, which balances the tail better than a persistent grid (measured);
// each workgroup stages the activations from L2 once.
template <int LPR, int U>
hipError_t launch_gemv5_t(const Gemv5Args& a, hipStream_t s) {
  constexpr int UR = (64 / LPR) * U;
  const size_t lds = (size_t)80 * a.nch;
  const int64_t units = ((int64_t)a.N + UR - 1) / UR;
  const int64_t blocks = (units + kP5Waves - 1) / kP5Waves;
  hipLaunchKernelGGL((gemv5_kernel<LPR, U>), dim3((unsigned)blocks), dim3(kP5Block), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int packed5_lanes_per_row(int64_t K) {
  // the lane count per row that leaves the fewest lanes idle (16 on a tie)
  const int64_t nch = (K + 79) / 80;
  const int64_t s8 = 8 * ((nch + 7) / 8), s16 = 16 * ((nch + 15) / 16);
  return s8 < s16 ? 8 : 16;
}

int64_t pack5_work_items(int64_t N) { return (N + kP5Waves - 1) / kP5Waves * kP5Block; }

int64_t gemv5_work_items(int64_t N, int64_t K) {
  const int64_t ur = (64 / packed5_lanes_per_row(K)) * (packed5_lanes_per_row(K) == 8 ? 2 : 4);
  return ((N + ur - 1) / ur + kP5Waves - 1) / kP5Waves * kP5Block;
}

hipError_t launch_pack5(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                        int32_t* rowsum, int32_t* bad, hipStream_t s) {
  const int words = (int)(4 * ((K + 79) / 80));
  const dim3 grid((unsigned)((N + kP5Waves - 1) / kP5Waves)), block(kP5Block);
  hipLaunchKernelGGL(pack5_kernel, grid, block, 0, s, w, N, (int)K, ldw, words, packed, rowsum, bad);
  return hipGetLastError();
}

hipError_t launch_gemv5(const uint8_t* packed, const float* s_row, const int32_t* rowsum, int64_t N,
                        int64_t K, const int8_t* q, const float* s_act, const int32_t* z, float* y,
                        int32_t* acc, hipStream_t s) {
  Gemv5Args a;
  a.packed = packed, a.s_row = s_row, a.rowsum = rowsum, a.q = q, a.s_act = s_act, a.z = z;
  a.y = y, a.acc = acc;
  a.N = (int32_t)N, a.K = (int32_t)K;
  a.nch = (int32_t)((K + 79) / 80);
  a.ld = 16 * a.nch;
  return packed5_lanes_per_row(K) == 8 ? launch_gemv5_t<8, 2>(a, s) : launch_gemv5_t<16, 4>(a, s);
}

}  // namespace tern
