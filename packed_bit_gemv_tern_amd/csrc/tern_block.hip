// tern_block.hip -- one token against a ternary matrix with block-wise scales.
//
// The article "Neutrino-1: quantization is a training decision, not a
// deployment one" ("What's actually ternary") groups each row's weights into
// fixed-size blocks along the input dimension, every block with its own
// higher-precision scale; one scale per row is the coarsest case.  With
// block size B (block b of a row = columns [b*B, (b+1)*B) below K):
//
//     acc_b = sum_{j in b} w_ij q_j - z * rowsum_b[i][b]          (int32, exact)
//     y_i   = (sum_b s_b[i][b] * acc_b) * s_act                    (fp32)
//
// The packed weights are the 2-bit layout of the per-row path.  A wave reads
// one row per load, lane r holding chunks r, r + 64, ... (64 weights each),
// so a block of B = 64 g columns is a group of g lanes.  As in the per-row
// VALU path the lane forms S = sum c qb over its chunk (codes c = w + 1,
// biased activations qb = q + 128, zero past K); the group sums S with DPP,
// subtracts the block's activation sum and (z + 128) * rowsum_b (exact), and
// converts.  The group's first lane puts s_b * acc_b (one rounding) into the
// wave's LDS row, and lane u then adds row u's products in block order from
// +0 (one rounding each) -- the order of the definition, so y has the bits
// of its left-to-right evaluation.
//
// Two units of U rows are in flight per wave (next unit's weights, block
// scales and block row sums loaded before the current unit is reduced), all
// through range-checked buffer loads, as in the per-row M = 1 kernel.
#include "tern_device.h"

#include <type_traits>

namespace tern {

namespace {

constexpr int kBlkBlock = 256;
constexpr int kBlkWaves = kBlkBlock / 64;
constexpr uint32_t kPlane0 = 0x03030303u, kPlane1 = 0x0C0C0C0Cu, kPlane2 = 0x30303030u,
                   kPlane3 = 0xC0C0C0C0u;
constexpr uint32_t kBias = 0x80808080u, kOnes = 0x01010101u;

__device__ __forceinline__ uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_udot4(a, b, c, false);
}

// Value of lane l ^ D.  The transposed steps below need exactly that lane:
// the partner must agree with l in every other bit, so the half-mirror
// exchange dpp_partner<4> (lane 7 - (l & 7)) is composed with a quad
// reversal (l ^ 3) to give l ^ 4.
template <int D>
__device__ __forceinline__ uint32_t partner(uint32_t v) {
  if constexpr (D == 32) {
    auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return p[0] ^ p[1] ^ v;  // the swapped copy: one of p[0], p[1] is v itself
  } else if constexpr (D == 16) {
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return p[0] ^ p[1] ^ v;
  } else if constexpr (D == 4) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x1B, 0xF, 0xF, false);
  } else {
    return dpp_partner<D>(v);  // l ^ 8 (row_ror:8), l ^ 2, l ^ 1 (quad_perm)
  }
}

// sum over aligned groups of g lanes (g a power of two, uniform)
__device__ __forceinline__ uint32_t group_sum_int(uint32_t v, int g) {
  if (g > 1) v += partner<1>(v);
  if (g > 2) v += partner<2>(v);
  if (g > 4) v += partner<4>(v);
  if (g > 8) v += partner<8>(v);
  if (g > 16) v += partner<16>(v);
  if (g > 32) v += partner<32>(v);
  return v;
}

struct BlkArgs {
  const uint8_t* packed;
  const float* s_b;
  const int32_t* rowsum_b;
  const int8_t* q;
  const float* s_act;
  const int32_t* z;
  float* y;
  int32_t N, K, ld, nch, nb, g;
};

template <int CPL>
struct BlkU {
  static constexpr int U = CPL == 1 ? 4 : CPL == 2 ? 2 : 1;
};

// LDS floats per wave for the row products: U rows of up to K / 64 blocks
// (K <= 64 * 64 * CPL), a pitch of a multiple of 4 plus 4
constexpr int kBlkProdWave = 288;

template <int CPL, int LG>
__global__ __launch_bounds__(kBlkBlock) void blocked_gemv_kernel(BlkArgs a) {
  constexpr int U = BlkU<CPL>::U;
  constexpr int g = 1 << LG;
  static_assert(U * (64 * CPL + 8) <= kBlkProdWave, "products per wave");
  __shared__ __attribute__((aligned(16))) float prods[kBlkWaves][kBlkProdWave];
  float* prow = prods[threadIdx.x >> 6];
  const int pitch = (a.nb + 3) / 4 * 4 + 4;
  const int lane = threadIdx.x & 63;
  const int gw = (int)blockIdx.x * kBlkWaves + (int)(threadIdx.x >> 6);
  const int nw = (int)gridDim.x * kBlkWaves;

  // biased activations of the lane's chunks (zero past K) and each chunk's
  // block activation sum
  uint32_t qc[CPL][16];
  uint32_t qbb[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int ch = lane + 64 * t;
    uint32_t qs = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t v = 0;
      if (ch < a.nch) {
        const int j0 = 64 * ch + 4 * i;
        if (j0 + 4 <= a.K) {
          v = (uint32_t)load_g(reinterpret_cast<const int32_t*>(a.q + j0)) ^ kBias;
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (j0 + b < a.K) v |= (uint32_t)((uint8_t)load_g(a.q + j0 + b) ^ 0x80u) << (8 * b);
        }
      }
      qc[t][i] = v;
      qs = udot4(v, kOnes, qs);
    }
    qbb[t] = group_sum_int(qs, g);
  }
  const float sa = load_g(a.s_act);
  const uint32_t zb = (uint32_t)(load_g(a.z) + 128);

  uint32_t woff[U][CPL], moff[U][CPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int ch = lane + 64 * t;
      woff[u][t] = ch < a.nch ? (uint32_t)u * (uint32_t)a.ld + 16u * (uint32_t)ch : kDropOffset;
      moff[u][t] = ch < a.nch ? 4u * ((uint32_t)u * (uint32_t)a.nb + (uint32_t)(ch / g)) : kDropOffset;
    }
  struct Unit {
    u32x4 w[U][CPL];
    float s[U][CPL];
    int32_t r[U][CPL];
  };
  auto issue = [&](int base, bool live, Unit& b) {
    const uint32_t n = live ? (uint32_t)min(U, a.N - base) : 0u;
    const auto rw = buffer_rsrc(const_cast<uint8_t*>(a.packed) + (int64_t)base * a.ld, n * (uint32_t)a.ld);
    const auto rs = buffer_rsrc(const_cast<float*>(a.s_b) + (int64_t)base * a.nb, 4u * n * (uint32_t)a.nb);
    const auto rr = buffer_rsrc(const_cast<int32_t*>(a.rowsum_b) + (int64_t)base * a.nb, 4u * n * (uint32_t)a.nb);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        b.w[u][t] = buffer_load_weights16(rw, woff[u][t]);
        b.s[u][t] = __uint_as_float(buffer_load_u32(rs, moff[u][t]));
        b.r[u][t] = (int32_t)buffer_load_u32(rr, moff[u][t]);
      }
  };
  auto finish = [&](const Unit& c, int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        uint32_t p[4] = {0, 0, 0, 0};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t x = c.w[u][t][d];
          p[0] = udot4(x & kPlane0, qc[t][4 * d + 0], p[0]);
          p[1] = udot4(x & kPlane1, qc[t][4 * d + 1], p[1]);
          p[2] = udot4(x & kPlane2, qc[t][4 * d + 2], p[2]);
          p[3] = udot4(x & kPlane3, qc[t][4 * d + 3], p[3]);
        }
        // sum c * qb of the chunk (plane k is 4^k-scaled), then of the block
        const uint32_t sc = p[0] + (p[1] >> 2) + (p[2] >> 4) + (p[3] >> 6);
        const uint32_t sb = group_sum_int(sc, g);
        const int32_t accb = (int32_t)(sb - qbb[t] - mul_zr((int32_t)zb, c.r[u][t]));
        const int ch = lane + 64 * t;
        if ((lane & (g - 1)) == 0 && ch < a.nch) prow[u * pitch + ch / g] = __fmul_rn(c.s[u][t], (float)accb);
      }
    }
    wait_lds();  // the wave's products are in LDS (its own accesses complete in order)
    float tot = 0.0f;
    if (lane < U) {
      const float* pr = prow + lane * pitch;
      for (int b = 0; b < a.nb; ++b) tot = __fadd_rn(tot, pr[b]);
    }
    const uint32_t rows = (uint32_t)min(U, a.N - base) * 4u;
    buffer_store_u32(__float_as_uint(__fmul_rn(tot, sa)), buffer_rsrc(a.y + base, rows),
                     lane < U ? 4u * (uint32_t)lane : kDropOffset);
    wait_lds();  // every row is read before the next unit's products go in
  };

  const int step = nw * U;
  if ((int64_t)gw * U >= a.N) return;
  int base = gw * U;
  Unit ua, ub;
  issue(base, true, ua);
#pragma unroll 1
  for (;;) {
    bool more = (int64_t)base + step < a.N;
    issue(more ? base + step : base, more, ub);
    __builtin_amdgcn_sched_barrier(0);
    finish(ua, base);
    if (!more) break;
    base += step;
    more = (int64_t)base + step < a.N;
    issue(more ? base + step : base, more, ua);
    __builtin_amdgcn_sched_barrier(0);
    finish(ub, base);
    if (!more) break;
    base += step;
  }
}

// Load-time block row sums from the packed weights: one thread per (row,
// block), summing code - 1 over the block's columns below K.
__global__ __launch_bounds__(kBlkBlock) void block_rowsum_kernel(const uint8_t* packed, int64_t N,
                                                                 int64_t K, int64_t B, int64_t ld,
                                                                 int64_t nb, int32_t* rowsum_b) {
  const int64_t e = (int64_t)blockIdx.x * kBlkBlock + threadIdx.x;
  if (e >= N * nb) return;
  const int64_t i = e / nb, b = e % nb;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(packed + i * ld);
  int32_t s = 0;
  for (int64_t j0 = b * B; j0 < K && j0 < (b + 1) * B; j0 += 16) {
    const uint32_t x = load_g(row + j0 / 16);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int byte = 0; byte < 4; ++byte) {
        const int64_t j = j0 + 4 * k + byte;  // weight 4k + byte of the word
        if (j < K) s += (int32_t)((x >> (8 * byte + 2 * k)) & 3u) - 1;
      }
  }
  rowsum_b[e] = s;
}

}  // namespace

hipError_t launch_blocked_gemv(const uint8_t* packed, const float* s_b, const int32_t* rowsum_b, int64_t N,
                               int64_t K, int64_t B, const int8_t* q, const float* s_act, const int32_t* z,
                               float* y, int grid_blocks, hipStream_t s) {
  BlkArgs a;
  a.packed = packed, a.s_b = s_b, a.rowsum_b = rowsum_b, a.q = q, a.s_act = s_act, a.z = z, a.y = y;
  a.N = (int32_t)N, a.K = (int32_t)K;
  a.ld = (int32_t)(16 * ((K + 63) / 64));
  a.nch = a.ld / 16;
  a.nb = (int32_t)((K + B - 1) / B);
  a.g = (int32_t)(B / 64);
  const int cpl = (a.nch + 63) / 64;
  int lg = 0;
  while ((1 << lg) < a.g) ++lg;
  const dim3 grid((unsigned)grid_blocks), block(kBlkBlock);
  auto go = [&](auto cpl_c) {
    constexpr int C = decltype(cpl_c)::value;
    switch (lg) {
      case 0: hipLaunchKernelGGL((blocked_gemv_kernel<C, 0>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((blocked_gemv_kernel<C, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((blocked_gemv_kernel<C, 2>), grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL((blocked_gemv_kernel<C, 3>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((blocked_gemv_kernel<C, 4>), grid, block, 0, s, a); break;
      case 5: hipLaunchKernelGGL((blocked_gemv_kernel<C, 5>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((blocked_gemv_kernel<C, 6>), grid, block, 0, s, a); break;
    }
  };
  switch (cpl) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    default: go(std::integral_constant<int, 4>{}); break;
  }
  return hipGetLastError();
}

int blocked_rows_per_wave(int64_t K) {
  const int64_t cpl = (16 * ((K + 63) / 64) / 16 + 63) / 64;
  return cpl == 1 ? BlkU<1>::U : cpl == 2 ? BlkU<2>::U : 1;
}

int64_t block_rowsum_work_items(int64_t N, int64_t K, int64_t B) {
  return (N * ((K + B - 1) / B) + kBlkBlock - 1) / kBlkBlock * kBlkBlock;
}

hipError_t launch_block_rowsum(const uint8_t* packed, int64_t N, int64_t K, int64_t B, int32_t* rowsum_b,
                               hipStream_t s) {
  const int64_t nb = (K + B - 1) / B;
  const int64_t total = N * nb;
  const dim3 grid((unsigned)((total + kBlkBlock - 1) / kBlkBlock)), block(kBlkBlock);
  hipLaunchKernelGGL(block_rowsum_kernel, grid, block, 0, s, packed, N, K, B, 16 * ((K + 63) / 64), nb,
                     rowsum_b);
  return hipGetLastError();
}

}  // namespace tern
