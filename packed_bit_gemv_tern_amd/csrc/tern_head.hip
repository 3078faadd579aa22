// tern_head.hip -- the int8 output head: logits of up to eight tokens.
//
// The output head (and the token embedding) stay int8 with one scale per
// row, because no long sum hides their rounding (Neutrino-1 8B model card,
// "Where the bytes live"; article "Neutrino-1: quantization is a training
// decision, not a deployment one", "What's actually ternary").  Against the
// same per-token activations as the ternary linears (int8 q, fp32 s_act,
// int32 zero point z):
//
//     acc[m][i] = sum_j W_ij q[m][j] - z[m] * rowsum_i       (int32, exact)
//     y[m][i]   = (s_row[i] * (float)acc[m][i]) * s_act[m]   (RNE, this order)
//
// with rowsum_i = sum_j W_ij computed once at load time (tern_head_rowsum).
// At 151,936 x 4,096 the head is 622 MB read once per pass: bound by HBM.
//
// A workgroup owns a contiguous range of rows.  It stages its tokens'
// activations (zero past K and past M) and its rows' scales and row sums in
// LDS, so nothing but the weight stream touches HBM in the loop.  Each wave
// takes units of U rows; a lane holds 16-byte chunks lane, lane + 64, ... of
// each row and forms v_dot4_i32_i8 products with the staged activations.
// The next step's U chunks are loaded before the current step is computed
// (two register buffers), through range-checked buffer loads: rows past the
// range and chunks past K read as zero.  At a unit's last step the U x MT
// sums are reduced over the wave with the transposed butterfly.
#include "tern_device.h"

namespace tern {

namespace {

constexpr int kHeadBlock = 256;
constexpr int kHeadWaves = kHeadBlock / 64;

// rows per unit for MT tokens: U * MT values go through one 64-lane reduction.
// Eight rows (eight 16-byte weight loads per lane and step) at every MT:
// with four at M > 1 the full 151,936 x 4,096 head took 105.8 us at M = 8
// against 102.1 with eight (M = 2 and 4 the same either way), the launches
// sized as below.
template <int MT>
struct HeadU {
  static constexpr int U = 8;
};

struct HeadArgs {
  const int8_t* W;
  const float* s_row;
  const int32_t* rowsum;
  const int8_t* q;
  const float* s_act;
  const int32_t* z;
  float* y;
  int32_t* acc;
  int64_t ldw;
  int32_t N, K, ldq, ldy, M;
  int32_t kpad;  // K rounded up to 16
  int32_t rows;  // rows per workgroup (a multiple of U * kHeadWaves)
};

__device__ __forceinline__ int32_t sdot4(uint32_t a, uint32_t b, int32_t c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

template <int MT>
__global__ __launch_bounds__(kHeadBlock) void head_kernel(HeadArgs a) {
  constexpr int U = HeadU<MT>::U;
  constexpr int NV = U * MT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* qs = smem;                                                    // MT x kpad
  float* srs = reinterpret_cast<float*>(smem + MT * a.kpad);             // rows
  int32_t* rss = reinterpret_cast<int32_t*>(smem + MT * a.kpad + 4 * a.rows);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int r0 = (int)blockIdx.x * a.rows;
  const int nrows = min(a.rows, a.N - r0);
  const int nck = a.kpad / 16;

  // stage activations (zero past K and for tokens past M) and metadata
  for (int e = threadIdx.x; e < MT * nck; e += kHeadBlock) {
    const int m = e / nck, c = e % nck;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (m < a.M) {
      const int8_t* src = a.q + (int64_t)m * a.ldq + 16 * c;
      if (16 * c + 16 <= a.K) {
        v = load16(src);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * c + i < a.K) v[i / 4] |= (uint32_t)(uint8_t)load_g(src + i) << (8 * (i % 4));
      }
    }
    *reinterpret_cast<u32x4*>(qs + m * a.kpad + 16 * c) = v;
  }
  for (int r = threadIdx.x; r < nrows; r += kHeadBlock) {
    srs[r] = load_g(a.s_row + r0 + r);
    rss[r] = load_g(a.rowsum + r0 + r);
  }
  float sa[MT];
  int32_t zt[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    sa[m] = m < a.M ? load_g(a.s_act + m) : 0.0f;
    zt[m] = m < a.M ? load_g(a.z + m) : 0;
  }
  __syncthreads();

  const int cpl = (nck + 63) / 64;  // chunks per lane per row
  const int nunits = (nrows + U - 1) / U;
  int unit = wave;
  if (unit >= nunits) return;

  // step (unit, t): chunk lane + 64 t of the unit's U rows
  auto issue = [&](int un, int t, bool live, u32x4 (&w)[U]) {
    const int rr = r0 + un * U;
    const uint32_t n = live ? (uint32_t)min(U, a.N - rr) : 0u;
    const auto rw = buffer_rsrc(const_cast<int8_t*>(a.W) + (int64_t)rr * a.ldw, n * (uint32_t)a.ldw);
    const int c = lane + 64 * t;
    const bool in_row = c < nck;  // past the row: read nothing (zero)
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = buffer_load_weights16(rw, in_row ? (uint32_t)u * (uint32_t)a.ldw + 16u * (uint32_t)c : kDropOffset);
  };
  int32_t acc[U][MT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[u][m] = 0;
  auto compute = [&](int t, const u32x4 (&w)[U]) {
    const int c = min(lane + 64 * t, nck - 1);  // its weights are zero when clamped
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(qs + m * a.kpad + 16 * c);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[u][m] = sdot4(w[u][d], qv[d], acc[u][m]);
    }
  };
  auto finish = [&](int un) {
    uint32_t v[NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        v[u * MT + m] = (uint32_t)acc[u][m];
        acc[u][m] = 0;
      }
    const uint32_t tot = reduce_split<64, NV>(v, lane);
    const int vidx = split_index<64, NV>(lane);
    const int mu = vidx / MT, mm = vidx % MT;
    const int lr = un * U + mu;  // row within the workgroup's range
    if ((lane % (64 / NV)) == 0 && mm < a.M && lr < nrows) {
      float s = 0.0f;
      int32_t zz = 0;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m == mm) s = sa[m], zz = zt[m];
      const int32_t av = (int32_t)(tot - (uint32_t)zz * (uint32_t)rss[lr]);
      const int64_t o = (int64_t)mm * a.ldy + r0 + lr;
      store_g(a.y + o, __fmul_rn(__fmul_rn(srs[lr], (float)av), s));
      if (a.acc) store_g(a.acc + o, av);
    }
  };
  // advance (unit, t) to the next step of this wave; false past the end
  auto next = [&](int& un, int& t) {
    if (++t == cpl) {
      t = 0;
      un += kHeadWaves;
    }
    return un < nunits;
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
    if (t == cpl - 1) finish(unit);
    if (!more) break;
    unit = nu, t = nt;
    nu = unit, nt = t;
    more = next(nu, nt);
    issue(more ? nu : unit, nt, more, wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(t, wb);
    if (t == cpl - 1) finish(unit);
    if (!more) break;
    unit = nu, t = nt;
  }
}

// ---- load-time row sums ----
__global__ __launch_bounds__(kHeadBlock) void head_rowsum_kernel(const int8_t* W, int64_t N, int64_t K,
                                                                 int64_t ldw, int32_t* rowsum) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kHeadWaves + (threadIdx.x >> 6);
  if (row >= N) return;
  const int8_t* r = W + row * ldw;
  int32_t s = 0;
  for (int64_t j = lane; j < K; j += 64) s += r[j];
  s = (int32_t)reduce_split<64, 1>(*reinterpret_cast<uint32_t(*)[1]>(&s), lane);
  if (lane == 0) rowsum[row] = s;
}

}  // namespace

int head_tokens(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

int64_t head_lds_bytes(int64_t M, int64_t K, int64_t rows) {
  return (int64_t)head_tokens(M) * (16 * ((K + 15) / 16)) + 8 * rows;
}

// Workgroups per CU the host sizes a launch for (each takes N / (that * CUs)
// rows).  Every workgroup stages its tokens' activations in LDS first, and
// fewer, longer workgroups ran faster: the full head at M = 1 / 8 took
// 96.6 / 105.8 us with four per CU (and four rows per unit at M = 8),
// 92.5 / 102.1 with two; one per CU was slower again (97.8 / 123.5).
int head_wg_per_cu() { return 2; }

int head_rows_per_unit(int64_t M) {
  switch (head_tokens(M)) {
    case 1: return HeadU<1>::U * kHeadWaves;
    case 2: return HeadU<2>::U * kHeadWaves;
    case 4: return HeadU<4>::U * kHeadWaves;
    default: return HeadU<8>::U * kHeadWaves;
  }
}

hipError_t launch_head(const int8_t* W, const float* s_row, const int32_t* rowsum, int64_t N, int64_t K,
                       int64_t ldw, int64_t M, const int8_t* q, int64_t ldq, const float* s_act,
                       const int32_t* z, float* y, int64_t ldy, int32_t* acc, int64_t rows_per_wg,
                       hipStream_t s) {
  HeadArgs a;
  a.W = W, a.s_row = s_row, a.rowsum = rowsum, a.q = q, a.s_act = s_act, a.z = z, a.y = y, a.acc = acc;
  a.ldw = ldw;
  a.N = (int32_t)N, a.K = (int32_t)K, a.ldq = (int32_t)ldq, a.ldy = (int32_t)ldy, a.M = (int32_t)M;
  a.kpad = (int32_t)(16 * ((K + 15) / 16));
  a.rows = (int32_t)rows_per_wg;
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), block(kHeadBlock);
  const size_t lds = (size_t)head_lds_bytes(M, K, rows_per_wg);
  switch (head_tokens(M)) {
    case 1: hipLaunchKernelGGL(head_kernel<1>, grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL(head_kernel<2>, grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL(head_kernel<4>, grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL(head_kernel<8>, grid, block, lds, s, a); break;
  }
  return hipGetLastError();
}

int64_t head_rowsum_work_items(int64_t N) { return (N + kHeadWaves - 1) / kHeadWaves * kHeadBlock; }

hipError_t launch_head_rowsum(const int8_t* W, int64_t N, int64_t K, int64_t ldw, int32_t* rowsum,
                              hipStream_t s) {
  const dim3 grid((unsigned)((N + kHeadWaves - 1) / kHeadWaves)), block(kHeadBlock);
  hipLaunchKernelGGL(head_rowsum_kernel, grid, block, 0, s, W, N, K, ldw, rowsum);
  return hipGetLastError();
}

}  // namespace tern
