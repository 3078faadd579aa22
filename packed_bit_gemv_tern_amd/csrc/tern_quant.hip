// tern_quant.hip -- per-token asymmetric int8 quantisation of activations.
//
// The ternary linears and the int8 head take each token's activations as
// int8 q with an fp32 scale s_act and an int32 zero point z (x ~= s_act *
// (q - z)).  The pages never describe how those are made, so this is the
// plainest reading: the token's range widened to contain zero, in 255 steps
// (zero stays exact and |z| <= 128):
//
//     lo = min(0, min_j x_j),  hi = max(0, max_j x_j)
//     s  = (hi - lo) / 255          (s = 1 when hi == lo: an all-zero token)
//     z  = -128 - rint(lo / s)
//     q_j = clamp(rint(x_j / s) + z, -128, 127)
//
// Every division is one correctly rounded fp32 division and rint rounds half
// to even, so the integer codes are a function of the fp32 inputs alone.
// One workgroup per token: a min/max pass over the row, then the codes.
#include "tern_prologue.h"

namespace tern {

namespace {

constexpr int kQuantBlock = 256;

__global__ __launch_bounds__(kQuantBlock) void quant_kernel(const float* x, int64_t K, int64_t ldx,
                                                            int8_t* q, int64_t ldq, float* s_act,
                                                            int32_t* z) {
  __shared__ float red[2][kQuantBlock / 64];
  const int64_t m = blockIdx.x;
  const float* r = x + m * ldx;
  float lo = 0.0f, hi = 0.0f;
  for (int64_t j = threadIdx.x; j < K; j += kQuantBlock) {
    const float v = load_g(r + j);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  lo = wave_min_f(lo);
  hi = wave_max_f(hi);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[0][w] = lo, red[1][w] = hi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kQuantBlock / 64; ++i) lo = fminf(lo, red[0][i]), hi = fmaxf(hi, red[1][i]);
  float s;
  int32_t zm;
  act_params(lo, hi, s, zm);
  int8_t* out = q + m * ldq;
  for (int64_t j = threadIdx.x; j < K; j += kQuantBlock) out[j] = (int8_t)act_code(load_g(r + j), s, zm);
  if (threadIdx.x == 0) {
    s_act[m] = s;
    z[m] = zm;
  }
}

// Weight quantiser (article, "What's actually ternary"): per block of B
// columns, scale = the mean absolute weight and state = the rounded, clamped
// ratio w / scale.  The mean is an fp64 sum in column order divided by the
// block's column count and rounded once to fp32, so it is a function of the
// inputs alone; a zero block has scale 0 and states 0.  One thread per
// (row, block); this runs once at load time, so it favours the fixed order
// over speed.
__global__ __launch_bounds__(kQuantBlock) void wquant_kernel(const float* W, int64_t N, int64_t K,
                                                             int64_t ldw, int64_t B, int64_t nb,
                                                             int8_t* t, int64_t ldt, float* s_b) {
  const int64_t idx = (int64_t)blockIdx.x * kQuantBlock + threadIdx.x;
  if (idx >= N * nb) return;
  const int64_t i = idx / nb, b = idx % nb;
  const float* row = W + i * ldw;
  const int64_t j0 = b * B, j1 = min(j0 + B, K);
  double total = 0.0;
  for (int64_t j = j0; j < j1; ++j) total += fabs((double)load_g(row + j));
  const float scale = (float)__ddiv_rn(total, (double)(j1 - j0));
  s_b[idx] = scale;
  int8_t* out = t + i * ldt;
  for (int64_t j = j0; j < j1; ++j) {
    float state = 0.0f;
    if (scale > 0.0f) {
      const float ratio = fminf(1.0f, fmaxf(-1.0f, __fdiv_rn(load_g(row + j), scale)));
      state = __builtin_rintf(ratio);
    }
    out[j] = (int8_t)state;
  }
}

}  // namespace

int64_t quantize_weights_work_items(int64_t N, int64_t K, int64_t B) {
  return (N * ((K + B - 1) / B) + kQuantBlock - 1) / kQuantBlock * kQuantBlock;
}

int64_t quantize_act_work_items(int64_t M) { return M * kQuantBlock; }

hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, int64_t ldw, int64_t B,
                                   int8_t* t, int64_t ldt, float* s_b, hipStream_t s) {
  const int64_t nb = (K + B - 1) / B;
  const int64_t blocks = (N * nb + kQuantBlock - 1) / kQuantBlock;
  hipLaunchKernelGGL(wquant_kernel, dim3((unsigned)blocks), dim3(kQuantBlock), 0, s, W, N, K, ldw, B,
                     nb, t, ldt, s_b);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               int64_t ldq, float* s_act, int32_t* z, hipStream_t s) {
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)M), dim3(kQuantBlock), 0, s, x, K, ldx, q, ldq,
                     s_act, z);
  return hipGetLastError();
}

}  // namespace tern
