// tern_pack.hip -- load-time packing of ternary int8 matrices into the 2-bit
// layout, plus unpack and validate kernels (test aids).
//
// The weights are packed once and then stay packed at rest; the runtime reads
// them without a decode pass at load (Fermion Research models page,
// "Neutrino-1 0.6B"; Neutrino-1 8B model card, "Overview").  Per-row
// metadata carries the row sum (model card, "Where the bytes live"), which
// the packing computes on the way.
//
// Layout: code = w + 1; row stride 16 * ceil(K / 64) bytes; weight j in the
// little-endian word j / 16 at bit 8 * (j % 4) + 2 * ((j % 16) / 4);
// padding code 01.  One wave handles one row, one lane one 16-weight word.
#include "tern_device.h"

namespace tern {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

__device__ __forceinline__ int field_shift(int t) { return 8 * (t & 3) + 2 * (t >> 2); }

__global__ __launch_bounds__(kBlock) void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(kBlock) void pack_kernel(const int8_t* __restrict__ w, int64_t N,
                                                      int K, int64_t ldw, int words,
                                                      uint8_t* __restrict__ packed,
                                                      int32_t* __restrict__ rowsum,
                                                      int32_t* __restrict__ bad) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= N) return;
  const int8_t* wr = w + row * ldw;
  uint32_t* out = reinterpret_cast<uint32_t*>(packed + row * (int64_t)words * 4);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(wr) & 15) == 0;
  int32_t sum = 0, nbad = 0;
  for (int wi = lane; wi < words; wi += 64) {
    const int j0 = 16 * wi;
    int8_t v[16];
    if (vec_ok && j0 + 16 <= K) {
      const u32x4 t = load16(wr + j0);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (int8_t)(t[i >> 2] >> (8 * (i & 3)));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (j0 + i < K) ? wr[j0 + i] : (int8_t)0;
    }
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      uint32_t code = 1u;  // weight 0, also for padding and out-of-set values
      if (j0 + t < K) {
        const int x = v[t];
        if (x >= -1 && x <= 1) {
          code = (uint32_t)(x + 1);
          sum += x;
        } else {
          ++nbad;
        }
      }
      word |= code << field_shift(t);
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

__global__ __launch_bounds__(kBlock) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                        int64_t N, int K, int words,
                                                        int8_t* __restrict__ w, int64_t ldw) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= N) return;
  const uint32_t* in = reinterpret_cast<const uint32_t*>(packed + row * (int64_t)words * 4);
  int8_t* wr = w + row * ldw;
  for (int wi = lane; wi < words; wi += 64) {
    const uint32_t word = in[wi];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int j = 16 * wi + t;
      if (j < K) {
        const uint32_t c = (word >> field_shift(t)) & 3u;
        wr[j] = (c == 3u) ? (int8_t)0 : (int8_t)((int)c - 1);
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void validate_kernel(const uint8_t* __restrict__ packed,
                                                          int64_t N, int K, int words,
                                                          int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= N) return;
  const uint32_t* in = reinterpret_cast<const uint32_t*>(packed + row * (int64_t)words * 4);
  int32_t invalid = 0, padding = 0;
  for (int wi = lane; wi < words; wi += 64) {
    const uint32_t word = in[wi];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t c = (word >> field_shift(t)) & 3u;
      if (16 * wi + t < K)
        invalid += (c == 3u);
      else
        padding += (c != 1u);
    }
  }
  invalid = (int32_t)group_sum<64>((uint32_t)invalid);
  padding = (int32_t)group_sum<64>((uint32_t)padding);
  if (lane == 0) {
    if (invalid) atomicAdd(&counts[0], invalid);
    if (padding) atomicAdd(&counts[1], padding);
  }
}

dim3 rows_grid(int64_t N) { return dim3((unsigned)((N + kWaves - 1) / kWaves)); }

}  // namespace

int64_t pack_work_items(int64_t N) { return (N + kWaves - 1) / kWaves * kBlock; }

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                       int32_t* rowsum, int32_t* bad, hipStream_t s) {
  const int words = (int)(4 * ((K + 63) / 64));
  hipLaunchKernelGGL(pack_kernel, rows_grid(N), dim3(kBlock), 0, s, w, N, (int)K, ldw, words,
                     packed, rowsum, bad);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, int64_t ldw,
                         hipStream_t s) {
  const int words = (int)(4 * ((K + 63) / 64));
  hipLaunchKernelGGL(unpack_kernel, rows_grid(N), dim3(kBlock), 0, s, packed, N, (int)K, words,
                     w, ldw);
  return hipGetLastError();
}

hipError_t launch_validate(const uint8_t* packed, int64_t N, int64_t K, int32_t* counts,
                           hipStream_t s) {
  const int words = (int)(4 * ((K + 63) / 64));
  hipLaunchKernelGGL(validate_kernel, rows_grid(N), dim3(kBlock), 0, s, packed, N, (int)K, words,
                     counts);
  return hipGetLastError();
}

}  // namespace tern
