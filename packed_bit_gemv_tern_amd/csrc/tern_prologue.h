// tern_prologue.h -- per-token activation quantisation shared by the
// quantiser kernel and the stack launch, and the stack launch's prologue:
// the fp32 inputs a stack names are quantised inside the launch, each
// distinct input once, and published to the waves that read them.
#pragma once

#include "tern_device.h"

namespace tern {

// Scale and zero point of a token whose range widened to contain zero is
// [lo, hi]: s = (hi - lo) / 255 (1 for an all-zero token), z = -128 -
// rint(lo / s); a value's code is clamp(rint(x / s) + z, -128, 127).  Every
// division is one correctly rounded fp32 division and rint rounds half to
// even, so the codes are a function of the fp32 inputs alone.
__device__ __forceinline__ void act_params(float lo, float hi, float& s, int32_t& zm) {
  s = __fdiv_rn(hi - lo, 255.0f);
  if (s == 0.0f) s = 1.0f;
  zm = -128 - (int32_t)__builtin_rintf(__fdiv_rn(lo, s));
}
__device__ __forceinline__ int32_t act_code(float x, float s, int32_t zm) {
  const int32_t v = (int32_t)__builtin_rintf(__fdiv_rn(x, s)) + zm;
  return min(127, max(-128, v));
}

__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fminf(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

// The SwiGLU gate of the model card's feed-forward layers, silu(g) * u,
// in fixed fp32 steps (round to nearest even, no fused multiply-add: the
// build keeps every product and sum as written) so that the result is a
// function of g and u alone:
//   t = clamp(-g, -87, 100); e = e^t by Cody and Waite's reduction
//   t = k ln2 + r (k = rint(t / ln 2), ln 2 split in a 15-bit head, whose
//   product with k is exact, and an fp32 tail) and the Taylor series of e^r
//   through r^7 by Horner's rule, scaled by 2^k (+inf past 88.7);
//   silu = g / (1 + e), correctly rounded; h = silu * u.
__device__ __forceinline__ float swiglu32(float g, float u) {
  constexpr double kLn2 = 0.69314718055994530942;
  constexpr float kInvLn2 = (float)(1.0 / kLn2);
  constexpr float kHead = 0.693145751953125f;
  constexpr float kTail = (float)(kLn2 - 0.693145751953125);
  const float t = fminf(fmaxf(-g, -87.0f), 100.0f);
  const float k = __builtin_rintf(__fmul_rn(t, kInvLn2));
  const float r = __fsub_rn(__fsub_rn(t, __fmul_rn(k, kHead)), __fmul_rn(k, kTail));
  float p = (float)(1.0 / 5040.0);
  p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 720.0));
  p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 120.0));
  p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 24.0));
  p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 6.0));
  p = __fadd_rn(__fmul_rn(p, r), 0.5f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  const float e = __builtin_ldexpf(p, (int)k);
  return __fmul_rn(__fdiv_rn(g, __fadd_rn(1.0f, e)), u);
}

// LDS a stack kernel lends the prologue: the claim just made (two slots,
// alternating) and the waves' partial minima and maxima.
struct PrologueLds {
  unsigned long long claim[2];
  float red[2][16];
};

// One token row of K floats quantised by the whole workgroup: a min/max
// pass, then the codes (thread t takes columns 4t + 4Ti .. +3, T threads,
// stored as one dword where the four lie inside K; q is 4-byte aligned).
// With x_up the row's values are swiglu32(x_j, x_up_j), formed in each pass.
__device__ __forceinline__ void quantize_row_wg(const float* x, const float* x_up, int K, int8_t* q,
                                                float* s_out, int32_t* z_out, PrologueLds& pl) {
  const int t = threadIdx.x, nt = blockDim.x, waves = blockDim.x >> 6;
  auto val = [&](int j) { return x_up ? swiglu32(load_g(x + j), load_g(x_up + j)) : load_g(x + j); };
  float lo = 0.0f, hi = 0.0f;
  for (int j0 = 4 * t; j0 < K; j0 += 4 * nt) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (j0 + u < K) {
        const float v = val(j0 + u);
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
    }
  }
  lo = wave_min_f(lo);
  hi = wave_max_f(hi);
  if ((t & 63) == 0) pl.red[0][t >> 6] = lo, pl.red[1][t >> 6] = hi;
  __syncthreads();
  for (int i = 0; i < waves; ++i) lo = fminf(lo, pl.red[0][i]), hi = fmaxf(hi, pl.red[1][i]);
  float s;
  int32_t zm;
  act_params(lo, hi, s, zm);
  for (int j0 = 4 * t; j0 < K; j0 += 4 * nt) {
    if (j0 + 3 < K) {
      uint32_t word = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) word |= ((uint32_t)act_code(val(j0 + u), s, zm) & 0xffu) << (8 * u);
      store_g(reinterpret_cast<uint32_t*>(q + j0), word);
    } else {
      for (int u = 0; j0 + u < K; ++u) store_g(q + j0 + u, (int8_t)act_code(val(j0 + u), s, zm));
    }
  }
  if (t == 0) {
    store_g(s_out, s);
    store_g(z_out, zm);
  }
}

// The prologue of a stack launch with quantisation jobs.  The claiming
// workgroups (a bit each in the plan: the first few of the grid and every
// one whose schedule reads a quantised input) take token rows (job, token)
// from the plan's counter one at a time, quantise them and set each row's
// flag to the launch's number; a workgroup leaves once a claim comes back
// past the last row.  Each claiming workgroup makes exactly one such claim,
// so one launch advances the counter by period = nitems + claimers, and
// counter / period numbers the launches from 0 (prepare clears the counter
// and the flags).  Every row is claimed by a running workgroup, which
// finishes it without waiting on anything, and a workgroup waits for rows
// only after its own claims have run out, so every wait ends whatever the
// order the workgroups run in.  Returns the flag value of this launch (0:
// no jobs, or a workgroup that reads no quantised input and does not claim).
__device__ __forceinline__ uint32_t stack_prologue(const StackHeader* h, StackSync* sy, PrologueLds& pl) {
  const int nitems = h->nitems;
  if (nitems == 0) return 0;
  const char* base = reinterpret_cast<const char*>(h);
  const uint32_t* part = reinterpret_cast<const uint32_t*>(base + h->off_part);
  if (((part[blockIdx.x >> 5] >> (blockIdx.x & 31)) & 1u) == 0) return 0;
  const QuantJob* jobs = reinterpret_cast<const QuantJob*>(base + h->off_job);
  uint32_t* flags = reinterpret_cast<uint32_t*>(sy + 1);
  const int M = h->M;
  const unsigned long long period = (unsigned long long)nitems + (unsigned long long)h->claimers;
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0)
      pl.claim[it & 1] = __hip_atomic_fetch_add(&sy->claim, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // (uniform: kept in scalar registers)
    const unsigned long long c0 = pl.claim[it & 1];
    const unsigned long long c =
        ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((int)(c0 >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)c0);
    const uint32_t launch1 = (uint32_t)(c / period) + 1u;
    const long long item = (long long)(c % period);
    if (item >= nitems) return launch1;
    const int job = (int)(item / M), m = (int)(item % M);
    const QuantJob jb = jobs[job];
    quantize_row_wg(jb.x + (int64_t)m * jb.ldx, jb.x_up ? jb.x_up + (int64_t)m * jb.ldx : nullptr, jb.K,
                    jb.q + (int64_t)m * jb.ldq, jb.s_act + m, jb.z + m, pl);
    // every wave's codes are visible device-wide before the row's flag
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flags + item, launch1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Polls a wave makes for one flag before it gives up (a poll is a load and
// a sleep of about 0.2 us; the bound is of the order of a second): the rows
// always finish, so it only turns a broken invariant into an error in place
// of a hang.
constexpr int kQuantSpinLimit = 1 << 20;

// Before a wave's first read of job `job`'s output: wait until every token
// row of the job carries this launch's flag, then acquire (the rows'
// writes are visible to the wave's loads that follow).
__device__ __forceinline__ void wait_quantized(const StackHeader* h, StackSync* sy, int job, uint32_t launch1) {
  const int M = h->M;
  const uint32_t* f = reinterpret_cast<const uint32_t*>(sy + 1) + (int64_t)job * M;
  const int lane = threadIdx.x & 63;
  bool gave_up = false;
  for (int m0 = 0; m0 < M && !gave_up; m0 += 64) {
    const int m = m0 + lane;
    for (int it = 0;; ++it) {
      const bool ok = m >= M || __hip_atomic_load(f + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == launch1;
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      if (it >= kQuantSpinLimit) {
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  if (gave_up && lane == 0) __hip_atomic_fetch_or(&sy->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Before a worker's first segment: wait for every quantised input its
// segments [s0, s1) read (done up front, where the kernels hold nothing in
// registers yet; the rows all finish within the launch's first
// microseconds).  launch1 = 0: the launch has no jobs.
__device__ __forceinline__ void wait_segment_inputs(const StackHeader* h, StackSync* sy, const LinearArgs* lin,
                                                    const Segment* seg, int s0, int s1, uint32_t launch1) {
  if (launch1 == 0) return;
  int waited = -1;
  for (int s = s0; s < s1; ++s) {
    const int qj = lin[seg[s].lin].qjob;
    if (qj >= 0 && qj != waited) wait_quantized(h, sy, waited = qj, launch1);
  }
}

}  // namespace tern
