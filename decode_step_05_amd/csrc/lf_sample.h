// Temperature sampling of the next token, one workgroup per row of logits.
//
// Stochastic decoding for pass@N (asector.ru summary, "Performance and
// infrastructure") draws several continuations of one prompt. The pages name
// no sampler; the one here draws from softmax(z / T) by inverting its
// cumulative distribution at a uniform u in [0, 1) that the caller supplies:
// token i covers u in [c_{i-1}, c_i), c_i = p_0 + ... + p_i, so the draw is the
// smallest i with c_i > u. Unnormalised: with w_i = exp((z_i - max z) / T) and
// S = sum w, the draw is the smallest i with w_0 + ... + w_i > u * S and
// w_i > 0; if fp32 rounding leaves none, the last i with w_i > 0.
//
// Layout: 1024 threads (16 waves); thread t owns the contiguous index range
// [t*C, t*C + C), C = ceil(n / 1024), so the partial sums in thread order are
// the cumulative sums in index order. A row that fits in LDS (up to 35,747
// logits) is first staged there with coalesced loads, one padding word per 32
// so that the threads' contiguous ranges fall in different banks, and each
// weight is computed once, in place. A longer row is read three times (max,
// sums, search) from global memory, the same arithmetic in the same order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;
constexpr int kSampleLdsFloats = 36 * 1024;  // 144 KB of the 160 KB per CU

// padded LDS slot of logit i: one spare word after every 32
__host__ __device__ constexpr int sample_slot(int i) { return i + (i >> 5); }
// whether a row of n >= 1 logits is staged in LDS
__host__ __device__ constexpr bool sample_fits_lds(int n) { return sample_slot(n - 1) < kSampleLdsFloats; }

__global__ __launch_bounds__(kSampleThreads) void k_sample(const float* __restrict__ logits, int n, float inv_t,
                                                           const float* __restrict__ u,
                                                           int32_t* __restrict__ tokens, int staged) {
  extern __shared__ float row_w[];  // staged rows: the logits, then their weights, at sample_slot(i)
  __shared__ float red[kSampleWaves];
  __shared__ float wave_off[kSampleWaves];
  __shared__ int hit, last_pos;
  const int row = blockIdx.x;
  const float* z = logits + static_cast<size_t>(row) * n;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int chunk = (n + kSampleThreads - 1) / kSampleThreads;
  const int i0 = min(t * chunk, n), i1 = min(i0 + chunk, n);
  if (t == 0) {
    hit = n;
    last_pos = -1;
  }

  // 1. row maximum (staged rows: while loading them, coalesced)
  float m = -INFINITY;
  if (staged) {
    for (int i = t; i < n; i += kSampleThreads) {
      const float v = z[i];
      row_w[sample_slot(i)] = v;
      m = fmaxf(m, v);
    }
  } else {
    for (int i = i0; i < i1; ++i) m = fmaxf(m, z[i]);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < kSampleWaves; ++w) m = fmaxf(m, red[w]);

  // 2. this thread's weight sum, then an exclusive scan over threads
  // (the barrier of the maximum also orders the staging stores before these reads)
  float s = 0.f;
  if (staged) {
    // eight LDS reads in flight, then the weights in index order
    for (int b = i0; b < i1; b += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = b + k < i1 ? row_w[sample_slot(b + k)] : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (b + k < i1) {
          const float w = __expf((v[k] - m) * inv_t);
          row_w[sample_slot(b + k)] = w;
          s += w;
        }
    }
  } else {
    for (int i = i0; i < i1; ++i) s += __expf((z[i] - m) * inv_t);
  }
  float inc = s;
  for (int d = 1; d < 64; d <<= 1) {
    const float v = __shfl_up(inc, d);
    if (lane >= d) inc += v;
  }
  __syncthreads();  // every wave has read red[] for the maximum
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  if (t == 0) {
    float acc = 0.f;
    for (int w = 0; w < kSampleWaves; ++w) {
      wave_off[w] = acc;
      acc += red[w];
    }
    red[0] = acc;  // the total S (all waves have read red[] above)
  }
  __syncthreads();
  const float total = red[0];
  const float off = wave_off[wave] + (inc - s);
  const float target = u[row] * total;

  // 3. the first index whose cumulative weight passes the target
  float c = off;
  int mine = n, pos = -1;
  for (int b = i0; b < i1 && mine == n; b += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = b + k >= i1 ? 0.f : staged ? row_w[sample_slot(b + k)] : __expf((z[b + k] - m) * inv_t);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = v[k];
      c += w;
      if (mine == n && b + k < i1 && w > 0.f) {
        pos = b + k;
        if (c > target) mine = b + k;
      }
    }
  }
  // without a hit the loop ran to the end: pos is the range's last positive index
  // one LDS atomic per wave: every thread past the hit also hits, on its first index
  for (int o = 32; o > 0; o >>= 1) {
    mine = min(mine, __shfl_xor(mine, o));
    pos = max(pos, __shfl_xor(pos, o));
  }
  if (lane == 0) {
    if (mine < n) atomicMin(&hit, mine);
    if (pos >= 0) atomicMax(&last_pos, pos);
  }
  __syncthreads();
  if (t == 0) tokens[row] = hit < n ? hit : last_pos;
}

}  // namespace lf
