// Device-side building blocks for gfx950 (CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 half_t;

constexpr int kWave = 64;
constexpr int kBlock = 256;          // threads per workgroup for every step kernel
constexpr int kWavesPerBlock = kBlock / kWave;

// Device-side sequence state (first bytes of the per-sequence buffer).
enum StateSlot : int {
  kLen = 0,       // positions in the cache = position of the next step
  kArgmax = 1,    // greedy token of the most recent position
  kFedEnd = 2,    // argmax of position p is stored as token p+1 only if p+1 >= kFedEnd
  kBadToken = 3,  // set when a token id outside [0, vocab) was clamped
};

// 16-byte weight load that bypasses cache residency (weights are read once per step).
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Read a value of a table that no one writes during the launch through the
// constant address space: a wave-uniform address then gives scalar loads,
// which (unlike vector loads, retired in issue order) do not wait behind the
// wave's weight loads.
template <class T>
__device__ __forceinline__ T cload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// acc + sum_i w[i] * x[i] over 8 fp16 weights and 8 fp32 inputs.
__device__ __forceinline__ float dot8(u32x4 w, f32x4 x0, f32x4 x1, float acc) {
  const h8 h = __builtin_bit_cast(h8, w);
  acc = fmaf(static_cast<float>(h[0]), x0.x, acc);
  acc = fmaf(static_cast<float>(h[1]), x0.y, acc);
  acc = fmaf(static_cast<float>(h[2]), x0.z, acc);
  acc = fmaf(static_cast<float>(h[3]), x0.w, acc);
  acc = fmaf(static_cast<float>(h[4]), x1.x, acc);
  acc = fmaf(static_cast<float>(h[5]), x1.y, acc);
  acc = fmaf(static_cast<float>(h[6]), x1.z, acc);
  acc = fmaf(static_cast<float>(h[7]), x1.w, acc);
  return acc;
}

__device__ __forceinline__ void unpack8(u32x4 w, float (&f)[8]) {
  const h8 h = __builtin_bit_cast(h8, w);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(h[i]);
}

// Butterfly sum over the whole wave; every lane receives the total.
// The value of lane (this lane ^ off) within a wave64. Offsets 1, 2 and 8
// are DPP moves (quad permutations; a rotation by 8 within each 16-lane row),
// 16 and 32 the gfx950 lane swaps between rows (v_permlane16_swap swaps the
// odd rows of its first operand with the even rows of its second,
// v_permlane32_swap the upper half of the first with the lower half of the
// second); only 4 goes through the LDS crossbar.
__device__ __forceinline__ float lane_xor(float v, int off) {
  const unsigned u = __float_as_uint(v);
  const unsigned lane = threadIdx.x & 63;
  switch (off) {
    case 1: return __uint_as_float(__builtin_amdgcn_update_dpp(0u, u, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    case 2: return __uint_as_float(__builtin_amdgcn_update_dpp(0u, u, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    case 8: return __uint_as_float(__builtin_amdgcn_update_dpp(0u, u, 0x128, 0xF, 0xF, false));  // row_ror:8
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      return __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    case 32: {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
    default: return __shfl_xor(v, off);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Butterfly sum within aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over the workgroup (kBlock threads); `red` is kWavesPerBlock floats of LDS.
// Fixed combination order, so the result is deterministic.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) t += red[i];
  __syncthreads();
  return t;
}

// (value, index) ordering for greedy choice: larger value wins, lower index on ties.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Signal that this workgroup has finished writing its results, and find out
// whether it is the last of `expected` workgroups sharing `counter`. Every
// thread must call it. The last workgroup sees all others' writes after it
// returns true, and resets the counter for the next launch.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, int* flag_lds) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(counter, 1u);
    *flag_lds = (prev == expected - 1) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag_lds != 0;
  if (last) __threadfence();
  return last;
}

__device__ __forceinline__ void reset_counter(unsigned* counter) {
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lf
