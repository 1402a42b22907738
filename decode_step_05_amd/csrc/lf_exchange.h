// Data exchange between workgroups of one launch through tagged words, and
// the split merge of attention built on it.
//
// Every value another workgroup reads is stored as one 64-bit word (fp32
// value, 32-bit tag) with a device-scope store; the tag names the producing
// launch (and phase), and a reader polls with device-scope loads until the
// words it needs carry the expected tag. Producers never wait for their
// stores, so an exchange costs one memory round trip after the data lands.
#pragma once
#include "lf_device.h"

namespace lf {

typedef unsigned long long u64;

constexpr unsigned kSSpin = 1u << 21;  // polls before a wait gives up (raises the abort flag)

// Buffers are addressed through buffer descriptors (scalar registers) with a
// per-lane byte offset and a wave-uniform one, so that few vector registers
// hold addresses. Reads past a descriptor's range return zero (and are masked
// out where used).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));

__device__ __forceinline__ rsrc_t rsrc_of(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Store tagged element e: one 64-bit store with the device-scope coherence
// bit (the form of a relaxed device-scope atomic store).
__device__ __forceinline__ void put_t(rsrc_t r, int e, float v, unsigned tag) {
  const u32x2 d = {__float_as_uint(v), tag};
  __builtin_amdgcn_raw_buffer_store_b64(d, r, e * 8, 0, 16);
}

// Store tagged element e for readers on the same XCD: a plain store, which
// lands in (and stays in) that XCD's L2, the cache the readers' device-scope
// loads are served from. Workgroups whose launch indices are congruent
// modulo 8 share an XCD (workgroups are dealt to the XCDs in turn; checked
// when a model is initialised). An exchange through the L2 costs about half a
// memory round trip.
__device__ __forceinline__ void put_t_xcd(rsrc_t r, int e, float v, unsigned tag) {
  const u32x2 d = {__float_as_uint(v), tag};
  __builtin_amdgcn_raw_buffer_store_b64(d, r, e * 8, 0, 0);
}

// Two tagged values (16 bytes at byte offset voff + soff) with a
// device-coherent load (the cache bypass of a device-scope atomic load; each
// 8-byte half is one tagged value, written by a single 64-bit store).
__device__ __forceinline__ u32x4 ld_t2(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 16);
}

__device__ __forceinline__ bool stale2(const u32x4& v, unsigned tag) { return v[1] != tag || v[3] != tag; }

// Poll budget shared by the waits of a wave: false once the launch is aborted
// (by another wave, or by this one when its budget runs out).
struct SPoll {
  unsigned* abort;
  unsigned spins;
  __device__ __forceinline__ bool next(int lane) {
    if (++spins >= kSSpin) {
      if (lane == 0) __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    if ((spins & 31) == 0 && __hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(1);
    return true;
  }
};

// Operand of the batched projections' matrix instructions (16x16x32): per
// k-step of 32 k, 64 slots of 8 fp16; lane 16 g + c takes k-group g (k
// 8g .. 8g + 7 of the step) of column c, where column s < 8 is the hi part
// of sequence s's value and column 8 + s its lo part. In memory a k-group's
// 16 columns are ordered by sequence, hi then lo (slot 16 g + 2 s + h), so
// the columns of n sequences are one run of 32 n bytes. Half index of
// (k, column):
__device__ __forceinline__ int frag_index(int k, int col) {
  return (((k >> 5) * 64 + ((k >> 3) & 3) * 16 + 2 * (col & 7) + (col >> 3)) << 3) + (k & 7);
}
// Store values v0, v1 at k, k + 1 (k even) of sequence s as hi and lo parts.
__device__ __forceinline__ void put_frag2(half_t* f, int k, int s, float v0, float v1) {
  typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
  const half_t h0 = static_cast<half_t>(v0), h1 = static_cast<half_t>(v1);
  const hh2 hi = {h0, h1};
  const hh2 lo = {static_cast<half_t>(v0 - static_cast<float>(h0)), static_cast<half_t>(v1 - static_cast<float>(h1))};
  *reinterpret_cast<hh2*>(f + frag_index(k, s)) = hi;
  *reinterpret_cast<hh2*>(f + frag_index(k, s + 8)) = lo;
}

// Fold softmax state (m2, l2, a0, a1) into (M, L, A0, A1): maxima in log2
// units; a state with maximum -inf holds nothing.
__device__ __forceinline__ void fold_state(float& M, float& L, float& A0, float& A1, float m2, float l2, float a0,
                                           float a1) {
  const float Mn = fmaxf(M, m2);
  if (Mn == -INFINITY) return;
  const float fo = exp2f(M - Mn), fn = exp2f(m2 - Mn);
  L = L * fo + l2 * fn;
  A0 = A0 * fo + a0 * fn;
  A1 = A1 * fo + a1 * fn;
  M = Mn;
}

// One wave of split si of kv head kvh: wait for the S partial states of the
// kv head's G query heads (part: [n_kv * G][S_max][HD + 2] tagged words:
// outputs, running max in log2 units, denominator) and store this split's
// share of the merged attention output to out ([n_kv * G * HD]; tagged words
// if TAGGED, else fp32 values for a later launch; outputs [si*per,
// si*per + per) of the G*HD, per even). In rounds of at most 64 output
// pairs: lane (pair pi, group sg) of NG groups (P pairs rounded up to a power
// of two per group) folds splits sg, sg + NG, ... of pair pi into a running
// (max, denominator, outputs) state, and the groups are folded by lane
// shuffles. Every load of a batch is issued before the first is waited for,
// so a batch whose states have landed costs one round trip. Returns false if
// the launch was aborted. frag (untagged only): store the outputs instead as
// column fcol of a matrix-core operand, split into fp16 hi and lo parts
// (frag_index), for a batched projection.
template <int HD, int G, bool TAGGED = true>
__device__ __forceinline__ bool attn_merge_share(const u64* part, void* out, int n_kv, int S_max, int kvh, int si,
                                                 int S, unsigned tag_part, unsigned tag_att, SPoll& poll, int lane,
                                                 half_t* frag = nullptr, int fcol = 0) {
  constexpr int ST = HD + 2;  // tagged words per (head, split)
  constexpr int NE = G * HD;  // outputs of the kv head's query heads
  const int per = ((NE + S - 1) / S + 1) & ~1;
  const int e_begin = si * per, e_end = min(NE, e_begin + per);
  const rsrc_t r = rsrc_of(part, n_kv * G * S_max * ST * 8);
  const rsrc_t ro = rsrc_of(out, n_kv * G * HD * 8);
  constexpr int MAXS = 4;  // splits per lane per batch of loads
  for (int e0 = e_begin; e0 < e_end; e0 += 2 * kWave) {
    const int P = min(kWave, (e_end - e0) / 2);  // output pairs of this round
    int PP = 1;
    while (PP < P) PP <<= 1;
    const int NG = kWave / PP;  // lane groups
    const int pi = lane & (PP - 1), sg = lane / PP;
    const bool active = pi < P;
    const int e = e0 + 2 * min(pi, P - 1);
    const int head = kvh * G + e / HD, d = e % HD;
    const int va_off = (head * S_max * ST + d) * 8, vm_off = (head * S_max * ST + HD) * 8;
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
    for (int t0 = sg; t0 < S; t0 += NG * MAXS) {
      u32x4 va[MAXS], vm[MAXS];
      int so[MAXS];
#pragma unroll
      for (int u = 0; u < MAXS; ++u) {
        const int t = t0 + u * NG;
        // per-lane offsets in the vector operand; splits past S read past the
        // descriptor's range, which returns zero without a memory access
        so[u] = active && t < S ? t * ST * 8 : 0x40000000;
        va[u] = ld_t2(r, va_off + so[u], 0);
        vm[u] = ld_t2(r, vm_off + so[u], 0);
      }
      unsigned stale = 0;
#pragma unroll
      for (int u = 0; u < MAXS; ++u)
        if (so[u] != 0x40000000 && (stale2(va[u], tag_part) || stale2(vm[u], tag_part))) stale |= 1u << u;
      while (__any(stale != 0)) {
        if (!poll.next(lane)) return false;
#pragma unroll
        for (int u = 0; u < MAXS; ++u) {
          const int o = (stale & (1u << u)) ? so[u] : 0x40000000;
          const u32x4 na = ld_t2(r, va_off + o, 0), nm = ld_t2(r, vm_off + o, 0);
          if (stale & (1u << u)) {
            va[u] = na;
            vm[u] = nm;
          }
        }
        unsigned still = 0;
#pragma unroll
        for (int u = 0; u < MAXS; ++u)
          if ((stale & (1u << u)) && (stale2(va[u], tag_part) || stale2(vm[u], tag_part))) still |= 1u << u;
        stale = still;
      }
#pragma unroll
      for (int u = 0; u < MAXS; ++u)
        if (so[u] != 0x40000000)
          fold_state(M, L, A0, A1, __uint_as_float(vm[u][0]), __uint_as_float(vm[u][2]), __uint_as_float(va[u][0]),
                     __uint_as_float(va[u][2]));
    }
    // fold the lane groups: lanes pi + PP * g, g < NG (unrolled, so that each
    // exchange has a constant offset)
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int off = 1 << k;
      if (off >= PP)
        fold_state(M, L, A0, A1, lane_xor(M, off), lane_xor(L, off), lane_xor(A0, off), lane_xor(A1, off));
    }
    if (sg == 0 && active) {
      if constexpr (TAGGED) {
        put_t(ro, head * HD + d, A0 / L, tag_att);
        put_t(ro, head * HD + d + 1, A1 / L, tag_att);
      } else if (frag) {
        put_frag2(frag, head * HD + d, fcol, A0 / L, A1 / L);
      } else {
        *reinterpret_cast<float2*>(static_cast<float*>(out) + head * HD + d) = make_float2(A0 / L, A1 / L);
      }
    }
  }
  return true;
}

}  // namespace lf
