// Kernels of one decode step (batch 1) for gfx950.
//
// Every projection is a GEMV y = W x with fp16 W (row-major [out, in]) read
// once per step with 16-byte non-temporal loads. Each wave owns row groups
// g, g + TW, g + 2 TW, ... (TW = all waves of the launch) and keeps the next
// group's loads in flight while it reduces the current one, so HBM stays busy
// through the reductions; the first two groups are issued before the
// workgroup stages its input vector in LDS (after it, for QKV). The input
// stage can apply RMSNorm
// (each workgroup reduces sum(x^2) itself: no separate norm kernel), and the
// epilogue fuses what follows the product: rotary embedding and the KV append
// (QKV), SwiGLU (gate/up), the residual add (O, down), or the logits and the
// greedy argmax (LM head). Attention splits each kv head's visible keys over
// workgroups; every split merges its share of the kv head's outputs from the
// partial softmax states of all splits.
//
// Data that another workgroup of the same launch reads is written with
// device-scope stores and read with device-scope loads (they bypass the
// per-XCD L2 without flushing it); a workgroup announces completion with one
// atomic after its stores have been acknowledged. No L2 writeback fences.
#pragma once
#include "lf_exchange.h"

namespace lf {

// ------------------------------------------------- device-scope data access

__device__ __forceinline__ void put_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 get_f32x2(const float2* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void put_f16(half_t* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned short*>(p), __builtin_bit_cast(unsigned short, static_cast<half_t>(v)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's stores are acknowledged, then count the workgroup in.
// Returns true in every thread of the last of `expected` workgroups.
// Workgroup barrier for data exchanged through LDS only: each wave waits for
// its own LDS operations, not for its global memory operations (loads may
// stay in flight across it, where the barrier of __syncthreads would wait for
// them). Whoever publishes global data waits for it explicitly.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bool arrive(unsigned* counter, unsigned expected, int* flag_lds) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_lds = (prev == expected - 1) ? 1 : 0;
  }
  __syncthreads();
  return *flag_lds != 0;
}


// ------------------------------------------------------------ reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Sum within aligned groups of W lanes (W = 4, 8 or 16) using DPP lane moves.
template <int W>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(W == 4 || W == 8 || W == 16, "DPP row reductions cover 4, 8 or 16 lanes");
  v += dpp<0xB1>(v);                   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);                   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if constexpr (W >= 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}
// Wave total, uniform across lanes.
__device__ __forceinline__ float wave_total(float v) {
  v = row_sum<16>(v);
  const int i = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(i, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(i, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(i, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(i, 48)));
}

// Greedy key: larger logit wins, then the lower index; 0 is below every key.
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  unsigned u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ties with +0.0, as better() compares them
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) | static_cast<unsigned>(0x7fffffff - i);
}
__device__ __forceinline__ int argmax_index(unsigned long long key) {
  return 0x7fffffff - static_cast<int>(key & 0xffffffffu);
}

// ------------------------------------------------------------------ GEMV

// Input of a GEMV: an fp32 vector, the same with RMSNorm, or RMSNorm of an
// embedding row. A compile-time parameter of the kernels: with one staging
// path per kernel, the wait for the staged input counts only the loads
// issued before it (a runtime choice between paths that issue it before and
// after the weights makes the compiler wait for every load at their join).
enum InKind : int { kInF32 = 0, kInNormF32 = 1, kInNormEmbed = 2 };
// kEpiQKVX: QKV whose queries and new keys and values also go to the
// exchange words of the attention that runs in the same launch.
enum Epi : int { kEpiQKV = 0, kEpiSwiGLU = 1, kEpiResid = 2, kEpiLogits = 3, kEpiQKVX = 4 };

struct GemvArgs {
  const half_t* W;        // [rows, K] (QKV and gate/up repacked so that epilogue pairs are adjacent rows)
  int rows, K;
  // input vector
  int in_kind;            // InKind; selects the kernel variant
  const float* x;         // fp32 source (kInF32, kInNormF32)
  const half_t* emb;      // embedding table [vocab, K] (kInNormEmbed)
  const half_t* gain;     // RMSNorm gain [K]
  float eps;
  int vocab;
  float* resid_copy;      // if set, every workgroup stores its slice of the raw source here
  // sequence state
  int32_t* state;
  int32_t* tokens;        // token history [max_ctx + 1]
  int max_ctx;
  // epilogue outputs
  float* y;               // kEpiResid: residual (y += Wx); kEpiSwiGLU: activation; kEpiLogits: logits
  float* q;               // kEpiQKV: rotated queries [Hq * hd]
  half_t* kc;             // kEpiQKV: this layer's K cache [lanes][max_ctx][kpl][hd]
  half_t* vc;             //          and V cache
  const float2* rope;     // (cos, sin) [max_ctx][hd / 2]
  int hd, qpl, kpl;
  u64* qkvx;              // kEpiQKVX: tagged words [Hkv][(G + 2) hd]: per kv head its G queries, key, value
  unsigned tag;           // kEpiQKVX: their tag
  // finishing work of the last workgroup (kEpiLogits: argmax + step end; kEpiResid: step end)
  unsigned* counter;      // null: none
  unsigned long long* best;  // kEpiLogits: packed greedy key
};

// Input staging in two halves so that its loads can be issued before the
// weight loads: the vector memory counter retires loads in issue order, so
// waiting for the input must not also wait for the weights.
template <int THREADS, int KMAX>
struct Stage {
  static constexpr int NV = (KMAX + THREADS * 8 - 1) / (THREADS * 8);  // 8-element pieces per thread
  float v[NV][8];
  u32x4 gn[NV];
};

// Issue the loads of the input vector (length K <= KMAX) and of the RMSNorm
// gains. COH: read the source with device-scope loads (written in this launch).
template <int THREADS, int KMAX, bool COH, int IN>
__device__ __forceinline__ void stage_load(Stage<THREADS, KMAX>& st, const GemvArgs& a, int p) {
  constexpr int NV = Stage<THREADS, KMAX>::NV;
  const int tid = threadIdx.x, K = a.K;
  constexpr bool norm = IN != kInF32;
  if constexpr (IN == kInNormEmbed) {
    int tok = a.tokens[p];
    if (tok < 0 || tok >= a.vocab) {
      tok = tok < 0 ? 0 : a.vocab - 1;
      if (tid == 0 && blockIdx.x == 0) a.state[kBadToken] = 1;
    }
    const half_t* row = a.emb + static_cast<size_t>(tok) * K;
    u32x4 e[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = min((tid + j * THREADS) * 8, K - 8);
      e[j] = ld16(row + i);
      st.gn[j] = ld16(a.gain + i);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) unpack8(e[j], st.v[j]);
    return;
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = min((tid + j * THREADS) * 8, K - 8);
    if (COH) {
      const float2* src = reinterpret_cast<const float2*>(a.x + i);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float2 f = get_f32x2(src + t);
        st.v[j][2 * t] = f.x;
        st.v[j][2 * t + 1] = f.y;
      }
    } else {
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(a.x + i);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(a.x + i + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        st.v[j][t] = f0[t];
        st.v[j][4 + t] = f1[t];
      }
    }
    if (norm) st.gn[j] = ld16(a.gain + i);
  }
}

// Finish the stage: RMSNorm (sum of squares over the workgroup, then
// x * rsqrt(mean + eps) * gain) if asked, the layer-0 residual copy, and the
// LDS store. LDS layout: two planes, plane h holding elements 8q+4h .. 8q+4h+3
// of every 8-element chunk q in the 16-byte word xs[h*K/8 + q]; a wave reading
// chunks q = lane + 64c touches consecutive 16-byte words: one ds_read_b128
// per plane, free of bank conflicts.
template <int THREADS, int KMAX, int IN>
__device__ __forceinline__ void stage_store(const Stage<THREADS, KMAX>& st, const GemvArgs& a, f32x4* xs, float* red) {
  constexpr int NW = THREADS / kWave;
  constexpr int NV = Stage<THREADS, KMAX>::NV;
  const int tid = threadIdx.x, K = a.K;
  const int per = (K + gridDim.x - 1) / gridDim.x;
  const int s0 = blockIdx.x * per, s1 = min(s0 + per, K);
  constexpr bool norm = IN != kInF32;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = (tid + j * THREADS) * 8;
    if (i >= K || tid >= THREADS) break;  // threads past THREADS only take part in the barriers
#pragma unroll
    for (int t = 0; t < 8; ++t) ss = fmaf(st.v[j][t], st.v[j][t], ss);
    if (a.resid_copy)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (i + t >= s0 && i + t < s1) put_f32(a.resid_copy + i + t, st.v[j][t]);
  }
  float r = 1.f;
  if (norm) {
    ss = wave_total(ss);
    if ((tid & (kWave - 1)) == 0 && tid < THREADS) red[tid / kWave] = ss;
    lds_barrier();  // not __syncthreads: its fence would wait for the weight loads in flight
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
    r = 1.0f / sqrtf(tot / static_cast<float>(K) + a.eps);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int q = tid + j * THREADS;
    if (q * 8 >= K || tid >= THREADS) break;
    float g[8];
    if (norm) unpack8(st.gn[j], g);
    f32x4 o0, o1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o0[t] = norm ? st.v[j][t] * r * g[t] : st.v[j][t];
      o1[t] = norm ? st.v[j][4 + t] * r * g[4 + t] : st.v[j][4 + t];
    }
    xs[q] = o0;
    xs[(K >> 3) + q] = o1;
  }
  lds_barrier();  // the weight loads stay in flight; each group is waited for where it is reduced
}

template <int NR, int KCH>
struct Rows {
  u32x4 w[NR][KCH];
  float res[NR];  // current residual values (residual epilogue)
};

// Issue the loads of rows [r, r+NR): lane covers 16-byte chunks lane + 64c.
// res_src (residual epilogue): also load the residual values of those rows.
template <int NR, int KCH>
__device__ __forceinline__ void issue_rows(Rows<NR, KCH>& b, const half_t* __restrict__ W, int r, int rows, int K,
                                           int lane, const float* res_src = nullptr) {
  // Out-of-range rows and chunks load from a clamped, in-bounds address and are
  // ignored where the values are used: no branches around the loads, so all
  // of them stay in flight together.
  const int K8 = K >> 3;
  if (res_src)
#pragma unroll
    for (int i = 0; i < NR; ++i) b.res[i] = get_f32(res_src + min(r + i, rows - 1));
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const half_t* row = W + static_cast<size_t>(min(r + i, rows - 1)) * K;
#pragma unroll
    for (int c = 0; c < KCH; ++c) b.w[i][c] = ld_stream(row + static_cast<size_t>(min(lane + kWave * c, K8 - 1)) * 8);
  }
}

// Where the QKV projection writes at position p.
struct QkvOut {
  float* q;
  half_t *kc, *vc;
  const float2* rope;
  int hd, qpl, kpl, max_ctx;
};

// Store the rotary pair of QKV rows (r, r+1) (r even; lane-major order: per
// lane its q heads, then k heads, then v heads, each head's rows as pairs
// (c, c + hd/2) of the half-split rotary embedding): rotate q and k by the
// angles of position p, then store q (fp32) or append k / v to the cache (fp16).
__device__ __forceinline__ void qkv_put(const QkvOut& a, int r, float y0, float y1, int p) {
  const int half_hd = a.hd >> 1, upl = a.qpl + 2 * a.kpl;
  const int u = r / a.hd, c = (r % a.hd) >> 1;
  const int ln = u / upl, j = u % upl;
  if (j < a.qpl + a.kpl) {  // rotary embedding on q and k
    // scalar load (one lane runs this; the row, hence the index, is the wave's)
    const int ri = __builtin_amdgcn_readfirstlane(p * half_hd + c);
    const float2 cs = __builtin_bit_cast(float2, cload(reinterpret_cast<const unsigned long long*>(a.rope + ri)));
    const float t0 = y0 * cs.x - y1 * cs.y;
    const float t1 = y0 * cs.y + y1 * cs.x;
    y0 = t0;
    y1 = t1;
  }
  if (j < a.qpl) {
    float* qh = a.q + static_cast<size_t>(ln * a.qpl + j) * a.hd;
    put_f32(qh + c, y0);
    put_f32(qh + c + half_hd, y1);
  } else {
    const bool is_k = j < a.qpl + a.kpl;
    const int h = is_k ? j - a.qpl : j - a.qpl - a.kpl;
    half_t* dst = (is_k ? a.kc : a.vc) + ((static_cast<size_t>(ln) * a.max_ctx + p) * a.kpl + h) * a.hd;
    put_f16(dst + c, y0);
    put_f16(dst + c + half_hd, y1);
  }
}

// qkv_put for QKV fused with attention: rotate as qkv_put, append k / v to
// the cache, and store the rotated queries and the new key and value as
// tagged words for the attention workgroups on this XCD (plain stores: they
// stay in the XCD's L2, where those workgroups read them).
__device__ __forceinline__ void qkv_put_x(const QkvOut& a, u64* x, unsigned tag, int r, float y0, float y1, int p) {
  const int half_hd = a.hd >> 1, upl = a.qpl + 2 * a.kpl, G = a.qpl / a.kpl;
  const int u = r / a.hd, c = (r % a.hd) >> 1;
  const int ln = u / upl, j = u % upl;
  if (j < a.qpl + a.kpl) {
    const int ri = __builtin_amdgcn_readfirstlane(p * half_hd + c);
    const float2 cs = __builtin_bit_cast(float2, cload(reinterpret_cast<const unsigned long long*>(a.rope + ri)));
    const float t0 = y0 * cs.x - y1 * cs.y;
    const float t1 = y0 * cs.y + y1 * cs.x;
    y0 = t0;
    y1 = t1;
  }
  int kvh, slot;  // exchange slot: G queries, then the key, then the value
  if (j < a.qpl) {
    kvh = ln * a.kpl + j / G;
    slot = j % G;
  } else {
    const bool is_k = j < a.qpl + a.kpl;
    const int h = is_k ? j - a.qpl : j - a.qpl - a.kpl;
    kvh = ln * a.kpl + h;
    slot = is_k ? G : G + 1;
    half_t* dst = (is_k ? a.kc : a.vc) + ((static_cast<size_t>(ln) * a.max_ctx + p) * a.kpl + h) * a.hd;
    dst[c] = static_cast<half_t>(y0);  // read by later launches only
    dst[c + half_hd] = static_cast<half_t>(y1);
  }
  u64* e = x + (static_cast<size_t>(kvh) * (G + 2) + slot) * a.hd + c;
  const u64 t = static_cast<u64>(tag) << 32;
  e[0] = t | __float_as_uint(y0);
  e[half_hd] = t | __float_as_uint(y1);
}

// This lane's chunks of the staged input in registers (zero past K): read
// from LDS once per wave instead of once per row group, for K up to 4096.
template <int KCH>
struct XRegs {
  static constexpr bool on = KCH <= 8;
  f32x4 x[2][on ? KCH : 1];
};

// Reduce rows [r, r+NR) against the input (xr if XRegs<KCH>::on, else xs in
// LDS) and run the epilogue (lane 0 stores). FULL: K is exactly 512*KCH, so
// every chunk of every lane is in range.
template <int EPI, int NR, int KCH, bool FULL>
__device__ __forceinline__ void finish_rows(const GemvArgs& a, const Rows<NR, KCH>& b, const f32x4* xs,
                                            const XRegs<KCH>& xr, int r, int lane, int p, float& bv, int& bi) {
  const int K8 = a.K >> 3;
  const f32x4* xs_hi = xs + K8;
  float acc[NR][2];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i][0] = acc[i][1] = 0.f;
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int ch = lane + kWave * c;
    if (XRegs<KCH>::on || FULL || ch < K8) {
      f32x4 x0, x1;
      if constexpr (XRegs<KCH>::on) {
        x0 = xr.x[0][c];
        x1 = xr.x[1][c];
      } else {
        x0 = xs[ch];
        x1 = xs_hi[ch];
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const h8 h = __builtin_bit_cast(h8, b.w[i][c]);
        // two independent chains (elements 0-3 and 4-7) keep the FMA pipe full
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[i][0] = fmaf(static_cast<float>(h[t]), x0[t], acc[i][0]);
          acc[i][1] = fmaf(static_cast<float>(h[4 + t]), x1[t], acc[i][1]);
        }
      }
    }
  }
  float out[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) out[i] = wave_total(acc[i][0] + acc[i][1]);
  if (lane != 0) return;
  if constexpr (EPI == kEpiQKV) {
    static_assert(NR == 2, "QKV rows come in rotary pairs");
    if (r >= a.rows) return;
    qkv_put(QkvOut{a.q, a.kc, a.vc, a.rope, a.hd, a.qpl, a.kpl, a.max_ctx}, r, out[0], out[1], p);
  } else if constexpr (EPI == kEpiQKVX) {
    static_assert(NR == 2, "QKV rows come in rotary pairs");
    if (r >= a.rows) return;
    qkv_put_x(QkvOut{a.q, a.kc, a.vc, a.rope, a.hd, a.qpl, a.kpl, a.max_ctx}, a.qkvx, a.tag, r, out[0], out[1], p);
  } else if constexpr (EPI == kEpiSwiGLU) {
    static_assert(NR == 2, "gate/up rows come in pairs");
    if (r >= a.rows) return;
    const float g = out[0], up = out[1];
    put_f32(a.y + (r >> 1), g / (1.0f + expf(-g)) * up);
  } else if constexpr (EPI == kEpiResid) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (r + i < a.rows) put_f32(a.y + r + i, b.res[i] + out[i]);
  } else {  // kEpiLogits
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (r + i < a.rows) {
        put_f32(a.y + r + i, out[i]);
        if (better(out[i], r + i, bv, bi)) {
          bv = out[i];
          bi = r + i;
        }
      }
  }
}

// Row group of wave gw (of TW) at its k-th group. MAP 0: gw + k TW. MAP 1,
// the QKV projection fused with attention (256 workgroups of 8 waves, two
// groups each; 16 kv heads of G + 2 heads of hd rows, G = qpl / kpl, and
// (G + 2) hd / 2 = 256 rotary pairs each): workgroup b's k-th groups are
// pairs of kv head (b mod 8) + 8 k, whose attention runs on the workgroups
// congruent to b modulo 8 (one XCD), pair (b / 8) * 8 + wave of the head's
// queries, key and value, in the lane-major row order of the repacked
// weights.
template <int MAP>
__device__ __forceinline__ int row_group(const GemvArgs& a, int gw, int TW, int k) {
  if constexpr (MAP == 0) {
    return gw + k * TW;
  } else {
    const int b = gw >> 3, w = gw & 7;
    const int kvh = (b & 7) + 8 * k, j = (b >> 3) * 8 + w;
    const int G = a.qpl / a.kpl, half = a.hd >> 1;
    const int u = j / half, jj = j % half;  // unit of the kv head: query u < G, key G, value G + 1
    const int ln = kvh / a.kpl, kvl = kvh % a.kpl;
    const int unit = u < G ? kvl * G + u : u == G ? a.qpl + kvl : a.qpl + a.kpl + kvl;
    return (ln * (a.qpl + 2 * a.kpl) + unit) * half + jj;
  }
}

// The GEMV work of one workgroup: wave gw of TW handles row groups gw + k*TW
// for k < GPW (the launch covers the matrix: GPW * TW >= groups). The loop is
// unrolled at compile time so that each group's loads are waited for exactly
// (the next group's loads stay in flight while this one is reduced).
// Must be called by every thread of the workgroup (the input stage has barriers).
// Returns false (in every thread) if the sequence is full and nothing was done.
struct NoLoads {
  __device__ void operator()(int) const {}
};

// pre(p): further loads of the caller at position p, issued before the
// input's wait and before the weights; with STH below THREADS only the
// waves that do not stage the input should issue any (a wave's loads
// complete in issue order, so the stagers' input wait would include them).
// STH: the threads (the first ones of the workgroup) that stage the input.
template <int EPI, int NR, int KCH, int GPW, int THREADS, bool COH, int IN, int MAP = 0, class Pre = NoLoads,
          int STH = THREADS>
__device__ __forceinline__ bool gemv_run(const GemvArgs& a, f32x4* xs, float* red, int gw, int TW, int& p, float& bv,
                                         int& bi, const Pre& pre = Pre{}) {
  const int lane = threadIdx.x & (kWave - 1);
  const int ng = (a.rows + NR - 1) / NR;
  const float* res = EPI == kEpiResid ? a.y : nullptr;
  const bool full = a.K == KCH * kWave * 8;
  constexpr int KMAX = KCH * kWave * 8;
  Rows<NR, KCH> buf[2];
  Stage<STH, KMAX> st;
  // Issue order: input vector, then weights (loads retire in issue order).
  // The embedding row needs the position first; that is one kernel per step.
  // Staging the input before requesting any weight leaves HBM idle for the
  // input's round trip at every launch, which was measured slower for every
  // GEMV but QKV: there every wave requests all its rows (four) at once, the
  // input comes back behind them, and the reduction of the four rows after
  // it costs more than the idle round trip.
  constexpr bool embed = IN == kInNormEmbed;
  constexpr bool stage_first = (EPI == kEpiQKV || EPI == kEpiQKVX) && !embed;
  // The position, read before any store of this launch (so with a scalar
  // load), is waited for only where it is first used.
  p = a.state[kLen];
  if constexpr (!embed)
    if (STH == THREADS || static_cast<int>(threadIdx.x) < STH) stage_load<STH, KMAX, COH, IN>(st, a, 0);
  pre(p);
  if constexpr (stage_first) stage_store<STH, KMAX, IN>(st, a, xs, red);
  issue_rows<NR, KCH>(buf[0], a.W, min(row_group<MAP>(a, gw, TW, 0), ng - 1) * NR, a.rows, a.K, lane, res);
  if (GPW > 1)
    issue_rows<NR, KCH>(buf[1], a.W, min(row_group<MAP>(a, gw, TW, 1), ng - 1) * NR, a.rows, a.K, lane, res);
  if (p >= a.max_ctx) return false;  // the host never launches a step on a full cache
  if constexpr (embed)
    if (STH == THREADS || static_cast<int>(threadIdx.x) < STH) stage_load<STH, KMAX, COH, IN>(st, a, p);
  if constexpr (!stage_first) stage_store<STH, KMAX, IN>(st, a, xs, red);
  XRegs<KCH> xr;
  if constexpr (XRegs<KCH>::on) {
    const int K8 = a.K >> 3;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = lane + kWave * c;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      xr.x[0][c] = ch < K8 ? xs[ch] : z;
      xr.x[1][c] = ch < K8 ? xs[K8 + ch] : z;
    }
  }
#pragma unroll
  for (int k = 0; k < GPW; ++k) {
    const int g = row_group<MAP>(a, gw, TW, k);
    if (g < ng) {
      if (full)
        finish_rows<EPI, NR, KCH, true>(a, buf[k & 1], xs, xr, g * NR, lane, p, bv, bi);
      else
        finish_rows<EPI, NR, KCH, false>(a, buf[k & 1], xs, xr, g * NR, lane, p, bv, bi);
    }
    if (k + 2 < GPW)
      issue_rows<NR, KCH>(buf[k & 1], a.W, min(row_group<MAP>(a, gw, TW, k + 2), ng - 1) * NR, a.rows, a.K, lane, res);
  }
  return true;
}

template <int EPI, int NR, int KCH, int GPW, int WAVES, int IN>
__global__ __launch_bounds__(WAVES * kWave) void k_gemv(GemvArgs a) {
  constexpr int THREADS = WAVES * kWave;
  extern __shared__ f32x4 xs[];  // the input vector, 16-byte words (see stage_store)
  __shared__ float red[WAVES];
  __shared__ float2 wbest[WAVES];
  __shared__ int flag;

  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  int p;
  if (!gemv_run<EPI, NR, KCH, GPW, THREADS, false, IN>(a, xs, red, blockIdx.x * WAVES + wave, gridDim.x * WAVES, p, bv,
                                                         bi))
    return;

  if (a.counter == nullptr) return;
  if constexpr (EPI == kEpiLogits) {
    if (lane == 0) wbest[wave] = make_float2(bv, __int_as_float(bi));
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < WAVES; ++w) {
        const int wi = __float_as_int(wbest[w].y);
        if (better(wbest[w].x, wi, bv, bi)) {
          bv = wbest[w].x;
          bi = wi;
        }
      }
      if (bi != 0x7fffffff)
        __hip_atomic_fetch_max(a.best, argmax_key(bv, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!arrive(a.counter, gridDim.x, &flag)) return;
    if (threadIdx.x == 0) {
      const unsigned long long key = __hip_atomic_load(a.best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int i = key ? argmax_index(key) : 0;  // key == 0 only if every logit is NaN
      if (i < 0 || i >= a.rows) i = 0;
      a.state[kArgmax] = i;
      if (p + 1 >= a.state[kFedEnd]) a.tokens[p + 1] = i;
      a.state[kLen] = p + 1;
      __hip_atomic_store(a.best, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    if (!arrive(a.counter, gridDim.x, &flag)) return;
    if (threadIdx.x == 0) {
      a.state[kLen] = p + 1;
      __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------- attention

// One layer's attention at position p: queries, the layer's cache, the
// window and the split plan (S work items per kv head, `chunk` keys each).
struct AttnArgs {
  const float* q;           // rotated queries [Hq * hd]
  const half_t* kc;         // this layer's K cache [lanes][max_ctx][kpl][hd]
  const half_t* vc;
  const int32_t* state;
  int max_ctx, window, S, chunk, kpl;
  float scale_log2;         // log2(e) / sqrt(hd)
};

// K and V loads of one iteration of an attention work item: U 16-byte pieces
// of K and of V per lane.
template <int U>
struct AttnLoads {
  u32x4 kk[U], vv[U];
};

// Where work item (split s, kv head kvh) reads at position p.
struct AttnSpan {
  const half_t *Kb, *Vb;  // this lane's piece of the first key of the split
  size_t key_stride;      // elements between consecutive keys
  int k0, nk;             // first key and number of keys of the split
};

template <int HD>
__device__ __forceinline__ AttnSpan attn_span(const AttnArgs& a, int s, int kvh, int p) {
  constexpr int LPR = HD / 8;
  const int lane = threadIdx.x & (kWave - 1);
  const int ln = kvh / a.kpl, kvl = kvh % a.kpl;
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  AttnSpan sp;
  sp.k0 = lo + s * a.chunk;
  sp.nk = max(0, min(sp.k0 + a.chunk, p + 1) - sp.k0);
  // key j of this kv head: ((ln * max_ctx + j) * kpl + kvl) * HD
  sp.key_stride = static_cast<size_t>(a.kpl) * HD;
  const size_t base =
      ((static_cast<size_t>(ln) * a.max_ctx + min(sp.k0, a.max_ctx - 1)) * a.kpl + kvl) * HD + (lane % LPR) * 8;
  sp.Kb = a.kc + base;
  sp.Vb = a.vc + base;
  return sp;
}

// Issue the loads of the iteration whose first wave row block is b0 (NW
// waves; a wave load covers KPW keys). Keys past the split load its last key
// (masked where used). Requires nk > 0.
template <int HD, int U, int NW>
__device__ __forceinline__ void attn_load(AttnLoads<U>& ld, const AttnSpan& sp, int b0) {
  constexpr int KPW = kWave / (HD / 8);
  const int kin = (threadIdx.x & (kWave - 1)) / (HD / 8);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = min((b0 + u * NW) * KPW + kin, sp.nk - 1);
    const size_t off = static_cast<size_t>(t) * sp.key_stride;
    ld.kk[u] = ld_stream(sp.Kb + off);
    ld.vv[u] = ld_stream(sp.Vb + off);
  }
}

// Prefetch of the first iteration of a work item (all NW waves).
template <int HD, int U, int NW>
__device__ __forceinline__ void attn_prefetch(AttnLoads<U>& ld, const AttnArgs& a, int s, int kvh, int p) {
  const AttnSpan sp = attn_span<HD>(a, s, kvh, p);
  if (sp.nk > 0) attn_load<HD, U, NW>(ld, sp, threadIdx.x / kWave);
}

// Fold the online-softmax state (m, l, acc) of lane ^ off into this lane's.
template <int G>
__device__ __forceinline__ void fold_xor(float (&m)[G], float (&l)[G], float (&acc)[G][8], int off) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float m2 = lane_xor(m[g], off), l2 = lane_xor(l[g], off);
    float a2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = lane_xor(acc[g][i], off);
    const float M = fmaxf(m[g], m2);
    if (M == -INFINITY) continue;
    const float f1 = exp2f(m[g] - M), f2 = exp2f(m2 - M);
    l[g] = l[g] * f1 + l2 * f2;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = acc[g][i] * f1 + a2[i] * f2;
    m[g] = M;
  }
}

// One iteration of a work item: the scores of the U key rows of this lane
// group (key (b0 + u NW) KPW + kin of the split; keys at or past nk are
// masked) against the G queries qr (this lane's 8 dimensions, scaled to log2
// units), then the online-softmax update of (m, l, acc) with their values.
template <int HD, int G, int U, int NW>
__device__ __forceinline__ void attn_step(const AttnLoads<U>& x, int b0, int kin, int nk, const float (&qr)[G][8],
                                          float (&m)[G], float (&l)[G], float (&acc)[G][8]) {
  constexpr int LPR = HD / 8, KPW = kWave / LPR;
  float sc[U][G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = (b0 + u * NW) * KPW + kin;
    float kf[8];
    unpack8(x.kk[u], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fmaf(qr[g][i], kf[i], d);
      d = row_sum<LPR>(d);
      sc[u][g] = t < nk ? d : -INFINITY;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = m[g];
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
    if (mx == -INFINITY) continue;
    const float al = exp2f(m[g] - mx);
    l[g] *= al;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] *= al;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = exp2f(sc[u][g] - mx);
      l[g] += pu;
      float vf[8];
      unpack8(x.vv[u], vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(pu, vf[i], acc[g][i]);
    }
    m[g] = mx;
  }
}

// LDS of the combine step: per-wave softmax states.
template <int HD, int G, int NW>
struct AttnCombine {
  float acc[NW][G][HD];
  float2 ml[NW][G];
};

// End of a work item (split si of kv head kvh) computed by waves 0 .. NW-1
// (every wave of the workgroup calls it; any further waves only take part
// in its barrier): fold each wave's key rows (lanes ch, ch + LPR, ...),
// combine the waves in LDS, and store the split's state (outputs, max,
// denominator) as tagged words (part: [n_kv * G][S_max][HD + 2]); XCD: for
// readers on this XCD.
template <int HD, int G, int NW, bool XCD>
__device__ __forceinline__ void attn_store_state(float (&m)[G], float (&l)[G], float (&acc)[G][8],
                                                 AttnCombine<HD, G, NW>& cb, u64* part, int n_kv, int S_max,
                                                 int kvh, int si, unsigned epoch) {
  constexpr int LPR = HD / 8;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1), ch = lane % LPR;
  if (wave < NW) {
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) fold_xor<G>(m, l, acc, off);
  }
  if (wave < NW && lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) cb.acc[wave][g][ch * 8 + i] = acc[g][i];
      if (ch == 0) cb.ml[wave][g] = make_float2(m[g], l[g]);
    }
  }
  lds_barrier();
  const rsrc_t rp = rsrc_of(part, n_kv * G * S_max * (HD + 2) * 8);
  for (int idx = tid; idx < G * HD; idx += NW * kWave) {
    const int d = idx % HD, g = idx / HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, cb.ml[w][g].x);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float2 ml = cb.ml[w][g];
        const float f = exp2f(ml.x - M);
        L = fmaf(ml.y, f, L);
        A = fmaf(cb.acc[w][g][d], f, A);
      }
    }
    const int base = ((kvh * G + g) * S_max + si) * (HD + 2);
    if constexpr (XCD) {
      put_t_xcd(rp, base + d, A, epoch);
      if (d == 0) {
        put_t_xcd(rp, base + HD, M, epoch);
        put_t_xcd(rp, base + HD + 1, L, epoch);
      }
    } else {
      put_t(rp, base + d, A, epoch);
      if (d == 0) {
        put_t(rp, base + HD, M, epoch);
        put_t(rp, base + HD + 1, L, epoch);
      }
    }
  }
}

struct AttnXArgs {
  AttnArgs t;
  u64* part;          // [Hq][S_max][hd + 2] tagged split states: outputs, running max (log2 units), denominator
  float* o;           // attention output [Hq * hd]
  unsigned* epochs;   // [Hkv] launch epoch per kv head (>= 1): the tag of its split states
  unsigned* abort;    // raised when a wait gives up; later waits give up at once
  int S_max, n_kv;
  half_t* ofrag;      // if set: the outputs go here as column fcol of a batched projection's operand (not to o)
  int fcol;
};

template <int HD, int G>
struct AttnXSmem {
  AttnCombine<HD, G, kWavesPerBlock> cb;
};

// Attention of work item (split s = blockIdx.x, kv head kvh = blockIdx.y):
// keys [lo + s*chunk, lo + (s+1)*chunk) of the visible ones (lo = p - W + 1
// under a window W, else 0) for the kv head's G query heads (grouped-query
// attention: query head i reads kv head i / G). Each of the kBlock/64 waves
// loads U 16-byte pieces of K and of V per lane per iteration (HD/8 lanes per
// key row), keeps an online softmax per key row in registers and folds its
// rows with lane shuffles; the workgroup combines the waves in LDS and stores
// the split's state as tagged words. Then wave 0 of every split merges its
// share of the kv head's outputs from the S states (one memory round trip:
// no counter, no last-workgroup pass) and stores them for the O projection.
// The S splits of a kv head wait for each other, so S must not exceed what
// the device holds at once (it holds many more). The tag is the kv head's
// epoch, which split 0 advances once it has read every split's state, hence
// after every split has read the epoch.
// XCD: the launch is one-dimensional (S * n_kv workgroups, n_kv a multiple
// of 8) and the splits of a kv head are the workgroups congruent to it
// modulo 8, so they run on one XCD and exchange their states through its
// L2; otherwise the grid is (S, n_kv) and the states go through memory.
// The work item (split si, kv head kvh) of one attention launch, run by a
// whole workgroup of kBlock threads (see k_attn). DB: the split spans several
// load rounds, which are double-buffered (the next round's loads are in
// flight while a round is computed; rounds past the split re-read its last
// key, L2 hits, and are masked).
template <int HD, int G, int U, bool XCD, bool DB = false>
__device__ __forceinline__ void attn_item(const AttnXArgs& a, int si, int kvh, AttnXSmem<HD, G>& sm) {
  constexpr int LPR = HD / 8, NW = kWavesPerBlock;
  const int p = a.t.state[kLen];
  if (p >= a.t.max_ctx) return;  // the host never launches a step on a full cache
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int kin = lane / LPR, ch = lane % LPR;
  constexpr int KPW = kWave / LPR;

  const AttnSpan sp = attn_span<HD>(a.t, si, kvh, p);
  AttnLoads<U> ld;
  if (sp.nk > 0) attn_load<HD, U, NW>(ld, sp, wave);
  float qr[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qp = a.t.q + static_cast<size_t>(kvh * G + g) * HD + ch * 8;
    const f32x4 q0 = reinterpret_cast<const f32x4*>(qp)[0], q1 = reinterpret_cast<const f32x4*>(qp)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qr[g][i] = q0[i] * a.t.scale_log2;
      qr[g][4 + i] = q1[i] * a.t.scale_log2;
    }
  }
  const unsigned epoch = a.epochs[kvh];  // every wave reads it before its part of the state is stored

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }
  const int nk = sp.nk;
  if constexpr (DB) {
    if (nk > 0) {
      AttnLoads<U> ld1;
      for (int b0 = wave; b0 * KPW < nk; b0 += 2 * NW * U) {
        attn_load<HD, U, NW>(ld1, sp, b0 + NW * U);
        __builtin_amdgcn_sched_barrier(0);
        attn_step<HD, G, U, NW>(ld, b0, kin, nk, qr, m, l, acc);
        __builtin_amdgcn_sched_barrier(0);
        attn_load<HD, U, NW>(ld, sp, b0 + 2 * NW * U);
        __builtin_amdgcn_sched_barrier(0);
        attn_step<HD, G, U, NW>(ld1, b0 + NW * U, kin, nk, qr, m, l, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (nk > 0) {
    attn_step<HD, G, U, NW>(ld, wave, kin, nk, qr, m, l, acc);
    for (int b0 = wave + NW * U; b0 * KPW < nk; b0 += NW * U) {
      attn_load<HD, U, NW>(ld, sp, b0);
      attn_step<HD, G, U, NW>(ld, b0, kin, nk, qr, m, l, acc);
    }
  }
  attn_store_state<HD, G, NW, XCD>(m, l, acc, sm.cb, a.part, a.n_kv, a.S_max, kvh, si, epoch);
  if (wave == 0) {
    SPoll poll{a.abort, 0u};
    attn_merge_share<HD, G, false>(a.part, a.o, a.n_kv, a.S_max, kvh, si, a.t.S, epoch, epoch, poll, lane, a.ofrag,
                                   a.fcol);
    if (si == 0 && lane == 0) a.epochs[kvh] = epoch + 1 == 0 ? 1u : epoch + 1;
  }
}

template <int HD, int G, int U, bool XCD>
__global__ __launch_bounds__(kBlock) void k_attn(AttnXArgs a) {
  __shared__ AttnXSmem<HD, G> sm;
  int si, kvh;
  if constexpr (XCD) {
    const int b = blockIdx.x, hpc = a.n_kv >> 3, r = b >> 3;  // hpc kv heads per XCD
    kvh = (b & 7) + 8 * (r % hpc);
    si = r / hpc;
  } else {
    si = blockIdx.x;
    kvh = blockIdx.y;
  }
  attn_item<HD, G, U, XCD>(a, si, kvh, sm);
}

// ------------------------------------------- QKV fused with attention

// One layer's QKV projection and attention in one launch of 256 workgroups
// of 8 waves, one attention work item each (16 kv heads x 16 splits). The
// kv heads of a class of workgroups congruent modulo 8 (one XCD) are
// computed and attended to by that class alone, so every exchange goes
// through the XCD's L2 (about 0.4 us per round trip, against 0.9 us through
// memory):
//  1. copy the work item's cached keys and values (before any weight load)
//     straight to LDS;
//  2. the QKV GEMV (row_group<1>): rotary embedding, KV append, and the
//     queries and new key / value as tagged words (kEpiQKVX);
//  3. wait for the kv head's queries (and, in the split that holds the new
//     position, its key and value) from the other workgroups of the class,
//     then attend to the split's keys from LDS as k_attn does;
//  4. store the split state and merge a share of the kv head's outputs.
// The tag of the launch is its class's epoch, read by every workgroup at its
// start; the workgroup holding the new position of the class's first kv head
// reads words from all 32 workgroups of the class, so after those reads it
// advances the epoch for the next launch.
struct QkvAttnArgs {
  GemvArgs g;              // the QKV GEMV (EPI kEpiQKVX; g.tag set in-kernel)
  AttnXArgs at;            // this layer's attention (at.t.q and at.epochs unused)
  unsigned* class_epochs;  // [8] epoch per class (>= 1)
};

template <int HD, int G, int UKV, int IN>
__global__ __launch_bounds__(8 * kWave) void k_qkv_attn(QkvAttnArgs a) {
  constexpr int NW = 8, THREADS = NW * kWave, LPR = HD / 8, KPW = kWave / LPR;
  constexpr int CH = NW * UKV * KPW;  // keys of a split held in LDS
  static_assert(HD == 128, "a wave reads 128 of the exchange words");
  static_assert(G * HD + sizeof(AttnCombine<HD, G, 4>) / 4 <= 4096, "combine states fit in the input stage");
  // Two LDS arrays: the compiler then knows that the copies to kv do not
  // write the input stage, and does not make the input's wait also wait for
  // them.
  __shared__ f32x4 xs[1024];           // GEMV input (K = 4096), then q + combine states
  __shared__ u32x4 kv[2 * CH * LPR];   // keys [CH][LPR], then values [CH][LPR]
  __shared__ float red[NW];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int b = blockIdx.x, cls = b & 7, idx = b >> 3;
  const int S = a.at.t.S;
  const int kvh = cls + 8 * (idx / S), si = idx % S;
  const unsigned epoch = a.class_epochs[cls];
  const int kin = lane / LPR, ch = lane % LPR;

  // 1. the split's cached keys and values to LDS, copied by waves 4-7 while
  // waves 0-3 load and stage the GEMV input, before any weight is requested
  // (keys past the split repeat its last key and are masked; the new
  // position's slot is replaced in 3.; an empty split copies its first
  // in-range key, unused)
  constexpr int NS = 4, UC = UKV * NW / (NW - NS);  // input-staging waves; copies per copying wave
  auto copy_kv = [&](int pos) {
    if (wave < NS) return;
    const AttnSpan sp = attn_span<HD>(a.at.t, si, kvh, pos);
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int t0 = (wave - NS + u * (NW - NS)) * KPW;
      const size_t off = static_cast<size_t>(max(0, min(t0 + kin, sp.nk - 1))) * sp.key_stride;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(sp.Kb + off),
                                       (__attribute__((address_space(3))) void*)(kv + t0 * LPR), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(sp.Vb + off),
                                       (__attribute__((address_space(3))) void*)(kv + (CH + t0) * LPR), 16, 0, 0);
    }
  };

  // 2. QKV
  GemvArgs ga = a.g;
  ga.tag = epoch;
  int p0;
  float bv = 0.f;
  int bi = 0;
  if (!gemv_run<kEpiQKVX, 2, 8, 2, THREADS, false, IN, 1, decltype(copy_kv), NS * kWave>(
          ga, xs, red, b * NW + wave, gridDim.x * NW, p0, bv, bi, copy_kv))
    return;  // the host never launches a step on a full cache
  const AttnSpan sp = attn_span<HD>(a.at.t, si, kvh, p0);

  // 3. every copy of step 1 has landed (a wave's loads complete in issue
  // order, and each wave has waited for its weights, requested after its
  // copies) and the input stage is free
  lds_barrier();
  float* qs = reinterpret_cast<float*>(xs);  // [G][HD]
  constexpr int NA = 4, UA = UKV * NW / NA;  // waves that attend (all keys), loads of each
  AttnCombine<HD, G, NA>& cb = *reinterpret_cast<AttnCombine<HD, G, NA>*>(qs + G * HD);
  const bool has_p = sp.nk > 0 && p0 < sp.k0 + sp.nk;  // the split holds the new position (its last key)
  SPoll poll{a.at.abort, 0u};
  {
    // wave w reads tagged words 128 w .. 128 w + 127 of the kv head's
    // [G queries][key][value]: waves 0 .. G-1 the queries, G and G+1 the key
    // and value (only where they are needed)
    const int nwaves = has_p ? G + 2 : G;
    if (wave < nwaves) {
      const rsrc_t rx = rsrc_of(a.g.qkvx + static_cast<size_t>(kvh) * (G + 2) * HD, (G + 2) * HD * 8);
      const int wo = (wave * kWave + lane) * 16;
      u32x4 v = ld_t2(rx, wo, 0);
      bool st = stale2(v, epoch);
      while (__any(st)) {
        if (!poll.next(lane)) break;
        const u32x4 nv = ld_t2(rx, st ? wo : 0x40000000, 0);
        if (st) v = nv;
        st = st && stale2(v, epoch);
      }
      const int e = 2 * (wave * kWave + lane);  // word index in the kv head's block
      if (e < G * HD) {
        qs[e] = __uint_as_float(v[0]);
        qs[e + 1] = __uint_as_float(v[2]);
      } else {
        const int d = (e - G * HD) % HD;
        const bool is_v = e >= (G + 1) * HD;
        half_t* row = reinterpret_cast<half_t*>(kv + ((is_v ? CH : 0) + (p0 - sp.k0)) * LPR);
        row[d] = static_cast<half_t>(__uint_as_float(v[0]));
        row[d + 1] = static_cast<half_t>(__uint_as_float(v[2]));
      }
    }
  }
  lds_barrier();
  float qr[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[g][i] = qs[g * HD + ch * 8 + i] * a.at.t.scale_log2;
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }
  if (wave < NA && sp.nk > 0) {
    AttnLoads<UA> ld;
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int t = (wave + u * NA) * KPW + kin;
      ld.kk[u] = kv[t * LPR + ch];
      ld.vv[u] = kv[(CH + t) * LPR + ch];
    }
    attn_step<HD, G, UA, NA>(ld, wave, kin, sp.nk, qr, m, l, acc);
  }

  // 4. split state, merge
  attn_store_state<HD, G, NA, true>(m, l, acc, cb, a.at.part, a.at.n_kv, a.at.S_max, kvh, si, epoch);
  if (wave == 0) {
    attn_merge_share<HD, G, false>(a.at.part, a.at.o, a.at.n_kv, a.at.S_max, kvh, si, S, epoch, epoch, poll, lane);
    if (has_p && kvh == cls && lane == 0) a.class_epochs[cls] = epoch + 1 == 0 ? 1u : epoch + 1;
  }
}

// ------------------------------------------------------------- utilities

// Weight repack. Mode 0 (QKV): packed unit u (lane-major: per lane, its q
// heads, then k heads, then v heads) holds rows (dim c, dim c + hd/2) at
// packed rows (2c, 2c+1), so a rotary pair lands in one wave. Mode 1
// (gate/up): packed row 2j = gate j, 2j+1 = up j.
struct RepackArgs {
  half_t* dst;
  const half_t* src;
  int rows, K, mode;
  int hd, n_q, n_kv, qpl, kpl, ffn;
};

__device__ __forceinline__ int repack_src_row(const RepackArgs& a, int r) {
  if (a.mode == 1) return (r & 1) ? a.ffn + (r >> 1) : (r >> 1);
  const int u = r / a.hd, i = r % a.hd;
  const int dim = (i & 1) ? (a.hd >> 1) + (i >> 1) : (i >> 1);
  const int upl = a.qpl + 2 * a.kpl;
  const int ln = u / upl, j = u % upl;
  if (j < a.qpl) return (ln * a.qpl + j) * a.hd + dim;
  if (j < a.qpl + a.kpl) return (a.n_q + ln * a.kpl + (j - a.qpl)) * a.hd + dim;
  return (a.n_q + a.n_kv + ln * a.kpl + (j - a.qpl - a.kpl)) * a.hd + dim;
}

__global__ __launch_bounds__(kBlock) void k_repack(RepackArgs a) {
  const int r = blockIdx.x;
  if (r >= a.rows) return;
  const int sr = repack_src_row(a, r);
  const u32x4* s = reinterpret_cast<const u32x4*>(a.src + static_cast<size_t>(sr) * a.K);
  u32x4* d = reinterpret_cast<u32x4*>(a.dst + static_cast<size_t>(r) * a.K);
  for (int c = threadIdx.x; c < (a.K >> 3); c += kBlock) d[c] = s[c];
}

// The XCD each workgroup runs on (hardware register XCC_ID, bits 3:0).
__global__ void k_xcd_ids(unsigned* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 0xFu;
}

__global__ void k_fill_u32(unsigned* p, unsigned v, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// Start a step with an explicit token, or set the length (d_token == null).
// After a length change the greedy token of position len may be recorded as
// token len+1 again (positions past len are discarded). abort (if not null):
// the model's give-up flag, cleared.
__global__ void k_set_pos(int32_t* state, int32_t* tokens, int32_t len, const int32_t* d_token, unsigned* abort) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  state[kLen] = len;
  if (abort) *abort = 0u;
  if (d_token) {
    tokens[len] = *d_token;
    state[kFedEnd] = len + 1;
  } else {
    state[kFedEnd] = min(state[kFedEnd], len + 1);
  }
}

// Copy n prompt tokens into the history at [len, len + n).
__global__ void k_put_tokens(int32_t* state, int32_t* tokens, int32_t len, const int32_t* src, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) tokens[len + i] = src[i];
  if (i == 0) {
    state[kLen] = len;
    state[kFedEnd] = len + n;
  }
}

// Streaming read of n 16-byte words (the practical HBM read ceiling):
// workgroup b reads its contiguous share of `per` words, each thread words
// i, i + 256, ... with non-temporal loads, 8 in flight, folded into one word
// that is stored only if it matches a value the data never produces (so the
// loads are kept).
__global__ __launch_bounds__(kBlock) void k_read_probe(const u32x4* __restrict__ p, size_t n, size_t per,
                                                        unsigned* sink) {
  const size_t b0 = static_cast<size_t>(blockIdx.x) * per, b1 = min(b0 + per, n);
  unsigned acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + 7 * kBlock < b1; i += 8 * kBlock) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld_stream(p + i + u * kBlock);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += kBlock) {
    const u32x4 v = ld_stream(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

__global__ void k_copy_out(float* dst, const float* src, int n, int32_t* argmax_dst, const int32_t* state) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
  if (i == 0 && argmax_dst) *argmax_dst = state[kArgmax];
}

}  // namespace lf
