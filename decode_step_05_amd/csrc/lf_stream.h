// One decode step in one cooperative launch, with the weights streamed
// through LDS ("stream" step kernel).
//
// A workgroup has kSW compute waves and one control wave. The compute waves
// only read weights and compute dot products: each streams its share of the
// step's GEMV weights (every layer's QKV, O, gate/up and down rows, then the
// LM head rows), 1 KB per wave instruction, with direct global-to-LDS loads
// into a private ring of RING slots, and keeps RING loads in flight across
// phase boundaries and grid barriers. Their results go to LDS.
// The control wave never has weight loads in flight, so its memory traffic is
// not queued behind them (vector memory operations retire in issue order): it
// stages each GEMV input into LDS (with RMSNorm), runs the epilogues (rotary
// embedding and KV append, residual adds, SwiGLU, logits and greedy argmax),
// makes every global store, and runs the grid barriers.
// Attention (one split work item per workgroup) is computed and stored by all
// waves: the compute waves' weight loads issued before it have landed by then,
// so waiting for their own stores costs them nothing.
//
// The weights of a GEMV phase are stored for this kernel in stream order:
// 1-KB slot j of compute wave gw at slot index j * kSTW + gw, so that
// neighbouring waves read neighbouring memory.
#pragma once
#include "lf_kernels.h"

namespace lf {

constexpr int kSW = 8;                        // compute waves per workgroup
constexpr int kSCtrl = kSW;                   // wave index of the control wave
constexpr int kSThreads = (kSW + 1) * kWave;  // threads per workgroup
constexpr int kSGrid = 256;                   // workgroups per launch
constexpr int kSTW = kSGrid * kSW;            // compute waves per launch
constexpr int kSResMax = 256;                 // GEMV rows per workgroup and phase, at most
constexpr int kSKMax = 8192;                  // GEMV input length, at most
constexpr int kSAttnU = 8;                    // K/V loads per lane and iteration of an attention item
constexpr int kSLdsMax = 160 * 1024;          // LDS per workgroup

enum SKind : int { kSQKV = 0, kSO = 1, kSGU = 2, kSDown = 3, kSLM = 4 };

// One GEMV phase of the weight stream.
struct SPhase {
  const u32x4* w;  // 16-byte piece `lane` of slot j of compute wave gw: w[(j * kSTW + gw) * 64 + lane]
  int rows, K;     // rows and input length of the matrix
  int kch, rpw;    // 1-KB slots per row (ceil(K / 512)), rows per compute wave
};

struct SLayer {
  const half_t *g1, *g2;  // RMSNorm gains before attention and before the FFN
  int window, S, chunk;   // attention window and split plan
};

struct StreamArgs {
  const SPhase* ph;       // [n_ph]: per layer QKV, O, gate/up, down; then the LM head
  const SLayer* layers;   // [L]
  int n_ph, L, d, qdim, ffn, vocab, hd, qpl, kpl, n_kv, max_ctx;
  float eps, scale_log2;
  const half_t *embed, *gf;
  const float2* rope;
  float *x, *q, *o, *act;
  float2* part_ml;
  float* part_acc;
  unsigned* attn_counters;  // [n_kv]
  unsigned long long* best;
  unsigned* bar;            // [0] barrier count, [1] exit count, [2] abort flag
  int32_t* state;
  int32_t* tokens;
  float* logits;
  half_t *kc, *vc;          // cache bases (layer l at l * layer_cache)
  size_t layer_cache;
  const float* x_in;        // hidden mode (vocab == 0)
  float* x_out;
};

template <int HD, int G>
struct SSmem {
  union {
    f32x4 xs[2 * (kSKMax / 8)];         // GEMV input, two planes
    AttnSmem<HD, G, kSW + 1> attn;
  };
  float res[kSResMax];                  // GEMV results of the workgroup's rows
  int flag;
};

template <int HD, int G>
constexpr int ssmem_bytes() {
  return static_cast<int>((sizeof(SSmem<HD, G>) + 1023) / 1024 * 1024);
}
// Ring slots per compute wave: what LDS leaves, at most 14.
template <int HD, int G>
constexpr int stream_ring() {
  const int r = (kSLdsMax - ssmem_bytes<HD, G>()) / (kSW * 1024);
  return r < 14 ? r : 14;
}
template <int HD, int G>
constexpr int stream_lds_bytes() {
  return ssmem_bytes<HD, G>() + kSW * stream_ring<HD, G>() * 1024;
}

// Wait until at most N vector memory operations of this wave are outstanding
// (they retire in issue order), and keep the compiler from moving memory
// accesses across the wait: the compiler does not track the LDS writes of
// global-to-LDS loads.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

// Wait until this wave's LDS reads have returned, and keep the compiler from
// moving a global-to-LDS load above the wait: such a load may write LDS before
// an earlier, still pending read of the same address has been served.
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("" ::: "memory");
}

// One wave copies 1 KB from global memory to LDS: lane i's 16 bytes land at
// dst + 16 i (dst is the same for all lanes).
__device__ __forceinline__ void dma_1k(const u32x4* src, u32x4* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
}

// Read a value of a table that no one writes during the launch through the
// constant address space: a wave-uniform address then gives scalar loads,
// which (unlike vector loads) do not wait behind the weight stream.
template <class T>
__device__ __forceinline__ T cload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}
__device__ __forceinline__ SPhase const_load(const SPhase* p) {
  SPhase r;
  r.w = cload(&p->w);
  r.rows = cload(&p->rows);
  r.K = cload(&p->K);
  r.kch = cload(&p->kch);
  r.rpw = cload(&p->rpw);
  return r;
}
__device__ __forceinline__ SLayer const_load(const SLayer* p) {
  SLayer r;
  r.g1 = cload(&p->g1);
  r.g2 = cload(&p->g2);
  r.window = cload(&p->window);
  r.S = cload(&p->S);
  r.chunk = cload(&p->chunk);
  return r;
}

// The weight stream of one compute wave: its slots of every phase in order;
// stream slot k goes to ring position k % RING. Past the end of the stream
// the last slot is loaded again, so that every consumed slot is followed by
// exactly one issue and RING loads are always in flight.
template <int RING>
struct SProducer {
  const SPhase* ph;
  const u32x4* w;
  u32x4* ring;
  int n_ph, phi, j, nsl, pos, gw, lane;

  __device__ __forceinline__ void init(const SPhase* phases, int n, int gw_, int lane_, u32x4* ring_) {
    ph = phases;
    n_ph = n;
    gw = gw_;
    lane = lane_;
    ring = ring_;
    phi = 0;
    j = 0;
    pos = 0;
    const SPhase p0 = const_load(ph);
    w = p0.w;
    nsl = p0.rpw * p0.kch;
  }

  __device__ __forceinline__ void issue() {
    dma_1k(w + (static_cast<size_t>(j) * kSTW + gw) * kWave + lane, ring + pos * kWave);
    pos = pos + 1 == RING ? 0 : pos + 1;
    if (++j == nsl) {
      if (phi + 1 < n_ph) {
        ++phi;
        const SPhase pn = const_load(ph + phi);
        w = pn.w;
        nsl = pn.rpw * pn.kch;
        j = 0;
      } else {
        j = nsl - 1;
      }
    }
  }
};

// Compute wave cw: the rows of phase P, slot by slot from the ring, each slot
// refilled with the stream slot RING ahead once read. Results go to
// res[cw * rpw + i].
template <int RING>
__device__ __forceinline__ void s_consume(const SPhase& P, SProducer<RING>& pr, const f32x4* xs, float* res, int cw,
                                          int lane, int& cpos, const u32x4* ring) {
  const int K8p = P.kch * kWave;  // offset of the second xs plane
  for (int i = 0; i < P.rpw; ++i) {
    float a0 = 0.f, a1 = 0.f;
    for (int c = 0; c < P.kch; ++c) {
      wait_vm<RING - 1>();
      const u32x4 wv = ring[cpos * kWave + lane];
      const f32x4 x0 = xs[c * kWave + lane], x1 = xs[K8p + c * kWave + lane];
      const h8 h = __builtin_bit_cast(h8, wv);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a0 = fmaf(static_cast<float>(h[t]), x0[t], a0);
        a1 = fmaf(static_cast<float>(h[4 + t]), x1[t], a1);
      }
      wait_lds_reads();  // the slot is read before its refill is issued
      pr.issue();
      cpos = cpos + 1 == RING ? 0 : cpos + 1;
    }
    const float out = wave_total(a0 + a1);
    if (lane == 0) res[cw * P.rpw + i] = out;
  }
}

// Control wave: stage a GEMV input of length K into xs as two planes (chunk
// q of 8 elements: elements 0-3 at xs[q], 4-7 at xs[kch*64 + q]), zero from K
// up to kch*512. With a gain: store x * gain and return the RMSNorm factor
// 1 / sqrt(mean(x^2) + eps), which the epilogue applies to the GEMV outputs
// (a scalar factor commutes with the matrix product); else store x, return 1.
// src: fp32 source, read with device-scope loads (written in this launch), or
// emb: an fp16 embedding row. resid_copy: also store this workgroup's slice
// of x there (the residual stream's first value).
__device__ __forceinline__ float s_stage(f32x4* xs, int K, int kch, const float* src, const half_t* emb,
                                         const half_t* gain, float eps, float* resid_copy, int lane) {
  const int K8p = kch * kWave;
  const int per = (K + gridDim.x - 1) / gridDim.x;
  const int s0 = blockIdx.x * per, s1 = min(s0 + per, K);
  float ss = 0.f;
  constexpr int B = 8;  // chunks per lane and batch of loads
  for (int i0 = 0; i0 < kch; i0 += B) {
    float v[B][8];
    u32x4 gn[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int el = min((lane + kWave * (i0 + b)) * 8, K - 8);  // clamped: loads stay in bounds
      if (emb) {
        unpack8(ld16(emb + el), v[b]);
      } else {
        const float2* s2 = reinterpret_cast<const float2*>(src + el);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float2 f = get_f32x2(s2 + t);
          v[b][2 * t] = f.x;
          v[b][2 * t + 1] = f.y;
        }
      }
      if (gain) gn[b] = ld16(gain + el);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = lane + kWave * (i0 + b);
      if (i0 + b >= kch) break;
      const bool valid = q * 8 < K;
      float g[8];
      if (gain) {
        unpack8(gn[b], g);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) g[t] = 1.f;
      }
      f32x4 o0, o1;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float x = valid ? v[b][t] : 0.f;
        ss = fmaf(x, x, ss);
        if (t < 4)
          o0[t] = x * g[t];
        else
          o1[t - 4] = x * g[t];
      }
      if (resid_copy && valid)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (q * 8 + t >= s0 && q * 8 + t < s1) put_f32(resid_copy + q * 8 + t, v[b][t]);
      xs[q] = o0;
      xs[K8p + q] = o1;
    }
  }
  if (!gain) return 1.f;
  ss = wave_total(ss);
  return 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
}

// Control wave: count this workgroup's arrival at the grid barrier once this
// wave's memory operations are acknowledged, and wait for the others. Every
// wait is bounded: on timeout the abort flag is raised. Returns false if the
// launch was aborted (uniform over the wave).
__device__ __forceinline__ bool s_grid_sync(unsigned* count, unsigned* abort, unsigned target, int lane) {
  __builtin_amdgcn_s_waitcnt(0);
  int ok = 1;
  if (lane == 0) {
    __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (unsigned spins = 0;; ++spins) {
      if (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        ok = 0;
        break;
      }
      if (spins >= (1u << 22)) {
        __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return __builtin_amdgcn_readfirstlane(ok) != 0;
}

// Largest packed (value, index) key over the wave (argmax_key order).
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned lo = __shfl_xor(static_cast<unsigned>(k), off);
    const unsigned hi = __shfl_xor(static_cast<unsigned>(k >> 32), off);
    const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}

template <int HD, int G>
__global__ __launch_bounds__(kSThreads) void k_stream(StreamArgs s) {
  constexpr int RING = stream_ring<HD, G>();
  static_assert(RING >= 4, "LDS leaves too few ring slots");
  extern __shared__ f32x4 s_lds[];
  SSmem<HD, G>& sm = *reinterpret_cast<SSmem<HD, G>*>(s_lds);
  u32x4* const ring_all = reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(s_lds) + ssmem_bytes<HD, G>());
  // wave index as a wave-uniform (scalar) value: the producer state derived
  // from it then stays in scalar registers and the phase table is read with
  // scalar loads, which do not queue behind the weight stream
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x & (kWave - 1);
  const bool ctrl = wave == kSCtrl;
  const int nb = gridDim.x;
  const bool hidden = s.vocab == 0;

  const int p = s.state[kLen];
  if (!(p < s.max_ctx && __hip_atomic_load(s.bar + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)) return;
  float* const resid = hidden ? s.x_out : s.x;
  u32x4* const ring = ring_all + (ctrl ? 0 : wave) * RING * kWave;

  SProducer<RING> pr;
  int cpos = 0;
  if (!ctrl) {
    pr.init(s.ph, s.n_ph, blockIdx.x * kSW + wave, lane, ring);
    for (int k = 0; k < RING; ++k) pr.issue();
  }

  unsigned nbar = 0;  // grid barriers passed (control wave)
  float rn = 1.f;     // RMSNorm factor of the current phase (control wave)

  // A GEMV phase: the control wave stages the input, the compute waves run
  // their rows, the control wave runs the epilogue and the grid barrier.
  auto gemv = [&](int phi, int kind, int l) -> bool {
    const SPhase P = const_load(s.ph + phi);
    const int n = kSW * P.rpw, r0 = blockIdx.x * n;
    float resv[kSResMax / kWave];
    if (ctrl) {
      const SLayer w = const_load(s.layers + (l < s.L ? l : s.L - 1));
      if (kind == kSQKV) {
        if (l == 0 && !hidden) {
          int tok = s.tokens[p];
          if (tok < 0 || tok >= s.vocab) {
            tok = tok < 0 ? 0 : s.vocab - 1;
            if (blockIdx.x == 0 && lane == 0) s.state[kBadToken] = 1;
          }
          rn = s_stage(sm.xs, P.K, P.kch, nullptr, s.embed + static_cast<size_t>(tok) * s.d, w.g1, s.eps, resid, lane);
        } else {
          rn = s_stage(sm.xs, P.K, P.kch, l == 0 ? s.x_in : resid, nullptr, w.g1, s.eps, l == 0 ? resid : nullptr,
                       lane);
        }
      } else if (kind == kSO) {
        rn = s_stage(sm.xs, P.K, P.kch, s.o, nullptr, nullptr, s.eps, nullptr, lane);
      } else if (kind == kSGU) {
        rn = s_stage(sm.xs, P.K, P.kch, resid, nullptr, w.g2, s.eps, nullptr, lane);
      } else if (kind == kSDown) {
        rn = s_stage(sm.xs, P.K, P.kch, s.act, nullptr, nullptr, s.eps, nullptr, lane);
      } else {
        rn = s_stage(sm.xs, P.K, P.kch, resid, nullptr, s.gf, s.eps, nullptr, lane);
      }
      if (kind == kSO || kind == kSDown)
#pragma unroll
        for (int k = 0; k < kSResMax / kWave; ++k) resv[k] = get_f32(resid + min(r0 + lane + kWave * k, P.rows - 1));
    }
    lds_barrier();
    if (!ctrl) s_consume<RING>(P, pr, sm.xs, sm.res, wave, lane, cpos, ring);
    lds_barrier();
    if (ctrl) {
      if (kind == kSQKV) {
        const QkvOut qo{s.q, s.kc + l * s.layer_cache, s.vc + l * s.layer_cache, s.rope, s.hd, s.qpl, s.kpl, s.max_ctx};
        for (int u = lane; 2 * u < n; u += kWave)
          if (r0 + 2 * u < P.rows) qkv_put(qo, r0 + 2 * u, sm.res[2 * u] * rn, sm.res[2 * u + 1] * rn, p);
      } else if (kind == kSGU) {
        for (int u = lane; 2 * u < n; u += kWave)
          if (r0 + 2 * u < P.rows) {
            const float g = sm.res[2 * u] * rn, up = sm.res[2 * u + 1] * rn;
            put_f32(s.act + ((r0 >> 1) + u), g / (1.0f + expf(-g)) * up);
          }
      } else if (kind == kSO || kind == kSDown) {
#pragma unroll
        for (int k = 0; k < kSResMax / kWave; ++k) {
          const int t = lane + kWave * k;
          if (t < n && r0 + t < P.rows) put_f32(resid + r0 + t, resv[k] + sm.res[t]);
        }
      } else {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int t = lane; t < n; t += kWave)
          if (r0 + t < P.rows) {
            const float z = sm.res[t] * rn;
            put_f32(s.logits + r0 + t, z);
            if (better(z, r0 + t, bv, bi)) {
              bv = z;
              bi = r0 + t;
            }
          }
        const unsigned long long key = wave_max_key(bi != 0x7fffffff ? argmax_key(bv, bi) : 0ull);
        if (lane == 0 && key) __hip_atomic_fetch_max(s.best, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const bool ok = s_grid_sync(s.bar, s.bar + 2, ++nbar * nb, lane);
      if (lane == 0) sm.flag = ok;
    }
    lds_barrier();
    return sm.flag != 0;
  };

  auto attention = [&](int l) -> bool {
    const SLayer w = const_load(s.layers + l);
    AttnArgs t{};
    t.q = s.q;
    t.kc = s.kc + l * s.layer_cache;
    t.vc = s.vc + l * s.layer_cache;
    t.state = s.state;
    t.part_ml = s.part_ml;
    t.part_acc = s.part_acc;
    t.o = s.o;
    t.counters = s.attn_counters;
    t.max_ctx = s.max_ctx;
    t.window = w.window;
    t.S = w.S;
    t.chunk = w.chunk;
    t.kpl = s.kpl;
    t.scale_log2 = s.scale_log2;
    const int items = w.S * s.n_kv;
    for (int it = blockIdx.x; it < items; it += nb)
      attn_item<HD, G, kSAttnU, kSW + 1, true>(t, sm.attn, it % w.S, it / w.S, p);
    if (ctrl) {
      const bool ok = s_grid_sync(s.bar, s.bar + 2, ++nbar * nb, lane);
      if (lane == 0) sm.flag = ok;
    }
    lds_barrier();
    return sm.flag != 0;
  };

  bool alive = true;
  for (int l = 0; l < s.L && alive; ++l) {
    alive = gemv(4 * l, kSQKV, l) && attention(l) && gemv(4 * l + 1, kSO, l) && gemv(4 * l + 2, kSGU, l) &&
            gemv(4 * l + 3, kSDown, l);
  }
  if (alive && !hidden) alive = gemv(4 * s.L, kSLM, s.L);

  // ---- step end (control wave of workgroup 0): greedy token, position
  if (alive && blockIdx.x == 0 && threadIdx.x == kSCtrl * kWave) {
    if (!hidden) {
      const unsigned long long key = __hip_atomic_load(s.best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int i = key ? argmax_index(key) : 0;  // key == 0 only if every logit is NaN
      if (i < 0 || i >= s.vocab) i = 0;
      s.state[kArgmax] = i;
      if (p + 1 >= s.state[kFedEnd]) s.tokens[p + 1] = i;
      __hip_atomic_store(s.best, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s.state[kLen] = p + 1;
  }
  // No global-to-LDS copy may land after the workgroup has ended.
  if (!ctrl) wait_vm<0>();
  // Leave: the last workgroup out resets the barrier counters for the next launch.
  lds_barrier();
  if (threadIdx.x == kSCtrl * kWave) {
    const unsigned prev = __hip_atomic_fetch_add(s.bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == static_cast<unsigned>(nb) - 1) {
      __hip_atomic_store(s.bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(s.bar + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Copy a row-major fp16 matrix [rows][K] (K a multiple of 8) into stream
// order: 16-byte piece `lane` of slot j of compute wave gw holds elements
// [c*512 + 8*lane, +8) of row r, where j = i*kch + c and
// r = (gw / kSW) * kSW * rpw + (gw % kSW) * rpw + i; zero past rows or K.
__global__ void k_stream_repack(const half_t* __restrict__ src, int rows, int K, int kch, int rpw,
                                u32x4* __restrict__ dst, size_t n_pieces) {
  for (size_t t = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n_pieces;
       t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int lane = static_cast<int>(t % kWave);
    const size_t sw = t / kWave;
    const int gw = static_cast<int>(sw % kSTW), j = static_cast<int>(sw / kSTW);
    const int i = j / kch, c = j % kch;
    const int r = (gw / kSW) * kSW * rpw + (gw % kSW) * rpw + i;
    const int e = c * 512 + lane * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows && e < K) v = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(r) * K + e);
    dst[t] = v;
  }
}

}  // namespace lf
