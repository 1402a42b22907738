// One decode step in one cooperative launch ("persistent" step kernel).
//
// The workgroups of the launch (all co-resident) run the step's phases in
// order, separated by grid barriers:
//   per layer: QKV (+ RMSNorm, rotary, KV append) | attention (+ split merge)
//              | O + residual | gate/up (+ RMSNorm, SwiGLU) | down + residual
//   then:      LM head (+ final RMSNorm, per-workgroup argmax) | step end.
// Weights do not depend on the previous phase, so before a workgroup waits at
// a barrier its waves issue the loads of their first two row groups of the
// next GEMV: HBM keeps streaming while the barrier resolves, which is the
// point of this kernel compared to one launch per phase.
//
// Cross-workgroup data is written with device-scope stores and read with
// device-scope loads; before arriving at a barrier a wave waits until its
// stores are acknowledged. The barrier counter grows monotonically within a
// launch; the last workgroup to leave resets it. Every spin is bounded: on
// timeout an abort flag is raised and all workgroups leave, so the launch
// always drains.
#pragma once
#include "lf_kernels.h"

namespace lf {

constexpr int kStepWaves = 8;                    // waves per workgroup
constexpr int kStepThreads = kStepWaves * kWave;
constexpr unsigned kSpinLimit = 1u << 22;        // polls before a barrier gives up

struct LayerW {
  const half_t *wqkv, *wo, *wgu, *wd, *g1, *g2;
  int window, S, chunk;
};

struct StepArgs {
  const LayerW* layers;     // device array [L]
  int L, d, qkv_rows, qdim, ffn, vocab, hd, qpl, kpl, n_kv, max_ctx;
  float eps, scale_log2;
  const half_t *embed, *lm, *gf;
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

struct Barrier {
  unsigned* count;
  unsigned* abort;
  unsigned nb, k;
  int* flag;  // LDS

  // All threads call this after their phase's stores were acknowledged.
  // Returns false if the launch was aborted.
  __device__ __forceinline__ bool sync() {
    ++k;
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned target = k * nb;
      __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int ok = 1;
      for (unsigned spins = 0;; ++spins) {
        if (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
        if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          ok = 0;
          break;
        }
        if (spins >= kSpinLimit) {
          __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      *flag = ok;
    }
    __syncthreads();
    return *flag != 0;
  }
};

// A GEMV phase: the first two row groups of each wave are issued by
// prefetch() (before the preceding barrier), run() stages the input and
// streams the rest, keeping two groups in flight.
template <int EPI, int NR, int KCH>
struct GemvPhase {
  Rows<NR, KCH> buf[2];

  __device__ __forceinline__ void prefetch(const GemvArgs& a, int gw, int TW) {
    const int lane = threadIdx.x & (kWave - 1);
    const int ng = (a.rows + NR - 1) / NR;
    const float* res = EPI == kEpiResid ? a.y : nullptr;
    issue_rows<NR, KCH>(buf[0], a.W, min(gw, ng - 1) * NR, a.rows, a.K, lane, res);
    issue_rows<NR, KCH>(buf[1], a.W, min(gw + TW, ng - 1) * NR, a.rows, a.K, lane, res);
  }

  __device__ __forceinline__ void run(const GemvArgs& a, f32x4* xs, float* red, int gw, int TW, int p, float& bv,
                                      int& bi) {
    constexpr int KMAX = KCH * kWave * 8;
    const int lane = threadIdx.x & (kWave - 1);
    const int ng = (a.rows + NR - 1) / NR;
    const float* res = EPI == kEpiResid ? a.y : nullptr;
    const bool full = a.K == KMAX;
    {
      Stage<kStepThreads, KMAX> st;
      stage_load<kStepThreads, KMAX, true>(st, a, p);
      stage_store<kStepThreads, KMAX>(st, a, xs, red);
    }
    // two buffers, statically indexed (a runtime index would spill them)
    int g = gw;
    while (g < ng) {
      step_group(a, buf[0], xs, g, full, lane, p, bv, bi);
      if (g + 2 * TW < ng) issue_rows<NR, KCH>(buf[0], a.W, (g + 2 * TW) * NR, a.rows, a.K, lane, res);
      g += TW;
      if (g >= ng) break;
      step_group(a, buf[1], xs, g, full, lane, p, bv, bi);
      if (g + 2 * TW < ng) issue_rows<NR, KCH>(buf[1], a.W, (g + 2 * TW) * NR, a.rows, a.K, lane, res);
      g += TW;
    }
  }

  __device__ __forceinline__ void step_group(const GemvArgs& a, const Rows<NR, KCH>& b, const f32x4* xs, int g,
                                             bool full, int lane, int p, float& bv, int& bi) {
    if (full)
      finish_rows<EPI, NR, KCH, true>(a, b, xs, g * NR, lane, p, bv, bi);
    else
      finish_rows<EPI, NR, KCH, false>(a, b, xs, g * NR, lane, p, bv, bi);
  }
};

template <int HD, int G, int KCH_D, int KCH_F>
struct StepSmem {
  union {
    f32x4 xs[(KCH_F > KCH_D ? KCH_F : KCH_D) * kWave * 2];  // GEMV input, two planes
    AttnSmem<HD, G, kStepWaves> attn;
  };
  float red[kStepWaves];
  float2 wbest[kStepWaves];
  int flag;
};

// KCH_D: 16-byte chunks per lane covering d_model and n_q_heads*head_dim;
// KCH_F: covering ffn.
template <int HD, int G, int KCH_D, int KCH_F>
__global__ __launch_bounds__(kStepThreads) void k_step(StepArgs s) {
  __shared__ StepSmem<HD, G, KCH_D, KCH_F> sm;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int nb = gridDim.x;
  const int gw = blockIdx.x * kStepWaves + wave, TW = nb * kStepWaves;
  Barrier bar{s.bar, s.bar + 2, static_cast<unsigned>(nb), 0u, &sm.flag};
  const bool hidden = s.vocab == 0;

  const int p = s.state[kLen];
  const bool run = p < s.max_ctx && __hip_atomic_load(s.bar + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
  float* resid = hidden ? s.x_out : s.x;

  GemvArgs base{};
  base.eps = s.eps;
  base.vocab = s.vocab;
  base.state = s.state;
  base.tokens = s.tokens;
  base.max_ctx = s.max_ctx;
  base.hd = s.hd;
  base.qpl = s.qpl;
  base.kpl = s.kpl;
  base.rope = s.rope;

  auto qkv_args = [&](int l) {
    GemvArgs a = base;
    const LayerW& w = s.layers[l];
    a.W = w.wqkv;
    a.rows = s.qkv_rows;
    a.K = s.d;
    a.gain = w.g1;
    if (l == 0) {
      a.in_kind = hidden ? kInNormF32 : kInNormEmbed;
      a.x = s.x_in;
      a.emb = s.embed;
      a.resid_copy = resid;
    } else {
      a.in_kind = kInNormF32;
      a.x = resid;
    }
    a.q = s.q;
    a.kc = s.kc + l * s.layer_cache;
    a.vc = s.vc + l * s.layer_cache;
    return a;
  };
  auto o_args = [&](int l) {
    GemvArgs a = base;
    a.W = s.layers[l].wo;
    a.rows = s.d;
    a.K = s.qdim;
    a.in_kind = kInF32;
    a.x = s.o;
    a.y = resid;
    return a;
  };
  auto gu_args = [&](int l) {
    GemvArgs a = base;
    a.W = s.layers[l].wgu;
    a.rows = 2 * s.ffn;
    a.K = s.d;
    a.in_kind = kInNormF32;
    a.x = resid;
    a.gain = s.layers[l].g2;
    a.y = s.act;
    return a;
  };
  auto down_args = [&](int l) {
    GemvArgs a = base;
    a.W = s.layers[l].wd;
    a.rows = s.d;
    a.K = s.ffn;
    a.in_kind = kInF32;
    a.x = s.act;
    a.y = resid;
    return a;
  };
  auto lm_args = [&]() {
    GemvArgs a = base;
    a.W = s.lm;
    a.rows = s.vocab;
    a.K = s.d;
    a.in_kind = kInNormF32;
    a.x = resid;
    a.gain = s.gf;
    a.y = s.logits;
    return a;
  };

  // Wait until this wave's stores (and loads) are acknowledged, before the
  // next phase's prefetch is issued and the barrier is entered.
  auto stores_done = [&]() { __builtin_amdgcn_s_waitcnt(0); };

  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool alive = run;
  // The loop is rotated so that no prefetched buffer is carried across its
  // back edge (a carried buffer holds registers in every phase):
  //   QKV(0) | for l: attention(l) O(l) gate/up(l) down(l) then QKV(l+1) or LM head
  if (alive) {
    GemvPhase<kEpiQKV, 2, KCH_D> ph;
    ph.prefetch(qkv_args(0), gw, TW);
    ph.run(qkv_args(0), sm.xs, sm.red, gw, TW, p, bv, bi);
    stores_done();
    alive = bar.sync();
  }
  for (int l = 0; l < s.L && alive; ++l) {
    // ---- attention: work items (split, kv head) over the workgroups.
    // 8 waves x 4 loads cover the same 128 keys (head_dim 128) as the
    // attention kernel's 4 waves x 8 loads, so the split plan is shared.
    {
      const LayerW& w = s.layers[l];
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
      for (int it = blockIdx.x; it < items; it += nb) attn_item<HD, G, 4, kStepWaves, true>(t, sm.attn, it % w.S, it / w.S, p);
    }
    stores_done();
    {
      GemvPhase<kEpiResid, 1, KCH_D> ph;
      ph.prefetch(o_args(l), gw, TW);
      if (!(alive = bar.sync())) break;
      // ---- O projection + residual
      ph.run(o_args(l), sm.xs, sm.red, gw, TW, p, bv, bi);
    }
    stores_done();
    {
      GemvPhase<kEpiSwiGLU, 2, KCH_D> ph;
      ph.prefetch(gu_args(l), gw, TW);
      if (!(alive = bar.sync())) break;
      // ---- gate/up (+ RMSNorm, SwiGLU)
      ph.run(gu_args(l), sm.xs, sm.red, gw, TW, p, bv, bi);
    }
    stores_done();
    {
      GemvPhase<kEpiResid, 1, KCH_F> ph;
      ph.prefetch(down_args(l), gw, TW);
      if (!(alive = bar.sync())) break;
      // ---- down + residual
      ph.run(down_args(l), sm.xs, sm.red, gw, TW, p, bv, bi);
    }
    stores_done();
    if (l + 1 < s.L) {
      // ---- QKV of the next layer (+ RMSNorm, rotary, KV append)
      GemvPhase<kEpiQKV, 2, KCH_D> ph;
      ph.prefetch(qkv_args(l + 1), gw, TW);
      if (!(alive = bar.sync())) break;
      ph.run(qkv_args(l + 1), sm.xs, sm.red, gw, TW, p, bv, bi);
      stores_done();
      alive = bar.sync();
    } else if (!hidden) {
      // ---- final RMSNorm + LM head + greedy argmax
      GemvPhase<kEpiLogits, 1, KCH_D> ph;
      ph.prefetch(lm_args(), gw, TW);
      if (!(alive = bar.sync())) break;
      ph.run(lm_args(), sm.xs, sm.red, gw, TW, p, bv, bi);
      if (lane == 0) sm.wbest[wave] = make_float2(bv, __int_as_float(bi));
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int w = 1; w < kStepWaves; ++w) {
          const int wi = __float_as_int(sm.wbest[w].y);
          if (better(sm.wbest[w].x, wi, bv, bi)) {
            bv = sm.wbest[w].x;
            bi = wi;
          }
        }
        if (bi != 0x7fffffff)
          __hip_atomic_fetch_max(s.best, argmax_key(bv, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      stores_done();
      alive = bar.sync();
    } else {
      alive = bar.sync();
    }
  }
  // ---- step end (workgroup 0): greedy token, position
  if (alive && blockIdx.x == 0 && threadIdx.x == 0) {
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
  // Leave: the last workgroup out resets the barrier counters for the next launch.
  if (run) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned prev = __hip_atomic_fetch_add(s.bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == static_cast<unsigned>(nb) - 1) {
        __hip_atomic_store(s.bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(s.bar + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace lf
