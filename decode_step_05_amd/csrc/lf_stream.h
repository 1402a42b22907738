// One decode step in one cooperative launch, with the weights streamed
// through LDS ("stream" step kernel).
//
// A workgroup has kSW compute waves and one control wave.
// The compute waves only read weights and compute dot products: each streams
// its share of the step's GEMV weights (every layer's QKV, O, gate/up and down
// rows, then the LM head rows), 1 KB per wave instruction, with direct
// global-to-LDS loads into a private ring of RING slots, and keeps RING loads
// in flight across phase boundaries. Their results go to LDS. They also run
// the attention math of the workgroup's work item, on K/V rows they load
// before the item's queries exist.
// The control wave never has weight loads in flight, so its memory traffic is
// not queued behind them (vector memory operations retire in issue order): it
// waits for and stages each GEMV input into LDS, runs the epilogues (RMSNorm
// scale, rotary embedding and KV append, residual adds, SwiGLU, logits and
// greedy argmax, attention split merge) and makes the global stores.
//
// Workgroups exchange data without grid barriers: every value another
// workgroup reads is stored as one 64-bit word (fp32 value, 32-bit tag), the
// tag naming the launch and the producing phase, and the reader polls until
// all it needs carries the expected tag. A buffer is rewritten only after
// every workgroup has consumed it: each phase needs the outputs of all
// workgroups of the phase before, which they produce only after reading their
// own inputs of the buffer's previous version.
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
constexpr int kSAttnU = 4;                    // K/V loads per lane and iteration of an attention item
constexpr int kSLdsMax = 160 * 1024;          // LDS per workgroup
constexpr int kSTagsPerLayer = 6;             // tag slots per layer (STag)
constexpr unsigned kSTagsPerLaunch = 512;     // tag slots per launch (layers <= 64)

enum SKind : int { kSQKV = 0, kSO = 1, kSGU = 2, kSDown = 3, kSLM = 4 };
// Producing phases, for tags.
enum STag : int { kTQKV = 0, kTPart = 1, kTAtt = 2, kTO = 3, kTGU = 4, kTDown = 5 };

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
  int n_ph, L, d, qdim, ffn, vocab, hd, qpl, kpl, n_kv, max_ctx, S_max;
  float eps, scale_log2;
  const half_t *embed, *gf;
  const float2* rope;
  // tagged exchange buffers (value, tag)
  u64* xt;     // [d] residual stream after each O and down phase
  u64* qt;     // [qdim] rotated queries
  u64* kvt;    // [2][n_kv][hd] rotated key and value at p, rounded to fp16
  u64* ot;     // [qdim] attention output
  u64* actt;   // [ffn] SwiGLU activation
  u64* partt;  // [n_q][S_max][hd + 2] split partial states: output, running max (log2 units), denominator
  unsigned long long* best;
  unsigned* bar;           // [1] exit count, [2] abort flag, [3] launch epoch (>= 1), [4] LM arrivals
  int32_t* state;
  int32_t* tokens;
  float* logits;
  half_t *kc, *vc;         // cache bases (layer l at l * layer_cache)
  size_t layer_cache;
  const float* x_in;       // hidden mode (vocab == 0)
  float* x_out;
};

// LDS of a workgroup (the weight rings follow it).
template <int HD, int G>
struct SSmem {
  static constexpr int KPW = kWave / (HD / 8);  // keys per wave load
  union {
    f32x4 xs[2 * (kSKMax / 8)];  // GEMV input, two planes
    struct {
      float acc[kSW][KPW][G][HD];
      float2 ml[kSW][KPW][G];
    } at;                        // attention: per-row-group softmax states
  };
  float q[G][HD];                // attention: scaled queries of the work item
  float kv_new[2][HD];           // attention: key and value at p
  float comb[G][HD];             // attention: combined state of the workgroup
  float2 comb_ml[G];
  float res[kSResMax];           // GEMV results of the workgroup's rows
  float resid[kSResMax];         // the residual stream rows the workgroup's O and down phases produce
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

// ---- tagged exchange (control wave)

__device__ __forceinline__ unsigned stag(unsigned epoch, int l, int kind) {
  return epoch * kSTagsPerLaunch + static_cast<unsigned>(l * kSTagsPerLayer + kind);
}

// Control wave: wait until the K tagged values src[0..K) carry `tag` and
// stage them into xs as two planes (chunk q of 8 elements: elements 0-3 at
// xs[q], 4-7 at xs[kch*64 + q]), zero from K up to kch*512. With a gain
// (loaded first, while the producers may still be running): xs = x * gain and
// rn = 1 / sqrt(mean(x^2) + eps), the RMSNorm factor the epilogue applies to
// the GEMV outputs (a scalar factor commutes with the matrix product); else
// xs = x and rn = 1. Returns false if the launch was aborted.
__device__ __forceinline__ bool s_stage_t(f32x4* xs, int K, int kch, const u64* src, unsigned tag,
                                          const half_t* gain, float eps, float& rn, SPoll& poll, int lane) {
  const int K8p = kch * kWave;
  if (gain)
    for (int b = 0; b < kch; ++b) {
      const int q = lane + kWave * b;
      float g[8];
      unpack8(ld16(gain + min(q * 8, K - 8)), g);
      xs[q] = f32x4{g[0], g[1], g[2], g[3]};
      xs[K8p + q] = f32x4{g[4], g[5], g[6], g[7]};
    }
  const rsrc_t r = rsrc_of(src, K * 8);
  float ss = 0.f;
  constexpr int B = 6;  // chunks per batch: 24 loads of 16 bytes per lane
  // chunk q = lane + 64 (i0 + b) holds bytes 64 q .. 64 q + 63
  const int voff = lane * 64;
  for (int i0 = 0; i0 < kch; i0 += B) {
    u32x4 d[B][4];
    unsigned stale = 0;
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) d[b][j] = ld_t2(r, voff, (i0 + b) * kWave * 64 + 16 * j);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + b < kch && (lane + kWave * (i0 + b)) * 8 < K && stale2(d[b][j], tag)) stale |= 1u << (4 * b + j);
    while (__any(stale != 0)) {
      if (!poll.next(lane)) return false;
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (stale & (1u << (4 * b + j))) d[b][j] = ld_t2(r, voff, (i0 + b) * kWave * 64 + 16 * j);
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if ((stale & (1u << (4 * b + j))) && !stale2(d[b][j], tag)) stale &= ~(1u << (4 * b + j));
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (i0 + b >= kch) break;
      const int q = lane + kWave * (i0 + b);
      const bool valid = q * 8 < K;
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = valid ? __uint_as_float(d[b][j][0]) : 0.f;
        v[2 * j + 1] = valid ? __uint_as_float(d[b][j][2]) : 0.f;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) ss = fmaf(v[t], v[t], ss);
      f32x4 o0 = f32x4{v[0], v[1], v[2], v[3]}, o1 = f32x4{v[4], v[5], v[6], v[7]};
      if (gain) {
        o0 *= xs[q];
        o1 *= xs[K8p + q];
      }
      xs[q] = o0;
      xs[K8p + q] = o1;
    }
  }
  rn = gain ? 1.0f / sqrtf(wave_total(ss) / static_cast<float>(K) + eps) : 1.f;
  return true;
}

// Control wave: stage an fp32 vector written before the launch (the layer-0
// input: an embedding row or the hidden-mode input), as s_stage_t does.
__device__ __forceinline__ void s_stage_plain(f32x4* xs, int K, int kch, const float* x, const half_t* emb,
                                              const half_t* gain, float eps, float& rn, int lane) {
  const int K8p = kch * kWave;
  float ss = 0.f;
  for (int b = 0; b < kch; ++b) {
    const int q = lane + kWave * b;
    const int e = min(q * 8, K - 8);
    const bool valid = q * 8 < K;
    float v[8], g[8];
    if (emb) {
      unpack8(ld16(emb + e), v);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(x + e), c = *reinterpret_cast<const f32x4*>(x + e + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] = a[t];
        v[4 + t] = c[t];
      }
    }
    if (gain) {
      unpack8(ld16(gain + e), g);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) g[t] = 1.f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      v[t] = valid ? v[t] : 0.f;
      ss = fmaf(v[t], v[t], ss);
    }
    xs[q] = f32x4{v[0] * g[0], v[1] * g[1], v[2] * g[2], v[3] * g[3]};
    xs[K8p + q] = f32x4{v[4] * g[4], v[5] * g[5], v[6] * g[6], v[7] * g[7]};
  }
  rn = gain ? 1.0f / sqrtf(wave_total(ss) / static_cast<float>(K) + eps) : 1.f;
}

// Control wave: wait for n tagged values at src (n even, 16-byte aligned) and
// store them to dst[i] * scale (LDS). Returns false if aborted.
__device__ __forceinline__ bool s_fetch_t(float* dst, const u64* src, int n, unsigned tag, float scale, SPoll& poll,
                                          int lane) {
  const rsrc_t r = rsrc_of(src, n * 8);
  const int voff = lane * 16;
  for (int i0 = 0; i0 < n; i0 += 2 * kWave * 8) {  // 8 loads of two values per lane per round
    u32x4 d[8];
    unsigned stale = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = i0 + 2 * (lane + kWave * u);
      d[u] = ld_t2(r, voff, (i0 + 2 * kWave * u) * 8);
      if (e < n && stale2(d[u], tag)) stale |= 1u << u;
    }
    while (__any(stale != 0)) {
      if (!poll.next(lane)) return false;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (stale & (1u << u)) {
          d[u] = ld_t2(r, voff, (i0 + 2 * kWave * u) * 8);
          if (!stale2(d[u], tag)) stale &= ~(1u << u);
        }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = i0 + 2 * (lane + kWave * u);
      if (e < n) {
        dst[e] = __uint_as_float(d[u][0]) * scale;
        dst[e + 1] = __uint_as_float(d[u][2]) * scale;
      }
    }
  }
  return true;
}

// Store the rotary pair of QKV rows (r, r+1) (lane-major order, see qkv_put):
// q to qt; k and v appended to the cache (fp16) and, rounded to fp16, to kvt.
__device__ __forceinline__ void qkv_put_t(const StreamArgs& s, rsrc_t rq, rsrc_t rkv, int l, int r, float y0, float y1,
                                          int p, unsigned tag) {
  const int hd = s.hd, half_hd = hd >> 1, upl = s.qpl + 2 * s.kpl;
  const int u = r / hd, c = (r % hd) >> 1;
  const int ln = u / upl, j = u % upl;
  if (j < s.qpl + s.kpl) {
    const float2 cs = s.rope[static_cast<size_t>(p) * half_hd + c];
    const float t0 = y0 * cs.x - y1 * cs.y;
    const float t1 = y0 * cs.y + y1 * cs.x;
    y0 = t0;
    y1 = t1;
  }
  if (j < s.qpl) {
    const int qh = (ln * s.qpl + j) * hd;
    put_t(rq, qh + c, y0, tag);
    put_t(rq, qh + c + half_hd, y1, tag);
  } else {
    const bool is_k = j < s.qpl + s.kpl;
    const int h = is_k ? j - s.qpl : j - s.qpl - s.kpl;
    const int kvh = ln * s.kpl + h;
    half_t* dst = (is_k ? s.kc : s.vc) + l * s.layer_cache + ((static_cast<size_t>(ln) * s.max_ctx + p) * s.kpl + h) * hd;
    const half_t h0 = static_cast<half_t>(y0), h1 = static_cast<half_t>(y1);
    put_f16(dst + c, y0);
    put_f16(dst + c + half_hd, y1);
    const int kv = ((is_k ? 0 : s.n_kv) + kvh) * hd;
    put_t(rkv, kv + c, static_cast<float>(h0), tag);
    put_t(rkv, kv + c + half_hd, static_cast<float>(h1), tag);
  }
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

// ---- attention (one work item per workgroup)

// Compute waves: the softmax-weighted sums over the work item's keys for its
// G query heads, as attn_item computes them, with the queries and the key and
// value at p taken from LDS (the cache slot at p is not read in this launch)
// and the first iteration's K/V loads issued beforehand (pre). Leaves each
// row group's state in sm.at.
template <int HD, int G, int U>
__device__ __forceinline__ void s_attn_rows(const AttnArgs& a, SSmem<HD, G>& sm, int s, int kvh, int p,
                                           const AttnLoads<U>& pre, int wave, int lane) {
  constexpr int LPR = HD / 8, KPW = kWave / LPR, NW = kSW;
  const int kin = lane / LPR, ch = lane % LPR;
  const AttnSpan sp = attn_span<HD>(a, s, kvh, p);
  const int nk = sp.nk;
  float qr[G][8], kn[8], vn[8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[g][i] = sm.q[g][ch * 8 + i];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    kn[i] = sm.kv_new[0][ch * 8 + i];
    vn[i] = sm.kv_new[1][ch * 8 + i];
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }
  // one iteration: U key rows per lane group, b0 the wave's first row block
  auto step = [&](const AttnLoads<U>& ld, int b0) {
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = (b0 + u * NW) * KPW + kin;
      const bool at_p = sp.k0 + min(t, nk - 1) == p;
      float kf[8];
      unpack8(ld.kk[u], kf);
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[i] = at_p ? kn[i] : kf[i];
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
        const int t = (b0 + u * NW) * KPW + kin;
        const bool at_p = sp.k0 + min(t, nk - 1) == p;
        const float pu = exp2f(sc[u][g] - mx);
        l[g] += pu;
        float vf[8];
        unpack8(ld.vv[u], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(pu, at_p ? vn[i] : vf[i], acc[g][i]);
      }
      m[g] = mx;
    }
  };
  // the first iteration on the prefetched loads, then fresh loads (peeled, so
  // that the prefetched registers are free for the later iterations)
  if (wave * KPW < nk) step(pre, wave);
  for (int b0 = wave + NW * U; b0 * KPW < nk; b0 += NW * U) {
    AttnLoads<U> ld;
    attn_load<HD, U, NW>(ld, sp, b0);
    step(ld, b0);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm.at.acc[wave][kin][g][ch * 8 + i] = acc[g][i];
    if (ch == 0) sm.at.ml[wave][kin][g] = make_float2(m[g], l[g]);
  }
}

// Threads tid < G*HD: combine the row-group states of sm.at into sm.comb
// (output sums, and per head the running max and denominator).
template <int HD, int G>
__device__ __forceinline__ void s_attn_combine(SSmem<HD, G>& sm, int tid) {
  constexpr int KPW = SSmem<HD, G>::KPW;
  if (tid >= G * HD) return;
  const int d = tid % HD, g = tid / HD;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kSW; ++w)
#pragma unroll
    for (int r = 0; r < KPW; ++r) M = fmaxf(M, sm.at.ml[w][r][g].x);
  float L = 0.f, A = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kSW; ++w)
#pragma unroll
      for (int r = 0; r < KPW; ++r) {
        const float2 ml = sm.at.ml[w][r][g];
        const float f = exp2f(ml.x - M);
        L = fmaf(ml.y, f, L);
        A = fmaf(sm.at.acc[w][r][g][d], f, A);
      }
  }
  sm.comb[g][d] = A;
  if (d == 0) sm.comb_ml[g] = make_float2(M, L);
}

// ---- the step kernel
//
// The control wave and the compute waves run separate loops over the same
// phase sequence, meeting at LDS barriers (two per GEMV phase, three per
// attention work item); a workgroup without an attention item skips those
// three. Separate loops keep each role's registers apart: the register
// allocator then needs the larger of the two, not their sum.

// What both roles need.
template <int HD, int G>
struct SCtx {
  const StreamArgs& s;
  SSmem<HD, G>& sm;
  int p, lane;
  unsigned epoch;
  bool hidden;

  __device__ __forceinline__ AttnArgs attn_args(int l) const {
    const SLayer w = const_load(s.layers + l);
    AttnArgs t{};
    t.kc = s.kc + l * s.layer_cache;
    t.vc = s.vc + l * s.layer_cache;
    t.max_ctx = s.max_ctx;
    t.window = w.window;
    t.S = w.S;
    t.chunk = w.chunk;
    t.kpl = s.kpl;
    return t;
  }
  // this workgroup's attention work item of layer l, if any
  __device__ __forceinline__ bool has_item(const AttnArgs& t) const {
    return static_cast<int>(blockIdx.x) < t.S * s.n_kv;
  }
};

// Compute wave `wave` (0 .. kSW-1).
template <int HD, int G, int RING>
__device__ __forceinline__ void s_compute_main(const SCtx<HD, G>& c, int wave, u32x4* ring) {
  const StreamArgs& s = c.s;
  SSmem<HD, G>& sm = c.sm;
  const int lane = c.lane;
  SProducer<RING> pr;
  pr.init(s.ph, s.n_ph, blockIdx.x * kSW + wave, lane, ring);
  for (int k = 0; k < RING; ++k) pr.issue();
  int cpos = 0;
  // one GEMV phase: false if the launch was aborted
  auto gemv = [&](int phi) -> bool {
    lds_barrier();  // input staged
    if (!sm.flag) return false;
    const SPhase P = const_load(s.ph + phi);
    s_consume<RING>(P, pr, sm.xs, sm.res, wave, lane, cpos, ring);
    return true;
  };
  bool alive = true;
  for (int l = 0; l < s.L && alive; ++l) {
    const AttnArgs t = c.attn_args(l);
    const bool item = c.has_item(t);
    const int si = blockIdx.x % t.S, kvh = blockIdx.x / t.S;
    if (!gemv(4 * l)) break;
    // The K/V rows before p do not depend on this step: load the first
    // iteration of the attention item now, before its queries exist.
    AttnLoads<kSAttnU> al;
    if (item) attn_prefetch<HD, kSAttnU, kSW>(al, t, si, kvh, c.p);
    lds_barrier();  // QKV results read
    if (item) {
      lds_barrier();  // queries and the new key and value staged
      if (!sm.flag) break;
      s_attn_rows<HD, G, kSAttnU>(t, sm, si, kvh, c.p, al, wave, lane);
      lds_barrier();  // row-group states written
      s_attn_combine<HD, G>(sm, threadIdx.x);
      lds_barrier();  // combined state written
    }
    alive = gemv(4 * l + 1);
    if (alive) lds_barrier();
    alive = alive && gemv(4 * l + 2);
    if (alive) lds_barrier();
    alive = alive && gemv(4 * l + 3);
    if (alive) lds_barrier();
  }
  if (alive && !c.hidden && gemv(4 * s.L)) lds_barrier();
  // No global-to-LDS copy may land after the workgroup has ended.
  wait_vm<0>();
}

// The control wave.
template <int HD, int G>
__device__ __forceinline__ void s_ctrl_main(const SCtx<HD, G>& c) {
  const StreamArgs& s = c.s;
  SSmem<HD, G>& sm = c.sm;
  const int lane = c.lane, p = c.p;
  const unsigned epoch = c.epoch;
  const int nb = gridDim.x;
  SPoll poll{s.bar + 2, 0u};
  const rsrc_t rx = rsrc_of(s.xt, s.d * 8), rq = rsrc_of(s.qt, s.qdim * 8), rkv = rsrc_of(s.kvt, 2 * s.n_kv * s.hd * 8),
               ract = rsrc_of(s.actt, s.ffn * 8), rpart = rsrc_of(s.partt, s.n_kv * G * s.S_max * (HD + 2) * 8);

  // The residual stream rows this workgroup's O and down phases produce
  // (rows rres0 + t) live in LDS, sm.resid[t].
  const int nres = kSW * const_load(s.ph + 1).rpw, rres0 = blockIdx.x * nres;
  const half_t* emb_row = nullptr;
  if (!c.hidden) {
    int tok = __builtin_amdgcn_readfirstlane(s.tokens[p]);
    if (tok < 0 || tok >= s.vocab) {
      tok = tok < 0 ? 0 : s.vocab - 1;
      if (blockIdx.x == 0 && lane == 0) s.state[kBadToken] = 1;
    }
    emb_row = s.embed + static_cast<size_t>(tok) * s.d;
  }
  for (int t = lane; t < nres; t += kWave) {
    const int r = min(rres0 + t, s.d - 1);
    sm.resid[t] = c.hidden ? s.x_in[r] : static_cast<float>(emb_row[r]);
  }

  // Stage the input of GEMV phase phi and meet the compute waves; false if
  // the launch was aborted.
  float rn = 1.f;
  auto stage = [&](int phi, int kind, int l) -> bool {
    const SPhase P = const_load(s.ph + phi);
    const SLayer w = const_load(s.layers + (l < s.L ? l : s.L - 1));
    bool ok = true;
    if (kind == kSQKV && l == 0)
      s_stage_plain(sm.xs, P.K, P.kch, s.x_in, emb_row, w.g1, s.eps, rn, lane);
    else if (kind == kSQKV)
      ok = s_stage_t(sm.xs, P.K, P.kch, s.xt, stag(epoch, l - 1, kTDown), w.g1, s.eps, rn, poll, lane);
    else if (kind == kSO)
      ok = s_stage_t(sm.xs, P.K, P.kch, s.ot, stag(epoch, l, kTAtt), nullptr, s.eps, rn, poll, lane);
    else if (kind == kSGU)
      ok = s_stage_t(sm.xs, P.K, P.kch, s.xt, stag(epoch, l, kTO), w.g2, s.eps, rn, poll, lane);
    else if (kind == kSDown)
      ok = s_stage_t(sm.xs, P.K, P.kch, s.actt, stag(epoch, l, kTGU), nullptr, s.eps, rn, poll, lane);
    else
      ok = s_stage_t(sm.xs, P.K, P.kch, s.xt, stag(epoch, s.L - 1, kTDown), s.gf, s.eps, rn, poll, lane);
    if (lane == 0) sm.flag = ok;
    lds_barrier();  // input staged
    if (!ok) return false;
    lds_barrier();  // results written
    return true;
  };

  // The epilogue of GEMV phase phi (results in sm.res).
  auto epilogue = [&](int phi, int kind, int l) {
    const SPhase P = const_load(s.ph + phi);
    const int n = kSW * P.rpw, r0 = blockIdx.x * n;
    if (kind == kSQKV) {
      const unsigned tag = stag(epoch, l, kTQKV);
      for (int u = lane; 2 * u < n; u += kWave)
        if (r0 + 2 * u < P.rows)
          qkv_put_t(s, rq, rkv, l, r0 + 2 * u, sm.res[2 * u] * rn, sm.res[2 * u + 1] * rn, p, tag);
    } else if (kind == kSGU) {
      const unsigned tag = stag(epoch, l, kTGU);
      for (int u = lane; 2 * u < n; u += kWave)
        if (r0 + 2 * u < P.rows) {
          const float g = sm.res[2 * u] * rn, up = sm.res[2 * u + 1] * rn;
          put_t(ract, (r0 >> 1) + u, g / (1.0f + expf(-g)) * up, tag);
        }
    } else if (kind == kSO || kind == kSDown) {
      const unsigned tag = stag(epoch, l, kind == kSO ? kTO : kTDown);
      const bool out = c.hidden && kind == kSDown && l == s.L - 1;
      for (int t = lane; t < n; t += kWave)
        if (r0 + t < P.rows) {
          const float v = sm.resid[t] + sm.res[t];
          sm.resid[t] = v;
          put_t(rx, r0 + t, v, tag);
          if (out) s.x_out[r0 + t] = v;
        }
    } else {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int t = lane; t < n; t += kWave)
        if (r0 + t < P.rows) {
          const float z = sm.res[t] * rn;
          s.logits[r0 + t] = z;
          if (better(z, r0 + t, bv, bi)) {
            bv = z;
            bi = r0 + t;
          }
        }
      const unsigned long long key = wave_max_key(bi != 0x7fffffff ? argmax_key(bv, bi) : 0ull);
      if (lane == 0 && key) __hip_atomic_fetch_max(s.best, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The last workgroup to finish its logits takes the greedy token and
      // ends the step.
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) {
        const unsigned prev = __hip_atomic_fetch_add(s.bar + 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == static_cast<unsigned>(nb) - 1) {
          const unsigned long long kb = __hip_atomic_load(s.best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          int i = kb ? argmax_index(kb) : 0;  // kb == 0 only if every logit is NaN
          if (i < 0 || i >= s.vocab) i = 0;
          s.state[kArgmax] = i;
          if (p + 1 >= s.state[kFedEnd]) s.tokens[p + 1] = i;
          s.state[kLen] = p + 1;
          __hip_atomic_store(s.best, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(s.bar + 4, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };

  bool alive = true;
  for (int l = 0; l < s.L && alive; ++l) {
    if (!stage(4 * l, kSQKV, l)) break;
    epilogue(4 * l, kSQKV, l);
    // attention: queries and the new key and value to LDS, the compute waves'
    // row-group math, the combined state stored; the split-0 workgroup of
    // each kv head merges
    const AttnArgs t = c.attn_args(l);
    if (c.has_item(t)) {
      const int si = blockIdx.x % t.S, kvh = blockIdx.x / t.S;
      const unsigned tq = stag(epoch, l, kTQKV);
      const bool ok =
          s_fetch_t(&sm.q[0][0], s.qt + static_cast<size_t>(kvh) * G * HD, G * HD, tq, s.scale_log2, poll, lane) &&
          s_fetch_t(&sm.kv_new[0][0], s.kvt + static_cast<size_t>(kvh) * HD, HD, tq, 1.f, poll, lane) &&
          s_fetch_t(&sm.kv_new[1][0], s.kvt + static_cast<size_t>(s.n_kv + kvh) * HD, HD, tq, 1.f, poll, lane);
      if (lane == 0) sm.flag = ok;
      lds_barrier();  // queries and the new key and value staged
      if (!ok) break;
      lds_barrier();  // row-group states written
      lds_barrier();  // combined state written
      const unsigned tp = stag(epoch, l, kTPart);
      for (int e = lane; e < G * HD; e += kWave) {
        const int g = e / HD, d = e % HD;
        put_t(rpart, ((kvh * G + g) * s.S_max + si) * (HD + 2) + d, sm.comb[g][d], tp);
      }
      if (lane < G) {
        const int ml = ((kvh * G + lane) * s.S_max + si) * (HD + 2) + HD;
        put_t(rpart, ml, sm.comb_ml[lane].x, tp);
        put_t(rpart, ml + 1, sm.comb_ml[lane].y, tp);
      }
      // every split merges its share of the outputs (an abort shows up at the next wait)
      attn_merge_share<HD, G>(s.partt, s.ot, s.n_kv, s.S_max, kvh, si, t.S, tp, stag(epoch, l, kTAtt), poll,
                              lane);
    }
    alive = stage(4 * l + 1, kSO, l);
    if (alive) epilogue(4 * l + 1, kSO, l);
    alive = alive && stage(4 * l + 2, kSGU, l);
    if (alive) epilogue(4 * l + 2, kSGU, l);
    alive = alive && stage(4 * l + 3, kSDown, l);
    if (alive) epilogue(4 * l + 3, kSDown, l);
  }
  if (alive && !c.hidden && stage(4 * s.L, kSLM, s.L)) epilogue(4 * s.L, kSLM, s.L);
  if (alive && c.hidden && blockIdx.x == 0 && lane == 0) s.state[kLen] = p + 1;
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
  const int p = __builtin_amdgcn_readfirstlane(s.state[kLen]);
  if (!(p < s.max_ctx && __hip_atomic_load(s.bar + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)) return;
  const unsigned epoch =
      __builtin_amdgcn_readfirstlane(__hip_atomic_load(s.bar + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const SCtx<HD, G> c{s, sm, p, lane, epoch, s.vocab == 0};
  if (wave == kSCtrl)
    s_ctrl_main<HD, G>(c);
  else
    s_compute_main<HD, G, RING>(c, wave, ring_all + wave * RING * kWave);
  // Leave: the last workgroup out advances the launch epoch.
  lds_barrier();
  if (threadIdx.x == kSCtrl * kWave) {
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned prev = __hip_atomic_fetch_add(s.bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == static_cast<unsigned>(gridDim.x) - 1) {
      __hip_atomic_store(s.bar + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(s.bar + 3, c.epoch + 1 == 0 ? 1u : c.epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
