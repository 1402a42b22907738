// Kernels of one decode step (batch 1) for gfx950.
//
// Every projection is a GEMV y = W x with fp16 W (row-major [out, in], rows
// streamed from HBM once per step with 16-byte non-temporal loads, one wave
// per group of rows, wave-shuffle reductions) and an fp32 input vector that
// each workgroup stages in LDS. The input stage can apply RMSNorm (the
// workgroup reduces sum(x^2) itself, so no separate norm kernel exists), and
// the epilogue fuses what follows the product: rotary embedding and the KV
// append (QKV), SwiGLU (gate/up), the residual add (O, down) or the logits
// and greedy argmax (LM head). Attention is split over key ranges; the last
// workgroup of a lane to finish merges the partial softmax states.
#pragma once
#include "lf_device.h"

namespace lf {

// ------------------------------------------------------------------ GEMV

enum InKind : int { kInF32 = 0, kInNormF32 = 1, kInNormEmbed = 2 };
enum Epi : int { kEpiQKV = 0, kEpiSwiGLU = 1, kEpiResid = 2, kEpiLogits = 3 };

struct GemvArgs {
  const half_t* W;        // [rows, K]
  int rows, K, rows_per_block;
  // input vector
  int in_kind;
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
  // finishing work of the last workgroup (kEpiLogits: argmax and step end; kEpiResid: step end)
  unsigned* counter;      // null: no finishing work
  float2* lm_part;        // per-workgroup (max, index) of the logits
};

// Stage the input vector of length K in LDS (fp32), applying RMSNorm if asked.
__device__ __forceinline__ void stage_input(const GemvArgs& a, float* xs, float* red) {
  const int tid = threadIdx.x, K = a.K;
  const int per = (K + gridDim.x - 1) / gridDim.x;
  const int s0 = blockIdx.x * per, s1 = min(s0 + per, K);
  float ss = 0.f;
  if (a.in_kind == kInNormEmbed) {
    const int p = a.state[kLen];
    int tok = a.tokens[p];
    if (tok < 0 || tok >= a.vocab) {
      tok = tok < 0 ? 0 : a.vocab - 1;
      if (tid == 0 && blockIdx.x == 0) a.state[kBadToken] = 1;
    }
    const half_t* row = a.emb + static_cast<size_t>(tok) * K;
    for (int i = tid * 8; i < K; i += kBlock * 8) {
      float f[8];
      unpack8(ld16(row + i), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xs[i + j] = f[j];
        ss = fmaf(f[j], f[j], ss);
        if (a.resid_copy && i + j >= s0 && i + j < s1) a.resid_copy[i + j] = f[j];
      }
    }
  } else {
    for (int i = tid * 4; i < K; i += kBlock * 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.x + i);
      *reinterpret_cast<f32x4*>(xs + i) = v;
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
      if (a.resid_copy) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i + j >= s0 && i + j < s1) a.resid_copy[i + j] = v[j];
      }
    }
  }
  if (a.in_kind != kInF32) {
    const float tot = block_sum(ss, red);  // its barrier also publishes xs
    const float r = 1.0f / sqrtf(tot / static_cast<float>(K) + a.eps);
    for (int i = tid; i < K; i += kBlock) xs[i] = xs[i] * r * static_cast<float>(a.gain[i]);
  }
  __syncthreads();
}

// Dot products of NR consecutive rows (row stride K) with xs; rows at or past
// `nvalid` are not read and give 0. Each lane covers 16-byte chunks
// lane, lane+64, ...; U chunks per row are in flight at once.
template <int NR, int U>
__device__ __forceinline__ void rows_dot(const half_t* __restrict__ W, int K, int nvalid,
                                         const float* __restrict__ xs, float (&out)[NR]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int K8 = K >> 3;
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  for (int c0 = lane; c0 < K8; c0 += kWave * U) {
    u32x4 w[NR][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + kWave * u;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        w[r][u] = (c < K8 && r < nvalid) ? ld_stream(W + static_cast<size_t>(r) * K + static_cast<size_t>(c) * 8)
                                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + kWave * u;
      if (c < K8) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(xs + c * 8);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(xs + c * 8 + 4);
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = dot8(w[r][u], x0, x1, acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) out[r] = wave_sum(acc[r]);
}

template <int EPI, int NR, int U>
__global__ __launch_bounds__(kBlock) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];
  __shared__ float red[kWavesPerBlock];
  __shared__ float2 wbest[kWavesPerBlock];
  __shared__ int flag;
  static_assert(NR % 2 == 0, "rows are processed in pairs");

  const int p = a.state[kLen];
  if (p >= a.max_ctx) return;  // the host never launches a step on a full cache
  stage_input(a, xs, red);

  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int rb = blockIdx.x * a.rows_per_block;
  const int re = min(rb + a.rows_per_block, a.rows);
  float bv = -INFINITY;
  int bi = 0x7fffffff;

  for (int r0 = rb + wave * NR; r0 < re; r0 += kWavesPerBlock * NR) {
    const int nvalid = min(NR, re - r0);
    float out[NR];
    rows_dot<NR, U>(a.W + static_cast<size_t>(r0) * a.K, a.K, nvalid, xs, out);
    if (lane != 0) continue;
    if constexpr (EPI == kEpiQKV) {
      const int half_hd = a.hd >> 1, upl = a.qpl + 2 * a.kpl;
#pragma unroll
      for (int k = 0; k < NR; k += 2) {
        if (k >= nvalid) break;
        const int r = r0 + k;
        const int u = r / a.hd, c = (r % a.hd) >> 1;
        const int ln = u / upl, j = u % upl;
        float y0 = out[k], y1 = out[k + 1];
        if (j < a.qpl + a.kpl) {  // rotary embedding on q and k
          const float2 cs = a.rope[static_cast<size_t>(p) * half_hd + c];
          const float t0 = y0 * cs.x - y1 * cs.y;
          const float t1 = y0 * cs.y + y1 * cs.x;
          y0 = t0;
          y1 = t1;
        }
        if (j < a.qpl) {
          float* qh = a.q + static_cast<size_t>(ln * a.qpl + j) * a.hd;
          qh[c] = y0;
          qh[c + half_hd] = y1;
        } else {
          const bool is_k = j < a.qpl + a.kpl;
          const int h = is_k ? j - a.qpl : j - a.qpl - a.kpl;
          half_t* dst = (is_k ? a.kc : a.vc) +
                        ((static_cast<size_t>(ln) * a.max_ctx + p) * a.kpl + h) * a.hd;
          dst[c] = static_cast<half_t>(y0);
          dst[c + half_hd] = static_cast<half_t>(y1);
        }
      }
    } else if constexpr (EPI == kEpiSwiGLU) {
#pragma unroll
      for (int k = 0; k < NR; k += 2) {
        if (k >= nvalid) break;
        const float g = out[k], u = out[k + 1];
        a.y[(r0 + k) >> 1] = g / (1.0f + expf(-g)) * u;
      }
    } else if constexpr (EPI == kEpiResid) {
#pragma unroll
      for (int k = 0; k < NR; ++k)
        if (k < nvalid) a.y[r0 + k] += out[k];
    } else {  // kEpiLogits
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        if (k < nvalid) {
          a.y[r0 + k] = out[k];
          if (better(out[k], r0 + k, bv, bi)) {
            bv = out[k];
            bi = r0 + k;
          }
        }
      }
    }
  }

  if (a.counter == nullptr) return;
  if constexpr (EPI == kEpiLogits) {
    if (lane == 0) wbest[wave] = make_float2(bv, __int_as_float(bi));
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = wbest[0].x;
      int i = __float_as_int(wbest[0].y);
      for (int w = 1; w < kWavesPerBlock; ++w) {
        const int wi = __float_as_int(wbest[w].y);
        if (better(wbest[w].x, wi, v, i)) {
          v = wbest[w].x;
          i = wi;
        }
      }
      a.lm_part[blockIdx.x] = make_float2(v, __int_as_float(i));
    }
    if (!arrive_last(a.counter, gridDim.x, &flag)) return;
    // Greedy choice over all workgroups' bests.
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (int b = threadIdx.x; b < static_cast<int>(gridDim.x); b += kBlock) {
      const float2 e = a.lm_part[b];
      const int ei = __float_as_int(e.y);
      if (better(e.x, ei, v, i)) {
        v = e.x;
        i = ei;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o);
      const int oi = __shfl_xor(i, o);
      if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
    if (lane == 0) wbest[wave] = make_float2(v, __int_as_float(i));
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kWavesPerBlock; ++w) {
        const int wi = __float_as_int(wbest[w].y);
        if (better(wbest[w].x, wi, v, i)) {
          v = wbest[w].x;
          i = wi;
        }
      }
      if (i < 0 || i >= a.rows) i = 0;  // only if every logit is NaN
      a.state[kArgmax] = i;
      if (p + 1 >= a.state[kFedEnd]) a.tokens[p + 1] = i;
      a.state[kLen] = p + 1;
    }
    reset_counter(a.counter);
  } else {
    if (!arrive_last(a.counter, gridDim.x, &flag)) return;
    if (threadIdx.x == 0) a.state[kLen] = p + 1;
    reset_counter(a.counter);
  }
}

// ------------------------------------------------------------- attention

struct AttnArgs {
  const float* q;           // rotated queries [Hq * hd]
  const half_t* kc;         // this layer's K cache [lanes][max_ctx][kpl][hd]
  const half_t* vc;
  const int32_t* state;
  float2* part_ml;          // [Hq][S] (running max in log2 units, denominator)
  float* part_acc;          // [Hq][S][hd] unnormalised outputs
  float* o;                 // attention output [Hq * hd]
  unsigned* counters;       // [lanes]
  int max_ctx, window, S, chunk, qpl, kpl;
  float scale_log2;         // log2(e) / sqrt(hd)
};

// Workgroup (split s, lane ln) reads the lane's key range
// [lo + s*chunk, lo + (s+1)*chunk) of all its kv heads as one contiguous tile
// (keys are lane-major: [pos][kv head in lane][hd]) and keeps an online
// softmax per (row group, query head) in registers. HD/8 lanes hold one
// 16-byte piece of a key row each; G query heads share each kv head.
template <int HD, int G, int U>
__global__ __launch_bounds__(kBlock) void k_attn(AttnArgs a) {
  constexpr int LPR = HD / 8;       // lanes per key row
  constexpr int RPW = kWave / LPR;  // key rows per wave load
  __shared__ float2 sm_ml[kWavesPerBlock][RPW][G];
  __shared__ float sm_acc[kWavesPerBlock][RPW][G][HD];
  __shared__ int flag;

  const int s = blockIdx.x, ln = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int p = a.state[kLen];
  if (p >= a.max_ctx) return;
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int k0 = lo + s * a.chunk;
  const int k1 = min(k0 + a.chunk, p + 1);
  const int nrows = k1 > k0 ? (k1 - k0) * a.kpl : 0;

  const int rin = lane / LPR, ch = lane % LPR, kvh = rin % a.kpl;
  const int head0 = ln * a.qpl + kvh * G;
  float qr[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qp = a.q + static_cast<size_t>(head0 + g) * HD + ch * 8;
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(qp);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(qp + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qr[g][i] = q0[i] * a.scale_log2;
      qr[g][4 + i] = q1[i] * a.scale_log2;
    }
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }

  const size_t base = (static_cast<size_t>(ln) * a.max_ctx + min(k0, a.max_ctx - 1)) * a.kpl * HD;
  const half_t* Kb = a.kc + base + ch * 8;
  const half_t* Vb = a.vc + base + ch * 8;
  for (int b0 = wave; b0 * RPW < nrows; b0 += kWavesPerBlock * U) {
    u32x4 kk[U], vv[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = (b0 + u * kWavesPerBlock) * RPW + rin;
      ok[u] = t < nrows;
      kk[u] = ok[u] ? ld_stream(Kb + static_cast<size_t>(t) * HD) : u32x4{0u, 0u, 0u, 0u};
      vv[u] = ok[u] ? ld_stream(Vb + static_cast<size_t>(t) * HD) : u32x4{0u, 0u, 0u, 0u};
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8(kk[u], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = fmaf(qr[g][i], kf[i], d);
        d = group_sum<LPR>(d);
        sc[u][g] = ok[u] ? d : -INFINITY;
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
        unpack8(vv[u], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(pu, vf[i], acc[g][i]);
      }
      m[g] = mx;
    }
  }

  // Combine the row groups of all waves that served the same kv head.
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm_acc[wave][rin][g][ch * 8 + i] = acc[g][i];
    if (ch == 0) sm_ml[wave][rin][g] = make_float2(m[g], l[g]);
  }
  __syncthreads();
  for (int idx = tid; idx < a.kpl * G * HD; idx += kBlock) {
    const int d = idx % HD, g = (idx / HD) % G, kh = idx / (HD * G);
    float M = -INFINITY;
    for (int w = 0; w < kWavesPerBlock; ++w)
      for (int r = kh; r < RPW; r += a.kpl) M = fmaxf(M, sm_ml[w][r][g].x);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kWavesPerBlock; ++w)
        for (int r = kh; r < RPW; r += a.kpl) {
          const float2 ml = sm_ml[w][r][g];
          const float f = exp2f(ml.x - M);
          L = fmaf(ml.y, f, L);
          A = fmaf(sm_acc[w][r][g][d], f, A);
        }
    }
    const int head = ln * a.qpl + kh * G + g;
    a.part_acc[(static_cast<size_t>(head) * a.S + s) * HD + d] = A;
    if (d == 0) a.part_ml[head * a.S + s] = make_float2(M, L);
  }

  // The last workgroup of this lane merges the splits.
  if (!arrive_last(&a.counters[ln], a.S, &flag)) return;
  const int n = p + 1 - lo;
  const int n_active = min(a.S, (n + a.chunk - 1) / a.chunk);
  for (int idx = tid; idx < a.qpl * HD; idx += kBlock) {
    const int d = idx % HD, head = ln * a.qpl + idx / HD;
    const float2* ml = a.part_ml + head * a.S;
    const float* pa = a.part_acc + static_cast<size_t>(head) * a.S * HD + d;
    float M = -INFINITY;
    for (int t = 0; t < n_active; ++t) M = fmaxf(M, ml[t].x);
    float L = 0.f, A = 0.f;
    for (int t = 0; t < n_active; ++t) {
      const float f = exp2f(ml[t].x - M);
      L = fmaf(ml[t].y, f, L);
      A = fmaf(pa[static_cast<size_t>(t) * HD], f, A);
    }
    a.o[static_cast<size_t>(head) * HD + d] = A / L;
  }
  reset_counter(&a.counters[ln]);
}

// ------------------------------------------------------------- utilities

// Weight repack. Mode 0 (QKV): packed unit u (lane-major: per lane, its q
// heads, then k heads, then v heads) holds rows (dim c, dim c + hd/2) at
// packed rows (2c, 2c+1), so a rotary pair lands in one wave. Mode 1
// (gate/up): packed row 2j = gate j, 2j+1 = up j. Mode 2: identity.
struct RepackArgs {
  half_t* dst;
  const half_t* src;
  int rows, K, mode;
  int hd, n_q, n_kv, qpl, kpl, ffn;
};

__device__ __forceinline__ int repack_src_row(const RepackArgs& a, int r) {
  if (a.mode == 1) return (r & 1) ? a.ffn + (r >> 1) : (r >> 1);
  if (a.mode == 2) return r;
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

__global__ void k_fill_u32(unsigned* p, unsigned v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Start a step with an explicit token, or set the length (d_token == null).
__global__ void k_set_pos(int32_t* state, int32_t* tokens, int32_t len, const int32_t* d_token) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  state[kLen] = len;
  if (d_token) {
    tokens[len] = *d_token;
    state[kFedEnd] = len + 1;
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

__global__ void k_copy_out(float* dst, const float* src, int n, int32_t* argmax_dst, const int32_t* state) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
  if (i == 0 && argmax_dst) *argmax_dst = state[kArgmax];
}

}  // namespace lf
