// Host side of lfdecode: configuration checks, memory layout, weight repack,
// launch plan of one decode step, hipGraph capture and replay, and the C ABI
// declared in include/lfdecode.h.
#include "lfdecode.h"
#include "lf_kernels.h"
#include "lf_prefill.h"
#include "lf_sample.h"
#include "lf_batch.h"

static_assert(LF_MAX_BATCH == lf::kMaxBatch, "the header states the batch limit");

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

using lf::half_t;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define LF_HIP(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) return fail(LF_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Attention split plan of one layer: S workgroups per lane, `chunk` keys each.
struct AttnPlan {
  int S, chunk;
};

// Attention splits each kv head's visible keys over at most kAttnSplits work
// items (16 kv heads x 16 = 256 workgroups: one per CU), or, with fewer kv
// heads, as many as make 256 work items in all (at most kMaxSplits per kv
// head), at least 64 keys each; every split's merge reads all S split states,
// so more splits than that cost more than they gain. A work item reads its keys in rounds of U loads of K
// and of V per lane (4 waves, 512/head_dim keys per wave load), U the
// smallest of 4, 8, 16 that covers its chunk in one round.
constexpr int kAttnSplits = 16;
constexpr int kMaxSplits = 64;  // partial-state buffers hold this many splits per head
constexpr int kFusedSplits = 16;  // splits per kv head of QKV fused with attention
AttnPlan split_plan(int visible, int S) {
  S = std::max(1, std::min(S, kMaxSplits));
  const int chunk = (visible + S - 1) / S;
  return {(visible + chunk - 1) / chunk, chunk};
}
int visible_keys(const lf_config& c, int layer) {
  return c.window[layer] > 0 ? std::min(c.window[layer], c.max_ctx) : c.max_ctx;
}
AttnPlan attn_plan(const lf_config& c, int layer) {
  const int visible = visible_keys(c, layer);
  // up to 256 work items in all: kv heads below 16 get more splits
  const int cap = std::max(kAttnSplits, std::min(kMaxSplits, 256 / c.n_kv_heads));
  return split_plan(visible, std::min(cap, (visible + 63) / 64));
}
int attn_loads_per_lane(int chunk, int head_dim) {
  const int per_load = lf::kWavesPerBlock * (512 / head_dim);  // keys per load round of the workgroup
  for (int u : {4, 8})
    if (u * per_load >= chunk) return u;
  return 16;
}

// Launch shape of a GEMV: (waves per workgroup, row groups per wave). Each
// candidate is a compiled variant; the first that gives a balanced grid of at
// least 256 workgroups (one per CU) wins, else the one with the most
// workgroups. Chosen from measurements of the decode shapes on MI355X.
struct GemvShape {
  int waves, gpw, blocks;
};

GemvShape gemv_shape(int epi, int rows) {
  static const int qkv[][2] = {{8, 2}, {8, 1}, {2, 1}}, glu[][2] = {{2, 7}, {8, 2}, {8, 1}, {2, 1}},
                   res[][2] = {{4, 4}, {8, 2}, {8, 1}, {2, 1}}, lgt[][2] = {{4, 16}, {8, 2}, {8, 1}, {2, 1}};
  const int(*cand)[2] = epi == lf::kEpiQKV ? qkv : epi == lf::kEpiSwiGLU ? glu : epi == lf::kEpiResid ? res : lgt;
  const int n = epi == lf::kEpiQKV ? 3 : 4;
  const int nr = (epi == lf::kEpiQKV || epi == lf::kEpiSwiGLU) ? 2 : 1;
  const int ng = (rows + nr - 1) / nr;
  GemvShape best{0, 0, 0};
  for (int i = 0; i < n; ++i) {
    const int w = cand[i][0], g = cand[i][1];
    const int b = (ng + w * g - 1) / (w * g);
    if (b >= 256 && (b % 256 == 0 || b > 480)) return {w, g, b};
    if (b > best.blocks) best = {w, g, b};
  }
  return best;
}

int validate(const lf_config* c) {
  if (!c) return fail(LF_EINVAL, "config is null");
  if (c->n_layers < 1 || c->n_layers > LF_MAX_LAYERS) return fail(LF_EINVAL, "n_layers %d out of [1, %d]", c->n_layers, LF_MAX_LAYERS);
  if (c->d_model < 8 || c->d_model % 8 || c->d_model > 8192) return fail(LF_EINVAL, "d_model %d: need a multiple of 8 in [8, 8192]", c->d_model);
  if (c->ffn < 8 || c->ffn % 8 || c->ffn > 8192) return fail(LF_EINVAL, "ffn %d: need a multiple of 8 in [8, 8192]", c->ffn);
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return fail(LF_EINVAL, "head_dim %d: need 32, 64 or 128", c->head_dim);
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads) return fail(LF_EINVAL, "n_q_heads %d must be a multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return fail(LF_EINVAL, "query heads per kv head %d: need 1, 2 or 4", G);
  if (c->n_lanes < 1 || c->n_q_heads % c->n_lanes || c->n_kv_heads % c->n_lanes || c->ffn % c->n_lanes)
    return fail(LF_EINVAL, "n_lanes %d must divide n_q_heads, n_kv_heads and ffn", c->n_lanes);
  const int kpl = c->n_kv_heads / c->n_lanes;
  if ((512 / c->head_dim) % kpl) return fail(LF_EINVAL, "kv heads per lane %d must divide %d", kpl, 512 / c->head_dim);
  if (static_cast<long>(c->n_q_heads) * c->head_dim > 8192) return fail(LF_EINVAL, "n_q_heads * head_dim exceeds 8192");
  if (c->vocab < 0) return fail(LF_EINVAL, "vocab %d < 0", c->vocab);
  if (c->max_ctx < 1 || c->max_ctx > 4096) return fail(LF_EINVAL, "max_ctx %d out of [1, 4096]", c->max_ctx);
  for (int l = 0; l < c->n_layers; ++l)
    if (c->window[l] < 0) return fail(LF_EINVAL, "window[%d] = %d < 0", l, c->window[l]);
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(LF_EINVAL, "rope_theta must be > 0 and rms_eps >= 0");
  return LF_OK;
}

struct Dims {
  int L, d, hq, hkv, hd, ffn, V, lanes, ctx, qkv_rows, qdim, qpl, kpl, G;
};

Dims dims(const lf_config& c) {
  Dims D;
  D.L = c.n_layers; D.d = c.d_model; D.hq = c.n_q_heads; D.hkv = c.n_kv_heads; D.hd = c.head_dim;
  D.ffn = c.ffn; D.V = c.vocab; D.lanes = c.n_lanes; D.ctx = c.max_ctx;
  D.qkv_rows = (D.hq + 2 * D.hkv) * D.hd; D.qdim = D.hq * D.hd;
  D.qpl = D.hq / D.lanes; D.kpl = D.hkv / D.lanes; D.G = D.hq / D.hkv;
  return D;
}

// Byte offsets of everything in the model workspace.
struct WsLayout {
  std::vector<size_t> wqkv, wo, wgu, wd, g1, g2;
  size_t embed = 0, lm = 0, gf = 0, rope, x, q, o, act, best, counters, abort, attn_epochs, total;
  // tagged exchange buffers of the attention kernels (one zeroed region)
  size_t attn_part, fpart, qkvx, tagged_begin, tagged_end;
  size_t class_epochs;  // QKV fused with attention: epoch per XCD class
  // batched step (lf_decode_step_batch): per-sequence activations, partial
  // sums of squares, greedy keys, split states and epochs
  size_t bx, bq, bfd, bfq, bff, bss, bbest, bcounter, bpart, bepochs;
  int S_max;
};

WsLayout ws_layout(const lf_config& c) {
  const Dims D = dims(c);
  WsLayout W;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const size_t h = sizeof(half_t);
  for (int l = 0; l < D.L; ++l) {
    W.wqkv.push_back(take(static_cast<size_t>(D.qkv_rows) * D.d * h));
    W.wo.push_back(take(static_cast<size_t>(D.d) * D.qdim * h));
    W.wgu.push_back(take(static_cast<size_t>(2) * D.ffn * D.d * h));
    W.wd.push_back(take(static_cast<size_t>(D.d) * D.ffn * h));
    W.g1.push_back(take(D.d * h));
    W.g2.push_back(take(D.d * h));
  }
  if (D.V) {
    W.embed = take(static_cast<size_t>(D.V) * D.d * h);
    W.lm = take(static_cast<size_t>(D.V) * D.d * h);
    W.gf = take(D.d * h);
  }
  W.rope = take(static_cast<size_t>(D.ctx) * (D.hd / 2) * sizeof(float2));
  W.x = take(D.d * sizeof(float));
  W.q = take(D.qdim * sizeof(float));
  W.o = take(D.qdim * sizeof(float));
  W.act = take(D.ffn * sizeof(float));
  W.S_max = kMaxSplits;
  W.best = take(sizeof(unsigned long long));
  W.counters = take((D.hkv + 4) * sizeof(unsigned));
  W.abort = take(sizeof(unsigned));  // raised when a wait between workgroups gives up
  W.attn_epochs = take(D.hkv * sizeof(unsigned));
  const size_t tw = sizeof(unsigned long long);
  W.tagged_begin = off;
  W.attn_part = take(static_cast<size_t>(D.hq) * W.S_max * (D.hd + 2) * tw);
  W.fpart = take(static_cast<size_t>(D.hq) * kFusedSplits * (D.hd + 2) * tw);
  W.qkvx = take(static_cast<size_t>(D.qkv_rows) * tw);
  W.bpart = take(static_cast<size_t>(lf::kMaxBatch) * D.hq * W.S_max * (D.hd + 2) * tw);
  W.tagged_end = off;
  W.class_epochs = take(8 * sizeof(unsigned));
  const size_t B = lf::kMaxBatch;
  W.bx = take(B * D.d * sizeof(float));
  W.bq = take(B * D.qdim * sizeof(float));
  // projection operands (frag_index): per k-step of 32, 64 lanes of 8 fp16,
  // and one more k-step that stays zero (read in place of k-steps past K)
  auto frag_bytes = [](int K) { return static_cast<size_t>((K + 31) / 32 + 1) * 64 * 8 * sizeof(half_t); };
  W.bfd = take(frag_bytes(D.d));
  W.bfq = take(frag_bytes(D.qdim));
  W.bff = take(frag_bytes(D.ffn));
  W.bss = take(B * lf::kSsStride * sizeof(float));
  W.bbest = take(B * sizeof(unsigned long long));
  W.bcounter = take(sizeof(unsigned));
  W.bepochs = take(B * D.hkv * sizeof(unsigned));
  W.total = off;
  return W;
}

// Byte offsets in the per-sequence buffer.
struct KvLayout {
  size_t state, tokens, logits, K, V, total, cache_bytes;
};

KvLayout kv_layout(const lf_config& c) {
  const Dims D = dims(c);
  KvLayout K;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  K.state = take(64 * sizeof(int32_t));
  K.tokens = take(static_cast<size_t>(D.ctx + 1) * sizeof(int32_t));
  K.logits = take(static_cast<size_t>(std::max(D.V, 1)) * sizeof(float));
  K.cache_bytes = static_cast<size_t>(D.L) * D.lanes * D.ctx * D.kpl * D.hd * sizeof(half_t);
  K.K = take(K.cache_bytes);
  K.V = take(K.cache_bytes);
  K.total = off;
  return K;
}

}  // namespace

struct BatchGraph {
  int n;
  lf_kv* kvs[lf::kMaxBatch];
  hipGraphExec_t exec;
};

struct GraphEntry {
  lf_kv* kv;
  const void* xin;
  void* xout;
  hipGraphExec_t exec;
};

struct lf_model {
  lf_config cfg;
  Dims D;
  WsLayout W;
  char* ws;
  hipStream_t capture_stream = nullptr;  // graphs are recorded here, replayed on the caller's stream
  std::vector<hipEvent_t> events;        // per-kernel brackets for lf_step_kernel_times
  std::vector<lf_kv*> kvs;               // live sequences; detached when the model is freed
  int mode = LF_MODE_GRAPH;
  bool xcd_classes = false;              // workgroups congruent modulo 8 share an XCD (probed at init)
  bool fused_ok = false;                 // QKV and attention can run as one kernel per layer
  std::vector<char> attn_xcd;            // per layer: k_attn runs with the XCD layout
  bool fused = false;                    // ... and do
  std::vector<GraphEntry> graphs;
  std::vector<BatchGraph> batch_graphs;
  int battn_room = 1;                    // batched attention workgroups the device holds at once
  int ncu = 256;                         // compute units of the device (read at init)
  void* scratch = nullptr;               // this device's address of the static prompt-pass scratch

  template <class T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
};

struct lf_kv {
  lf_model* m;
  char* buf;
  KvLayout K;
  int32_t len;
  int32_t* state() const { return reinterpret_cast<int32_t*>(buf + K.state); }
  int32_t* tokens() const { return reinterpret_cast<int32_t*>(buf + K.tokens); }
  float* logits() const { return reinterpret_cast<float*>(buf + K.logits); }
  half_t* kc() const { return reinterpret_cast<half_t*>(buf + K.K); }
  half_t* vc() const { return reinterpret_cast<half_t*>(buf + K.V); }
};

namespace {

template <int EPI> constexpr int gemv_nr() { return (EPI == lf::kEpiQKV || EPI == lf::kEpiSwiGLU) ? 2 : 1; }

// 16-byte chunks per lane per row: the smallest instantiated count covering K.
int gemv_kch(int K) {
  const int need = ((K >> 3) + lf::kWave - 1) / lf::kWave;
  for (int k : {1, 2, 4, 8, 14, 16})
    if (need <= k) return k;
  return 0;
}

// The input kinds each epilogue is launched with: QKV takes the normed
// residual (or, at layer 0, an embedding row), gate/up and the LM head the
// normed residual, O and down a plain vector.
template <int EPI>
constexpr bool gemv_takes(int in) {
  return EPI == lf::kEpiQKV ? in != lf::kInF32 : EPI == lf::kEpiResid ? in == lf::kInF32 : in == lf::kInNormF32;
}

template <int EPI, int KCH, int GPW, int WAVES, int IN>
const void* gemv_fn() {
  if constexpr (gemv_takes<EPI>(IN))
    return reinterpret_cast<const void*>(&lf::k_gemv<EPI, gemv_nr<EPI>(), KCH, GPW, WAVES, IN>);
  else
    return nullptr;
}

template <int EPI, int KCH, int IN>
const void* gemv_fn_k(int waves, int gpw) {
  if (waves == 2 && gpw == 7) return gemv_fn<EPI, KCH, 7, 2, IN>();
  if (waves == 4 && gpw == 4) return gemv_fn<EPI, KCH, 4, 4, IN>();
  if (waves == 4 && gpw == 16) return gemv_fn<EPI, KCH, 16, 4, IN>();
  if (waves == 8 && gpw == 2) return gemv_fn<EPI, KCH, 2, 8, IN>();
  if (waves == 2 && gpw == 1) return gemv_fn<EPI, KCH, 1, 2, IN>();
  return gemv_fn<EPI, KCH, 1, 8, IN>();
}

template <int EPI, int IN>
const void* gemv_kernel_in(int K, int waves, int gpw) {
  switch (gemv_kch(K)) {
    case 1: return gemv_fn_k<EPI, 1, IN>(waves, gpw);
    case 2: return gemv_fn_k<EPI, 2, IN>(waves, gpw);
    case 4: return gemv_fn_k<EPI, 4, IN>(waves, gpw);
    case 8: return gemv_fn_k<EPI, 8, IN>(waves, gpw);
    case 14: return gemv_fn_k<EPI, 14, IN>(waves, gpw);
    default: return gemv_fn_k<EPI, 16, IN>(waves, gpw);
  }
}

// The kernel variant for (input kind, K, launch shape); null if EPI never
// takes that input.
template <int EPI>
const void* gemv_kernel(int K, int waves, int gpw, int in) {
  switch (in) {
    case lf::kInF32: return gemv_kernel_in<EPI, lf::kInF32>(K, waves, gpw);
    case lf::kInNormF32: return gemv_kernel_in<EPI, lf::kInNormF32>(K, waves, gpw);
    default: return gemv_kernel_in<EPI, lf::kInNormEmbed>(K, waves, gpw);
  }
}

template <int EPI>
void launch_gemv(const lf::GemvArgs& a, hipStream_t st) {
  const GemvShape sh = gemv_shape(EPI, a.rows);
  const void* fn = gemv_kernel<EPI>(a.K, sh.waves, sh.gpw, a.in_kind);
  void* args[] = {const_cast<lf::GemvArgs*>(&a)};
  (void)hipLaunchKernel(fn, dim3(sh.blocks), dim3(sh.waves * lf::kWave), args, static_cast<size_t>(a.K) * sizeof(float),
                        st);
}

template <int EPI>
int set_lds_limit_epi() {
  const int bytes = 8192 * sizeof(float);
  static const int shapes[][2] = {{2, 7}, {4, 4}, {4, 16}, {8, 2}, {8, 1}, {2, 1}};  // (waves, row groups per wave)
  for (int in : {lf::kInF32, lf::kInNormF32, lf::kInNormEmbed})
    for (int K : {512, 1024, 2048, 4096, 7168, 8192})
      for (const auto& wg : shapes)
        if (const void* fn = gemv_kernel<EPI>(K, wg[0], wg[1], in))
          LF_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
  return LF_OK;
}

// The attention kernel variant for (head_dim, query heads per kv head, loads
// per lane, layout). XCD layout: a one-dimensional grid of S * n_kv
// workgroups in which the splits of a kv head are the workgroups congruent to
// it modulo 8 (one XCD, exchanges through its L2); else a grid (S, n_kv).
template <int HD, int G, bool XCD>
const void* attn_fn_u(int u) {
  return u == 4   ? reinterpret_cast<const void*>(&lf::k_attn<HD, G, 4, XCD>)
         : u == 8 ? reinterpret_cast<const void*>(&lf::k_attn<HD, G, 8, XCD>)
                  : reinterpret_cast<const void*>(&lf::k_attn<HD, G, 16, XCD>);
}
template <int HD, int G>
const void* attn_fn_t(int u, bool xcd) {
  return xcd ? attn_fn_u<HD, G, true>(u) : attn_fn_u<HD, G, false>(u);
}
const void* attn_kernel(int hd, int G, int u, bool xcd) {
#define LF_ATTN_CASE(H, GG) if (hd == H && G == GG) return attn_fn_t<H, GG>(u, xcd);
  LF_ATTN_CASE(32, 1) LF_ATTN_CASE(32, 2) LF_ATTN_CASE(32, 4)
  LF_ATTN_CASE(64, 1) LF_ATTN_CASE(64, 2) LF_ATTN_CASE(64, 4)
  LF_ATTN_CASE(128, 1) LF_ATTN_CASE(128, 2) LF_ATTN_CASE(128, 4)
#undef LF_ATTN_CASE
  return nullptr;
}

void launch_attn(const lf::AttnXArgs& a, int hd, int G, int n_kv, bool xcd, hipStream_t st) {
  const dim3 grid = xcd ? dim3(a.t.S * n_kv) : dim3(a.t.S, n_kv);
  void* args[] = {const_cast<lf::AttnXArgs*>(&a)};
  (void)hipLaunchKernel(attn_kernel(hd, G, attn_loads_per_lane(a.t.chunk, hd), xcd), grid, dim3(lf::kBlock), args, 0,
                        st);
}

// QKV fused with attention (k_qkv_attn): the decoder shape of 16 kv heads of
// 128 dimensions, 2 query heads each, d 4096, whose QKV GEMV runs as 256
// workgroups of 8 waves with two rotary pairs each, on a device whose
// workgroups congruent modulo 8 share an XCD. Every layer has kFusedSplits
// splits per kv head (one work item per workgroup); a split's keys must fit
// in LDS.
bool fused_shape(const Dims& D) {
  const GemvShape sh = gemv_shape(lf::kEpiQKV, D.qkv_rows);
  return D.hd == 128 && D.G == 2 && D.hkv == 16 && D.d == 4096 && sh.waves == 8 && sh.gpw == 2 && sh.blocks == 256 &&
         D.hkv * kFusedSplits == sh.blocks;
}
AttnPlan fused_plan(const lf_config& c, int layer) {
  const int visible = visible_keys(c, layer);
  return {kFusedSplits, (visible + kFusedSplits - 1) / kFusedSplits};
}
// Loads per lane per wave that cover a split of `chunk` keys (8 waves, 4 keys per wave load).
int fused_ukv(int chunk) {
  for (int u : {1, 2, 4, 8})
    if (32 * u >= chunk) return u;
  return 0;
}

template <int UKV, int IN>
const void* qkv_attn_fn() {
  return reinterpret_cast<const void*>(&lf::k_qkv_attn<128, 2, UKV, IN>);
}
template <int IN>
const void* qkv_attn_fn_in(int ukv) {
  switch (ukv) {
    case 1: return qkv_attn_fn<1, IN>();
    case 2: return qkv_attn_fn<2, IN>();
    case 4: return qkv_attn_fn<4, IN>();
    default: return qkv_attn_fn<8, IN>();
  }
}
const void* qkv_attn_kernel(int ukv, int in) {
  return in == lf::kInNormEmbed ? qkv_attn_fn_in<lf::kInNormEmbed>(ukv) : qkv_attn_fn_in<lf::kInNormF32>(ukv);
}

void launch_qkv_attn(const lf::QkvAttnArgs& a, hipStream_t st) {
  const int ukv = fused_ukv(a.at.t.chunk);
  void* args[] = {const_cast<lf::QkvAttnArgs*>(&a)};
  (void)hipLaunchKernel(qkv_attn_kernel(ukv, a.g.in_kind), dim3(256), dim3(8 * lf::kWave), args, 0, st);
}

// Which attention launches a device can run. Workgroups that wait on each
// other must all be resident at once: a wait on a workgroup that has not been
// dispatched ends only by giving up (the abort flag), so a plan is chosen
// from the device's room for each kernel (workgroups per CU x CUs):
//  * QKV fused with attention: one launch of 16 kv heads x 16 splits = 256
//    workgroups that wait on their XCD class: needs the fused shape, the XCD
//    dealing, room for all 256 at once and every split's keys in LDS;
//  * k_attn with the XCD layout: the splits of a kv head are spread over the
//    whole grid, so all S * n_kv workgroups must fit at once;
//  * k_attn with the two-dimensional grid: the S splits of a kv head are
//    consecutive workgroups, dispatched in order, so S of them must fit; a
//    configuration that cannot is rejected.
int plan_attention(const lf_config& c, int n_cu, int attn_per_cu, int fused_per_cu, bool xcd, bool& fused_ok,
                   std::vector<char>& xcd_layer) {
  const Dims D = dims(c);
  fused_ok = xcd && fused_shape(D) && static_cast<long>(fused_per_cu) * n_cu >= D.hkv * kFusedSplits;
  for (int l = 0; l < D.L && fused_ok; ++l) fused_ok = fused_ukv(fused_plan(c, l).chunk) > 0;
  const long room = static_cast<long>(attn_per_cu) * n_cu;
  xcd_layer.assign(D.L, 0);
  for (int l = 0; l < D.L; ++l) {
    const AttnPlan P = attn_plan(c, l);
    if (P.S > room)
      return fail(LF_EINVAL, "layer %d: %d attention splits cannot be resident at once (room for %ld)", l, P.S, room);
    xcd_layer[l] = xcd && D.hkv % 8 == 0 && static_cast<long>(P.S) * D.hkv <= room;
  }
  return LF_OK;
}

// Workgroups per CU the device holds of the attention kernels this model
// launches (the smallest over its layers and both layouts), and of its QKV
// fused with attention kernels (0 if the shape has none).
int attention_room(const lf_config& c, int& attn_per_cu, int& fused_per_cu) {
  const Dims D = dims(c);
  attn_per_cu = 1 << 20;
  fused_per_cu = 0;
  for (int l = 0; l < D.L; ++l) {
    const int u = attn_loads_per_lane(attn_plan(c, l).chunk, D.hd);
    for (bool x : {false, true}) {
      int n = 0;
      LF_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_kernel(D.hd, D.G, u, x), lf::kBlock, 0));
      attn_per_cu = std::min(attn_per_cu, n);
    }
  }
  if (!fused_shape(D)) return LF_OK;
  fused_per_cu = 1 << 20;
  for (int l = 0; l < D.L; ++l) {
    const int ukv = fused_ukv(fused_plan(c, l).chunk);
    if (ukv == 0) return fused_per_cu = 0, LF_OK;
    int n = 0;
    const int in = (l == 0 && D.V) ? lf::kInNormEmbed : lf::kInNormF32;
    LF_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, qkv_attn_kernel(ukv, in), 8 * lf::kWave, 0));
    fused_per_cu = std::min(fused_per_cu, n);
  }
  return LF_OK;
}

int set_lds_limits() {
  int rc;
  if ((rc = set_lds_limit_epi<lf::kEpiQKV>()) || (rc = set_lds_limit_epi<lf::kEpiSwiGLU>()) ||
      (rc = set_lds_limit_epi<lf::kEpiResid>()) || (rc = set_lds_limit_epi<lf::kEpiLogits>()))
    return rc;
  LF_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&lf::k_pf_gemm_db<lf::kPfStore>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lf::kPf2Lds));
  LF_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&lf::k_pf_gemm_db<lf::kPfAccum>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lf::kPf2Lds));
  LF_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&lf::k_pf_gemm_db<lf::kPfSwiGLU>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lf::kPf2Lds));
  return LF_OK;
}

// Optional per-kernel event brackets around each launch of enqueue_step.
struct StepTimer {
  hipEvent_t* ev;   // 2 per kernel (null: no events)
  int32_t* kinds;
  int cap, n;
  hipError_t err = hipSuccess;
  // only_kind >= 0: enqueue nothing but `reps` launches of that kernel of
  // layer only_layer (of every layer, in order, if only_layer < 0)
  int only_kind = -1, only_layer = -1, reps = 1;
  void before(hipStream_t st) {
    if (ev && n < cap && err == hipSuccess) err = hipEventRecord(ev[2 * n], st);
  }
  void after(hipStream_t st, int kind) {
    if (ev && n < cap && err == hipSuccess) {
      err = hipEventRecord(ev[2 * n + 1], st);
      kinds[n] = kind;
    }
    ++n;
  }
};

// Launch one kernel of a step (kind, layer l) through `launch`, bracketed by
// the timer's events, or as the timer's filter asks.
template <class F>
void emit_kernel(StepTimer* tm, hipStream_t st, int kind, int l, F&& launch) {
  if (!tm) {
    launch();
  } else if (tm->only_kind >= 0) {
    if (kind == tm->only_kind && (tm->only_layer < 0 || l == tm->only_layer))
      for (int r = 0; r < tm->reps; ++r) launch();
  } else {
    tm->before(st);
    launch();
    tm->after(st, kind);
  }
}

// Enqueue every kernel of one step. xin/xout: hidden mode input/output (null in token mode).
int enqueue_step(lf_model* m, lf_kv* kv, const float* xin, float* xout, hipStream_t st, StepTimer* tm = nullptr) {
  const Dims& D = m->D;
  const WsLayout& W = m->W;
  const lf_config& c = m->cfg;
  const bool hidden = D.V == 0;
  float* resid = hidden ? xout : m->at<float>(W.x);
  unsigned* counters = m->at<unsigned>(W.counters);
  const size_t layer_cache = static_cast<size_t>(D.lanes) * D.ctx * D.kpl * D.hd;

  lf::GemvArgs base{};
  base.eps = c.rms_eps;
  base.vocab = D.V;
  base.state = kv->state();
  base.tokens = kv->tokens();
  base.max_ctx = D.ctx;
  base.hd = D.hd;
  base.qpl = D.qpl;
  base.kpl = D.kpl;
  base.rope = m->at<float2>(W.rope);

  for (int l = 0; l < D.L; ++l) {
    // RMSNorm + QKV + rotary + KV append
    lf::GemvArgs a = base;
    a.W = m->at<half_t>(W.wqkv[l]);
    a.rows = D.qkv_rows;
    a.K = D.d;
    a.gain = m->at<half_t>(W.g1[l]);
    if (l == 0) {
      a.in_kind = hidden ? lf::kInNormF32 : lf::kInNormEmbed;
      a.x = xin;
      a.emb = hidden ? nullptr : m->at<half_t>(W.embed);
      a.resid_copy = resid;
    } else {
      a.in_kind = lf::kInNormF32;
      a.x = resid;
    }
    a.q = m->at<float>(W.q);
    a.kc = kv->kc() + l * layer_cache;
    a.vc = kv->vc() + l * layer_cache;

    // attention over the visible keys, split over key ranges, merged in-kernel
    const AttnPlan P = m->fused ? fused_plan(c, l) : attn_plan(c, l);
    lf::AttnXArgs t{};
    t.t.q = m->at<float>(W.q);
    t.t.kc = kv->kc() + l * layer_cache;
    t.t.vc = kv->vc() + l * layer_cache;
    t.t.state = kv->state();
    t.t.max_ctx = D.ctx;
    t.t.window = c.window[l];
    t.t.S = P.S;
    t.t.chunk = P.chunk;
    t.t.kpl = D.kpl;
    t.t.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D.hd)));
    t.part = m->at<lf::u64>(W.attn_part);
    t.o = m->at<float>(W.o);
    t.epochs = m->at<unsigned>(W.attn_epochs);
    t.abort = m->at<unsigned>(W.abort);
    t.S_max = W.S_max;
    t.n_kv = D.hkv;
    if (m->fused) {
      lf::QkvAttnArgs f{};
      f.g = a;
      f.g.qkvx = m->at<lf::u64>(W.qkvx);
      f.at = t;
      f.at.part = m->at<lf::u64>(W.fpart);
      f.at.S_max = kFusedSplits;
      f.class_epochs = m->at<unsigned>(W.class_epochs);
      emit_kernel(tm, st, LF_KERNEL_QKV_ATTN, l, [&] { launch_qkv_attn(f, st); });
    } else {
      emit_kernel(tm, st, LF_KERNEL_QKV, l, [&] { launch_gemv<lf::kEpiQKV>(a, st); });
      emit_kernel(tm, st, LF_KERNEL_ATTN, l, [&] { launch_attn(t, D.hd, D.G, D.hkv, m->attn_xcd[l] != 0, st); });
    }

    // O projection + residual
    a = base;
    a.W = m->at<half_t>(W.wo[l]);
    a.rows = D.d;
    a.K = D.qdim;
    a.in_kind = lf::kInF32;
    a.x = m->at<float>(W.o);
    a.y = resid;
    emit_kernel(tm, st, LF_KERNEL_O, l, [&] { launch_gemv<lf::kEpiResid>(a, st); });

    // RMSNorm + gate/up + SwiGLU
    a = base;
    a.W = m->at<half_t>(W.wgu[l]);
    a.rows = 2 * D.ffn;
    a.K = D.d;
    a.in_kind = lf::kInNormF32;
    a.x = resid;
    a.gain = m->at<half_t>(W.g2[l]);
    a.y = m->at<float>(W.act);
    emit_kernel(tm, st, LF_KERNEL_GATE_UP, l, [&] { launch_gemv<lf::kEpiSwiGLU>(a, st); });

    // down projection + residual (the last layer ends the step in hidden mode)
    a = base;
    a.W = m->at<half_t>(W.wd[l]);
    a.rows = D.d;
    a.K = D.ffn;
    a.in_kind = lf::kInF32;
    a.x = m->at<float>(W.act);
    a.y = resid;
    if (hidden && l == D.L - 1) a.counter = counters + D.hkv;
    emit_kernel(tm, st, LF_KERNEL_DOWN, l, [&] { launch_gemv<lf::kEpiResid>(a, st); });
  }
  if (!hidden) {
    // final RMSNorm + LM head + greedy argmax; ends the step
    lf::GemvArgs a = base;
    a.W = m->at<half_t>(W.lm);
    a.rows = D.V;
    a.K = D.d;
    a.in_kind = lf::kInNormF32;
    a.x = resid;
    a.gain = m->at<half_t>(W.gf);
    a.y = kv->logits();
    a.counter = counters + D.hkv;
    a.best = m->at<unsigned long long>(W.best);
    emit_kernel(tm, st, LF_KERNEL_LM_HEAD, D.L, [&] { launch_gemv<lf::kEpiLogits>(a, st); });
  }
  LF_HIP(hipPeekAtLastError());
  if (tm && tm->err != hipSuccess) return fail(LF_EHIP, "hipEventRecord: %s", hipGetErrorString(tm->err));
  return LF_OK;
}

// Recorded graphs a model keeps (single-sequence and batched, each): a key
// past that (a new sequence, hidden-state buffers or batch) runs its kernels
// eagerly, with the same results, rather than growing the cache without bound.
constexpr size_t kMaxGraphs = 64;

int run_step(lf_model* m, lf_kv* kv, const float* xin, float* xout, hipStream_t st) {
  if (m->mode == LF_MODE_EAGER) return enqueue_step(m, kv, xin, xout, st);
  hipGraphExec_t exec = nullptr;
  for (const GraphEntry& g : m->graphs)
    if (g.kv == kv && g.xin == xin && g.xout == xout) exec = g.exec;
  if (!exec && m->graphs.size() >= kMaxGraphs) return enqueue_step(m, kv, xin, xout, st);
  if (!exec) {
    // Record on the library's own stream (the caller's may be the legacy
    // default stream, which cannot be captured); nothing executes here.
    hipStream_t cs = m->capture_stream;
    LF_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
    const int rc = enqueue_step(m, kv, xin, xout, cs);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(cs, &graph);
    if (rc != LF_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return fail(LF_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
    const hipError_t ei = hipGraphInstantiateWithFlags(&exec, graph, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return fail(LF_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(ei));
    m->graphs.push_back({kv, xin, xout, exec});
  }
  LF_HIP(hipGraphLaunch(exec, st));
  return LF_OK;
}

void drop_graphs(lf_model* m, lf_kv* kv) {
  std::vector<GraphEntry> keep;
  for (const GraphEntry& g : m->graphs) {
    if (kv == nullptr || g.kv == kv)
      (void)hipGraphExecDestroy(g.exec);
    else
      keep.push_back(g);
  }
  m->graphs.swap(keep);
  std::vector<BatchGraph> bkeep;
  for (const BatchGraph& g : m->batch_graphs) {
    bool hit = kv == nullptr;
    for (int i = 0; i < g.n; ++i) hit = hit || g.kvs[i] == kv;
    if (hit)
      (void)hipGraphExecDestroy(g.exec);
    else
      bkeep.push_back(g);
  }
  m->batch_graphs.swap(bkeep);
}

// ------------------------------------------------------------ batched step

// Launch shape of a skinny GEMM: TPW tiles of 16 rows per workgroup (the
// largest of 4, 2, 1 that still gives 256 workgroups, one per CU) and KB
// k-steps per batch of loads: 8 KB of weights per wave and batch where the
// grid fits one workgroup per CU, half that where it is larger, so that two
// workgroups fit per CU (fewer registers) and the whole grid is resident at
// once; KB is even (k-steps are loaded in pairs) and at least 2.
struct BShape {
  int tpw, kb, blocks;
};
BShape bgemm_shape(int rows) {
  const int tiles = (rows + 15) / 16;
  int tpw = 1;
  for (int t : {4, 2})
    if ((tiles + t - 1) / t >= 256) {
      tpw = t;
      break;
    }
  const int blocks = (tiles + tpw - 1) / tpw;
  return {tpw, std::max(2, (blocks > 256 ? 4 : 8) / tpw), blocks};
}

template <int EPI, bool NORM>
const void* bgemm_fn(const BShape& sh) {
  if constexpr (EPI == lf::kBEpiResid && NORM) {
    return nullptr;  // a residual GEMM's input (attention output, SwiGLU) is never normalised
  } else {
#define LF_BGEMM(T, KB) if (sh.tpw == T && sh.kb == KB) return reinterpret_cast<const void*>(&lf::k_bgemm<EPI, T, NORM, KB>);
    LF_BGEMM(1, 8) LF_BGEMM(1, 4) LF_BGEMM(2, 4) LF_BGEMM(2, 2) LF_BGEMM(4, 2)
#undef LF_BGEMM
    return nullptr;
  }
}

template <int EPI, bool NORM>
int launch_bgemm(const lf::BGemmArgs& a, hipStream_t st) {
  const BShape sh = bgemm_shape(a.rows);
  void* args[] = {const_cast<lf::BGemmArgs*>(&a)};
  (void)hipLaunchKernel(bgemm_fn<EPI, NORM>(sh), dim3(sh.blocks), dim3(8 * lf::kWave), args, 0, st);
  return sh.blocks;  // partial sums of squares a residual GEMM writes per sequence
}

// The batched attention's splits: as many as keep about two workgroups per CU
// for the n sequences at once (the whole grid resident), at most kMaxSplits
// and at least 128 keys each; a split of more than 128 keys is read in
// double-buffered rounds of 128 (4 waves x 8 loads per lane).
// The S splits of one (sequence, kv head) are consecutive workgroups that
// wait on each other, so S is also capped by the device's room for the
// attention kernel (room: workgroups per CU x CUs, read at init).
AttnPlan batch_attn_plan(const lf_config& c, int layer, int n, int room) {
  const int visible = visible_keys(c, layer);
  const int want = std::max(1, 512 / (c.n_kv_heads * n));
  return split_plan(visible, std::min({want, (visible + 127) / 128, std::max(room, 1)}));
}
int batch_attn_u(int chunk, int hd) {
  const int per8 = lf::kWavesPerBlock * 8 * (512 / hd);  // keys per round at 8 loads per lane
  return chunk > per8 ? 0 : attn_loads_per_lane(chunk, hd);  // 0: rounds of 8, double-buffered
}

template <int HD, int G>
const void* battn_fn(int u) {
  return u == 4   ? reinterpret_cast<const void*>(&lf::k_battn<HD, G, 4, false>)
         : u == 8 ? reinterpret_cast<const void*>(&lf::k_battn<HD, G, 8, false>)
         : u == 0 ? reinterpret_cast<const void*>(&lf::k_battn<HD, G, 8, true>)
                  : reinterpret_cast<const void*>(&lf::k_battn<HD, G, 16, false>);
}
const void* battn_kernel(int hd, int G, int u) {
#define LF_BATTN_CASE(H, GG) if (hd == H && G == GG) return battn_fn<H, GG>(u);
  LF_BATTN_CASE(32, 1) LF_BATTN_CASE(32, 2) LF_BATTN_CASE(32, 4)
  LF_BATTN_CASE(64, 1) LF_BATTN_CASE(64, 2) LF_BATTN_CASE(64, 4)
  LF_BATTN_CASE(128, 1) LF_BATTN_CASE(128, 2) LF_BATTN_CASE(128, 4)
#undef LF_BATTN_CASE
  return nullptr;
}

// Enqueue every kernel of one batched step of the n sequences kvs[0..n).
int enqueue_batch_step(lf_model* m, lf_kv* const* kvs, int n, hipStream_t st) {
  const Dims& D = m->D;
  const WsLayout& W = m->W;
  const lf_config& c = m->cfg;
  const size_t layer_cache = static_cast<size_t>(D.lanes) * D.ctx * D.kpl * D.hd;
  lf::BatchSeqs q{};
  for (int i = 0; i < lf::kMaxBatch; ++i) {  // slots past n repeat sequence 0 (valid addresses)
    lf_kv* kv = kvs[i < n ? i : 0];
    q.state[i] = kv->state();
    q.tokens[i] = kv->tokens();
    q.kc[i] = kv->kc();
    q.vc[i] = kv->vc();
    q.logits[i] = kv->logits();
  }
  float* x = m->at<float>(W.bx);
  float* ss = m->at<float>(W.bss);
  half_t* fd = m->at<half_t>(W.bfd);
  half_t* fq = m->at<half_t>(W.bfq);
  half_t* ff = m->at<half_t>(W.bff);
  lf::BEmbedArgs ea{q, m->at<half_t>(W.embed), m->at<half_t>(W.g1[0]), x, fd, ss, D.d, D.V, D.ctx};
  hipLaunchKernelGGL(lf::k_bembed, dim3(n), dim3(lf::kBlock), 0, st, ea);
  int ss_n = 1;

  lf::BGemmArgs base{};
  base.eps = c.rms_eps;
  base.n = n;
  base.seq = q;
  base.layer_cache = layer_cache;
  base.rope = m->at<float2>(W.rope);
  base.hd = D.hd;
  base.qpl = D.qpl;
  base.kpl = D.kpl;
  base.max_ctx = D.ctx;
  base.ss = ss;
  base.ss_out = ss;
  for (int l = 0; l < D.L; ++l) {
    lf::BGemmArgs a = base;
    a.layer = l;
    a.W = m->at<half_t>(W.wqkv[l]);
    a.rows = D.qkv_rows;
    a.K = D.d;
    a.B = fd;
    a.ss_n = ss_n;
    a.y = m->at<float>(W.bq);
    a.y_stride = D.qdim;
    launch_bgemm<lf::kBEpiQKV, true>(a, st);

    const AttnPlan P = batch_attn_plan(c, l, n, m->battn_room);
    lf::AttnBArgs b{};
    b.a.t.max_ctx = D.ctx;
    b.a.t.window = c.window[l];
    b.a.t.S = P.S;
    b.a.t.chunk = P.chunk;
    b.a.t.kpl = D.kpl;
    b.a.t.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D.hd)));
    b.a.abort = m->at<unsigned>(W.abort);
    b.a.S_max = W.S_max;
    b.a.n_kv = D.hkv;
    b.seq = q;
    b.layer_cache = layer_cache;
    b.layer = l;
    b.q = m->at<float>(W.bq);
    b.ofrag = fq;
    b.part = m->at<lf::u64>(W.bpart);
    b.part_stride = static_cast<size_t>(D.hq) * W.S_max * (D.hd + 2);
    b.epochs = m->at<unsigned>(W.bepochs);
    b.q_dim = D.qdim;
    {
      void* args[] = {&b};
      (void)hipLaunchKernel(battn_kernel(D.hd, D.G, batch_attn_u(P.chunk, D.hd)), dim3(P.S, D.hkv, n),
                            dim3(lf::kBlock), args, 0, st);
    }

    a = base;
    a.layer = l;
    a.W = m->at<half_t>(W.wo[l]);
    a.rows = D.d;
    a.K = D.qdim;
    a.B = fq;
    a.y = x;
    a.y_stride = D.d;
    a.frag_out = fd;
    a.next_gain = m->at<half_t>(W.g2[l]);
    ss_n = launch_bgemm<lf::kBEpiResid, false>(a, st);

    a = base;
    a.layer = l;
    a.W = m->at<half_t>(W.wgu[l]);
    a.rows = 2 * D.ffn;
    a.K = D.d;
    a.B = fd;
    a.ss_n = ss_n;
    a.frag_out = ff;
    launch_bgemm<lf::kBEpiSwiGLU, true>(a, st);

    a = base;
    a.layer = l;
    a.W = m->at<half_t>(W.wd[l]);
    a.rows = D.d;
    a.K = D.ffn;
    a.B = ff;
    a.y = x;
    a.y_stride = D.d;
    a.frag_out = fd;
    a.next_gain = m->at<half_t>(l + 1 < D.L ? W.g1[l + 1] : W.gf);
    ss_n = launch_bgemm<lf::kBEpiResid, false>(a, st);
  }
  lf::BGemmArgs a = base;
  a.W = m->at<half_t>(W.lm);
  a.rows = D.V;
  a.K = D.d;
  a.B = fd;
  a.ss_n = ss_n;
  a.counter = m->at<unsigned>(W.bcounter);
  a.best = m->at<unsigned long long>(W.bbest);
  launch_bgemm<lf::kBEpiLogits, true>(a, st);
  LF_HIP(hipPeekAtLastError());
  return LF_OK;
}

// Scratch of the batched prompt pass for chunks of mc positions.
struct PfLayout {
  size_t x, y, h, q, total;
};

PfLayout pf_layout(const Dims& D, int mc) {
  PfLayout P;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const size_t rows = static_cast<size_t>(mc);
  P.x = take(rows * D.d * sizeof(float));
  P.y = take(rows * std::max(D.qkv_rows, 2 * D.ffn) * sizeof(float));
  P.h = take(rows * std::max(std::max(D.d, D.ffn), D.qdim) * sizeof(float));
  P.q = take(rows * D.qdim * sizeof(float));
  P.total = off;
  return P;
}

// Device scratch that a prompt-pass GEMM may use for the sums of split
// tiles: `pieces` blocks of kPfBM x kPf2BN fp32 at p (none if p is null).
struct PfPart {
  float* p;
  int pieces;
};
constexpr size_t kPfPieceBytes = static_cast<size_t>(lf::kPfBM) * lf::kPf2BN * sizeof(float);

// The free bytes [from, to) of the chunk scratch as a PfPart.
PfPart pf_part(char* ws, size_t from, size_t to) {
  from = align_up(from);
  if (to <= from) return {nullptr, 0};
  const size_t n = std::min<size_t>((to - from) / kPfPieceBytes, 1 << 20);
  return {n ? reinterpret_cast<float*>(ws + from) : nullptr, static_cast<int>(n)};
}

// How many K pieces to cut each tile of the last, partly filled round into
// (0: none). With one workgroup per CU and T tiles of equal work the launch
// takes ceil(T / ncu) rounds; splitting the R = T mod ncu tail tiles into s
// pieces makes it floor(T / ncu) + ceil(R s / ncu) / s rounds, plus a fixup
// pass that reads the pieces once. Taken where it saves at least a quarter of
// a round; each piece keeps at least 4 K steps, and the XCD mapping of
// k_pf_gemm_db wants the whole tiles and the pieces in multiples of 8.
int pf_split(int T, int K, int ncu, int cap) {
  const int R = T % ncu, nsteps = (K + lf::kPfBK - 1) / lf::kPfBK;
  if (R == 0 || (T - R) % 8) return 0;
  const double whole = T / ncu + 1;
  double best = whole - 0.25;
  int pick = 0;
  for (int s = 2; s <= 8; ++s) {
    if ((R * s) % 8 || R * s > cap || nsteps < 4 * s) continue;
    const double rounds = T / ncu + static_cast<double>((R * s + ncu - 1) / ncu) / s;
    if (rounds < best - 1e-9) {
      best = rounds;
      pick = s;
    }
  }
  return pick;
}

// The double-buffered 128 x 256 kernel where its grid gives every CU a
// workgroup (it holds one per CU), its tail tiles split over K where that
// shortens the launch (part: scratch for their sums); else the 128 x 128
// kernel (two per CU).
template <int EPI>
void launch_pf_gemm(const half_t* A, const half_t* W, float* C, int M, int N, int K, int ncu, PfPart part,
                    hipStream_t st) {
  const int tm = (M + lf::kPfBM - 1) / lf::kPfBM, tn2 = (N + lf::kPf2BN - 1) / lf::kPf2BN;
  const int T = tm * tn2;
  if (T >= ncu) {
    lf::PfGemmArgs g{A, W, C, M, N, K, tm, tn2};
    const int s = part.p ? pf_split(T, K, ncu, part.pieces) : 0;
    if (s == 0) {
      hipLaunchKernelGGL(lf::k_pf_gemm_db<EPI>, dim3(T), dim3(lf::kPf2Threads), lf::kPf2Lds, st, g);
      return;
    }
    const int R = T % ncu;
    g.full = T - R;
    g.split = s;
    g.part = part.p;
    hipLaunchKernelGGL(lf::k_pf_gemm_db<EPI>, dim3(g.full + R * s), dim3(lf::kPf2Threads), lf::kPf2Lds, st, g);
    hipLaunchKernelGGL(lf::k_pf_fixup<EPI>, dim3(R, lf::kPfBM), dim3(lf::kPf2BN), 0, st, g);
    return;
  }
  lf::PfGemmArgs g{A, W, C, M, N, K, tm, (N + lf::kPfBN - 1) / lf::kPfBN};
  hipLaunchKernelGGL(lf::k_pf_gemm<EPI>, dim3(g.tiles_m * g.tiles_n), dim3(lf::kPfThreads), 0, st, g);
}

// Two blocks of 32 queries per workgroup share its key / value tiles where
// the group has at most 2 query heads (4 waves), one block for 4 query heads.
void launch_pf_attn(const lf::PfAttnArgs& a, int hd, int G, int n_kv, hipStream_t st) {
#define LF_PF_ATTN(HD, GG)                                                                          \
  if (hd == HD && G == GG) {                                                                        \
    constexpr int QB = GG <= 2 ? 2 : 1;                                                             \
    hipLaunchKernelGGL((lf::k_pf_attn<HD, GG, QB>), dim3((a.M + 32 * QB - 1) / (32 * QB) * n_kv),    \
                       dim3(QB * GG * lf::kWave), 0, st, a);                                        \
    return;                                                                                         \
  }
  LF_PF_ATTN(128, 1) LF_PF_ATTN(128, 2) LF_PF_ATTN(128, 4)
  LF_PF_ATTN(64, 1) LF_PF_ATTN(64, 2) LF_PF_ATTN(64, 4)
  LF_PF_ATTN(32, 1) LF_PF_ATTN(32, 2) LF_PF_ATTN(32, 4)
#undef LF_PF_ATTN
}

// One chunk of the batched prompt pass: M positions from pos0 through every
// layer (the residual rows end in P.x).
void enqueue_pf_chunk(lf_model* m, lf_kv* kv, char* ws, const PfLayout& P, int M, int pos0, hipStream_t st) {
  const Dims& D = m->D;
  const WsLayout& W = m->W;
  const lf_config& c = m->cfg;
  const size_t layer_cache = static_cast<size_t>(D.lanes) * D.ctx * D.kpl * D.hd;
  float* x = reinterpret_cast<float*>(ws + P.x);
  float* y = reinterpret_cast<float*>(ws + P.y);
  half_t* h = reinterpret_cast<half_t*>(ws + P.h);  // GEMM inputs: split rows (4 bytes per activation)
  half_t* ys = reinterpret_cast<half_t*>(ws + P.y);  // the SwiGLU output, split rows
  float* q = reinterpret_cast<float*>(ws + P.q);
  // Scratch free during each GEMM, for split-tile sums: past the normed
  // input in h through q (QKV, gate/up), y (O: its QKV rows are consumed),
  // h through q (down: its input is y).
  const size_t rows = static_cast<size_t>(M);
  const PfPart past_norm = pf_part(ws, P.h + rows * D.d * sizeof(float), P.total);
  const PfPart in_y = pf_part(ws, P.y, P.h), from_h = pf_part(ws, P.h, P.total);
  for (int l = 0; l < D.L; ++l) {
    lf::PfNormArgs na{x, h, m->at<half_t>(W.g1[l]), l == 0 ? m->at<half_t>(W.embed) : nullptr, kv->tokens(), kv->state(),
                      M, D.d, D.V, pos0, c.rms_eps};
    hipLaunchKernelGGL(lf::k_pf_norm, dim3(M), dim3(lf::kBlock), 0, st, na);
    launch_pf_gemm<lf::kPfStore>(h, m->at<half_t>(W.wqkv[l]), y, M, D.qkv_rows, D.d, m->ncu, past_norm, st);
    lf::PfQkvArgs qa{y, q, kv->kc() + l * layer_cache, kv->vc() + l * layer_cache, m->at<float2>(W.rope),
                     M, D.qkv_rows, D.hd, D.qpl, D.kpl, D.hq, D.ctx, pos0};
    hipLaunchKernelGGL(lf::k_pf_qkv, dim3((D.qkv_rows / 8 + lf::kBlock - 1) / lf::kBlock, M), dim3(lf::kBlock), 0, st, qa);
    lf::PfAttnArgs aa{q, kv->kc() + l * layer_cache, kv->vc() + l * layer_cache, h, M, pos0, D.ctx, c.window[l], D.kpl,
                      D.hq, D.hkv, static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D.hd)))};
    launch_pf_attn(aa, D.hd, D.G, D.hkv, st);
    launch_pf_gemm<lf::kPfAccum>(h, m->at<half_t>(W.wo[l]), x, M, D.d, D.qdim, m->ncu, in_y, st);
    na.gain = m->at<half_t>(W.g2[l]);
    na.emb = nullptr;
    hipLaunchKernelGGL(lf::k_pf_norm, dim3(M), dim3(lf::kBlock), 0, st, na);
    // gate/up with SwiGLU in its epilogue: the activations [M][ffn] land in y as split rows
    launch_pf_gemm<lf::kPfSwiGLU>(h, m->at<half_t>(W.wgu[l]), y, M, 2 * D.ffn, D.d, m->ncu, past_norm, st);
    launch_pf_gemm<lf::kPfAccum>(ys, m->at<half_t>(W.wd[l]), x, M, D.d, D.ffn, m->ncu, from_h, st);
  }
}

// Arguments shared by both prompt-pass entry points.
int prefill_check(lf_model* m, lf_kv* kv, int n, int chunk) {
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  if (m->D.V == 0) return fail(LF_EINVAL, "the prompt pass needs vocab > 0");
  if (n < 1) return fail(LF_EINVAL, "n = %d < 1", n);
  if (chunk < 1 || chunk > LF_MAX_PREFILL_CHUNK) return fail(LF_EINVAL, "chunk %d out of [1, %d]", chunk, LF_MAX_PREFILL_CHUNK);
  if (static_cast<long>(kv->len) + n > m->D.ctx) return fail(LF_ERANGE, "len %d + n %d > max_ctx %d", kv->len, n, m->D.ctx);
  return LF_OK;
}

// The prompt pass over n positions in chunks of `chunk`, with its scratch at
// ws (at least pf_layout(D, chunk).total bytes, 256-byte aligned).
int prefill_run(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int n, int chunk, char* ws, hipStream_t st) {
  const Dims& D = m->D;
  const WsLayout& W = m->W;
  const PfLayout P = pf_layout(D, chunk);
  hipLaunchKernelGGL(lf::k_put_tokens, dim3((n + 255) / 256), dim3(256), 0, st, kv->state(), kv->tokens(), kv->len, d_tokens, n);
  int last = 0;
  for (int c0 = 0; c0 < n; c0 += chunk) {
    last = std::min(chunk, n - c0);
    enqueue_pf_chunk(m, kv, ws, P, last, kv->len + c0, st);
  }
  hipLaunchKernelGGL(lf::k_pf_finish, dim3(1), dim3(lf::kBlock), 0, st,
                     reinterpret_cast<const float*>(ws + P.x) + static_cast<size_t>(last - 1) * D.d, m->at<float>(W.x), D.d,
                     kv->state(), kv->len + n - 1);
  // final RMSNorm + LM head + greedy argmax of the last position (the decode step's kernel)
  lf::GemvArgs a{};
  a.eps = m->cfg.rms_eps;
  a.vocab = D.V;
  a.state = kv->state();
  a.tokens = kv->tokens();
  a.max_ctx = D.ctx;
  a.hd = D.hd;
  a.qpl = D.qpl;
  a.kpl = D.kpl;
  a.rope = m->at<float2>(W.rope);
  a.W = m->at<half_t>(W.lm);
  a.rows = D.V;
  a.K = D.d;
  a.in_kind = lf::kInNormF32;
  a.x = m->at<float>(W.x);
  a.gain = m->at<half_t>(W.gf);
  a.y = kv->logits();
  a.counter = m->at<unsigned>(W.counters) + D.hkv;
  a.best = m->at<unsigned long long>(W.best);
  launch_gemv<lf::kEpiLogits>(a, st);
  LF_HIP(hipPeekAtLastError());
  kv->len += n;
  return LF_OK;
}

}  // namespace

// Scratch of lf_prefill_batched_static, for callers that cannot allocate
// device memory. Each device the library runs on holds its own copy until the
// process ends; every call on a device shares it (calls that overlap on one
// device race). Host code never uses the name as an address: the device
// address comes from hipGetSymbolAddress, once per device (static_scratch).
constexpr size_t kStaticScratchBytes = LF_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes == size_t(32) << 20, "the header states 32 MiB");
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// The current device's address of `scratch`, looked up on the first call for
// that device (with it current) and kept.
int static_scratch(void** out) {
  int dev = 0;
  LF_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(LF_EINVAL, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(LF_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LF_OK;
}

// The largest chunk whose prompt-pass scratch fits the static scratch (0 if
// not even one position fits).
int static_chunk_max(const Dims& D) {
  if (pf_layout(D, 1).total > kStaticScratchBytes) return 0;
  int lo = 1, hi = LF_MAX_PREFILL_CHUNK;  // the scratch grows with the chunk
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (pf_layout(D, mid).total <= kStaticScratchBytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace

// ===================================================================== C ABI

extern "C" {

const char* lf_last_error(void) { return g_err.c_str(); }

size_t lf_workspace_bytes(const lf_config* cfg) {
  if (validate(cfg) != LF_OK) return 0;
  return ws_layout(*cfg).total;
}

size_t lf_kv_bytes(const lf_config* cfg) {
  if (validate(cfg) != LF_OK) return 0;
  return kv_layout(*cfg).total;
}

// Whether workgroups whose launch indices are congruent modulo 8 run on one
// XCD (workgroups are dealt to the XCDs in turn, continuing from where the
// previous launch stopped): read each workgroup's XCD in launches of 256,
// 37 and 256 workgroups. Uses the attention state buffer as scratch and
// zeroes it again.
static int probe_xcd_classes(lf_model* m, hipStream_t st) {
  unsigned* ids = m->at<unsigned>(m->W.attn_part);
  hipLaunchKernelGGL(lf::k_xcd_ids, dim3(256), dim3(64), 0, st, ids);
  hipLaunchKernelGGL(lf::k_xcd_ids, dim3(37), dim3(64), 0, st, ids + 256);
  hipLaunchKernelGGL(lf::k_xcd_ids, dim3(256), dim3(64), 0, st, ids + 512);
  std::vector<unsigned> h(768);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(h.data(), ids, h.size() * sizeof(unsigned), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(256), 0, st, ids, 0u, h.size());
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) return fail(LF_EHIP, "XCD probe: %s", hipGetErrorString(e));
  bool ok = true;
  for (int b = 0; b < 256; ++b) ok = ok && h[b] == h[b % 8] && h[512 + b] == h[512 + b % 8];
  m->xcd_classes = ok;
  return LF_OK;
}

int lf_model_init(const lf_config* cfg, const lf_weight_ptrs* w, void* d_workspace, size_t ws_bytes,
                  void* stream, lf_model** out) {
  if (!out) return fail(LF_EINVAL, "out is null");
  *out = nullptr;
  int rc = validate(cfg);
  if (rc) return rc;
  if (!w || !d_workspace) return fail(LF_EINVAL, "weights or workspace is null");
  if (reinterpret_cast<uintptr_t>(d_workspace) % kAlign) return fail(LF_EINVAL, "workspace not 256-byte aligned");
  const Dims D = dims(*cfg);
  const WsLayout W = ws_layout(*cfg);
  if (ws_bytes < W.total) return fail(LF_EINVAL, "workspace %zu bytes < %zu needed", ws_bytes, W.total);
  if (!w->attn_norm || !w->wqkv || !w->wo || !w->ffn_norm || !w->wgate_up || !w->wdown)
    return fail(LF_EINVAL, "per-layer weight arrays must not be null");
  for (int l = 0; l < D.L; ++l)
    if (!w->attn_norm[l] || !w->wqkv[l] || !w->wo[l] || !w->ffn_norm[l] || !w->wgate_up[l] || !w->wdown[l])
      return fail(LF_EINVAL, "layer %d has a null weight pointer", l);
  if (D.V && (!w->embed || !w->lm_head || !w->final_norm)) return fail(LF_EINVAL, "embed, lm_head and final_norm required when vocab > 0");
  if ((rc = set_lds_limits())) return rc;

  lf_model* m = new (std::nothrow) lf_model();
  if (!m) return fail(LF_EINVAL, "out of host memory");
  m->cfg = *cfg;
  m->D = D;
  m->W = W;
  m->ws = static_cast<char*>(d_workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto bail = [&](int code) {
    if (m->capture_stream) (void)hipStreamDestroy(m->capture_stream);
    delete m;
    return code;
  };
  if (hipStreamCreateWithFlags(&m->capture_stream, hipStreamNonBlocking) != hipSuccess)
    return bail(fail(LF_EHIP, "capture stream: %s", hipGetErrorString(hipGetLastError())));
  const size_t h = sizeof(half_t);

  for (int l = 0; l < D.L; ++l) {
    lf::RepackArgs r{};
    r.K = D.d; r.hd = D.hd; r.n_q = D.hq; r.n_kv = D.hkv; r.qpl = D.qpl; r.kpl = D.kpl; r.ffn = D.ffn;
    r.dst = m->at<half_t>(W.wqkv[l]);
    r.src = static_cast<const half_t*>(w->wqkv[l]);
    r.rows = D.qkv_rows;
    r.mode = 0;
    hipLaunchKernelGGL(lf::k_repack, dim3(r.rows), dim3(lf::kBlock), 0, st, r);
    r.dst = m->at<half_t>(W.wgu[l]);
    r.src = static_cast<const half_t*>(w->wgate_up[l]);
    r.rows = 2 * D.ffn;
    r.mode = 1;
    hipLaunchKernelGGL(lf::k_repack, dim3(r.rows), dim3(lf::kBlock), 0, st, r);
    if (hipMemcpyAsync(m->at<half_t>(W.wo[l]), w->wo[l], static_cast<size_t>(D.d) * D.qdim * h, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(m->at<half_t>(W.wd[l]), w->wdown[l], static_cast<size_t>(D.d) * D.ffn * h, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(m->at<half_t>(W.g1[l]), w->attn_norm[l], D.d * h, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(m->at<half_t>(W.g2[l]), w->ffn_norm[l], D.d * h, hipMemcpyDeviceToDevice, st))
      return bail(fail(LF_EHIP, "weight copy failed: %s", hipGetErrorString(hipGetLastError())));
  }
  if (D.V) {
    if (hipMemcpyAsync(m->at<half_t>(W.embed), w->embed, static_cast<size_t>(D.V) * D.d * h, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(m->at<half_t>(W.lm), w->lm_head, static_cast<size_t>(D.V) * D.d * h, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(m->at<half_t>(W.gf), w->final_norm, D.d * h, hipMemcpyDeviceToDevice, st))
      return bail(fail(LF_EHIP, "embedding/head copy failed: %s", hipGetErrorString(hipGetLastError())));
  }
  // Rotary table: angle p * theta^(-2c/hd) evaluated in double, stored as fp32 (cos, sin).
  std::vector<float2> rope(static_cast<size_t>(D.ctx) * (D.hd / 2));
  for (int p = 0; p < D.ctx; ++p)
    for (int c = 0; c < D.hd / 2; ++c) {
      const double inv = std::pow(static_cast<double>(cfg->rope_theta), -2.0 * c / D.hd);
      const double ang = p * inv;
      rope[static_cast<size_t>(p) * (D.hd / 2) + c] = make_float2(static_cast<float>(std::cos(ang)), static_cast<float>(std::sin(ang)));
    }
  if (hipMemcpyAsync(m->at<float2>(W.rope), rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice, st))
    return bail(fail(LF_EHIP, "rope upload failed: %s", hipGetErrorString(hipGetLastError())));
  const int nctr = D.hkv + 4;
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.counters), 0u, size_t(nctr));
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.best), 0u, size_t(2));
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.abort), 0u, size_t(1));
  // tagged exchange words start with tag 0 (no epoch is 0)
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(256), dim3(256), 0, st, m->at<unsigned>(W.tagged_begin), 0u,
                     (W.tagged_end - W.tagged_begin) / sizeof(unsigned));
  // attention: split states are tagged with the kv head's epoch, which starts at 1
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.attn_epochs), 1u, size_t(D.hkv));
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.class_epochs), 1u, size_t(8));
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.bepochs), 1u,
                     size_t(lf::kMaxBatch) * D.hkv);
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.bbest), 0u, size_t(2 * lf::kMaxBatch));
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, st, m->at<unsigned>(W.bcounter), 0u, size_t(1));
  // batched step buffers zeroed: the operands are zero past K and in the
  // columns of sequences a batch does not use
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(64), dim3(256), 0, st, m->at<unsigned>(W.bx), 0u,
                     (W.bss + lf::kMaxBatch * lf::kSsStride * sizeof(float) - W.bx) / sizeof(unsigned));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return bail(fail(LF_EHIP, "model setup: %s", hipGetErrorString(e)));
  if ((rc = probe_xcd_classes(m, st))) return bail(rc);
  if ((rc = static_scratch(&m->scratch))) return bail(rc);
  int dev = 0, ncu = 0, attn_per_cu = 0, fused_per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return bail(fail(LF_EHIP, "device query: %s", hipGetErrorString(hipGetLastError())));
  if ((rc = attention_room(*cfg, attn_per_cu, fused_per_cu))) return bail(rc);
  if ((rc = plan_attention(*cfg, ncu, attn_per_cu, fused_per_cu, m->xcd_classes, m->fused_ok, m->attn_xcd)))
    return bail(rc);
  m->fused = m->fused_ok;
  m->ncu = ncu;
  if (m->D.V) {  // the batched step's attention kernels (lf_decode_step_batch needs a vocabulary)
    int per_cu = 1 << 20;
    for (int u : {4, 8, 16, 0}) {
      int k = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&k, battn_kernel(m->D.hd, m->D.G, u), lf::kBlock, 0) != hipSuccess)
        k = 0;  // then one split per (sequence, kv head): nothing waits on another workgroup
      per_cu = std::min(per_cu, k);
    }
    (void)hipGetLastError();
    m->battn_room = per_cu * ncu;
  }
  *out = m;
  return LF_OK;
}

int lf_plan_attention(const lf_config* cfg, int32_t n_cu, int32_t attn_wg_per_cu, int32_t fused_wg_per_cu,
                      int32_t xcd_classes, int32_t* fused, int32_t* xcd_layers) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!fused || !xcd_layers) return fail(LF_EINVAL, "null argument");
  if (n_cu < 1 || attn_wg_per_cu < 0 || fused_wg_per_cu < 0) return fail(LF_EINVAL, "need n_cu >= 1 and rooms >= 0");
  bool f = false;
  std::vector<char> x;
  if ((rc = plan_attention(*cfg, n_cu, attn_wg_per_cu, fused_wg_per_cu, xcd_classes != 0, f, x))) return rc;
  *fused = f ? 1 : 0;
  for (int l = 0; l < cfg->n_layers; ++l) xcd_layers[l] = x[l];
  return LF_OK;
}

void lf_model_free(lf_model* m) {
  if (!m) return;
  // Sequences may outlive their model (lf_kv_free may come later): detach
  // them so that they never touch the freed model.
  for (lf_kv* kv : m->kvs) kv->m = nullptr;
  drop_graphs(m, nullptr);
  if (m->capture_stream) (void)hipStreamDestroy(m->capture_stream);
  for (hipEvent_t e : m->events) (void)hipEventDestroy(e);
  delete m;
}

int lf_model_set_graph(lf_model* m, int enabled) {
  if (!m) return fail(LF_EINVAL, "model is null");
  m->mode = enabled ? LF_MODE_GRAPH : LF_MODE_EAGER;
  return LF_OK;
}

int lf_model_set_mode(lf_model* m, int mode) {
  if (!m) return fail(LF_EINVAL, "model is null");
  if (mode != LF_MODE_EAGER && mode != LF_MODE_GRAPH) return fail(LF_EINVAL, "unknown mode %d", mode);
  m->mode = mode;
  return LF_OK;
}

int lf_model_mode(const lf_model* m) { return m ? m->mode : -1; }

int lf_model_set_fused(lf_model* m, int enabled) {
  if (!m) return fail(LF_EINVAL, "model is null");
  if (enabled && !m->fused_ok) return fail(LF_EINVAL, "QKV and attention cannot run fused for this shape or device");
  if (m->fused != (enabled != 0)) drop_graphs(m, nullptr);  // recorded graphs hold the other kernels
  m->fused = enabled != 0;
  return LF_OK;
}

int lf_model_fused(const lf_model* m) { return m ? (m->fused ? 1 : 0) : -1; }

int lf_model_raise_give_up(lf_model* m, void* stream) {
  if (!m) return fail(LF_EINVAL, "model is null");
  hipLaunchKernelGGL(lf::k_fill_u32, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), m->at<unsigned>(m->W.abort),
                     1u, size_t(1));
  LF_HIP(hipPeekAtLastError());
  return LF_OK;
}

int lf_kv_alloc(lf_model* m, void* d_buf, size_t bytes, lf_kv** out) {
  if (!m || !d_buf || !out) return fail(LF_EINVAL, "null argument");
  *out = nullptr;
  if (reinterpret_cast<uintptr_t>(d_buf) % kAlign) return fail(LF_EINVAL, "sequence buffer not 256-byte aligned");
  const KvLayout K = kv_layout(m->cfg);
  if (bytes < K.total) return fail(LF_EINVAL, "sequence buffer %zu bytes < %zu needed", bytes, K.total);
  LF_HIP(hipMemset(static_cast<char*>(d_buf) + K.state, 0, K.tokens - K.state + (m->D.ctx + 1) * sizeof(int32_t)));
  LF_HIP(hipDeviceSynchronize());
  lf_kv* kv = new (std::nothrow) lf_kv();
  if (!kv) return fail(LF_EINVAL, "out of host memory");
  kv->m = m;
  kv->buf = static_cast<char*>(d_buf);
  kv->K = K;
  kv->len = 0;
  m->kvs.push_back(kv);
  *out = kv;
  return LF_OK;
}

void lf_kv_free(lf_kv* kv) {
  if (!kv) return;
  if (lf_model* m = kv->m) {
    drop_graphs(m, kv);
    for (size_t i = 0; i < m->kvs.size(); ++i)
      if (m->kvs[i] == kv) {
        m->kvs.erase(m->kvs.begin() + i);
        break;
      }
  }
  delete kv;
}

int lf_kv_cache_ptrs(const lf_kv* kv, void** d_k, void** d_v) {
  if (!kv || !d_k || !d_v) return fail(LF_EINVAL, "null argument");
  *d_k = kv->kc();
  *d_v = kv->vc();
  return LF_OK;
}

int32_t lf_kv_len(const lf_kv* kv) { return kv ? kv->len : -1; }

int lf_kv_tokens(const lf_kv* kv, int32_t* d_out, int32_t start, int32_t n, void* stream) {
  if (!kv || !d_out) return fail(LF_EINVAL, "null argument");
  if (!kv->m) return fail(LF_EINVAL, "the sequence's model was freed");
  if (start < 0 || n < 0 || static_cast<long>(start) + n > kv->m->D.ctx + 1)
    return fail(LF_ERANGE, "tokens [%d, %d) outside [0, %d]", start, start + n, kv->m->D.ctx + 1);
  if (n == 0) return LF_OK;
  LF_HIP(hipMemcpyAsync(d_out, kv->tokens() + start, static_cast<size_t>(n) * sizeof(int32_t), hipMemcpyDeviceToDevice,
                        static_cast<hipStream_t>(stream)));
  return LF_OK;
}

int lf_kv_set_len(lf_kv* kv, int32_t len, void* stream) {
  if (!kv) return fail(LF_EINVAL, "kv is null");
  if (!kv->m) return fail(LF_EINVAL, "the sequence's model was freed");
  if (len < 0 || len > kv->m->D.ctx) return fail(LF_ERANGE, "length %d out of [0, %d]", len, kv->m->D.ctx);
  hipLaunchKernelGGL(lf::k_set_pos, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), kv->state(), kv->tokens(), len,
                     static_cast<const int32_t*>(nullptr), kv->m->at<unsigned>(kv->m->W.abort));
  LF_HIP(hipPeekAtLastError());
  kv->len = len;
  return LF_OK;
}

int lf_prefill(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int32_t n, void* stream) {
  if (!m || !kv || !d_tokens) return fail(LF_EINVAL, "null argument");
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  if (m->D.V == 0) return fail(LF_EINVAL, "lf_prefill needs vocab > 0");
  if (n < 1) return fail(LF_EINVAL, "n = %d < 1", n);
  if (static_cast<long>(kv->len) + n > m->D.ctx) return fail(LF_ERANGE, "len %d + n %d > max_ctx %d", kv->len, n, m->D.ctx);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(lf::k_put_tokens, dim3((n + 255) / 256), dim3(256), 0, st, kv->state(), kv->tokens(), kv->len, d_tokens, n);
  LF_HIP(hipPeekAtLastError());
  for (int i = 0; i < n; ++i) {
    const int rc = run_step(m, kv, nullptr, nullptr, st);
    if (rc) return rc;
    kv->len += 1;
  }
  return LF_OK;
}

size_t lf_prefill_workspace_bytes(const lf_config* cfg, int32_t chunk) {
  if (validate(cfg) != LF_OK || chunk < 1 || chunk > LF_MAX_PREFILL_CHUNK) return 0;
  return pf_layout(dims(*cfg), chunk).total;
}

int lf_prefill_batched(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int32_t n, int32_t chunk, void* d_workspace,
                       size_t ws_bytes, void* stream) {
  if (!m || !kv || !d_tokens || !d_workspace) return fail(LF_EINVAL, "null argument");
  int rc = prefill_check(m, kv, n, chunk);
  if (rc) return rc;
  if (reinterpret_cast<uintptr_t>(d_workspace) % kAlign) return fail(LF_EINVAL, "workspace not 256-byte aligned");
  const size_t need = pf_layout(m->D, chunk).total;
  if (ws_bytes < need) return fail(LF_EINVAL, "workspace %zu bytes < %zu needed for chunk %d", ws_bytes, need, chunk);
  return prefill_run(m, kv, d_tokens, n, chunk, static_cast<char*>(d_workspace), static_cast<hipStream_t>(stream));
}

int lf_prefill_batched_static(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int32_t n, int32_t chunk, void* stream) {
  if (!m || !kv || !d_tokens) return fail(LF_EINVAL, "null argument");
  const int fit = static_chunk_max(m->D);
  if (fit < 1) return fail(LF_EINVAL, "one position of this shape needs more than the %zu-byte static scratch", kStaticScratchBytes);
  if (chunk == 0) chunk = std::min(fit, std::max(n, 1));
  int rc = prefill_check(m, kv, n, chunk);
  if (rc) return rc;
  if (chunk > fit)
    return fail(LF_EINVAL, "chunk %d needs %zu bytes of scratch; the static scratch holds %zu (at most %d positions per chunk)",
                chunk, pf_layout(m->D, chunk).total, kStaticScratchBytes, fit);
  if (!m->scratch) return fail(LF_EINVAL, "no static scratch address for the model's device");
  return prefill_run(m, kv, d_tokens, n, chunk, static_cast<char*>(m->scratch), static_cast<hipStream_t>(stream));
}

int lf_decode_step(lf_model* m, lf_kv* kv, const int32_t* d_token, void* stream) {
  if (!m || !kv) return fail(LF_EINVAL, "null argument");
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  if (m->D.V == 0) return fail(LF_EINVAL, "lf_decode_step needs vocab > 0; use lf_decode_step_hidden");
  if (kv->len >= m->D.ctx) return fail(LF_ERANGE, "sequence is full (%d positions)", m->D.ctx);
  if (!d_token && kv->len == 0) return fail(LF_EINVAL, "no previous position to take a greedy token from");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_token) {
    hipLaunchKernelGGL(lf::k_set_pos, dim3(1), dim3(64), 0, st, kv->state(), kv->tokens(), kv->len, d_token,
                       static_cast<unsigned*>(nullptr));
    LF_HIP(hipPeekAtLastError());
  }
  const int rc = run_step(m, kv, nullptr, nullptr, st);
  if (rc) return rc;
  kv->len += 1;
  return LF_OK;
}

int lf_decode_step_batch(lf_model* m, lf_kv* const* kvs, int32_t n, const int32_t* d_tokens, void* stream) {
  if (!m || !kvs) return fail(LF_EINVAL, "null argument");
  if (m->D.V == 0) return fail(LF_EINVAL, "lf_decode_step_batch needs vocab > 0");
  if (n < 1 || n > LF_MAX_BATCH) return fail(LF_EINVAL, "n = %d out of [1, %d]", n, LF_MAX_BATCH);
  for (int i = 0; i < n; ++i) {
    lf_kv* kv = kvs[i];
    if (!kv) return fail(LF_EINVAL, "sequence %d is null", i);
    if (kv->m != m) return fail(LF_EINVAL, "sequence %d belongs to another model", i);
    for (int j = 0; j < i; ++j)
      if (kvs[j] == kv) return fail(LF_EINVAL, "sequence %d appears twice", i);
    if (kv->len >= m->D.ctx) return fail(LF_ERANGE, "sequence %d is full (%d positions)", i, m->D.ctx);
    if (!d_tokens && kv->len == 0) return fail(LF_EINVAL, "sequence %d has no previous position to take a greedy token from", i);
  }
  // one sequence: the single-sequence step is faster (its GEMVs use every
  // lane; the batched GEMMs would fill 1 of their 16 operand columns)
  if (n == 1) return lf_decode_step(m, kvs[0], d_tokens, stream);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_tokens) {
    lf::BTokArgs t{};
    for (int i = 0; i < n; ++i) {
      t.seq.state[i] = kvs[i]->state();
      t.seq.tokens[i] = kvs[i]->tokens();
      t.len[i] = kvs[i]->len;
    }
    t.tokens = d_tokens;
    t.n = n;
    hipLaunchKernelGGL(lf::k_bset_tokens, dim3(1), dim3(64), 0, st, t);
    LF_HIP(hipPeekAtLastError());
  }
  hipGraphExec_t exec = nullptr;
  if (m->mode != LF_MODE_EAGER)
    for (const BatchGraph& g : m->batch_graphs) {
      bool same = g.n == n;
      for (int i = 0; same && i < n; ++i) same = g.kvs[i] == kvs[i];
      if (same) exec = g.exec;
    }
  if (m->mode == LF_MODE_EAGER || (!exec && m->batch_graphs.size() >= kMaxGraphs)) {
    const int rc = enqueue_batch_step(m, kvs, n, st);
    if (rc) return rc;
  } else {
    if (!exec) {
      hipStream_t cs = m->capture_stream;
      LF_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
      const int rc = enqueue_batch_step(m, kvs, n, cs);
      hipGraph_t graph = nullptr;
      const hipError_t e = hipStreamEndCapture(cs, &graph);
      if (rc != LF_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
      }
      if (e != hipSuccess) return fail(LF_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
      const hipError_t ei = hipGraphInstantiateWithFlags(&exec, graph, 0);
      (void)hipGraphDestroy(graph);
      if (ei != hipSuccess) return fail(LF_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(ei));
      BatchGraph g{n, {}, exec};
      for (int i = 0; i < n; ++i) g.kvs[i] = kvs[i];
      m->batch_graphs.push_back(g);
    }
    LF_HIP(hipGraphLaunch(exec, st));
  }
  for (int i = 0; i < n; ++i) kvs[i]->len += 1;
  return LF_OK;
}

int lf_decode_steps(lf_model* m, lf_kv* kv, int32_t n, void* stream) {
  if (!m || !kv) return fail(LF_EINVAL, "null argument");
  if (n < 0) return fail(LF_EINVAL, "n = %d < 0", n);
  if (static_cast<long>(kv->len) + n > m->D.ctx) return fail(LF_ERANGE, "len %d + n %d > max_ctx %d", kv->len, n, m->D.ctx);
  for (int i = 0; i < n; ++i) {
    const int rc = lf_decode_step(m, kv, nullptr, stream);
    if (rc) return rc;
  }
  return LF_OK;
}

int lf_decode_step_hidden(lf_model* m, lf_kv* kv, const float* d_x_in, float* d_x_out, void* stream) {
  if (!m || !kv || !d_x_in || !d_x_out) return fail(LF_EINVAL, "null argument");
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  if (m->D.V != 0) return fail(LF_EINVAL, "lf_decode_step_hidden needs vocab == 0");
  if (kv->len >= m->D.ctx) return fail(LF_ERANGE, "sequence is full (%d positions)", m->D.ctx);
  const int rc = run_step(m, kv, d_x_in, d_x_out, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  kv->len += 1;
  return LF_OK;
}

int lf_logits(const lf_model* m, const lf_kv* kv, float* d_logits, int32_t* d_argmax, void* stream) {
  if (!m || !kv || !d_logits) return fail(LF_EINVAL, "null argument");
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  if (m->D.V == 0) return fail(LF_EINVAL, "no logits when vocab == 0");
  if (kv->len == 0) return fail(LF_EINVAL, "no position decoded yet");
  const int n = m->D.V;
  hipLaunchKernelGGL(lf::k_copy_out, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), d_logits,
                     kv->logits(), n, d_argmax, kv->state());
  LF_HIP(hipPeekAtLastError());
  return LF_OK;
}

int lf_kv_status(const lf_kv* kv, int32_t out[3], void* stream) {
  if (!kv || !out) return fail(LF_EINVAL, "null argument");
  if (!kv->m) return fail(LF_EINVAL, "the sequence's model was freed");
  int32_t s[4];
  unsigned abort_flag = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  LF_HIP(hipMemcpyAsync(s, kv->state(), sizeof s, hipMemcpyDeviceToHost, st));
  LF_HIP(hipMemcpyAsync(&abort_flag, kv->m->at<unsigned>(kv->m->W.abort), sizeof abort_flag, hipMemcpyDeviceToHost, st));
  LF_HIP(hipStreamSynchronize(st));
  out[0] = s[lf::kLen];
  out[1] = s[lf::kArgmax];
  out[2] = (s[lf::kBadToken] ? 1 : 0) | (abort_flag ? 2 : 0);
  return LF_OK;
}

int lf_step_kernel_times(lf_model* m, lf_kv* kv, const int32_t* d_token, const float* d_x_in, float* d_x_out,
                         float* ms, int32_t* kinds, int32_t cap, int32_t* n_out, void* stream) {
  if (!m || !kv || !ms || !kinds || !n_out || cap < 1) return fail(LF_EINVAL, "null argument or cap < 1");
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  const bool hidden = m->D.V == 0;
  if (hidden && (!d_x_in || !d_x_out)) return fail(LF_EINVAL, "hidden mode needs d_x_in and d_x_out");
  if (!hidden && !d_token && kv->len == 0) return fail(LF_EINVAL, "no previous position to take a greedy token from");
  if (kv->len >= m->D.ctx) return fail(LF_ERANGE, "sequence is full (%d positions)", m->D.ctx);
  const int nk = 5 * m->D.L + (hidden ? 0 : 1);
  if (cap < nk) return fail(LF_EINVAL, "cap %d < %d kernels per step", cap, nk);
  while (static_cast<int>(m->events.size()) < 2 * nk) {
    hipEvent_t e;
    LF_HIP(hipEventCreate(&e));
    m->events.push_back(e);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_token) {
    hipLaunchKernelGGL(lf::k_set_pos, dim3(1), dim3(64), 0, st, kv->state(), kv->tokens(), kv->len, d_token,
                       static_cast<unsigned*>(nullptr));
    LF_HIP(hipPeekAtLastError());
  }
  StepTimer tm{m->events.data(), kinds, cap, 0};
  const int rc = enqueue_step(m, kv, hidden ? d_x_in : nullptr, hidden ? d_x_out : nullptr, st, &tm);
  if (rc) return rc;
  LF_HIP(hipStreamSynchronize(st));
  kv->len += 1;
  for (int i = 0; i < tm.n; ++i) LF_HIP(hipEventElapsedTime(&ms[i], m->events[2 * i], m->events[2 * i + 1]));
  *n_out = tm.n;
  return LF_OK;
}

int lf_sample(const float* d_logits, int32_t rows, int32_t n, float temperature, const float* d_u, int32_t* d_tokens,
              void* stream) {
  if (!d_logits || !d_u || !d_tokens) return fail(LF_EINVAL, "null argument");
  if (rows < 1 || n < 1 || n > (1 << 24)) return fail(LF_EINVAL, "need rows >= 1 and 1 <= n <= 2^24");
  if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(1.f / temperature))
    return fail(LF_EINVAL, "temperature must be positive and finite, with a finite reciprocal");
  const bool staged = lf::sample_fits_lds(n);
  const size_t lds = staged ? sizeof(float) * (lf::sample_slot(n - 1) + 1) : 0;
  // the kernel's LDS limit is raised once per device (two threads racing here set the same value)
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> lds_set[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(LF_EHIP, "no usable current device for sampling");
  if (!lds_set[dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(lf::k_sample),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             sizeof(float) * lf::kSampleLdsFloats);
    if (e != hipSuccess) return fail(LF_EHIP, "sampling kernel LDS limit: %s", hipGetErrorString(e));
    lds_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(lf::k_sample, dim3(rows), dim3(lf::kSampleThreads), lds, static_cast<hipStream_t>(stream),
                     d_logits, n, 1.f / temperature, d_u, d_tokens, staged ? 1 : 0);
  LF_HIP(hipPeekAtLastError());
  return LF_OK;
}

int lf_read_bandwidth(const void* d_buf, size_t bytes, int32_t iters, void* d_sink, float* gbs, void* stream) {
  if (!d_buf || !d_sink || !gbs) return fail(LF_EINVAL, "null argument");
  if (reinterpret_cast<uintptr_t>(d_buf) % 16 || bytes < 16 || iters < 1)
    return fail(LF_EINVAL, "need a 16-byte aligned buffer of at least 16 bytes and iters >= 1");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n = bytes / 16;
  const dim3 grid(1024), block(lf::kBlock);
  const size_t per = (n + grid.x - 1) / grid.x;
  const auto* p = static_cast<const lf::u32x4*>(d_buf);
  auto* sink = static_cast<unsigned*>(d_sink);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(LF_EHIP, "event create: %s", hipGetErrorString(hipGetLastError()));
  }
  hipLaunchKernelGGL(lf::k_read_probe, grid, block, 0, st, p, n, per, sink);  // warm-up
  hipError_t e = hipEventRecord(e0, st);
  for (int i = 0; i < iters && e == hipSuccess; ++i) {
    hipLaunchKernelGGL(lf::k_read_probe, grid, block, 0, st, p, n, per, sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(LF_EHIP, "read probe: %s", hipGetErrorString(e));
  *gbs = static_cast<float>(static_cast<double>(n) * 16 * iters / (ms * 1e-3) / 1e9);
  return LF_OK;
}

int lf_kernel_time(lf_model* m, lf_kv* kv, int32_t kind, int32_t layer, int32_t reps, int32_t iters,
                   const float* d_x_in, float* d_x_out, float* avg_ms, void* stream) {
  if (!m || !kv || !avg_ms) return fail(LF_EINVAL, "null argument");
  if (kv->m != m) return fail(LF_EINVAL, "sequence belongs to another model");
  const bool hidden = m->D.V == 0;
  if ((kind < LF_KERNEL_QKV || kind > LF_KERNEL_DOWN) && kind != LF_KERNEL_QKV_ATTN)
    return fail(LF_EINVAL, "kind %d cannot be repeated", kind);
  if ((kind == LF_KERNEL_QKV_ATTN) != m->fused && (kind == LF_KERNEL_QKV || kind == LF_KERNEL_ATTN || kind == LF_KERNEL_QKV_ATTN))
    return fail(LF_EINVAL, "kind %d is not launched by this model (QKV and attention %s)", kind,
                m->fused ? "run fused" : "run apart");
  if (layer < -1 || layer >= m->D.L) return fail(LF_EINVAL, "layer %d out of range", layer);
  if (hidden && kind == LF_KERNEL_DOWN && (layer == m->D.L - 1 || layer < 0))
    return fail(LF_EINVAL, "the last down projection ends the step in hidden mode");
  if (hidden && (!d_x_in || !d_x_out)) return fail(LF_EINVAL, "hidden mode needs d_x_in and d_x_out");
  if (reps < 1 || reps > 256 || iters < 1) return fail(LF_EINVAL, "reps must be in [1, 256], iters >= 1");
  if (kv->len >= m->D.ctx) return fail(LF_ERANGE, "sequence is full (%d positions)", m->D.ctx);
  while (m->events.size() < 2) {
    hipEvent_t e;
    LF_HIP(hipEventCreate(&e));
    m->events.push_back(e);
  }
  StepTimer tm{nullptr, nullptr, 0, 0};
  tm.only_kind = kind;
  tm.only_layer = layer;
  tm.reps = reps;
  hipStream_t cs = m->capture_stream, st = static_cast<hipStream_t>(stream);
  LF_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
  const int rc = enqueue_step(m, kv, hidden ? d_x_in : nullptr, hidden ? d_x_out : nullptr, cs, &tm);
  hipGraph_t graph = nullptr;
  const hipError_t e = hipStreamEndCapture(cs, &graph);
  if (rc != LF_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc != LF_OK ? rc : fail(LF_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiateWithFlags(&exec, graph, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) return fail(LF_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(ei));
  hipError_t er = hipGraphLaunch(exec, st);  // warm-up
  if (er == hipSuccess) er = hipEventRecord(m->events[0], st);
  for (int i = 0; i < iters && er == hipSuccess; ++i) er = hipGraphLaunch(exec, st);
  if (er == hipSuccess) er = hipEventRecord(m->events[1], st);
  if (er == hipSuccess) er = hipStreamSynchronize(st);
  float ms = 0.f;
  if (er == hipSuccess) er = hipEventElapsedTime(&ms, m->events[0], m->events[1]);
  (void)hipGraphExecDestroy(exec);
  if (er != hipSuccess) return fail(LF_EHIP, "kernel timing: %s", hipGetErrorString(er));
  *avg_ms = ms / (static_cast<float>(iters) * reps * (layer < 0 ? m->D.L : 1));
  return LF_OK;
}

}  // extern "C"
