// Batched decode step for gfx950: one decode step of up to kMaxBatch
// sequences of one model, for stochastic decoding of several continuations
// of one prompt (the asector.ru summary, "Performance and infrastructure",
// proposes sampling N completions per problem, scored as pass@N). Every
// weight is read from HBM once per step for all the sequences; each sequence
// keeps its own cache, position and tokens.
//
// Every projection is a skinny GEMM Y[s][row] = sum_k W[row][k] X[s][k] on
// the matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation). The
// instruction multiplies a 16 x 32 block of fp16 weights (16 rows) by a
// 32 x 16 block whose 16 columns are the fp16 hi and lo parts of the fp32
// activations of 8 sequences (hi = fp16(x), lo = fp16(x - hi), about 22
// significant bits, as in the prompt pass): column s holds sequence s's hi
// part, column 8 + s its lo part, and the row's result is the sum of the two
// columns. Lane l holds, of its operands, weight row l % 16 and column
// l % 16 with the 8 consecutive k of group l / 16; of the result, column
// l % 16 and rows 4 (l / 16) .. 4 (l / 16) + 3. Every kernel that produces
// a projection's input (the embedding gather, attention, the residual and
// SwiGLU epilogues) writes it already in that operand layout (frag_index),
// split and, for a normalised input, multiplied by the gain, so each lane of
// the projection loads one 16-byte operand piece per k-step. The 8 waves of
// a workgroup split K; their partial results are summed in LDS in a fixed
// order.
//
// RMSNorm: the producer of a normalised input also writes, per workgroup,
// the partial sums of squares of the new residual; the consumer sums them in
// a fixed order and scales its outputs by 1/sqrt(mean + eps).
#pragma once
#include "lf_kernels.h"

namespace lf {

constexpr int kMaxBatch = 8;
constexpr int kSsStride = 1024;  // partial sums of squares per sequence (one per producing workgroup)
constexpr int kSsMax = 512;      // most partials a consumer reads per sequence

// Per-sequence buffers of one batched step (entries past n repeat entry 0,
// so that every entry is a valid address: loads need no condition).
struct BatchSeqs {
  int32_t* state[kMaxBatch];
  int32_t* tokens[kMaxBatch];
  half_t* kc[kMaxBatch];  // each sequence's K cache (layer 0; layer l at + l * layer_cache)
  half_t* vc[kMaxBatch];
  float* logits[kMaxBatch];
};

// The position of each sequence slot, read with scalar loads (the state
// pointers are kernel arguments) before any vector load of the caller; no
// condition on a load, so that all eight are in flight together.
__device__ __forceinline__ void batch_positions(const BatchSeqs& q, int (&pos)[kMaxBatch]) {
#pragma unroll
  for (int s = 0; s < kMaxBatch; ++s) pos[s] = cload(q.state[s] + kLen);
}

__device__ __forceinline__ int pick(const int (&v)[kMaxBatch], int s) {
  int r = v[0];
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i) r = s == i ? v[i] : r;
  return r;
}

// ---------------------------------------------------------- skinny GEMM

enum BEpi : int { kBEpiQKV = 0, kBEpiSwiGLU = 1, kBEpiResid = 2, kBEpiLogits = 3 };

struct BGemmArgs {
  const half_t* W;     // [rows, K] fp16 (QKV and gate/up rows repacked as for the batch-1 kernels)
  int rows, K;         // K a multiple of 8
  const half_t* B;     // the input as the instruction's operand (frag_index), gain applied; zero past K,
                       // and allocated one k-step past the last (all zero)
  const float* ss;     // normalised input: partial sums of squares of the raw input, [kMaxBatch][kSsStride]
  int ss_n;            // partials per sequence (<= kSsMax); 0: the input is not normalised
  float eps;
  int n;               // sequences (1 .. kMaxBatch)
  BatchSeqs seq;
  size_t layer_cache;  // elements between two layers' caches
  int layer;
  float* y;            // QKV: queries [s][q_dim]; residual: x [s][rows] (+=)
  int y_stride;
  half_t* frag_out;    // residual, SwiGLU: the output as the next projection's operand
  const half_t* next_gain;  // residual: RMSNorm gain of the next projection's input [rows]
  float* ss_out;       // residual: partial sums of squares of the new residual [kMaxBatch][kSsStride]
  const float2* rope;  // (cos, sin) [max_ctx][hd / 2]
  int hd, qpl, kpl, max_ctx;
  unsigned* counter;          // logits: workgroups done (the last one ends the step)
  unsigned long long* best;   // logits: packed greedy key per sequence
};

// QKV epilogue of one sequence: rotary pair of packed rows (r, r + 1) at
// position p (as qkv_put; cs: the pair's (cos, sin) at p, loaded early).
__device__ __forceinline__ void bqkv_put(const BGemmArgs& a, int s, int p, int r, float y0, float y1, float2 cs) {
  const int half_hd = a.hd >> 1, upl = a.qpl + 2 * a.kpl;
  const int u = r / a.hd, c = (r % a.hd) >> 1;
  const int ln = u / upl, j = u % upl;
  if (j < a.qpl + a.kpl) {
    const float t0 = y0 * cs.x - y1 * cs.y;
    const float t1 = y0 * cs.y + y1 * cs.x;
    y0 = t0;
    y1 = t1;
  }
  if (j < a.qpl) {
    float* qh = a.y + static_cast<size_t>(s) * a.y_stride + static_cast<size_t>(ln * a.qpl + j) * a.hd;
    qh[c] = y0;
    qh[c + half_hd] = y1;
  } else {
    const bool is_k = j < a.qpl + a.kpl;
    const int h = is_k ? j - a.qpl : j - a.qpl - a.kpl;
    half_t* base = (is_k ? a.seq.kc[s] : a.seq.vc[s]) + a.layer_cache * a.layer;
    half_t* dst = base + ((static_cast<size_t>(ln) * a.max_ctx + p) * a.kpl + h) * a.hd;
    dst[c] = static_cast<half_t>(y0);
    dst[c + half_hd] = static_cast<half_t>(y1);
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int off) {
  const unsigned lo = __float_as_uint(lane_xor(__uint_as_float(static_cast<unsigned>(v)), off));
  const unsigned hi = __float_as_uint(lane_xor(__uint_as_float(static_cast<unsigned>(v >> 32)), off));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Weight and operand loads of KB k-step slots of one wave.
template <int KB, int TPW>
struct BBatch {
  u32x4 w[KB][TPW];
  u32x4 b[KB];
};

// Workgroup: TPW tiles of 16 rows and all K. Its 8 waves take the k-steps in
// turn (wave w: k-steps w, w + 8, ...), so the workgroup streams each row as
// one moving window; a wave loads KB of its k-steps at a time, two batches in
// flight, and the waves' partial results are summed in LDS.
template <int EPI, int TPW, bool NORM, int KB>
__global__ __launch_bounds__(8 * kWave) void k_bgemm(BGemmArgs a) {
  constexpr int NW = 8;
  static_assert(NW == kMaxBatch, "wave w sums sequence w's partial sums of squares");
  __shared__ float red[NW][TPW][4][kWave];
  __shared__ float rs[kMaxBatch];
  __shared__ float ssw[TPW][kMaxBatch];
  __shared__ unsigned long long wkey[TPW][kMaxBatch];
  __shared__ int flag;
  __shared__ u32x4 wt[NW][16 * 144 / 16];  // per wave: one 16-row x 64-k weight block (rows 144 B apart)
  static_assert(KB % 2 == 0, "weights are loaded in pairs of k-steps");
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4, col = lane & 15;
  const int nks = (a.K + 31) >> 5;
  const int J = 2 * (((nks + 1) / 2 + NW - 1) / NW);  // k-step slots per wave (pairs of k-steps)
  // Runs of consecutive tiles share an XCD: when the grid is a multiple of 8
  // (workgroups are dealt to the 8 XCDs in turn), XCD c takes the c-th eighth
  // of the tiles, so that for the lane-major QKV rows the queries, keys and
  // values of one lane are computed, and their cache lines assembled, in one
  // L2 (measured: QKV 16.8 -> 15.8 us, gate/up 22.5 -> 21.7 us per launch at
  // 8 sequences; the mapping is a permutation either way).
  const int bx = (gridDim.x & 7) == 0 ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int ntiles = (a.rows + 15) >> 4, tile0 = bx * TPW;

  int pos[kMaxBatch];
  if constexpr (EPI == kBEpiQKV || EPI == kBEpiLogits) batch_positions(a.seq, pos);
  // Loaded before the weights (a wave's loads complete in issue order), all
  // from clamped in-range addresses without a condition (a condition around
  // a load makes the compiler wait for it at once): the partial sums of
  // squares of sequence `wave` (summed at the end), and what the epilogue
  // reads. Wave t < TPW finishes tile tile0 + t; lane (g, col) holds rows
  // 16 tile + 4 g + r (r < 4) of sequence col.
  float ssv[kSsMax / kWave];
  if constexpr (NORM) {
    const float* sp = a.ss + min(wave, a.n - 1) * kSsStride;
    const int last = max(a.ss_n - 1, 0);
#pragma unroll
    for (int j = 0; j < kSsMax / kWave; ++j) ssv[j] = sp[min(lane + kWave * j, last)];
  }
  const bool epi = wave < TPW && tile0 + wave < ntiles;
  const int s = col;
  const int sl = min(s, a.n - 1);  // the sequence this lane's loads use
  const bool act = epi && s < a.n;
  const int row0 = 16 * (tile0 + wave) + 4 * g;
  f32x4 xres = {0.f, 0.f, 0.f, 0.f};
  float gnext[4] = {0.f, 0.f, 0.f, 0.f};
  float2 cs[2] = {{1.f, 0.f}, {1.f, 0.f}};
  if constexpr (EPI == kBEpiResid) {
    const float* xp = a.y + static_cast<size_t>(sl) * a.y_stride;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(row0 + r, a.rows - 1);
      xres[r] = xp[row];
      gnext[r] = static_cast<float>(a.next_gain[row]);
    }
  } else if constexpr (EPI == kBEpiQKV) {
    const int p = min(pick(pos, sl), a.max_ctx - 1), half_hd = a.hd >> 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = ((min(row0 + 2 * h, a.rows - 2)) % a.hd) >> 1;
      cs[h] = a.rope[static_cast<size_t>(p) * half_hd + c];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // Weight loads: a 16-row x 64-k block of a tile (k-steps 2p and 2p + 1)
  // is read as two instructions of 8 rows x 128 bytes, lane l taking row
  // l / 8 (+ 8) and 16 bytes at chunk l % 8: whole 128-byte lines per
  // instruction, which streams about a quarter faster than the operand
  // layout's 16 rows x 64 bytes. compute() passes each block through a
  // wave-private LDS tile to put it in the operand layout. A wave takes the
  // k-step pairs in turn with the other waves (pair w, w + 8, ...); slots past
  // its last pair load its first pair again (an L2 hit) and are masked.
  const half_t* wr[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    wr[t] = a.W + static_cast<size_t>(min(16 * min(tile0 + t, ntiles - 1) + (lane >> 3), a.rows - 1)) * a.K;
  const size_t half_rows = static_cast<size_t>(8) * a.K;  // rows 8 .. 15 of a tile
  const int npair = (nks + 1) >> 1;
  const int first_pair = min(wave, npair - 1);
  // This lane's operand slot (frag_index): the columns of sequences past n
  // read those of sequence n - 1 instead (the same bytes, so an instruction
  // reads 32 n bytes per k-group); their results are never used.
  const int bslot = (lane & 48) + 2 * min(lane & 7, a.n - 1) + ((lane >> 3) & 1);
  auto pair_of = [&](int j) { return wave + NW * (j >> 1); };
  auto issue = [&](BBatch<KB, TPW>& b, int j0) {
#pragma unroll
    for (int j = 0; j < KB; j += 2) {
      const int p0 = pair_of(j0 + j);
      const int p = p0 < npair ? p0 : first_pair;
      const int k = min(64 * p + 8 * (lane & 7), a.K - 8);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int rt = 16 * min(tile0 + t, ntiles - 1) + (lane >> 3);
        b.w[j][t] = ld_stream(wr[t] + k);
        b.w[j + 1][t] = ld_stream(wr[t] + (rt + 8 < a.rows ? half_rows : 0) + k);
      }
      // k-steps past the last (and the slots past the wave's last pair) read
      // k-step nks of the operand, which is zero
      const int ks0 = p0 < npair ? 2 * p0 : nks, ks1 = p0 < npair && 2 * p0 + 1 < nks ? 2 * p0 + 1 : nks;
      b.b[j] = ld16(a.B + (static_cast<size_t>(ks0) * kWave + bslot) * 8);
      b.b[j + 1] = ld16(a.B + (static_cast<size_t>(ks1) * kWave + bslot) * 8);
    }
  };
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int kRowB = 144;  // LDS bytes per row of a block (128 + 16: rows 4 banks apart)
  char* tile_lds = reinterpret_cast<char*>(wt[wave]);
  auto compute = [&](const BBatch<KB, TPW>& b, int j0) {
#pragma unroll
    for (int j = 0; j < KB; j += 2) {
      const h8 f0 = __builtin_bit_cast(h8, b.b[j]), f1 = __builtin_bit_cast(h8, b.b[j + 1]);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        // lane l wrote row l / 8 (+ 8), chunk l % 8; lane (g, m) reads row m,
        // chunk g (k-step 2p) and chunk g + 4 (k-step 2p + 1). The same
        // wave's LDS operations execute in order; the compiler barriers keep
        // the reads after the writes.
        *reinterpret_cast<u32x4*>(tile_lds + (lane >> 3) * kRowB + (lane & 7) * 16) = b.w[j][t];
        *reinterpret_cast<u32x4*>(tile_lds + ((lane >> 3) + 8) * kRowB + (lane & 7) * 16) = b.w[j + 1][t];
        asm volatile("" ::: "memory");
        const h8 a0 = *reinterpret_cast<const h8*>(tile_lds + col * kRowB + g * 16);
        const h8 a1 = *reinterpret_cast<const h8*>(tile_lds + col * kRowB + (g + 4) * 16);
        asm volatile("" ::: "memory");
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, f0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, f1, acc[t], 0, 0, 0);
      }
    }
  };
  // Two batches in flight, in a loop without any condition on an issue (one
  // makes the compiler wait for every load before it) and a peeled last pair;
  // the batch count is rounded up to even (an extra batch repeats the last
  // k-step, masked). The scheduling barriers keep each batch's loads
  // together, ahead of the other batch's arithmetic (the scheduler would
  // otherwise move loads next to their uses and leave few in flight).
  const int nb = ((J + KB - 1) / KB + 1) & ~1;
  BBatch<KB, TPW> b0, b1;
  issue(b0, 0);
  int i = 0;
  for (; i + 2 < nb; i += 2) {
    issue(b1, (i + 1) * KB);
    __builtin_amdgcn_sched_barrier(0);
    compute(b0, i * KB);
    __builtin_amdgcn_sched_barrier(0);
    issue(b0, (i + 2) * KB);
    __builtin_amdgcn_sched_barrier(0);
    compute(b1, (i + 1) * KB);
    __builtin_amdgcn_sched_barrier(0);
  }
  issue(b1, (i + 1) * KB);
  __builtin_amdgcn_sched_barrier(0);
  compute(b0, i * KB);
  __builtin_amdgcn_sched_barrier(0);
  compute(b1, (i + 1) * KB);

  // sum the waves' partial results in LDS (fixed order); the norm scale
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][t][r][lane] = acc[t][r];
  if constexpr (NORM) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kSsMax / kWave; ++j) sum += lane + kWave * j < a.ss_n ? ssv[j] : 0.f;
    sum = wave_total(sum);
    if (lane == 0 && wave < a.n) rs[wave] = 1.0f / sqrtf(sum / static_cast<float>(a.K) + a.eps);
  }
  lds_barrier();

  float y[4] = {0.f, 0.f, 0.f, 0.f};
  if (epi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][wave][r][lane];
      y[r] = v + lane_xor(v, 8);  // hi column + lo column
    }
  }
  const float sc = NORM && act ? rs[s] : 1.f;
  if constexpr (EPI == kBEpiQKV) {
    if (act) {
      const int p = pick(pos, s);
#pragma unroll
      for (int r = 0; r < 4; r += 2)
        if (row0 + r < a.rows) bqkv_put(a, s, p, row0 + r, y[r] * sc, y[r + 1] * sc, cs[r >> 1]);
    }
  } else if constexpr (EPI == kBEpiSwiGLU) {
    if (act) {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float gt = y[2 * h] * sc, up = y[2 * h + 1] * sc;
        v[h] = gt / (1.0f + expf(-gt)) * up;
      }
      // rows = 2 ffn, a multiple of 16: a lane's four rows exist together
      if (row0 < a.rows) put_frag2(a.frag_out, row0 >> 1, s, v[0], v[1]);
    }
  } else if constexpr (EPI == kBEpiResid) {
    float sq = 0.f;
    if (act) {
      float* xp = a.y + static_cast<size_t>(s) * a.y_stride + row0;
      float xn[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xn[r] = xres[r] + y[r];
        if (row0 + r < a.rows) {
          xp[r] = xn[r];
          sq = fmaf(xn[r], xn[r], sq);
        }
      }
      // rows = d_model, a multiple of 8: a lane's four rows exist together
      if (row0 < a.rows) {
        put_frag2(a.frag_out, row0, s, xn[0] * gnext[0], xn[1] * gnext[1]);
        put_frag2(a.frag_out, row0 + 2, s, xn[2] * gnext[2], xn[3] * gnext[3]);
      }
    }
    if (wave < TPW) {
      sq += lane_xor(sq, 16);
      sq += lane_xor(sq, 32);
      if (lane < kMaxBatch) ssw[wave][lane] = sq;
    }
    lds_barrier();
    if (tid < a.n) {
      float tot = 0.f;
#pragma unroll
      for (int t = 0; t < TPW; ++t) tot += ssw[t][tid];
      a.ss_out[tid * kSsStride + blockIdx.x] = tot;
    }
  } else {  // kBEpiLogits
    unsigned long long key = 0;
    if (act) {
      float* z = a.seq.logits[s];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row0 + r < a.rows) {
          const float v = y[r] * sc;
          z[row0 + r] = v;
          if (v == v) key = max(key, argmax_key(v, row0 + r));  // a NaN logit never wins
        }
    }
    if (wave < TPW) {
      key = max(key, shfl_xor_u64(key, 16));
      key = max(key, shfl_xor_u64(key, 32));
      if (lane < kMaxBatch) wkey[wave][lane] = key;
    }
    lds_barrier();
    if (tid < a.n) {
      unsigned long long k = 0;
#pragma unroll
      for (int t = 0; t < TPW; ++t) k = max(k, wkey[t][tid]);
      if (k) __hip_atomic_fetch_max(a.best + tid, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!arrive(a.counter, gridDim.x, &flag)) return;
    if (tid < a.n) {
      const unsigned long long k = __hip_atomic_load(a.best + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int i = k ? argmax_index(k) : 0;  // k == 0 only if every logit is NaN
      if (i < 0 || i >= a.rows) i = 0;
      int32_t* st = a.seq.state[tid];
      const int p = pick(pos, tid);
      st[kArgmax] = i;
      if (p + 1 >= st[kFedEnd]) a.seq.tokens[tid][p + 1] = i;
      st[kLen] = p + 1;
      __hip_atomic_store(a.best + tid, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// --------------------------------------------------- embedding, attention

struct BEmbedArgs {
  BatchSeqs seq;
  const half_t* emb;   // [vocab, d]
  const half_t* gain;  // RMSNorm gain of layer 0's QKV input [d]
  float* x;            // residual [s][d]
  half_t* frag;        // layer 0's QKV operand (frag_index)
  float* ss;           // partial sums of squares [kMaxBatch][kSsStride] (one partial per sequence)
  int d, vocab, max_ctx;
};

// Workgroup s: the embedding row of sequence s's token at its position, as
// the fp32 residual and as the gain-scaled operand of layer 0's QKV
// projection, and its sum of squares.
__global__ __launch_bounds__(kBlock) void k_bembed(BEmbedArgs a) {
  __shared__ float red[kWavesPerBlock];
  const int s = blockIdx.x;
  int32_t* st = a.seq.state[s];
  const int p = st[kLen];
  if (p >= a.max_ctx) return;  // the host never launches a step on a full cache
  int tok = a.seq.tokens[s][p];
  if (tok < 0 || tok >= a.vocab) {
    tok = tok < 0 ? 0 : a.vocab - 1;
    if (threadIdx.x == 0) st[kBadToken] = 1;
  }
  const half_t* e = a.emb + static_cast<size_t>(tok) * a.d;
  float* x = a.x + static_cast<size_t>(s) * a.d;
  float sq = 0.f;
  for (int i = 2 * threadIdx.x; i < a.d; i += 2 * kBlock) {  // d is a multiple of 8
    const float v0 = static_cast<float>(e[i]), v1 = static_cast<float>(e[i + 1]);
    x[i] = v0;
    x[i + 1] = v1;
    put_frag2(a.frag, i, s, v0 * static_cast<float>(a.gain[i]), v1 * static_cast<float>(a.gain[i + 1]));
    sq = fmaf(v0, v0, fmaf(v1, v1, sq));
  }
  sq = block_sum(sq, red);
  if (threadIdx.x == 0) a.ss[s * kSsStride] = sq;
}

struct AttnBArgs {
  AttnXArgs a;          // shared fields (t.q, t.kc, t.vc, t.state, part, o, epochs per sequence below)
  BatchSeqs seq;
  size_t layer_cache;
  int layer;
  const float* q;       // queries [s][q_dim]
  half_t* ofrag;        // outputs, as the O projection's operand (frag_index; column s)
  u64* part;            // split states, per sequence part_stride words
  size_t part_stride;
  unsigned* epochs;     // [s][n_kv]
  int q_dim;
};

// Attention of work item (split blockIdx.x, kv head blockIdx.y) of sequence
// blockIdx.z: k_attn's two-dimensional layout (the splits of a kv head are
// consecutive workgroups), with the sequence's cache, position, queries,
// split states and epochs; the outputs go to column s of the O projection's
// operand. DB: splits of several load rounds, double-buffered.
template <int HD, int G, int U, bool DB>
__global__ __launch_bounds__(kBlock) void k_battn(AttnBArgs b) {
  __shared__ AttnXSmem<HD, G> sm;
  const int s = blockIdx.z;
  AttnXArgs a = b.a;
  a.t.q = b.q + static_cast<size_t>(s) * b.q_dim;
  a.t.kc = b.seq.kc[s] + b.layer_cache * b.layer;
  a.t.vc = b.seq.vc[s] + b.layer_cache * b.layer;
  a.t.state = b.seq.state[s];
  a.part = b.part + b.part_stride * s;
  a.ofrag = b.ofrag;
  a.fcol = s;
  a.epochs = b.epochs + static_cast<size_t>(s) * a.n_kv;
  attn_item<HD, G, U, false, DB>(a, blockIdx.x, blockIdx.y, sm);
}

// Start a batched step: sequence s's token at its position is d_tokens[s]
// (each sequence's length is given by the host, as for k_set_pos).
struct BTokArgs {
  BatchSeqs seq;
  int len[kMaxBatch];
  const int32_t* tokens;
  int n;
};

__global__ void k_bset_tokens(BTokArgs a) {
  const int s = threadIdx.x;
  if (blockIdx.x != 0 || s >= a.n) return;
  int32_t* st = a.seq.state[s];
  st[kLen] = a.len[s];
  a.seq.tokens[s][a.len[s]] = a.tokens[s];
  st[kFedEnd] = a.len[s] + 1;
}

}  // namespace lf
