// Batched prompt pass (prefill) for gfx950: the decoder applied to a chunk of
// prompt positions at once. Every projection becomes a GEMM of the chunk's
// activations with the layer's fp16 weights on the matrix cores
// (v_mfma_f32_32x32x16_f16, fp32 accumulation), attention is causal / sliding
// window over the cache with the same matrix instructions, and the keys and
// values land in the cache layout the decode step reads. It computes the same
// function as one decode step per prompt position (the decoder of the
// Laneformer blog post, "Designing the architecture": pre-norm GQA decoder,
// sliding-window attention on some layers). Activations stay fp32 as in the
// decode step: an fp32 operand of a matrix instruction is fed as the sum of
// two fp16 parts (hi = fp16(a), lo = fp16(a - hi), about 22 significant bits),
// each multiplied with the fp16 weights or values, fp32 accumulation. The
// kernels that produce a GEMM's activations store them already split (see
// split4), so that the split is done once per element rather than once per
// weight tile that reads it.
#pragma once
#include "lf_device.h"
#include "lf_kernels.h"  // lds_barrier

namespace lf {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Split activations: a row of K fp32 values a[k] is stored as K / 4 groups
// of 16 bytes, group g holding fp16 hi parts of a[4g .. 4g + 3], then their
// lo parts (hi = fp16(a), lo = fp16(a - hi)), so a row takes the bytes of its
// fp32 values and a GEMM's loader copies hi and lo straight into LDS.
__device__ __forceinline__ u32x4 split4(f32x4 v) {
  h8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = static_cast<half_t>(v[e]);
    o[e + 4] = static_cast<half_t>(v[e] - static_cast<float>(o[e]));
  }
  return __builtin_bit_cast(u32x4, o);
}

// Element k of a split row (2 K halves from row).
__device__ __forceinline__ void put_split(half_t* row, int k, float v) {
  const half_t hi = static_cast<half_t>(v);
  half_t* g = row + (k >> 2) * 8 + (k & 3);
  g[0] = hi;
  g[4] = static_cast<half_t>(v - static_cast<float>(hi));
}

// ---------------------------------------------------------------- GEMM
// C[M][N] (=, +=) A[M][K] · W[N][K]^T. A: activations, split rows (above);
// W: a weight matrix as the model stores it, fp16 row-major [out][in]; C
// fp32 (split rows of N / 2 for SwiGLU).
// Workgroup tile 128 x 128, K step 64, four waves of 64 x 64 (2 x 2 blocks of
// 32 x 32). A 32x32x16 matrix instruction takes, in lane l, row l % 32 of its
// A block and column l % 32 of its B block with 8 consecutive k each (k group
// l / 32), and returns in lane l column l % 32, rows 8 (r / 4) + 4 (l / 32) +
// r % 4 of register r. Both operands are K-contiguous rows here (activation
// rows, weight rows), so each lane reads 16 contiguous bytes per operand.
constexpr int kPfBM = 128, kPfBN = 128, kPfBK = 64, kPfThreads = 256;
constexpr int kPfLd = kPfBK + 8;  // LDS row stride in halves (144 B: rows 4 banks apart)

// kPfStore: C = A W^T; kPfAccum: C += A W^T; kPfSwiGLU: the gate/up product
// (gate f and up f in weight rows 2f, 2f + 1) goes through SwiGLU into C
// [M][N / 2] as split rows: C[m][f] = silu(gate) * up.
enum PfEpi : int { kPfStore = 0, kPfAccum = 1, kPfSwiGLU = 2 };

struct PfGemmArgs {
  const half_t* A;  // split rows: 2 K halves each
  const half_t* W;
  float* C;
  int M, N, K;  // K a multiple of 8
  int tiles_m, tiles_n;
  // k_pf_gemm_db only: tiles [full, tiles_m * tiles_n) are each computed as
  // `split` pieces over equal runs of K steps (split 0: none), whose raw sums
  // go to part ([piece][kPfBM][kPf2BN] fp32) for k_pf_fixup
  int full, split;
  float* part;
};

// Write, or add to C, a wave's 64 x 64 block of results at (mw, nw): lane l
// holds columns nw + 32 j + l % 32 and rows mw + 32 i + 8 (r / 4) +
// 4 (l / 32) + r % 4 of register r of block (i, j). The accumulating form
// reads a block's 16 old values first, from clamped in-range addresses
// without a condition (a condition around each load made the compiler wait
// for each in turn), then adds and stores the elements inside the matrix;
// one block at a time keeps the registers within two waves per SIMD. The
// SwiGLU form pairs column n (gate, even lanes) with column n + 1 (up, the
// next lane) and stores one value per pair.
template <int EPI>
__device__ __forceinline__ void pf_write(const PfGemmArgs& a, const f32x16 (&acc)[2][2], int mw, int nw, int lane) {
  auto row = [&](int i, int r) { return mw + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };
  if constexpr (EPI == kPfSwiGLU) {
    half_t* C = reinterpret_cast<half_t*>(a.C);  // split rows of N / 2 (N even): N halves each
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nw + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[i][j][r], up = lane_xor(g, 1);
          const int m = row(i, r);
          if ((lane & 1) == 0 && m < a.M && n < a.N)
            put_split(C + static_cast<size_t>(m) * a.N, n >> 1, g / (1.0f + expf(-g)) * up);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nw + j * 32 + (lane & 31);
      f32x16 old;
      if constexpr (EPI == kPfAccum) {
        const int nc = min(n, a.N - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) old[r] = a.C[static_cast<size_t>(min(row(i, r), a.M - 1)) * a.N + nc];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = row(i, r);
        if (m < a.M && n < a.N)
          a.C[static_cast<size_t>(m) * a.N + n] = EPI == kPfAccum ? old[r] + acc[i][j][r] : acc[i][j][r];
      }
    }
}

template <int EPI>
__global__ __launch_bounds__(kPfThreads) void k_pf_gemm(PfGemmArgs a) {
  __shared__ __attribute__((aligned(16))) half_t As[kPfBM * kPfLd];  // hi parts of the activations
  __shared__ __attribute__((aligned(16))) half_t Al[kPfBM * kPfLd];  // lo parts
  __shared__ __attribute__((aligned(16))) half_t Bs[kPfBN * kPfLd];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // Workgroups are dealt to the 8 XCDs in turn: give each XCD a contiguous
  // run of tiles, N-major, so the M tiles that share a weight tile share an L2.
  const int T = a.tiles_m * a.tiles_n, b = blockIdx.x;
  const int t = (T & 7) ? b : (b & 7) * (T >> 3) + (b >> 3);
  const int m0 = (t % a.tiles_m) * kPfBM, n0 = (t / a.tiles_m) * kPfBN;

  // loader: per K step a thread loads NA chunks of 4 activations (rows
  // tid / ACR + ARS i, floats (tid % ACR) * 4) and NB chunks of 8 weights
  // (rows tid / BCR + BRS i, halves (tid % BCR) * 8)
  constexpr int ACR = kPfBK / 4, ARS = kPfThreads / ACR, NA = kPfBM / ARS;
  constexpr int BCR = kPfBK / 8, BRS = kPfThreads / BCR, NB = kPfBN / BRS;
  const int lrow = tid / BCR, lcol = (tid % BCR) * 8;
  const int arow = tid / ACR, acol = (tid % ACR) * 4;
  const half_t* ap[NA];  // split rows: 4 activations in 8 halves
  const half_t* bp[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) ap[i] = a.A + (static_cast<size_t>(min(m0 + arow + ARS * i, a.M - 1)) * a.K + acol) * 2;
#pragma unroll
  for (int i = 0; i < NB; ++i) bp[i] = a.W + static_cast<size_t>(min(n0 + lrow + BRS * i, a.N - 1)) * a.K + lcol;
  u32x4 ra[NA];
  u32x4 rb[NB];
  auto load = [&](int k0) {
    const bool ina = k0 + acol < a.K, inb = k0 + lcol < a.K;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = ina ? ld16(ap[i] + 2 * k0) : z;
#pragma unroll
    for (int i = 0; i < NB; ++i) rb[i] = inb ? ld16(bp[i] + k0) : z;
  };

  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load(0);
  for (int k0 = 0; k0 < a.K; k0 += kPfBK) {
    __syncthreads();  // every wave is done reading the previous K step
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const u32x2 hi = {ra[i][0], ra[i][1]}, lo = {ra[i][2], ra[i][3]};
      *reinterpret_cast<u32x2*>(&As[(arow + ARS * i) * kPfLd + acol]) = hi;
      *reinterpret_cast<u32x2*>(&Al[(arow + ARS * i) * kPfLd + acol]) = lo;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4*>(&Bs[(lrow + BRS * i) * kPfLd + lcol]) = rb[i];
    __syncthreads();
    if (k0 + kPfBK < a.K) load(k0 + kPfBK);
#pragma unroll
    for (int kk = 0; kk < kPfBK / 16; ++kk) {
      h8 af[2], al[2], bf[2];
      const int col = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const h8*>(&As[(wm * 64 + i * 32 + (lane & 31)) * kPfLd + col]);
        al[i] = *reinterpret_cast<const h8*>(&Al[(wm * 64 + i * 32 + (lane & 31)) * kPfLd + col]);
        bf[i] = *reinterpret_cast<const h8*>(&Bs[(wn * 64 + i * 32 + (lane & 31)) * kPfLd + col]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  pf_write<EPI>(a, acc, m0 + wm * 64, n0 + wn * 64, lane);
}

// The same product on a 128 x 256 workgroup tile of eight 64 x 64 waves, for
// grids that fill the device (one workgroup per CU: 144 KB of LDS). Measured
// on the prompt pass's shapes, the single-buffered kernel above waits on its
// global loads: they are issued one K step ahead, and without them it runs
// about 40% faster. Here the LDS holds two K steps and the registers two
// more, so a step's loads have two compute phases to land: K step s is read
// into a register set during step s - 2, written to LDS stage s % 2 (A's
// hi and lo parts to their own arrays) at the end of step s - 1, and
// multiplied during step s,
// with one barrier per step. The wider tile reads a third fewer bytes of
// operands from L2 per flop. Loads go through buffer descriptors (one per
// operand, from the tile's first row) with a 32-bit per-lane offset, which
// keeps 64-bit addresses out of the vector registers; the K step is a scalar
// offset. K steps past the last (an odd count is rounded up to even) load the
// last step again, and the k past K of a part-filled last step read past the
// row (the next row, or zeros past the descriptor's range); both are written
// to LDS as zeros.
constexpr int kPf2BN = 256, kPf2Threads = 512;
constexpr int kPf2Stage = (2 * kPfBM + kPf2BN) * kPfLd;  // halves per LDS stage (A hi, A lo, W)
constexpr int kPf2Lds = 2 * kPf2Stage * static_cast<int>(sizeof(half_t));

//
// The last, partly filled round of tiles would leave CUs idle (one
// workgroup per CU, all tiles alike): those tiles can instead be split into
// pieces over K steps, which fill the round, with their sums added by
// k_pf_fixup. Workgroup b runs on XCD b mod 8; each XCD takes its eighth of
// the whole tiles as a contiguous run in pf_tile's order (tiles that share
// operands share an L2), then the pieces, dealt in turn, last.
//
// Tile t of a k_pf_gemm_db launch: N-major in blocks of 4 weight tiles, so
// that 32 consecutive tiles (one XCD's share of a round) are 8 activation
// tiles x 4 weight tiles rather than 16 x 2 (a third fewer operand bytes
// into that XCD's L2 per K step).
__device__ __forceinline__ void pf_tile(int t, int tm, int tn, int& m0, int& n0) {
  const int blk = t / (4 * tm), w = t % (4 * tm), nb = min(4, tn - 4 * blk);
  m0 = (w / nb) * kPfBM;
  n0 = (4 * blk + w % nb) * kPf2BN;
}

template <int EPI>
__global__ __launch_bounds__(kPf2Threads) void k_pf_gemm_db(PfGemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) half_t pf2_lds[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int T = a.tiles_m * a.tiles_n, b = blockIdx.x;
  const int nsteps_all = (a.K + kPfBK - 1) / kPfBK;
  int t, piece = -1, s_begin = 0, s_end = nsteps_all;
  if (a.split == 0) {
    t = (T & 7) ? b : (b & 7) * (T >> 3) + (b >> 3);
  } else {  // full and the number of pieces are multiples of 8
    const int c = b & 7, r = b >> 3, per = a.full >> 3;
    if (r < per) {
      t = c * per + r;
    } else {
      piece = (r - per) * 8 + c;
      t = a.full + piece / a.split;
      const int q = (nsteps_all + a.split - 1) / a.split, j = piece % a.split;
      s_begin = min(j * q, nsteps_all);
      s_end = min(s_begin + q, nsteps_all);
    }
  }
  int m0, n0;
  pf_tile(t, a.tiles_m, a.tiles_n, m0, n0);

  // loader: per K step a thread loads NA chunks of 4 activations (rows
  // arow + ARS i, floats acol ..) and NB chunks of 8 weights (rows lrow + BRS i,
  // halves lcol ..); rows past the matrix load its last row (results unused)
  constexpr int ACR = kPfBK / 4, ARS = kPf2Threads / ACR, NA = kPfBM / ARS;
  constexpr int BCR = kPfBK / 8, BRS = kPf2Threads / BCR, NB = kPf2BN / BRS;
  const int lrow = tid / BCR, lcol = (tid % BCR) * 8;
  const int arow = tid / ACR, acol = (tid % ACR) * 4;
  const size_t abytes = static_cast<size_t>(a.M - m0) * a.K * 4;  // split rows: 4 bytes per activation
  const size_t bbytes = static_cast<size_t>(a.N - n0) * a.K * sizeof(half_t);
  const rsrc_t ar = rsrc_of(a.A + static_cast<size_t>(m0) * a.K * 2, static_cast<int>(min(abytes, size_t(0x7fffffff))));
  const rsrc_t br = rsrc_of(a.W + static_cast<size_t>(n0) * a.K, static_cast<int>(min(bbytes, size_t(0x7fffffff))));
  // byte offsets of this thread's chunks at k = 0 from the descriptors' bases;
  // a step adds k0 as the scalar offset. Chunks of the last step past K read
  // the next row, or zeros past a descriptor's range, and are zeroed in LDS.
  int avo[NA], bvo[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) avo[i] = (min(arow + ARS * i, a.M - 1 - m0) * a.K + acol) * 4;
#pragma unroll
  for (int i = 0; i < NB; ++i) bvo[i] = (min(lrow + BRS * i, a.N - 1 - n0) * a.K + lcol) * static_cast<int>(sizeof(half_t));
  const int kend = min(a.K, s_end * kPfBK);  // k past this are zero (a piece's K run ends here)

  u32x4 ra0[NA], ra1[NA];
  u32x4 rb0[NB], rb1[NB];
  auto load = [&](u32x4 (&ra)[NA], u32x4 (&rb)[NB], int step) {
    const int k0 = max(min(step, s_end - 1), 0) * kPfBK;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, avo[i], k0 * 4, 0);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(br, bvo[i], k0 * static_cast<int>(sizeof(half_t)), 0);
  };
  auto store = [&](const u32x4 (&ra)[NA], const u32x4 (&rb)[NB], int step, half_t* stage) {
    half_t* As = stage;
    half_t* Al = As + kPfBM * kPfLd;
    half_t* Bs = Al + kPfBM * kPfLd;
    const int k0 = step * kPfBK;
    if (k0 + kPfBK <= kend) {  // the whole step inside K (uniform): plain copies
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const u32x2 hi = {ra[i][0], ra[i][1]}, lo = {ra[i][2], ra[i][3]};
        *reinterpret_cast<u32x2*>(&As[(arow + ARS * i) * kPfLd + acol]) = hi;
        *reinterpret_cast<u32x2*>(&Al[(arow + ARS * i) * kPfLd + acol]) = lo;
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4*>(&Bs[(lrow + BRS * i) * kPfLd + lcol]) = rb[i];
      return;
    }
    const bool ina = k0 + acol < kend, inb = k0 + lcol < kend;  // K is a multiple of 8
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const u32x2 hi = {ina ? ra[i][0] : 0u, ina ? ra[i][1] : 0u}, lo = {ina ? ra[i][2] : 0u, ina ? ra[i][3] : 0u};
      *reinterpret_cast<u32x2*>(&As[(arow + ARS * i) * kPfLd + acol]) = hi;
      *reinterpret_cast<u32x2*>(&Al[(arow + ARS * i) * kPfLd + acol]) = lo;
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4*>(&Bs[(lrow + BRS * i) * kPfLd + lcol]) = inb ? rb[i] : z;
  };

  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto compute = [&](const half_t* stage) {
    const half_t* As = stage;
    const half_t* Al = As + kPfBM * kPfLd;
    const half_t* Bs = Al + kPfBM * kPfLd;
#pragma unroll
    for (int kk = 0; kk < kPfBK / 16; ++kk) {
      h8 af[2], al[2], bf[2];
      const int col = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const h8*>(&As[(wm * 64 + i * 32 + (lane & 31)) * kPfLd + col]);
        al[i] = *reinterpret_cast<const h8*>(&Al[(wm * 64 + i * 32 + (lane & 31)) * kPfLd + col]);
        bf[i] = *reinterpret_cast<const h8*>(&Bs[(wn * 64 + i * 32 + (lane & 31)) * kPfLd + col]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
  };

  half_t* st0 = pf2_lds;
  half_t* st1 = pf2_lds + kPf2Stage;
  load(ra0, rb0, s_begin);
  load(ra1, rb1, s_begin + 1);
  store(ra0, rb0, s_begin, st0);
  __syncthreads();
  // Each step issues its loads first (the scheduling barriers keep them
  // there), then multiplies its stage, then writes the next step's stage
  // (free since the barrier that ended the step before). A wave raises its
  // priority while it multiplies, so that of the two waves on a SIMD the one
  // with matrix work ready issues first (35.45 -> 34.95 ms per prompt pass).
  for (int s = s_begin; s < s_end; s += 2) {
    load(ra0, rb0, s + 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    compute(st0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    store(ra1, rb1, s + 1, st1);
    __syncthreads();
    load(ra1, rb1, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    compute(st1);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    store(ra0, rb0, s + 2, st0);
    __syncthreads();
  }

  if (piece >= 0) {  // raw sums of the piece, tile-local [kPfBM][kPf2BN]
    float* pp = a.part + static_cast<size_t>(piece) * kPfBM * kPf2BN;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          pp[row * kPf2BN + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][r];
        }
    return;
  }
  pf_write<EPI>(a, acc, m0 + wm * 64, n0 + wn * 64, lane);
}

// The split tiles of a k_pf_gemm_db launch: the sum of each element's
// pieces in a fixed order, then the launch's epilogue as pf_write applies
// it. Workgroup (u, row): tile full + u, that row of it; thread c column c of
// the tile (for SwiGLU, gate and up columns in adjacent lanes). A row per
// workgroup keeps enough loads in flight over few split tiles.
template <int EPI>
__global__ __launch_bounds__(kPf2BN) void k_pf_fixup(PfGemmArgs a) {
  const int u = blockIdx.x, row = blockIdx.y, c = threadIdx.x;
  int m0, n0;
  pf_tile(a.full + u, a.tiles_m, a.tiles_n, m0, n0);
  const int m = m0 + row, n = n0 + c;
  const float* pp = a.part + static_cast<size_t>(u) * a.split * kPfBM * kPf2BN + row * kPf2BN + c;
  float v = 0.f;
  for (int j = 0; j < a.split; ++j) v += pp[static_cast<size_t>(j) * kPfBM * kPf2BN];
  if constexpr (EPI == kPfSwiGLU) {
    const float up = lane_xor(v, 1);
    if ((c & 1) == 0 && m < a.M && n < a.N)
      put_split(reinterpret_cast<half_t*>(a.C) + static_cast<size_t>(m) * a.N, n >> 1, v / (1.0f + expf(-v)) * up);
  } else if (m < a.M && n < a.N) {
    float* dst = a.C + static_cast<size_t>(m) * a.N + n;
    *dst = EPI == kPfAccum ? *dst + v : v;
  }
}

// ---------------------------------------------------------- attention
// Causal attention of a chunk of query positions over the cache, with the
// sliding window where the layer has one: keys j with p - W < j <= p for the
// query at position p (all j <= p when W = 0). Workgroup: QB blocks of 32
// consecutive query positions and one kv head; wave w handles block w / G and
// query head G·kvh + w % G (the G query heads of a kv head and the QB blocks
// share the workgroup's key and value tiles; a tile outside a wave's own
// range is fully masked for it). Per 32-key tile a wave forms
// S^T = K · Q^T (so lane l owns query l % 32 and 16 of the 32 keys; its
// partner lane l ^ 32 holds the other 16), applies the mask, updates an online
// softmax (running max and denominator per query), and adds V^T · P^T into
// O^T (HD x 32 queries). Q^T and P^T are fed as hi + lo fp16 parts. Each key
// tile is staged once per workgroup in LDS: K as rows, V transposed (so that a
// lane reads its keys for one head dimension contiguously); the next tile's
// loads are in flight meanwhile.
struct PfAttnArgs {
  const float* q;    // [M][n_q][hd] rotated queries of the chunk
  const half_t* kc;  // this layer's K cache [lanes][max_ctx][kpl][hd], keys 0..pos0+M-1 written
  const half_t* vc;
  half_t* o;         // [M][n_q * hd] attention outputs as split rows (input of the O projection)
  int M, pos0, max_ctx, window, kpl, n_q, n_kv;
  float scale_log2;  // log2(e) / sqrt(hd)
};

template <int HD, int G, int QB>
__global__ __launch_bounds__(QB * G * kWave) __attribute__((amdgpu_waves_per_eu(2))) void k_pf_attn(PfAttnArgs a) {
  constexpr int NW = QB * G;    // waves
  constexpr int VLD = 32 + 4;   // V^T row stride in halves
  constexpr int KLD = HD + 8;   // key row stride in halves (rows 4 banks apart)
  // K staging unit: 8 head dimensions of one key (unit c: key c / (HD / 8))
  constexpr int NKU = 32 * HD / 8;
  constexpr int NK = (NKU + NW * kWave - 1) / (NW * kWave);
  // V staging unit: 8 head dimensions of two adjacent keys, written to V^T as
  // 8 32-bit key pairs; unit c is key pair c % 16, dimensions 8 (c / 16) ..,
  // so 16 lanes fill 16 consecutive words of a V^T row and the 4 rows a wave
  // writes at once start 16 banks apart
  constexpr int NU = 2 * HD;
  constexpr int NV = (NU + NW * kWave - 1) / (NW * kWave);
  __shared__ __attribute__((aligned(16))) half_t Vt[HD * VLD];
  __shared__ __attribute__((aligned(16))) half_t Ks[32 * KLD];  // the tile's keys, staged once for all waves
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  // Workgroup b runs on XCD b mod 8. With n_kv a multiple of 8, the query
  // blocks of kv head kvh all go to XCD kvh / (n_kv / 8), so a kv head's keys
  // and values are read through one L2 (2 heads of a 3584-position cache:
  // 3.7 MB); kv heads innermost, the query blocks in reverse, so that the
  // blocks with the most keys (causal rows grow with the position) start
  // first and the short ones fill in behind them.
  int kvh, qb;
  {
    const int b = blockIdx.x, r = b % a.n_kv;
    qb = (gridDim.x / a.n_kv) - 1 - b / a.n_kv;
    kvh = (a.n_kv & 7) ? r : (r & 7) * (a.n_kv >> 3) + (r >> 3);
  }
  const int head = kvh * G + w % G;
  const int ln = kvh / a.kpl, hk = kvh % a.kpl;
  const int q_first = a.pos0 + qb * QB * 32;  // the workgroup's query range
  const int q_last = min(q_first + QB * 32 - 1, a.pos0 + a.M - 1);
  const int qrow = (qb * QB + w / G) * 32 + (lane & 31);  // chunk row of this lane's query (may pass M)
  const int qpos = a.pos0 + qrow;
  const int qbase = qpos - (lane & 31);  // the wave's 32 queries: positions qbase .. qbase + 31
  const int grp = lane >> 5;

  // This lane's query fragments (B operand of S^T: query l % 32, head
  // dimensions 16 kk + 8 grp ..), split into hi and lo parts.
  h8 qf[HD / 16], ql[HD / 16];
  {
    const float* qp = a.q + (static_cast<size_t>(min(qrow, a.M - 1)) * a.n_q + head) * HD + grp * 8;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(qp + kk * 16);
      const f32x4 u1 = *reinterpret_cast<const f32x4*>(qp + kk * 16 + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = e < 4 ? u0[e] : u1[e - 4];
        qf[kk][e] = static_cast<half_t>(v);
        ql[kk][e] = static_cast<half_t>(v - static_cast<float>(qf[kk][e]));
      }
    }
  }
  const size_t kstride = static_cast<size_t>(a.kpl) * HD;  // between consecutive positions
  const size_t base = (static_cast<size_t>(ln) * a.max_ctx * a.kpl + hk) * HD;
  const half_t* kbase = a.kc + base;
  const half_t* vbase = a.vc + base;
  const int k_lo = (a.window ? max(0, q_first - a.window + 1) : 0) & ~31;
  const int k_hi = q_last;

  // one key tile's loads: this thread's pieces of K and of V; keys past k_hi
  // are clamped to it (masked below), so every address is a written position
  auto load_tile = [&](int k0, h8 (&kr)[NK], h8 (&vr)[NV][2]) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int c = min(tid + i * NW * kWave, NKU - 1);
      kr[i] = *reinterpret_cast<const h8*>(kbase + static_cast<size_t>(min(k0 + c / (HD / 8), k_hi)) * kstride +
                                           (c % (HD / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = min(tid + i * NW * kWave, NU - 1);
      const int key = k0 + 2 * (c % 16), d8 = (c / 16) * 8;
      vr[i][0] = *reinterpret_cast<const h8*>(vbase + static_cast<size_t>(min(key, k_hi)) * kstride + d8);
      vr[i][1] = *reinterpret_cast<const h8*>(vbase + static_cast<size_t>(min(key + 1, k_hi)) * kstride + d8);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 ot[HD / 32];
#pragma unroll
  for (int th = 0; th < HD / 32; ++th)
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[th][r] = 0.f;

  h8 kr[NK], vr[NV][2];
  load_tile(k_lo, kr, vr);
  for (int k0 = k_lo; k0 <= k_hi; k0 += 32) {
    lds_barrier();  // every wave is done reading the previous tile's K and V^T
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = tid + i * NW * kWave;
      if (NU % (NW * kWave) == 0 || c < NU) {
        const int key = 2 * (c % 16), d8 = (c / 16) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const h2 pr = {vr[i][0][e], vr[i][1][e]};
          *reinterpret_cast<h2*>(&Vt[(d8 + e) * VLD + key]) = pr;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int c = tid + i * NW * kWave;
      if (NKU % (NW * kWave) == 0 || c < NKU)
        *reinterpret_cast<h8*>(&Ks[(c / (HD / 8)) * KLD + (c % (HD / 8)) * 8]) = kr[i];
    }
    // the next tile's loads fly while this one is computed (issued every
    // iteration: a conditional load would make the compiler wait at the join)
    h8 kn[NK], vn[NV][2];
    load_tile(k0 + 32, kn, vn);
    lds_barrier();  // K and V^T of this tile staged by every wave

    // S^T = K Q^T: keys (A operand: key l % 32, head dimensions 16 kk + 8 grp ..) from LDS
    f32x16 sa, sb;
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = sb[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
      const h8 kf = *reinterpret_cast<const h8*>(&Ks[(lane & 31) * KLD + kk * 16 + grp * 8]);
      sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, ql[kk], sb, 0, 0, 0);
    }

    float s[16];
    float mx = -INFINITY;
    if (k0 + 31 <= qbase && (a.window == 0 || k0 > qbase + 31 - a.window)) {  // the wave sees every key of the tile
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = (sa[r] + sb[r]) * a.scale_log2;
        mx = fmaxf(mx, s[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * grp + (r & 3);
        const bool vis = key <= qpos && (a.window == 0 || key > qpos - a.window);
        s[r] = vis ? (sa[r] + sb[r]) * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    // v_exp_f32 directly: exp2(-inf) = 0, and results below 2^-126, whose
    // handling is what the library's exp2f adds, vanish in the fp16 parts
    // and the sums anyway. A query that has seen no key yet (m_new = -inf)
    // subtracts 0 instead, so that its masked scores give 0, not NaN.
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    h8 pf[2], pl[2];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r] - m_ref);
      ps += p;
      pf[r >> 3][r & 7] = static_cast<half_t>(p);
      pl[r >> 3][r & 7] = static_cast<half_t>(p - static_cast<float>(pf[r >> 3][r & 7]));
    }
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__ballot(alpha != 1.f))  // a running max moved (once the maxima settle, most tiles skip this)
#pragma unroll
      for (int th = 0; th < HD / 32; ++th)
#pragma unroll
        for (int r = 0; r < 16; ++r) ot[th][r] *= alpha;
    // P^T in B-operand order: register r = 8 mm + s holds key 16 mm + 8 (s / 4) + 4 grp + s % 4,
    // which is where the A operand (V^T) takes its k slot s from
#pragma unroll
    for (int th = 0; th < HD / 32; ++th)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const half_t* vp = &Vt[(th * 32 + (lane & 31)) * VLD + 16 * mm + 4 * grp];
        const h4 v0 = *reinterpret_cast<const h4*>(vp);
        const h4 v1 = *reinterpret_cast<const h4*>(vp + 8);
        const h8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        ot[th] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[mm], ot[th], 0, 0, 0);
        ot[th] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pl[mm], ot[th], 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < NK; ++i) kr[i] = kn[i];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      vr[i][0] = vn[i][0];
      vr[i][1] = vn[i][1];
    }
  }

  if (qrow < a.M) {  // registers 4 u .. 4 u + 3: head dimensions th 32 + 8 u + 4 grp + 0..3, one split group
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    half_t* op = a.o + (static_cast<size_t>(qrow) * a.n_q * HD + head * HD) * 2;
#pragma unroll
    for (int th = 0; th < HD / 32; ++th)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 v = {ot[th][4 * u] * inv, ot[th][4 * u + 1] * inv, ot[th][4 * u + 2] * inv, ot[th][4 * u + 3] * inv};
        *reinterpret_cast<u32x4*>(op + (th * 32 + 8 * u + 4 * grp) * 2) = split4(v);
      }
  }
}

// ------------------------------------------------------- elementwise
// RMSNorm of each residual row (x / sqrt(mean(x^2) + eps) · gain);
// with emb set, the row is first loaded from the embedding of its token.
struct PfNormArgs {
  float* x;            // [M][d] residual
  half_t* h;           // [M][d] split rows (the GEMMs' input)
  const half_t* gain;
  const half_t* emb;   // [vocab][d], or null
  const int32_t* tokens;
  int32_t* state;
  int M, d, vocab, tok0;  // row t holds token tokens[tok0 + t]
  float eps;
};

// One workgroup per row; a thread holds 4 consecutive elements per step in
// registers between the sum of squares and the scaled store (d <= 8192 and
// a multiple of 8: 16-byte loads and stores).
__global__ __launch_bounds__(kBlock) void k_pf_norm(PfNormArgs a) {
  constexpr int NV = 8192 / (4 * kBlock);
  __shared__ float red[kWavesPerBlock];
  const int t = blockIdx.x;
  float* x = a.x + static_cast<size_t>(t) * a.d;
  const half_t* e = nullptr;
  if (a.emb) {
    int tok = a.tokens[a.tok0 + t];
    if (tok < 0 || tok >= a.vocab) {
      tok = tok < 0 ? 0 : a.vocab - 1;
      if (threadIdx.x == 0) a.state[kBadToken] = 1;
    }
    e = a.emb + static_cast<size_t>(tok) * a.d;
  }
  f32x4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = (threadIdx.x + k * kBlock) * 4;
    if (i < a.d) {
      if (e) {
        const h4 eh = *reinterpret_cast<const h4*>(e + i);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[k][c] = static_cast<float>(eh[c]);
        *reinterpret_cast<f32x4*>(x + i) = v[k];
      } else {
        v[k] = *reinterpret_cast<const f32x4*>(x + i);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) ss = fmaf(v[k][c], v[k][c], ss);
    }
  }
  const float inv = rsqrtf(block_sum(ss, red) / a.d + a.eps);
  half_t* h = a.h + static_cast<size_t>(t) * a.d * 2;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = (threadIdx.x + k * kBlock) * 4;
    if (i < a.d) {
      const h4 g = *reinterpret_cast<const h4*>(a.gain + i);
      f32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = v[k][c] * inv * static_cast<float>(g[c]);
      *reinterpret_cast<u32x4*>(h + 2 * i) = split4(o);
    }
  }
}

// Rotary embedding and cache append for the QKV GEMM's output, whose columns
// follow the model's lane-major row order (per lane: its query heads, key
// heads, value heads; within a head, dimensions c and c + hd/2 adjacent).
struct PfQkvArgs {
  const float* y;  // [M][rows]
  float* q;        // [M][n_q][hd]
  half_t* kc;      // this layer's cache
  half_t* vc;
  const float2* rope;  // [max_ctx][hd/2] (cos, sin)
  int M, rows, hd, qpl, kpl, n_q, max_ctx, pos0;
};

// Thread i takes column pairs 4 i .. 4 i + 3 of row t: dimensions c .. c + 3
// and c + hd/2 .. c + hd/2 + 3 of one head (hd a multiple of 8), 16-byte
// loads and 16- / 8-byte stores.
__global__ __launch_bounds__(kBlock) void k_pf_qkv(PfQkvArgs a) {
  const int i = blockIdx.x * kBlock + threadIdx.x, t = blockIdx.y;
  if (8 * i >= a.rows) return;
  const float* yr = a.y + static_cast<size_t>(t) * a.rows + 8 * i;
  const f32x4 ya = *reinterpret_cast<const f32x4*>(yr), yb = *reinterpret_cast<const f32x4*>(yr + 4);
  const int r = 8 * i, half_hd = a.hd >> 1, upl = a.qpl + 2 * a.kpl, p = a.pos0 + t;
  const int u = r / a.hd, c = (r % a.hd) >> 1;
  const int ln = u / upl, j = u % upl;
  const float y0[4] = {ya[0], ya[2], yb[0], yb[2]}, y1[4] = {ya[1], ya[3], yb[1], yb[3]};
  f32x4 o0, o1;  // dimensions c .. c + 3 and c + hd/2 ..
  if (j < a.qpl + a.kpl) {
    const f32x4* rp = reinterpret_cast<const f32x4*>(a.rope + static_cast<size_t>(p) * half_hd + c);
    const f32x4 ca = rp[0], cb = rp[1];  // (cos, sin) of pairs c, c + 1 and c + 2, c + 3
    const float cs[4] = {ca[0], ca[2], cb[0], cb[2]}, sn[4] = {ca[1], ca[3], cb[1], cb[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = y0[e] * cs[e] - y1[e] * sn[e];
      o1[e] = y0[e] * sn[e] + y1[e] * cs[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = y0[e];
      o1[e] = y1[e];
    }
  }
  if (j < a.qpl) {
    float* qh = a.q + (static_cast<size_t>(t) * a.n_q + ln * a.qpl + j) * a.hd;
    *reinterpret_cast<f32x4*>(qh + c) = o0;
    *reinterpret_cast<f32x4*>(qh + c + half_hd) = o1;
  } else {
    const bool is_k = j < a.qpl + a.kpl;
    const int h = is_k ? j - a.qpl : j - a.qpl - a.kpl;
    half_t* dst = (is_k ? a.kc : a.vc) + ((static_cast<size_t>(ln) * a.max_ctx + p) * a.kpl + h) * a.hd;
    const h4 k0 = {static_cast<half_t>(o0[0]), static_cast<half_t>(o0[1]), static_cast<half_t>(o0[2]), static_cast<half_t>(o0[3])};
    const h4 k1 = {static_cast<half_t>(o1[0]), static_cast<half_t>(o1[1]), static_cast<half_t>(o1[2]), static_cast<half_t>(o1[3])};
    *reinterpret_cast<h4*>(dst + c) = k0;
    *reinterpret_cast<h4*>(dst + c + half_hd) = k1;
  }
}

// Hand the last prompt position's residual to the decode step's LM head and
// point the sequence at that position (its LM head then advances it).
__global__ __launch_bounds__(kBlock) void k_pf_finish(const float* xrow, float* x, int d, int32_t* state, int32_t pos) {
  for (int i = threadIdx.x; i < d; i += kBlock) x[i] = xrow[i];
  if (threadIdx.x == 0) state[kLen] = pos;
}

}  // namespace lf
