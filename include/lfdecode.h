/*
 * lfdecode — batch-1 decode step of a Laneformer-2B-shaped decoder on MI355X
 * (gfx950), behind a plain C ABI.
 *
 * What one step computes (Kog Laneformer 2B blog, "Designing the
 * architecture"): a pre-norm decoder transformer with causal grouped-query
 * attention (query head i reads key/value head floor(i*Hkv/Hq)), heads spread
 * evenly over lanes, sliding-window attention on some layers, a KV cache that
 * every new token reads, and a greedy next token. The blog's "The idea" and
 * "Designing the architecture" sections state that at batch 1 the step is
 * bound by the bytes it streams from HBM: every weight once plus the visible
 * cache. Inference is FP16 at batch 1 (asector.ru summary, "Performance and
 * infrastructure"); the context is at most 4,096 tokens (same summary,
 * "Operational risks").
 *
 * Numerics: fp16 weights and KV cache; fp32 accumulation, residual stream,
 * softmax and logits.
 *
 * Memory ownership: the caller allocates every device buffer (weights,
 * workspace, KV/sequence buffer, token and logits buffers) and keeps it alive
 * while the library uses it. The library never allocates or frees device
 * memory after lf_model_init returns, and never frees caller memory. Handles
 * (lf_model, lf_kv) are small host objects owned by the library.
 *
 * Streams: every call that takes `stream` (a hipStream_t passed as void*)
 * enqueues its device work on that stream and returns without waiting, except
 * lf_model_init, which waits for its own setup work. Calls on one model must
 * be serialised on one stream: all sequences of a model share its workspace.
 *
 * Errors: functions return 0 on success or a negative LF_E* code; no C++
 * exception crosses the ABI. lf_last_error() returns a thread-local text for
 * the last failure of the calling thread.
 */
#ifndef LFDECODE_H
#define LFDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LF_OK 0
#define LF_EINVAL (-1)   /* null pointer, invalid configuration, undersized buffer, wrong mode */
#define LF_ERANGE (-2)   /* the sequence would pass max_ctx positions */
#define LF_EHIP (-3)     /* a HIP runtime call failed; see lf_last_error() */

#define LF_MAX_LAYERS 64

/*
 * Decoder shape. All sizes in elements.
 *   n_q_heads % n_kv_heads == 0; n_q_heads, n_kv_heads and ffn divisible by n_lanes;
 *   head_dim in {32, 64, 128}; (512 / head_dim) divisible by n_kv_heads / n_lanes;
 *   d_model, ffn multiples of 8 and at most 8192; n_q_heads * head_dim at most 8192;
 *   1 <= max_ctx <= 4096; 1 <= n_layers <= LF_MAX_LAYERS.
 * vocab == 0 selects hidden-in / hidden-out mode: no embedding, no LM head,
 * lf_decode_step_hidden is the step call.
 * window[l] == 0: layer l is full causal; window[l] == W > 0: position p sees
 * keys j with p - W < j <= p (the current key counts toward W).
 * Rotary embedding: pairs (c, c + head_dim/2), angle p * rope_theta^(-2c/head_dim).
 */
typedef struct lf_config {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_lanes, max_ctx;
  int32_t window[LF_MAX_LAYERS];
  float rope_theta, rms_eps;
} lf_config;

/*
 * Caller-owned device pointers to fp16 weights, matrices row-major [out, in].
 * The per-layer members are HOST arrays of n_layers DEVICE pointers.
 *   embed, lm_head  [vocab, d_model]   (unused when vocab == 0)
 *   final_norm      [d_model]          (unused when vocab == 0)
 *   attn_norm, ffn_norm [d_model] RMSNorm gains
 *   wqkv     [(n_q_heads + 2 n_kv_heads) head_dim, d_model]: all q rows, then k rows, then v rows
 *   wo       [d_model, n_q_heads head_dim]
 *   wgate_up [2 ffn, d_model]: gate rows, then up rows
 *   wdown    [d_model, ffn]
 * lf_model_init copies (and repacks) everything it needs into the workspace;
 * after it returns the caller may release these buffers.
 */
typedef struct lf_weight_ptrs {
  const void* embed;
  const void* lm_head;
  const void* final_norm;
  const void* const* attn_norm;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* ffn_norm;
  const void* const* wgate_up;
  const void* const* wdown;
} lf_weight_ptrs;

typedef struct lf_model lf_model;
typedef struct lf_kv lf_kv;

/* Bytes of device workspace a model of this shape needs (0 if the config is
 * invalid): the weights once (repacked, row-major), the rotary table, the
 * activations and the exchange buffers of the attention kernels. */
size_t lf_workspace_bytes(const lf_config* cfg);

/* Bytes of the per-sequence device buffer (state, token history, logits, K and V caches). */
size_t lf_kv_bytes(const lf_config* cfg);

/*
 * Validate cfg, bind the caller's workspace (d_workspace, >= lf_workspace_bytes,
 * 256-byte aligned), copy and repack the weights into it, build the rotary
 * table, and wait for that setup on `stream` (the stream argument is an
 * addition to the four calls of the path: the setup copies run on it). It
 * also reads which XCD each workgroup of three probe launches runs on, and
 * the device's room for the attention kernels, to choose their layouts
 * (lf_plan_attention). *out receives the handle.
 * LF_EINVAL for a bad config, null or misaligned pointers, a small workspace,
 * or a shape whose attention splits cannot all be resident at once.
 */
int lf_model_init(const lf_config* cfg, const lf_weight_ptrs* w, void* d_workspace, size_t ws_bytes,
                  void* stream, lf_model** out);
/* Free the handle. Sequences of the model become unusable (calls on them
 * fail with LF_EINVAL) but must still be released with lf_kv_free, in any
 * order relative to this call. The caller's buffers stay the caller's. */
void lf_model_free(lf_model* m);

/*
 * How a step is launched. Both modes compute the same function with the same
 * kernels (bitwise the same results).
 *   LF_MODE_GRAPH (default): one kernel per phase, captured per (sequence,
 *     in/out pointers) into a hipGraph on first use and replayed. A model
 *     keeps at most 64 such graphs (and 64 of lf_decode_step_batch); a step
 *     of a key beyond those launches its kernels one by one instead (same
 *     results). lf_kv_free drops the graphs of its sequence.
 *   LF_MODE_EAGER: one kernel per phase, launched one by one.
 * lf_model_set_mode returns LF_EINVAL for any other value.
 * lf_model_set_graph(m, 1/0) selects LF_MODE_GRAPH / LF_MODE_EAGER.
 */
#define LF_MODE_EAGER 0
#define LF_MODE_GRAPH 1
int lf_model_set_mode(lf_model* m, int mode);
int lf_model_mode(const lf_model* m);
int lf_model_set_graph(lf_model* m, int enabled);

/*
 * QKV fused with attention: one kernel per layer computes the QKV projection
 * and the layer's attention (instead of LF_KERNEL_QKV then LF_KERNEL_ATTN),
 * with each kv head's exchanges kept on one XCD of the device. Available for
 * 16 kv heads of head_dim 128 with 2 query heads each and d_model 4096, on a
 * device of at least 256 CUs that deals a launch's workgroups to its XCDs in
 * turn (probed by lf_model_init); the default where available.
 * lf_model_set_fused(m, 1) returns LF_EINVAL where it is not;
 * lf_model_set_fused(m, 0) selects the two kernels. A switch applies from the
 * next step (recorded graphs are discarded). The same computation either way
 * (the order of floating-point sums inside attention differs).
 * lf_model_fused returns 1 or 0 (-1 for a null model).
 */
int lf_model_set_fused(lf_model* m, int enabled);
int lf_model_fused(const lf_model* m);

/*
 * Raise the model's give-up flag (lf_kv_status bit 1) on stream, as an
 * attention wait that ran out of polls would: every wait of the following
 * steps gives up at once, their results are invalid, and the flag reads set
 * until lf_kv_set_len on one of the model's sequences clears it. For callers
 * and tests that check how an invalid step is reported and recovered from;
 * no kernel faults or hangs. LF_EINVAL for a null model.
 */
int lf_model_raise_give_up(lf_model* m, void* stream);

/*
 * Launch planning of the attention kernels (host only, no device work): what
 * lf_model_init chooses for a device with n_cu compute units that holds
 * attn_wg_per_cu workgroups of the split-KV attention kernel and
 * fused_wg_per_cu of the QKV fused with attention kernel per CU at once, and
 * deals a launch's workgroups to its 8 XCDs in turn if xcd_classes != 0.
 * The splits of a kv head wait for each other's partial softmax states, so
 * every layout is used only where all the workgroups that wait on each other
 * can be resident at once:
 *   *fused = 1 if QKV and attention can run as one launch (the fused shape,
 *     xcd_classes, and room for its 256 workgroups);
 *   xcd_layers[l] = 1 (host array of n_layers) if layer l's attention launch
 *     keeps each kv head's splits on one XCD (room for all S * n_kv
 *     workgroups, n_kv a multiple of 8), else 0 (a grid of S x n_kv in
 *     which each kv head's S splits are consecutive).
 * LF_EINVAL for a bad config, null pointers, n_cu < 1, negative rooms, or a
 * layer whose S splits do not fit at once.
 */
int lf_plan_attention(const lf_config* cfg, int32_t n_cu, int32_t attn_wg_per_cu, int32_t fused_wg_per_cu,
                      int32_t xcd_classes, int32_t* fused, int32_t* xcd_layers);

/*
 * Bind a caller buffer (>= lf_kv_bytes, 256-byte aligned) as one sequence with
 * length 0: the KV cache that every generated token reads (blog, "Designing
 * the architecture": with grouped-query and sliding-window attention the
 * cache is what each new token streams besides the weights), for at most
 * max_ctx <= 4096 positions (asector.ru summary, "Operational risks": a
 * context of 4,096 tokens). Zeroes the sequence state (synchronously).
 * Layout of the caches, so a caller can fill them (K holds keys
 * after the rotary embedding):
 *   K[layer][lane][pos][kv_head_in_lane][head_dim] fp16, V likewise,
 * kv head h lives in lane h / (n_kv_heads / n_lanes). lf_kv_cache_ptrs gives
 * the two device addresses.
 */
int lf_kv_alloc(lf_model* m, void* d_buf, size_t bytes, lf_kv** out);
void lf_kv_free(lf_kv* kv);
int lf_kv_cache_ptrs(const lf_kv* kv, void** d_k, void** d_v);

/*
 * Set the sequence length to len (0 <= len <= max_ctx): rewinds, or adopts
 * cache content the caller wrote for positions [0, len). Token len of the
 * history is kept as the input of the next step; greedy tokens of the
 * following steps are recorded from token len+1 on. Also clears the model's
 * give-up flag (lf_kv_status bit 1). Enqueued on stream (an argument beyond
 * the path's four calls: the caller orders it with its own work).
 * LF_ERANGE if len is outside [0, max_ctx].
 */
int lf_kv_set_len(lf_kv* kv, int32_t len, void* stream);
int32_t lf_kv_len(const lf_kv* kv);

/*
 * Copy token ids [start, start + n) of the sequence's history to d_out (device
 * int32, caller-owned): prompt tokens, tokens given to lf_decode_step, and the
 * greedy token of every decoded position p (stored as token p+1 once p+1 is
 * past the tokens given by the caller). 0 <= start, start + n <= max_ctx + 1,
 * else LF_ERANGE. Enqueued on stream.
 */
int lf_kv_tokens(const lf_kv* kv, int32_t* d_out, int32_t start, int32_t n, void* stream);

/*
 * Prefill: append n positions whose token ids are d_tokens[0..n) (device
 * int32, each in [0, vocab); ids outside are clamped and flagged, see
 * lf_kv_status), one decode step per position, so the prompt's keys and
 * values enter the cache exactly as generated tokens' do (blog, "Designing
 * the architecture"). Leaves the logits and greedy argmax of the last of
 * them. LF_EINVAL for null arguments, n < 1 or vocab == 0; LF_ERANGE if
 * len + n > max_ctx (asector.ru summary, "Operational risks": 4,096-token
 * context). Enqueued on stream.
 */
int lf_prefill(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int32_t n, void* stream);

/*
 * Batched prompt pass. The prompt is consumed in one pass before decoding (the
 * asector summary, "Performance and infrastructure", times a whole generation
 * pass), and across the prompt's positions every projection of the decoder
 * (the blog post, "Designing the architecture") is a matrix product.
 *
 * Same result and state as lf_prefill: it appends n positions (tokens
 * d_tokens[0..n), device int32), writes their keys and values to the cache, and
 * leaves the logits and greedy argmax of the last position. The positions are
 * taken `chunk` at a time (1 <= chunk <= LF_MAX_PREFILL_CHUNK). In each chunk,
 * each layer runs:
 *   - the projections as matrix-core GEMMs of the fp32 activations with the
 *     fp16 weights, fp32 accumulation. Each activation goes in as two fp16
 *     parts, hi = fp16(a) and lo = fp16(a - hi), about 22 significant bits;
 *     the residual stays fp32 as in the decode step;
 *   - causal / sliding-window attention over the cache, on the matrix cores,
 *     with the queries and the softmax weights split the same way.
 *
 * d_workspace: caller-owned device scratch, 256-byte aligned, at least
 * lf_prefill_workspace_bytes(cfg, chunk) bytes. Its contents do not matter
 * before or after the call. It must not be used by another call until the
 * stream has passed this one.
 * LF_EINVAL: null arguments, vocab == 0, n < 1, bad chunk, or a small or
 * unaligned workspace. LF_ERANGE: len + n > max_ctx. Enqueued on stream.
 */
#define LF_MAX_PREFILL_CHUNK 4096
size_t lf_prefill_workspace_bytes(const lf_config* cfg, int32_t chunk);  /* 0 if cfg or chunk is invalid */
int lf_prefill_batched(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int32_t n, int32_t chunk, void* d_workspace,
                       size_t ws_bytes, void* stream);

/*
 * The batched prompt pass without a caller workspace, for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, result and state as
 * lf_prefill_batched, with the scratch in an array of LF_STATIC_SCRATCH_BYTES
 * that the library holds on each device it runs on until the process ends
 * (its address is looked up once per device, in lf_model_init). Allocates
 * nothing. Every call on a device shares that array and it keeps the last
 * call's contents: calls that overlap on one device (on different streams,
 * or from different threads) race.
 * chunk: positions per pass, from 1 to the largest whose scratch fits the
 * array (282 for d_model 4096, 32 q / 16 kv heads of 128 and SwiGLU 7168), or
 * 0 for that largest. LF_EINVAL for a larger chunk (lf_last_error states the
 * limit), null arguments, vocab == 0 or n < 1; LF_ERANGE if len + n > max_ctx.
 * Enqueued on stream.
 */
#define LF_STATIC_SCRATCH_BYTES (32u << 20)
int lf_prefill_batched_static(lf_model* m, lf_kv* kv, const int32_t* d_tokens, int32_t n, int32_t chunk, void* stream);

/*
 * The decode step: append one position. Every weight of the model is read
 * once plus the cache keys each layer sees, which is what bounds its speed
 * at batch 1 (blog, "The idea" and "Designing the architecture"); FP16
 * weights and cache at batch 1 (asector.ru summary, "Performance and
 * infrastructure"). d_token (device int32) gives its token id; NULL feeds
 * the greedy argmax of the previous position (blog, TL;DR: greedy decoding),
 * which stays on the device. Leaves the logits and argmax of the new
 * position. LF_EINVAL for null handles, vocab == 0, or d_token NULL at
 * length 0; LF_ERANGE if len == max_ctx. Enqueued on stream (graph replay or
 * eager launches, per lf_model_set_mode).
 */
int lf_decode_step(lf_model* m, lf_kv* kv, const int32_t* d_token, void* stream);

/* n chained greedy steps (lf_decode_step with d_token == NULL, n times). */
int lf_decode_steps(lf_model* m, lf_kv* kv, int32_t n, void* stream);

/*
 * Batched decode step: one decode step of each of n sequences of one model
 * (1 <= n <= LF_MAX_BATCH), with every weight read from HBM once for all of
 * them. The asector.ru summary ("Performance and infrastructure") proposes
 * stochastic decoding scored as pass@N: N sampled continuations of one
 * prompt, which is n sequences that step together. Each sequence keeps its
 * own cache, length and token history, and after the call holds the logits
 * and greedy argmax of its new position exactly as after lf_decode_step
 * (lf_logits, lf_kv_status, lf_kv_tokens per sequence); the lengths may
 * differ. d_tokens: device int32 [n], the token of each sequence's new
 * position (e.g. drawn by lf_sample from the rows of lf_logits), or NULL to
 * feed each sequence its own greedy token of the previous position.
 * kvs: host array of n distinct sequence handles of model m.
 * Numerics: for n >= 2 the projections run on the matrix cores with each
 * fp32 activation split into two fp16 parts (hi = fp16(a), lo = fp16(a - hi)),
 * fp32 accumulation; attention, softmax and logits in fp32 as in the
 * single-sequence step. n == 1 runs lf_decode_step itself (bitwise the
 * same). LF_EINVAL for null or repeated handles, n out of range, vocab == 0,
 * or d_tokens NULL for an empty sequence; LF_ERANGE if a sequence is full.
 * Graph mode records one hipGraph per (n, handles) and replays it (at most 64
 * per model, as for lf_decode_step). Enqueued on stream.
 */
#define LF_MAX_BATCH 8
int lf_decode_step_batch(lf_model* m, lf_kv* const* kvs, int32_t n, const int32_t* d_tokens, void* stream);

/*
 * Hidden mode (vocab == 0): append one position whose input hidden vector is
 * d_x_in (fp32 [d_model]) and write the last layer's output residual to
 * d_x_out (fp32 [d_model]; may equal d_x_in).
 */
int lf_decode_step_hidden(lf_model* m, lf_kv* kv, const float* d_x_in, float* d_x_out, void* stream);

/*
 * Copy the logits of the most recent position (fp32 [vocab]) to d_logits and,
 * if d_argmax is not NULL, its greedy token (blog, TL;DR: greedy decoding;
 * the lowest index among maximal logits, +0.0 and -0.0 equal) to d_argmax
 * (device int32). Both buffers caller-owned. LF_EINVAL for null arguments,
 * vocab == 0 or an empty sequence. Enqueued on stream.
 */
int lf_logits(const lf_model* m, const lf_kv* kv, float* d_logits, int32_t* d_argmax, void* stream);

/*
 * Read back (synchronously on stream) the device-side sequence state:
 * out[0] = length, out[1] = last argmax, out[2] = flags: bit 0 set if a token
 * id outside [0, vocab) was clamped since lf_kv_alloc; bit 1 set if, in a
 * step of this model (any of its sequences) since lf_model_init or the last
 * lf_kv_set_len on one of its sequences, an attention workgroup gave up
 * waiting for another workgroup's data (a bounded poll ran out). The results
 * of those steps are invalid, and until the flag is cleared every later wait
 * gives up at once.
 */
int lf_kv_status(const lf_kv* kv, int32_t out[3], void* stream);

/*
 * Profiling aid (not needed to decode): run one step exactly as lf_decode_step
 * (token mode; d_token may be NULL) or lf_decode_step_hidden (hidden mode)
 * would, but with the per-phase kernels launched one by one, each bracketed
 * by two HIP events on `stream`; wait for it and write, in launch order, each
 * kernel's elapsed milliseconds (launch gaps included) to ms[] and its kind
 * (LF_KERNEL_*) to kinds[].
 * cap must be at least 5 * n_layers (+ 1 in token mode); *n_out receives the
 * kernel count. Appends one position like the step calls.
 */
#define LF_KERNEL_QKV 0      /* RMSNorm + QKV GEMV + rotary + KV append */
#define LF_KERNEL_ATTN 1     /* split-KV GQA attention + merge */
#define LF_KERNEL_O 2        /* O GEMV + residual */
#define LF_KERNEL_GATE_UP 3  /* RMSNorm + gate/up GEMV + SwiGLU */
#define LF_KERNEL_DOWN 4     /* down GEMV + residual */
#define LF_KERNEL_LM_HEAD 5  /* RMSNorm + LM head + greedy argmax */
#define LF_KERNEL_QKV_ATTN 6 /* QKV (as LF_KERNEL_QKV) and attention in one kernel */
int lf_step_kernel_times(lf_model* m, lf_kv* kv, const int32_t* d_token, const float* d_x_in, float* d_x_out,
                         float* ms, int32_t* kinds, int32_t cap, int32_t* n_out, void* stream);

/*
 * Profiling aid: the average duration of one per-phase kernel of the step's
 * graph, launched back to back as graph replays run it. Captures `reps`
 * launches (1..256) of the kernel of kind `kind` (LF_KERNEL_QKV .. DOWN, or
 * LF_KERNEL_QKV_ATTN, whichever the model launches; not
 * the LM head, nor in hidden mode the last layer's down projection, which end
 * the step) of layer `layer` (layer -1: of every layer in order, so that each
 * launch streams other weights, as in a step) with the arguments of the
 * sequence's next step, replays that graph `iters` times between two events
 * on `stream`, waits, and writes the time per launch in milliseconds to
 * *avg_ms. The sequence's
 * position does not change, but its activations and the KV entry at that
 * position are left unspecified (the next step recomputes them).
 */
int lf_kernel_time(lf_model* m, lf_kv* kv, int32_t kind, int32_t layer, int32_t reps, int32_t iters,
                   const float* d_x_in, float* d_x_out, float* avg_ms, void* stream);

/*
 * Measurement aid: the practical HBM read ceiling. Reads the device buffer
 * d_buf (bytes long, 16-byte aligned; caller-owned, not modified) `iters`
 * times with a plain streaming kernel of 16-byte non-temporal loads (1024
 * workgroups of 256 threads, each reading a contiguous share, 8 loads in
 * flight per thread), after one
 * untimed pass, between two HIP events on `stream`; waits and writes the
 * read rate in GB/s (1e9 bytes) to *gbs. d_sink: 4 bytes of device memory the
 * kernel may write. Use a buffer well above the 256 MB last-level cache.
 * LF_EINVAL for null pointers, misalignment, bytes < 16 or iters < 1.
 */
int lf_read_bandwidth(const void* d_buf, size_t bytes, int32_t iters, void* d_sink, float* gbs, void* stream);

/*
 * Temperature sampling of the next token, for stochastic (pass@N) decoding,
 * which the asector.ru summary ("Performance and infrastructure") proposes for
 * code: several sampled continuations of one prompt. The pages name no
 * sampler; this one inverts the cumulative distribution of
 * p = softmax(z / temperature) at a caller-given uniform u: for each row r,
 * d_tokens[r] = the smallest i with p_0 + ... + p_i > d_u[r] (token i covers
 * u in [c_{i-1}, c_i)); tokens of probability 0 are never drawn, and if fp32
 * rounding leaves the total below u the last token of positive probability is
 * drawn. Computed in fp32 (weights exp((z_i - max z) / T), cumulative sums in
 * index order), one workgroup per row.
 *
 * d_logits: device fp32 [rows, n], row-major, finite values (the logits that
 * lf_logits copies out, or any others). d_u: device fp32 [rows], each in
 * [0, 1); a value below 0 draws the first token of positive probability, a
 * value of 1 or more (or NaN) the last. d_tokens: device int32 [rows], written. All
 * three are caller-owned; nothing is allocated. Asynchronous on `stream`; to
 * continue a sequence with the drawn token pass d_tokens + r to lf_decode_step.
 * LF_EINVAL for null pointers, rows < 1, n < 1 or n > 2^24, or a temperature
 * that is not positive and finite or whose reciprocal is not finite (greedy
 * decoding is lf_decode_step's own argmax); LF_EHIP if the launch fails.
 */
int lf_sample(const float* d_logits, int32_t rows, int32_t n, float temperature, const float* d_u, int32_t* d_tokens,
              void* stream);

/* Text of the calling thread's last error ("" if none). */
const char* lf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LFDECODE_H */
