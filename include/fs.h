/*
 * fs.h - C ABI of the dense GQA decoder forward pass for gfx950 (MI355X).
 *
 * The library computes the forward pass of a small dense decoder-only
 * transformer of the Qwen3-0.6B kind: token embedding, N blocks of
 * (RMSNorm, Q/K/V projection, per-head q/k RMSNorm, rotate-half RoPE,
 * grouped-query causal attention over a KV cache, output projection and
 * residual, RMSNorm, SwiGLU MLP and residual), a final RMSNorm and the tied
 * embedding as lm_head, of the last row only.  Sources on the pages:
 *   - pipeline ids -> embedding -> blocks -> final norm -> last row -> logits:
 *     "Coming back to Failed Star", section "Second sitting" (data-flow figure);
 *     "Milestones", section M2;
 *   - GQA, RoPE, SwiGLU, RMSNorm: "Failed Star (fs)", section "How it's built";
 *   - Linear weights stored [out, in]: "Coming back to Failed Star",
 *     section "First sitting", item 3;
 *   - tied head: "Failed Star (fs)", section "Status";
 *   - KV cache, one-token decode work, cached == uncached: "Milestones", M4;
 *   - greedy selection (finite logits, lowest ID wins a tie) and the
 *     position budget: "Coming back to Failed Star", section "Next".
 *
 * Conventions for every entry point:
 *   - Return FS_OK (0) or a negative fs_status.  On an error nothing has been
 *     enqueued and fs_last_error() describes it.  No exception crosses the ABI.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; results are valid once the
 *     stream has reached that point.  Device faults surface at the caller's
 *     next synchronisation.
 *   - "device" pointers are HIP device allocations on the current device;
 *     "host" pointers are ordinary CPU memory read before the call returns.
 *   - A model handle is not thread-safe: serialise calls on it, all on one
 *     stream (or order the streams yourself).
 */
#ifndef FS_H
#define FS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FS_OK = 0,
  FS_ERR_INVALID_ARG = -1,   /* NULL pointer, bad size, bad slot, position mismatch */
  FS_ERR_OOM = -2,           /* device allocation failed */
  FS_ERR_HIP = -3,           /* a HIP runtime call or kernel launch failed */
  FS_ERR_CAPACITY = -4,      /* sequence would run past max_ctx (context exhausted) */
  FS_ERR_UNSUPPORTED = -5    /* dtype or shape this build does not implement */
} fs_status;

typedef enum { FS_F32 = 0, FS_BF16 = 1 } fs_dtype;

/* Storage of the matrices (wq, wk, wv, wo, w_gate, w_up, w_down and the tied
 * embedding / head).  The low-bit option answers "Milestones", M7 (decide
 * from measurements whether low-bit weights pay for themselves; "ferrite",
 * What it does, lists the 8-bit block formats it reads):
 *   FS_WEIGHTS_DTYPE:  kept in cfg.dtype;
 *   FS_WEIGHTS_I8_ROW: signed 8-bit codes with one fp32 scale per output row,
 *     made by fs_model_create from the cfg.dtype weights with the
 *     fs_quantize_rows_i8 rule.  Products use code * scale exactly (the scale
 *     multiplies each row's fp32 dot product); the embedding lookup reads the
 *     same codes, so the head stays tied.  Norm weights, activations and the
 *     KV cache keep cfg.dtype.
 *   FS_WEIGHTS_F8_ROW: 8-bit floating-point codes (e4m3: 1 sign, 4 exponent
 *     bits with bias 7, 3 mantissa bits, largest 448; the gfx950 matrix
 *     units' fp8 operand format) with one power-of-two fp32 scale per output
 *     row, made by fs_model_create with the fs_quantize_rows_f8 rule; the
 *     tied embedding / head likewise.  The RMSNorm outputs that feed the
 *     Q/K/V projection, the gate/up projection and the head are quantized per
 *     row by the same rule, so those products are sums of products of two fp8
 *     values (the prefill computes the large ones on the fp8 matrix
 *     instructions); the output and down projections are weight-only.
 *     Requires cfg.dtype = FS_BF16 or FS_F32. */
typedef enum { FS_WEIGHTS_DTYPE = 0, FS_WEIGHTS_I8_ROW = 1, FS_WEIGHTS_F8_ROW = 2 } fs_weight_format;

/* Model shape and KV capacity.
 *   n_heads % n_kv_heads == 0; query head h reads KV head h / (n_heads/n_kv_heads).
 *   head_dim in {64, 128, 256}; hidden, n_heads*head_dim and ffn multiples of 64.
 *   rms_eps: the eps of every RMSNorm, inside the square root.
 *   rope_theta: base of the rotary frequencies theta^(-2i/head_dim).
 *   dtype: element type of every weight, the KV cache, and GEMM operands.
 *          Accumulation and the residual stream are always fp32.
 *   max_seqs: number of KV slots; max_ctx: positions per slot.
 */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps, rope_theta;
  int32_t dtype;             /* fs_dtype */
  int32_t max_seqs, max_ctx;
  /* Gated-attention variant ("ferrite", What it does: gated attention output,
   * rotate-half RoPE on 64 of 256 head dims, q/gate split per head). */
  int32_t rope_dim;          /* rotated dims per head: 0 = all of head_dim; else a multiple of 16 <= head_dim */
  int32_t attn_gate;         /* 0 or 1: wq also carries a sigmoid gate per head */
  int32_t weight_format;     /* fs_weight_format */
} fs_config;

/* One layer's weights, device pointers of cfg.dtype, row-major [out, in]:
 *   attn_norm [hidden], wq [n_heads*head_dim, hidden], wk/wv [n_kv_heads*head_dim, hidden],
 *   q_norm/k_norm [head_dim] (shared by all heads), wo [hidden, n_heads*head_dim],
 *   mlp_norm [hidden], w_gate/w_up [ffn, hidden], w_down [hidden, ffn].
 * With attn_gate, wq is [2*n_heads*head_dim, hidden]: head h's query rows
 * [2h*head_dim, (2h+1)*head_dim) then its gate rows [(2h+1)*head_dim,
 * (2h+2)*head_dim); the head's attention output is multiplied by
 * sigmoid(gate) before wo.  Only the first rope_dim dims of q and k rotate,
 * by p * rope_theta^(-2i/rope_dim), pairs (i, i + rope_dim/2). */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo,
             *mlp_norm, *w_gate, *w_up, *w_down;
} fs_layer_weights;

/* embed [vocab, hidden] (also the lm_head), final_norm [hidden], both device;
 * layers: host array of n_layers entries. */
typedef struct {
  const void *embed, *final_norm;
  const fs_layer_weights *layers;
} fs_weights;

typedef struct fs_model fs_model;

/* Creates a model on the current device.  Synchronous: copies and repacks
 * the weights into library-owned device memory (fused QKV, paired gate/up),
 * so the caller may free its tensors on return (a bf16 model also keeps an
 * fp8 copy of its Q/K/V and gate/up matrices, half their bf16 bytes, for the
 * remainder pass of large prefills).  Allocates the KV cache
 * (max_seqs * max_ctx positions per layer) and the RoPE tables.  All slots
 * start empty.  *out receives the handle (NULL on error).
 * Environment read here, for measurement and tests (results agree to
 * rounding either way): FS_DECODE_GRAPHS=0 launches decode steps one kernel
 * at a time instead of replaying captured graphs; FS_DECODE_ATTN=split or
 * =onepass forces one form of the decode attention (split-K chunks plus a
 * merge launch, or one workgroup per sequence and KV head) where it exists;
 * FS_DECODE_MIN_CHUNK=32|64|128|256 sets the shortest split-K chunk;
 * FS_PREFILL_FUSE_ROPE=0 keeps the per-head q/k norm + RoPE + K/V write of a
 * large prefill in a pass of its own instead of the QKV GEMM's epilogue;
 * FS_GEMM_NORM_REMAINDER=0..3 selects which normalised inputs of the MFMA
 * (bf16) block carry a bf16 remainder pass (1 attention input, 2 MLP input;
 * default 3, both); FS_GEMM_REMAINDER_F8=0 keeps those passes in bf16 on the
 * large prefill GEMM too (by default there they run on fp8 copies of the
 * remainder and of the Q/K/V and gate/up weights, at half the cost);
 * FS_GEMM_TILE_GROUP=0..16 sets how many 256-row tile rows the large GEMMs'
 * workgroups walk together across the columns (default 2; 0 or 1 row-major;
 * read once per process, at the first large GEMM, not per model);
 * FS_PREFILL_F8_MFMA=0 keeps an FS_WEIGHTS_F8_ROW model's prefill on widened
 * (bf16) weights instead of the fp8 matrix instructions (the same values:
 * code * scale is exact in bf16);
 * FS_DECODE_PERSIST=1 runs batch-1 decode steps of the 0.6B shape as one
 * persistent launch (all 256 CUs resident, workgroups exchanging activations
 * in memory; measured slower than the default, see fs_decode_trace);
 * FS_DECODE_TRACE=1 (with it) records the clock stamps fs_decode_trace reads;
 * FS_PREFILL_FIXED_SHIFT=0 keeps the running-max softmax in the head_dim-128
 * prefill attention (by default a layer whose q/k-norm score bound,
 * log2(e) sqrt(d) max|g_q| max|g_k|, is at most 63 takes no softmax shift). */
fs_status fs_model_create(const fs_config *cfg, const fs_weights *w,
                          void *stream, fs_model **out);

/* Frees everything the model owns (waits for its pending work).  NULL is a no-op. */
void fs_model_destroy(fs_model *m);

/* Uncached scorer that also fills the KV cache.
 *   tokens: device int32 [B, S], row b is the prompt for slots[b], token IDs in [0, vocab).
 *   slots:  host int32 [B], distinct, in [0, max_seqs); each slot is reset.
 *   logits: device fp32 [B, vocab]; receives the logits of the LAST position
 *           of each row ("Coming back to Failed Star", First sitting, item 4).
 * Positions are 0..S-1 (no implicit BOS).  After the call slot length = S.
 * Errors: INVALID_ARG for NULL pointers, B <= 0 or > max_seqs, S <= 0 (empty
 * input), bad or duplicate slots; CAPACITY for S > max_ctx.
 * Token IDs are device data, checked on the device: an ID outside [0, vocab)
 * turns its sequence's residual row NaN (that row's logits are NaN, its greedy
 * ID -1, and the slot's cache holds NaN) and is recorded in pinned host memory;
 * the next fs_prefill, fs_decode_step or fs_generate on the model (or the same
 * fs_generate, which is synchronous) returns INVALID_ARG naming the ID and
 * enqueues nothing.  The record is cleared once reported. */
fs_status fs_prefill(fs_model *m, const int32_t *tokens, int32_t B, int32_t S,
                     const int32_t *slots, float *logits, void *stream);

/* One KV-cached decode step for B sequences.
 *   tokens:    device int32 [B] (e.g. the previous step's `next`; may alias `next`).
 *   positions: host int32 [B], positions[i] must equal the current length of slots[i].
 *   slots:     host int32 [B], distinct, in [0, max_seqs).
 *   logits:    device fp32 [B, vocab] or NULL.
 *   next:      device int32 [B] or NULL: greedy ID per row (argmax over finite
 *              logits, lowest ID on an exact tie, -1 if none is finite).
 * Appends K/V at positions[i] and attends over 0..positions[i]; afterwards
 * the slot length is positions[i]+1.
 * Errors: INVALID_ARG (NULL tokens, B out of range, bad/duplicate slot,
 * position != slot length, both outputs NULL, or an out-of-range token ID
 * recorded by an earlier call, see fs_prefill); CAPACITY if positions[i] >= max_ctx.
 * An out-of-range ID in `tokens` makes that row's logits NaN and its `next` -1. */
fs_status fs_decode_step(fs_model *m, const int32_t *tokens, const int32_t *positions,
                         const int32_t *slots, int32_t B, float *logits, int32_t *next,
                         void *stream);

/* Greedy selection over rows of logits.
 *   logits: device fp32 [B, V]; out: device int32 [B].
 * out[b] = index of the largest finite logit of row b, the lowest index among
 * exact ties ("Coming back to Failed Star", section "Next", Selection);
 * -1 if the row holds no finite value.  Errors: INVALID_ARG for NULL or B, V <= 0. */
fs_status fs_argmax(const float *logits, int32_t B, int32_t V, int32_t *out, void *stream);

/* Per-row symmetric int8 quantization (the FS_WEIGHTS_I8_ROW rule).
 *   src:    device [rows, cols] of dtype (fs_dtype), row-major.
 *   codes:  device int8 [rows, cols]; scales: device fp32 [rows].
 * scale[r] = max_k |src[r, k]| / 127 and codes[r, k] = nearest integer to
 * src[r, k] / scale[r] (ties to even), both quotients correctly rounded fp32;
 * a row of zeros gets scale 0 and zero codes.  Rows whose largest magnitude
 * is below the fp32 normal range are outside the rule's contract.
 * Errors: INVALID_ARG for NULL pointers, rows or cols <= 0, cols % 8 != 0;
 * UNSUPPORTED for an unknown dtype. */
fs_status fs_quantize_rows_i8(const void *src, int32_t dtype, int32_t rows, int32_t cols,
                              int8_t *codes, float *scales, void *stream);

/* Per-row fp8 quantization (the FS_WEIGHTS_F8_ROW rule, also the rule of its
 * activation rows).
 *   src:    device [rows, cols] of dtype (fs_dtype), row-major.
 *   codes:  device uint8 [rows, cols] (e4m3 codes); scales: device fp32 [rows].
 * scale[r] = the smallest power of two >= fl32(max_k |src[r, k]| / 448)
 * (fl32: the correctly rounded fp32 quotient), codes[r, k] = the e4m3 value
 * nearest to src[r, k] / scale[r] (an exact quotient; ties to the even
 * mantissa; magnitudes past 448 saturate); a row of zeros gets scale 0 and
 * zero codes.  Errors: INVALID_ARG for NULL pointers, rows or cols <= 0,
 * cols % 8 != 0, misaligned pointers (src 16 B, codes 8 B, scales 4 B);
 * UNSUPPORTED for an unknown dtype. */
fs_status fs_quantize_rows_f8(const void *src, int32_t dtype, int32_t rows, int32_t cols,
                              uint8_t *codes, float *scales, void *stream);

/* Product of two e4m3 code matrices with one power-of-two scale per row: the
 * arithmetic of the FS_WEIGHTS_F8_ROW model's Q/K/V and gate/up products at
 * prefill sizes, where both the weights and the quantized norm outputs are
 * codes ("Milestones", M7: the low-bit path measured against the baseline).
 *   a_codes: device uint8 [M, K], a_scales: device fp32 [M];
 *   w_codes: device uint8 [N, K], w_scales: device fp32 [N] (both as
 *            fs_quantize_rows_f8 writes them; K contiguous);
 *   out:     device fp32 [M, N], row-major:
 *            out[m, n] = a_scales[m] * w_scales[n] * sum_k e4m3(a[m, k]) * e4m3(w[n, k]).
 * Each product of two codes is exact; the sum is accumulated in fp32.  Runs
 * the model's fp8 matrix-instruction kernel (256x256 tiles) whatever M.  A NaN
 * code (0x7f, 0xff) makes its row / column NaN.  Asynchronous on stream.
 * Errors: INVALID_ARG for NULL pointers, M, N or K <= 0, K % 64 != 0,
 * N % 8 != 0, misaligned pointers (codes, out and w_scales 16 B, a_scales 4 B). */
fs_status fs_gemm_f8(const uint8_t *a_codes, const float *a_scales, const uint8_t *w_codes,
                     const float *w_scales, int32_t M, int32_t N, int32_t K, float *out, void *stream);

/* Parameters of the sampling chain temperature -> top-k -> top-p ->
 * renormalise -> draw ("Coming back to Failed Star", section "Next": the
 * sampling arc with an explicit filter order; "ferrite", What it does). */
typedef struct {
    float temperature;   /* > 0 samples; 0 selects greedily (the fs_argmax rule) */
    int32_t top_k;       /* keep logits >= the k-th largest (ties kept); 0 = no limit */
    float top_p;         /* in (0, 1]: keep tokens at least as probable as the one at which
                            the ranked mass of the top-k set first reaches top_p; 1 = keep all */
} fs_sampling;

/* Draws one token per row of logits.
 *   logits: device fp32 [B, V]; u: device fp32 [B], uniform draws in [0, 1)
 *           supplied by the caller (e.g. from a seeded generator; ignored when
 *           temperature is 0); out: device int32 [B].
 * Only finite logits take part.  The kept probabilities (computed in fp32 as
 * 2^((x - max) log2(e) / temperature)) are renormalised and u is mapped
 * through their cumulative distribution in increasing token ID: out[b] is the
 * first kept ID whose cumulative probability exceeds u[b]; -1 for a row with
 * no finite logit.  Uses the model's sampling scratch (allocated on the first
 * call, rows up to cfg.max_seqs); calls on one model must not overlap.
 * Errors: INVALID_ARG (NULL pointer, B outside [1, max_seqs], V <= 0,
 * temperature < 0 or not finite, top_k < 0, top_p outside (0, 1]), OOM, HIP. */
fs_status fs_sample(fs_model *m, const float *logits, int32_t B, int32_t V,
                    const fs_sampling *sampling, const float *u, int32_t *out, void *stream);

/* fs_sample for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, rule and results as fs_sample, without a model handle; the
 * per-row histograms live in a static device array of the library
 * (FS_SAMPLE_NOALLOC_MAX_ROWS rows, about 68 KB each; one copy per GPU, held
 * until the process ends), whose address is looked up once per device on the
 * first call there.  Allocates nothing; each call clears the rows it uses.
 * Every call on one GPU shares that array: calls that overlap on a GPU (on
 * different streams, or from different threads) race and must be serialised
 * by the caller.
 * Errors: CAPACITY for B > FS_SAMPLE_NOALLOC_MAX_ROWS; otherwise as fs_sample
 * (INVALID_ARG for NULL pointers, B <= 0, V <= 0 or bad sampling
 * parameters; HIP). */
#define FS_SAMPLE_NOALLOC_MAX_ROWS 64
fs_status fs_sample_noalloc(const float *logits, int32_t B, int32_t V, const fs_sampling *sampling,
                            const float *u, int32_t *out, void *stream);

/* Why fs_generate stopped. */
typedef enum {
    FS_STOP_NONE = 0,
    FS_STOP_EOS = 1,       /* the selected token is in the EOS set */
    FS_STOP_BUDGET = 2,    /* max_new_tokens tokens are out (or the budget was 0) */
    FS_STOP_CONTEXT = 3    /* the last token would be forwarded at position max_ctx */
} fs_stop_reason;

/* Settings of one generation. */
typedef struct {
    int32_t max_new_tokens;        /* >= 0; 0 returns at once without any forward pass */
    const int32_t *eos_ids;        /* host int32 [n_eos]: the explicit EOS set (may be empty) */
    int32_t n_eos;
    int32_t include_stop_id;       /* nonzero: the EOS ID that stops the loop is returned as the last ID */
    const fs_sampling *sampling;   /* NULL or temperature 0: greedy (the fs_argmax rule) */
    const float *uniforms;         /* device fp32 [max_new_tokens] when sampling: token i draws with uniforms[i] */
} fs_generation;

/* Greedy or sampled generation for one sequence, under the contract the
 * pages ask to settle first ("Coming back to Failed Star", section "Next:
 * one complete deterministic generation arc"): raw token IDs, no implicit
 * BOS; an explicit EOS set; a token budget that may be zero; never a forward
 * pass at a position >= max_ctx; distinct stop reasons.
 *   prompt: device int32 [S], S >= 1; slot: the sequence's slot (reset, as by
 *   fs_prefill); out_ids: host int32 [max_new_tokens]; *n_out: IDs written;
 *   *stop_reason: an fs_stop_reason.
 * Token i is selected from the logits of position S-1+i.  After selecting it:
 * an EOS ID stops the loop (FS_STOP_EOS; appended only with include_stop_id);
 * otherwise the ID is appended; a full budget stops (FS_STOP_BUDGET); if the
 * token's own position S+i is >= max_ctx it cannot be forwarded and the loop
 * stops with the token kept (FS_STOP_CONTEXT); else one decode step (graph
 * replay) forwards it.  The host reads each 4-byte token back to check the
 * stop rules while the step forwarding it already runs; a step issued for a
 * token that then stops the loop is discarded (the slot length counts only
 * the forwarded tokens: S plus the IDs fed back).  Synchronous.
 * Errors: INVALID_ARG (NULL pointer, S <= 0, bad slot, max_new_tokens < 0,
 * n_eos < 0, bad sampling parameters); CAPACITY (S > max_ctx); UNSUPPORTED
 * (a step's logits hold no finite value: the loop stops, *n_out and
 * *stop_reason = FS_STOP_NONE describe what was produced); OOM, HIP. */
fs_status fs_generate(fs_model *m, const int32_t *prompt, int32_t S, int32_t slot,
                      const fs_generation *gen, int32_t *out_ids, int32_t *n_out,
                      int32_t *stop_reason, void *stream);

/* Current length (positions filled) of a slot, or -1 for a bad handle/slot. */
int32_t fs_slot_length(const fs_model *m, int32_t slot);

/* Copies cached K (normed and rotated) and V of one layer, slot and KV head,
 * positions [pos0, pos0+n), into device buffers k_out, v_out of cfg.dtype,
 * [n, head_dim] each.  For inspection and tests.  Errors: INVALID_ARG. */
fs_status fs_kv_read(const fs_model *m, int32_t layer, int32_t slot, int32_t kv_head,
                     int32_t pos0, int32_t n, void *k_out, void *v_out, void *stream);

/* Measurement hook.  fs_timing(m, 1) waits for the device, clears earlier
 * records and starts recording: every kernel this model launches is then
 * bracketed by a pair of HIP events on the call's stream, labelled with the
 * step it implements ("embed", "norm", "qkv", "rope_kv", "attn", "combine",
 * "attn_gate", "wconv", "o_proj", "gate_up", "down", "head", "argmax"; a
 * prefill whose QKV GEMM does the q/k norm + RoPE + K/V write in its epilogue
 * has no "rope_kv" launches), and decode steps run
 * without graph replay.  fs_timing(m, 0) stops recording (records are kept
 * until the next fs_timing call).  Errors: INVALID_ARG for a NULL model. */
fs_status fs_timing(fs_model *m, int32_t enable);

/* Sum of the recorded launch intervals of one label: *total_ms (milliseconds)
 * and *launches.  Waits for the recorded events.  Errors: INVALID_ARG. */
fs_status fs_timing_read(fs_model *m, const char *label, double *total_ms, int64_t *launches);

/* Measurement hook: average duration of one decode-shaped (batch 1) launch
 * of the kernel that implements `label` ("qkv", "attn", "attn_split",
 * "attn_onepass", "combine", "o_proj", "gate_up", "down" or "head"), as it
 * runs inside a decode step; "empty" launches a kernel of 256 workgroups that
 * does nothing, in the same chain, so its figure is the per-launch floor the
 * step's dependent kernels each pay; "mfma" launches 256 workgroups of 8
 * waves, each wave 8192 32x32x16 bf16 matrix instructions on registers in
 * eight independent chains (2 * 32 * 32 * 16 * 8192 * 2048 flops per launch),
 * the matrix unit's own throughput; "hbm" reads the model's whole allocation
 * of matrices (embedding / head and every layer's projections, as stored)
 * once per launch with 16-byte loads, the HBM read rate a streaming kernel
 * reaches.  "attn" is the form of the decode attention a
 * batch-1 step at this position takes (one pass over the whole context with
 * no merge launch for short contexts, split-K chunks plus the "combine"
 * merge otherwise); "attn_split" and "attn_onepass" force one form.  One launch per layer,
 * each with that layer's weights, captured back to back in a graph and
 * replayed `reps` times between two HIP events on `stream` (so the figure
 * includes the per-launch dispatch cost of graph replay).  *avg_us receives
 * microseconds per launch.  The call overwrites the model's activation
 * scratch; "attn" also reads context 0..position of `slot` and writes K/V row
 * `position` of that slot with values derived from the scratch, so use a
 * slot that holds nothing of value ("combine" merges the partials of a
 * context of position+1).  Other labels ignore slot and position.
 * Synchronous.  Errors: INVALID_ARG (unknown label, bad slot/position,
 * reps <= 0), UNSUPPORTED ("attn_onepass" for a head shape without that
 * form), HIP. */
fs_status fs_kernel_bench(fs_model *m, const char *label, int32_t slot, int32_t position,
                          int32_t reps, double *avg_us, void *stream);

/* Measurement hook of the persistent batch-1 decode step (the one-launch
 * step the 0.6B shape takes at batch 1): with FS_DECODE_TRACE=1 set when the
 * model is created, each such step records the GPU's 100 MHz real-time clock
 * at fixed points of workgroup 0 into a 1024-entry device buffer (entry 0:
 * start; 8l+1..8l+6: layer l's waits done in the control wave, 8l+7: polls
 * its first wait took; 512+8l..: the compute wave's phase boundaries; 511,
 * 1023: the end); fs_decode_trace
 * copies the first n entries of the last step's record to host `out`
 * (synchronous).  Errors: INVALID_ARG, UNSUPPORTED (no trace buffer). */
fs_status fs_decode_trace(fs_model *m, int64_t *out, int32_t n);

/* Message of the last error on this thread ("" if none); valid until the
 * next fs_* call on this thread. */
const char *fs_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FS_H */
