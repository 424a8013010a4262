/*
 * dflash2.h -- C ABI of the DFlash2 block draft -> select -> verify step on
 * AMD Instinct MI355X (gfx950).
 *
 * The step (per sequence):
 *   1. append the target hidden-state taps of newly verified positions to the
 *      draft's context (feature projection + RMSNorm, then every layer's
 *      key/value projection with RoPE) -- NeMo AutoModel, "Train a DFlash
 *      Drafter for Speculative Decoding", section "What is DFlash?";
 *   2. run one non-causal forward of the draft stack over a block of
 *      block_size slots (slot 0 = the real anchor token, the rest = the
 *      reserved mask id), with a two-tap in-block depthwise convolution before
 *      every sublayer -- same page, sections "What is DFlash?" and "Variants"
 *      (row "DFlash 2"), and "Data" (mask token);
 *   3. project slots 1..block_size-1 through the shared lm_head and keep the
 *      selector_top_k best candidates per slot -- same page, "Variants";
 *   4. pick one coherent path through the candidate lattice with a rank-r
 *      pairwise selector solved by max-sum dynamic programming -- same page,
 *      "Variants" and "Objective"; llama-cpp-python wiki "DFlash2 Speculative
 *      Decoding", "Complete Runnable Code" (selector lattice);
 *   5. verify the path greedily against the target's logits and return the
 *      longest accepted prefix plus the target's own next token -- NeMo
 *      SpeechLM "DFlash speculative decoding with vLLM", intro and
 *      "Validation"; llama-cpp-python wiki, "Prerequisites".
 *
 * Conventions for every call:
 *   - Pointers marked [device] are device addresses on the current HIP
 *     device; [host] are host addresses.  The library never allocates device
 *     memory and never synchronises: work is enqueued on `stream` and the call
 *     returns.  The caller owns every buffer and must keep inputs alive and
 *     outputs unread until the stream reaches the enqueued work.
 *   - All linear weights are row-major [out, in]: y = x * W^T.
 *   - Element types: "act" is float32 when config.weight_dtype == FP32 and
 *     bf16 (uint16 bit pattern) otherwise; "param" (embedding, conv taps,
 *     norm gains) follows act; weights of the linears follow weight_dtype
 *     (fp8 = OCP e4m3fn codes with one float32 scale per output row).
 *   - Tuning: the environment variable DFLASH2_LMHEAD_TILES_PER_BLOCK
 *     (1..64), read at each dflash2_draft_block call, sets how many
 *     256-id vocabulary tiles one lm_head block sweeps when the batch has
 *     more than 64 rows (default: chosen from the shapes), and
 *     DFLASH2_TILED_MAX_SPLITS (1..16, default 16), read by
 *     dflash2_workspace_size and dflash2_draft_block, caps the K splits of
 *     those batches' linears (one
 *     split lets the GEMM apply SwiGLU and the QKV RoPE itself), and
 *     DFLASH2_STREAM_BLOCK_OVERHEAD (0..65536, default 256), read by the same
 *     calls, is the fixed cost of one weight-streaming block (batches of at
 *     most 64 rows), in k, in the model that picks their K splits, and
 *     DFLASH2_STREAM_MAX_ROW_BYTES (256..1048576, default 3072), read by the
 *     same calls, is the longest stretch of one weight row a streaming block
 *     reads (the planner prefers splits that keep within it).  Results agree
 *     to rounding either way.
 *   - Every call returns DFLASH2_OK or an error code; on error nothing was
 *     enqueued and dflash2_last_error() (thread-local) describes it.  Device
 *     data (ids, lengths, offsets) cannot be checked on the host; kernels
 *     skip any access such data would push outside its buffer, so a bad
 *     value gives wrong results for that sequence, never a fault.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH2_OK = 0,
  DFLASH2_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum   */
  DFLASH2_ERR_SHAPE = 2,       /* sizes inconsistent with the handle       */
  DFLASH2_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. K % 32)  */
  DFLASH2_ERR_WORKSPACE = 4,   /* workspace null, misaligned or too small  */
  DFLASH2_ERR_HIP = 5          /* a HIP runtime call failed                */
} dflash2_status;

typedef enum { DFLASH2_FP32 = 0, DFLASH2_BF16 = 1, DFLASH2_FP8_E4M3 = 2 } dflash2_dtype;

/* Draft configuration.  Field names follow the dflash_config keys (NeMo
 * SpeechLM page, "DFlash2 inference") and the recipe keys (NeMo AutoModel
 * page, "Key Config Fields" table).  target_layer_ids enter only through
 * num_taps and the order of the taps in new_taps. */
typedef struct {
  int32_t hidden;           /* draft width H                                  */
  int32_t num_layers;       /* draft_num_hidden_layers                        */
  int32_t num_q_heads;      /* draft_num_attention_heads                      */
  int32_t num_kv_heads;     /* draft_num_key_value_heads (divides num_q_heads) */
  int32_t head_dim;         /* draft_head_dim (even, <= 256)                  */
  int32_t ffn;              /* SwiGLU width F                                 */
  int32_t vocab;            /* V, shared with the target                      */
  int32_t num_taps;         /* len(target_layer_ids)                          */
  int32_t tap_width;        /* target hidden width of one tap                 */
  int32_t block_size;       /* num_speculative_tokens + 1, >= 2               */
  int32_t conv_kernel_size; /* taps of the in-block convolution, 1..block_size */
  int32_t selector_top_k;   /* candidates per slot, 1..64, <= vocab           */
  int32_t selector_rank;    /* rank r of the pairwise selector, 1..256        */
  int32_t max_batch;        /* sequences a cache holds (its batch dimension)  */
  int32_t max_context;      /* rows a cache holds per sequence and kv head    */
  int32_t sliding_window;   /* draft_sliding_window; 0 = attend to all rows   */
  int32_t mask_token_id;    /* reserved id filling slots 1..block_size-1      */
  int32_t weight_dtype;     /* dflash2_dtype of the linears and lm_head       */
  int32_t conv_group_size;  /* 0: static per-channel taps (conv_attn/conv_ffn);
                               > 0: dynamic taps, one set per group of this
                               many channels, computed from the slot's input
                               (dconv_attn/dconv_ffn); must divide hidden   */
  float rms_eps;            /* RMSNorm epsilon                                */
  float rope_theta;         /* RoPE base                                      */
  float input_embedding_scale;   /* scales the embedded block (1 = identity);
                                    must be finite                             */
  float output_multiplier;       /* logit transform multiplier (1 = identity);
                                    must be finite and > 0, so that the
                                    transform keeps the ranking of the logits */
  float final_logit_softcapping; /* logit soft cap; 0 = off; finite, >= 0      */
} dflash2_config;

/* Per-layer weights [device].  *_scale are float32 [out rows], required for
 * FP8_E4M3 and ignored otherwise. */
typedef struct {
  const void* conv_attn;     /* [conv_kernel_size, H] param: tap j multiplies slot t-j
                                (static taps; unused with conv_group_size > 0) */
  const void* attn_norm;     /* [H] param                                     */
  const void* wqkv;          /* [(nq + 2 nkv) * d, H]: q heads, k heads, v heads */
  const float* wqkv_scale;
  const void* wo;            /* [H, nq * d]                                   */
  const float* wo_scale;
  const void* conv_ffn;      /* [conv_kernel_size, H] param                   */
  const void* ffn_norm;      /* [H] param                                     */
  const void* w_gate_up;     /* [2F, H]: rows 0..F-1 gate, F..2F-1 up         */
  const float* w_gate_up_scale;
  const void* w_down;        /* [H, F]                                        */
  const float* w_down_scale;
  /* Dynamic convolution (conv_group_size G > 0, NeMo SpeechLM page, "DFlash2
   * inference": DFlash2 adds dynamic convolutions; NeMo AutoModel page, "Key
   * Config Fields": conv_group_size channels per dynamic correction).  Slot
   * t's taps are c[t] = W x_t with W [(H/G) * conv_kernel_size, H] (weight
   * dtype), row g * conv_kernel_size + j = tap j of channel group g, and
   * y_t[ch] = x_t[ch] + sum_j c[t][ch / G][j] * x_{t-j}[ch].  Ignored (may be
   * null) when conv_group_size is 0; the static conv_* are then used. */
  const void* dconv_attn;
  const float* dconv_attn_scale;
  const void* dconv_ffn;
  const float* dconv_ffn_scale;
} dflash2_layer_weights;

/* Draft weights.  Device pointers, not owned: they must outlive the handle.
 * `layers` is a [host] array of num_layers entries, copied at create. */
typedef struct {
  const void* embed;         /* [V, H] param: the target's embed_tokens       */
  const void* lm_head;       /* [V, H] weight dtype: the target's lm_head     */
  const float* lm_head_scale;
  const void* proj;          /* [H, num_taps * tap_width] feature projection  */
  const float* proj_scale;
  const void* proj_norm;     /* [H] param                                     */
  const void* final_norm;    /* [H] param                                     */
  const float* sel_tl;       /* [V, r] float32 left selector factors          */
  const float* sel_tr;       /* [V, r] float32 right selector factors         */
  const dflash2_layer_weights* layers;
} dflash2_weights;

typedef struct dflash2_handle dflash2_handle;

/* Validate the configuration and weight table and build a handle.  Rejects
 * (before any device work, the same rule the NIM page states for draft heads
 * in "Bring Your Own DFlash2 Head"): block_size outside 2..4096,
 * max_batch * block_size > 2^30, num_q_heads not a multiple of
 * num_kv_heads, odd or oversized head_dim, conv_kernel_size outside
 * 1..block_size, conv_group_size that is negative or does not
 * divide hidden, selector_top_k outside 1..min(64, vocab), selector_rank
 * outside 1..256, mask_token_id outside [0, vocab), an unknown weight_dtype,
 * a null weight (the static conv taps when conv_group_size is 0, the dynamic
 * ones otherwise), a missing fp8 scale, a weight or scale pointer that is not
 * 16-byte aligned (the kernels read 16 bytes at a time), a non-finite rms_eps, rope_theta,
 * input_embedding_scale or softcap, an output_multiplier that is not finite
 * and > 0 (top-k ranks the raw logits and transforms the kept values, which
 * needs a strictly increasing transform), and (UNSUPPORTED) any contraction
 * length (hidden, ffn, nq*head_dim, num_taps*tap_width) that is not a
 * multiple of 32 or exceeds 2^20 (the GEMM tiles use 32-bit offsets from a
 * 64-bit tile base), hidden > 16384 or max_context not a multiple of 8.  The
 * handle keeps a host copy of the config and the pointer table only; it is
 * immutable and may be shared across threads and streams. */
dflash2_status dflash2_create(const dflash2_config* config, const dflash2_weights* weights,
                              dflash2_handle** out);
void dflash2_destroy(dflash2_handle* handle);

/* Bytes of device workspace dflash2_draft_block needs for `batch` sequences
 * and at most `max_new_rows` appended context rows in total. */
dflash2_status dflash2_workspace_size(const dflash2_handle* handle, int32_t batch,
                                      int64_t max_new_rows, size_t* bytes);

/* Steps 1-3 for `batch` sequences (1 <= batch <= max_batch).
 *   anchor_ids  [device] int32 [batch]: the last verified token of each
 *               sequence; it fills slot 0.
 *   new_taps    [device] act [max_new_rows, num_taps, tap_width]: target
 *               hidden states of the newly verified positions, sequence by
 *               sequence, taps in target_layer_ids order.
 *   new_offsets [device] int32 [batch + 1]: prefix sums of the rows each
 *               sequence appends; new_offsets[batch] <= max_new_rows.
 *   ctx_lens    [device] int32 [batch]: context length L_b after the append;
 *               the new rows take positions L_b - n_b .. L_b - 1 and the
 *               block's slots positions L_b .. L_b + block_size - 1, so
 *               L_b + block_size <= max_context is required.
 *   max_new_rows [host]: upper bound on new_offsets[batch] (sizes grids and
 *               the workspace; block_size * batch bounds a warm step).
 *   k_cache     [device] act [num_layers][max_batch][num_kv_heads][max_context][head_dim]
 *   v_cache     [device] act [num_layers][max_batch][num_kv_heads][head_dim][max_context]
 *               (values are stored transposed: position is the fastest axis).
 *               Keys are stored after RoPE.  The call writes context rows
 *               [L_b - n_b, L_b) and uses rows [L_b, L_b + block_size) as
 *               scratch for the block's own keys/values; nothing else.  A
 *               rejected block therefore needs no rollback: the next step's
 *               append overwrites the scratch rows it reaches.
 *   topk_ids    [device] int32 [batch, block_size-1, selector_top_k]: per slot
 *               1.. the best ids under (logit desc, id asc), -0.0 ranked as +0.0.
 *   topk_vals   [device] float [batch, block_size-1, selector_top_k]: the
 *               logit transform applied to those logits.
 *   debug_logits [device, nullable] float [batch, block_size-1, vocab]: the
 *               float32 logits the ranking used (before the transform).
 *   debug_hidden [device, nullable] float [batch, block_size, hidden]: the
 *               residual stream after the last layer.
 *   workspace   [device] >= dflash2_workspace_size bytes, 256-byte aligned;
 *               scratch only, contents need no initialisation.
 * new_taps, k_cache, v_cache, debug_logits and debug_hidden must be 16-byte
 * aligned (DFLASH2_ERR_INVALID_ARG otherwise). */
dflash2_status dflash2_draft_block(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                   const int32_t* anchor_ids, const void* new_taps,
                                   const int32_t* new_offsets, const int32_t* ctx_lens,
                                   int64_t max_new_rows, void* k_cache, void* v_cache,
                                   int32_t* topk_ids, float* topk_vals, float* debug_logits,
                                   float* debug_hidden, void* workspace, size_t workspace_bytes);

/* Step 4.  One coherent path per sequence through the candidate lattice:
 *   c_0 = anchor, c_t = topk_ids[b, t-1, path_t], maximising
 *   sum_t pi(c_{t-1}, c_t) + topk_vals[b, t-1, path_t]  with
 *   pi(a, b) = sum_m sel_tl[a, m] * sel_tr[b, m]
 * evaluated in float32 exactly as: multiply, then add, m ascending from +0;
 * S_1 = pi(c_0, .) + z_1; S_t = max_i (S_{t-1}[i] + pi) + z_t.  Ties take
 * the smallest predecessor rank and the smallest final rank.
 *   anchor_ids [device] int32 [batch]; topk_ids/topk_vals as produced above
 *   (any candidates may be passed: ids are only used to index the tables).
 *   path_idx   [device] int32 [batch, block_size-1]: chosen candidate rank.
 *   draft_tokens [device] int32 [batch, block_size-1]: chosen token ids.
 *   path_score [device, nullable] float [batch].
 *   debug_pair [device, nullable] float [batch, block_size-1, k, k]: pair
 *              scores pi(c_{t-1,i}, c_{t,j}); slab 0 repeats pi(anchor, c_{1,j})
 *              in every row i.
 * No workspace; 1 <= batch <= max_batch. */
dflash2_status dflash2_select_path(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                   const int32_t* anchor_ids, const int32_t* topk_ids,
                                   const float* topk_vals, int32_t* path_idx,
                                   int32_t* draft_tokens, float* path_score, float* debug_pair);

/* Step 4 with the draft-length rule (llama-cpp-python wiki, "DFlash2
 * Speculative Decoding", "Configuration Notes": a positive draft_p_min stops
 * a path before a low-confidence selector transition; draft_n_max caps the
 * draft at block_size-1; "Complete Runnable Code": SpecConfig also carries
 * draft_n_min).  The path, drafts and score are exactly those of
 * dflash2_select_path.  Then, per position t, the transition's confidence is
 * the softmax over the k candidates of the lattice's float32 scores
 * pi(c_prev, c_j) + topk_vals[b, t, j], c_prev being the predecessor the path
 * took (the anchor at t = 0), taken at the chosen candidate (float32 expf).
 * draft_lens[b] = min(n_max', first t >= n_min' with conf < p_min, else
 * block_size-1), where n_max' = n_max clamped to [0, block_size-1] and
 * n_min' = n_min clamped to [0, n_max'].  p_min = 0 never stops a path.
 *   p_min      in [0, 1], else DFLASH2_ERR_INVALID_ARG.
 *   draft_lens [device] int32 [batch] (required).
 *   path_conf  [device, nullable] float [batch, block_size-1].
 *   path_score [device, nullable] float [batch].
 * No workspace; 1 <= batch <= max_batch. */
dflash2_status dflash2_select_path_stop(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                        const int32_t* anchor_ids, const int32_t* topk_ids,
                                        const float* topk_vals, float p_min, int32_t n_min,
                                        int32_t n_max, int32_t* path_idx, int32_t* draft_tokens,
                                        int32_t* draft_lens, float* path_conf, float* path_score);

/* Steps 1-4 in one call (NeMo AutoModel page, "Variants", row DFlash 2:
 * each position's top-k candidates and one path through them): exactly
 * dflash2_draft_block followed by dflash2_select_path on its outputs, with
 * the same arguments and results (topk_ids / topk_vals are still written),
 * except that the per-row candidate merge runs inside the selector's
 * kernel, one launch instead of two, when selector_top_k <= 16 and the
 * lm_head left at most 64 candidate lists per row (the LDS-tiled lm_head
 * of more than 64 rows, or a vocabulary of at most 8192 ids).
 * debug_hidden and debug_pair are not offered; path_score may be null.
 * Workspace: dflash2_workspace_size, as for dflash2_draft_block. */
dflash2_status dflash2_draft_select(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                    const int32_t* anchor_ids, const void* new_taps,
                                    const int32_t* new_offsets, const int32_t* ctx_lens,
                                    int64_t max_new_rows, void* k_cache, void* v_cache, int32_t* topk_ids,
                                    float* topk_vals, int32_t* path_idx, int32_t* draft_tokens,
                                    float* path_score, float* debug_logits, void* workspace,
                                    size_t workspace_bytes);

/* Bytes of device workspace dflash2_verify_accept needs.  Every stateless
 * step-5 and loss entry point below requires 2 <= block_size <= 4096,
 * batch >= 1, batch * block_size <= 2^30 and vocab >= 1, else
 * DFLASH2_ERR_SHAPE. */
dflash2_status dflash2_verify_workspace_size(int32_t batch, int32_t block_size, int32_t vocab,
                                             size_t* bytes);

/* Step 5, stateless.  Row i of target_logits [device] float [batch,
 * block_size, vocab] is the target's prediction after block slot i (slot 0 =
 * the anchor).  g_i = argmax (ties to the smallest id, -0.0 as +0.0, NaN
 * never wins).  accepted[b] = the largest n <= block_size-1 with
 * g_i == draft_tokens[b, i] for all i < n; bonus[b] = g_n.  The step emits
 * accepted[b] drafts plus the bonus token.
 *   draft_tokens [device] int32 [batch, block_size-1]
 *   accepted, bonus [device] int32 [batch]
 *   target_argmax [device, nullable] int32 [batch, block_size]
 *   workspace [device] >= dflash2_verify_workspace_size bytes, 256-aligned. */
dflash2_status dflash2_verify_accept(hipStream_t stream, int32_t batch, int32_t block_size,
                                     int32_t vocab, const int32_t* draft_tokens,
                                     const float* target_logits, int32_t* accepted,
                                     int32_t* bonus, int32_t* target_argmax, void* workspace,
                                     size_t workspace_bytes);

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): dflash2_verify_accept with its scratch in a fixed device
 * array inside the library (1 MiB per GPU, held until the process ends)
 * instead of a workspace argument.  Same arguments, kernels and results as
 * dflash2_verify_accept.  batch * block_size must be <= 131072, else
 * DFLASH2_ERR_WORKSPACE (before any device work).  The array's device
 * address is looked up once per GPU, on the first call with a stream of
 * that GPU; no call allocates.  All calls on one GPU share the array:
 * calls that overlap on one GPU (concurrent streams or threads) race, and
 * must be serialised by the caller. */
dflash2_status dflash2_verify_accept_noalloc(hipStream_t stream, int32_t batch, int32_t block_size,
                                             int32_t vocab, const int32_t* draft_tokens,
                                             const float* target_logits, int32_t* accepted,
                                             int32_t* bonus, int32_t* target_argmax);

/* Bytes of device workspace dflash2_verify_sample needs (>= the greedy
 * verification's). */
dflash2_status dflash2_verify_sample_workspace_size(int32_t batch, int32_t block_size, int32_t vocab,
                                                    size_t* bytes);

/* Step 5 with sampling, stateless (NeMo AutoModel page, "Key Config Fields",
 * paragraph on spec_generate: temperature, top-p and top-k truncate the
 * target's distribution and rejection sampling verifies the drafts against
 * it, so sampled decoding keeps the target's output distribution).  Row i of
 * target_logits [device] float [batch, block_size, vocab] is the target's
 * prediction after block slot i.  Per row the target distribution is
 *   p_v = e_v / S over the kept set,  e_v = exp((z_v - m) / temperature),
 * m = the row maximum; NaN logits weigh 0, +inf acts as FLT_MAX, entries
 * equal to m weigh 1.  The kept set: top_k (0 or >= vocab: off) keeps every
 * entry >= the top_k-th largest value (ties kept); then top_p (>= 1: off)
 * keeps an entry while the kept mass strictly above its value is below
 * top_p times the kept mass (equal values kept or dropped together).
 * The draft path is deterministic (a point mass on each draft), so draft i
 * (i < draft_lens[b]) is accepted while u_i < p_i(d_i); at the first
 * rejection the bonus is drawn from p_i with d_i struck out; when every
 * proposed draft is accepted it is drawn from row draft_lens[b].  A draw is
 * the smallest id j (ascending ids) whose cumulative mass exceeds v * total.
 * Weights are 64-bit fixed point (e_v * 2^(52 - ceil(log2 vocab)), rounded),
 * so all sums and decisions are exact and deterministic; they differ from
 * real arithmetic by at most vocab * 2^-(53 - ceil(log2 vocab)) of the mass.
 * temperature 0 is the greedy rule of dflash2_verify_accept (uniforms unused).
 *   draft_tokens [device] int32 [batch, block_size-1]
 *   draft_lens   [device, nullable] int32 [batch]: drafts proposed per
 *                sequence, clamped to [0, block_size-1]; null = all.
 *   uniforms     [device] float [batch, block_size] in [0, 1): column i
 *                (< block_size-1) is u_i, the last column is v (a value
 *                outside [0, 1) gives some token of the row, unspecified).
 *   temperature  finite, >= 0; top_k >= 0; top_p > 0; else
 *                DFLASH2_ERR_INVALID_ARG.
 *   accepted, bonus [device] int32 [batch]
 *   draft_prob   [device, nullable] float [batch, block_size-1]: p_i(d_i)
 *                for i < draft_lens[b], 0 beyond.
 *   workspace    [device] >= dflash2_verify_sample_workspace_size bytes,
 *                256-aligned. */
dflash2_status dflash2_verify_sample(hipStream_t stream, int32_t batch, int32_t block_size, int32_t vocab,
                                     const int32_t* draft_tokens, const int32_t* draft_lens,
                                     const float* target_logits, const float* uniforms, float temperature,
                                     int32_t top_k, float top_p, int32_t* accepted, int32_t* bonus,
                                     float* draft_prob, void* workspace, size_t workspace_bytes);

/* Bytes of device workspace dflash2_draft_losses needs. */
dflash2_status dflash2_draft_losses_workspace_size(int32_t batch, int32_t block_size, int32_t vocab,
                                                  size_t* bytes);

/* Training-side forward losses on given logits and labels (NeMo AutoModel
 * page, "Objective"): slots 1..block_size-1 are supervised; slot k's
 * cross-entropy on the transformed logits (output_multiplier, then
 * final_logit_softcapping, as in decoding) is weighted by
 * w_k = exp(-(k-1) / loss_decay_gamma); DFlash 2 adds, weighted by
 * selector_loss_weight, a cross-entropy over slot k's top-k candidates
 * scored as the lattice scores them, pi(true_{k-1}, c_kj) + topk_vals[kj]
 * (float32, multiply then add, m ascending), against the ground-truth
 * predecessor true_{k-1} (the anchor for k = 1, else labels[k-2]).
 *   labels   [device] int32 [batch, block_size-1]: true token of slots
 *            1..block_size-1; outside [0, vocab) = unsupervised (no term,
 *            not counted).
 *   logits   [device] float [batch, block_size-1, vocab]: the draft's
 *            pre-transform logits (as dflash2_draft_block's debug_logits);
 *            NaN logits give unspecified losses.
 *   topk_ids, topk_vals as dflash2_draft_block produces them.
 *   loss_decay_gamma > 0 (+inf: equal weights); selector_loss_weight finite;
 *            else DFLASH2_ERR_INVALID_ARG.
 *   block_ce    [device, nullable] float [batch, block_size-1]: CE per slot
 *               (NaN where unsupervised).
 *   selector_ce [device, nullable] float [batch, block_size-1]: selector CE
 *               where the label is among the candidates and its predecessor
 *               is known, NaN elsewhere.
 *   losses   [device] float [4]: total = block + weight * selector, block =
 *            sum w_k CE_k / sum w_k over supervised slots, selector = mean
 *            selector CE over slots with a signal (0 if none),
 *            candidate_recall = supervised slots whose label is among the
 *            candidates / supervised slots.
 * logsumexp runs in float32 (per-chunk online maxima and sums merged in a
 * fixed order); the sums over slots and sequences in double, in order. */
dflash2_status dflash2_draft_losses(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                    const int32_t* anchor_ids, const int32_t* labels, const float* logits,
                                    const int32_t* topk_ids, const float* topk_vals, float loss_decay_gamma,
                                    float selector_loss_weight, float* block_ce, float* selector_ce,
                                    float* losses, void* workspace, size_t workspace_bytes);

/* Optional per-kernel timing (instrumentation for benchmarks and profiling).
 * While a trace is attached on a thread, every kernel that calls from this
 * thread enqueue is bracketed by hipEventRecord(entry.start / entry.stop) on
 * the call's stream, and the entry receives the kernel kind and its
 * algorithmic traffic and work: bytes = every input read once plus every
 * output written once (split-K partial sums and other scratch excluded;
 * appended rows and context lengths counted at their host-side bounds),
 * flops = multiply-adds x 2.  The caller creates the events (hipEventCreate)
 * and reads them after synchronising.  At most `capacity` launches are
 * recorded; later launches run untraced. */
typedef enum {
  DFLASH2_K_GEMM = 0,         /* weight-streaming linear (draft linears, projections) */
  DFLASH2_K_LMHEAD_TOPK = 1,  /* lm_head with the fused per-group top-k      */
  DFLASH2_K_TOPK_MERGE = 2,
  DFLASH2_K_NORM = 3,         /* residual + conv + RMSNorm                   */
  DFLASH2_K_QKV_EPILOGUE = 4,
  DFLASH2_K_KV_APPEND = 5,
  DFLASH2_K_SWIGLU = 6,
  DFLASH2_K_ATTENTION = 7,
  DFLASH2_K_ATTN_COMBINE = 8,
  DFLASH2_K_SELECT = 9,
  DFLASH2_K_VERIFY_PARTIAL = 10,
  DFLASH2_K_VERIFY_FINAL = 11,
  DFLASH2_K_SAMPLE_ROWS = 12,  /* sampled verification: per-row truncation */
  DFLASH2_K_SAMPLE_PICK = 13,  /* sampled verification: accept walk + draw */
  DFLASH2_K_LOSS_ROWS = 14,    /* forward losses: per-chunk logsumexp       */
  DFLASH2_K_LOSS_SEQ = 15,     /* forward losses: per-slot terms and totals */
  DFLASH2_K_MERGE_SELECT = 16  /* dflash2_draft_select: candidate merge + selector */
} dflash2_kernel_kind;

typedef struct {
  hipEvent_t start, stop;     /* [host] created by the caller               */
  int32_t kind;               /* dflash2_kernel_kind, filled by the library */
  int32_t reserved;
  int64_t bytes;              /* algorithmic bytes of this launch           */
  int64_t flops;              /* algorithmic flops of this launch           */
} dflash2_trace_entry;

/* Attach [host] entries[capacity] to the calling thread (replaces any
 * attached trace).  Not for use while another call on this thread runs. */
dflash2_status dflash2_trace_attach(dflash2_trace_entry* entries, int32_t capacity);
/* Detach; returns the number of entries filled (<= capacity). */
int32_t dflash2_trace_detach(void);

/* Description of the last error on the calling thread ("" if none). */
const char* dflash2_last_error(void);

/* Measured ceilings (benchmark utilities, not part of the step).  They give
 * the rates this chip sustains, reported beside the nominal MI355X peaks
 * (dense bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s).
 *
 * dflash2_peak_mfma: `blocks` blocks of 4 waves (one per SIMD), each wave
 * running `iters` rounds of 16 independent v_mfma_f32_32x32x16_bf16 on
 * operands held in registers: 16 * 32768 flops per wave and round.  With
 * zero_operands != 0 every operand is 0.0, otherwise a per-lane pseudo-random
 * bf16 value in +-[0.5, 2).  out [device] float [blocks * 4] receives one sum
 * per wave.  Time the call with events on `stream`.
 *
 * dflash2_peak_read: `blocks` blocks of 256 threads read `bytes` (multiple
 * of 16; src 16-byte aligned) of src [device] once, 16 bytes per lane with
 * non-temporal loads; out [device] uint32 [blocks * 256] receives per-thread
 * checksums.
 * Errors: DFLASH2_ERR_INVALID_ARG for bad sizes or pointers. */
dflash2_status dflash2_peak_mfma(hipStream_t stream, int32_t blocks, int32_t iters, int32_t zero_operands,
                                 float* out);
dflash2_status dflash2_peak_read(hipStream_t stream, const void* src, size_t bytes, int32_t blocks,
                                 uint32_t* out);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH2_H */
