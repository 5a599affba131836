/*
 * mtp.h -- C ABI of the MI355X (gfx950) MTP speculative-decoding step.
 *
 * One round of speculative decoding with a Multi-Token-Prediction draft head:
 *   1. the draft head runs D times serially     (mtp_draft_step, mtp_draft_loop)
 *   2. the D+1 target positions are verified    (spec_verify)
 *   3. the KV cache is cropped and recurrent state restored on rejection
 *                                               (kv_crop, mtp_state_snapshot, mtp_state_restore)
 *
 * Sources (web pages, cited by title and section):
 *   [HB14] "14. MTP: speculative decoding with the built-in draft head" (Transformer by Hand)
 *   [DLM]  "The decoding loop and MTP" (agent-loop-visualizer docs)
 *   [YL]   "MTP (Multi-Token Prediction) 原理详解"
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never allocates,
 *     frees or synchronises inside a compute call.  Work is enqueued on `stream` and runs
 *     asynchronously.  Struct arguments (mtp_config, mtp_weights, mtp_kv, mtp_sampling) are
 *     HOST memory read during the call only.
 *   - Activations, hiddens and logits are float32; token ids, lengths and counts are int32.
 *     Weights and the KV cache use cfg->wdtype (MTP_F32 or MTP_BF16).
 *   - Matrices are row-major [out][in] (the nn.Linear layout).  All device pointers must be
 *     16-byte aligned.
 *   - Return value: MTP_OK (0) or a negative mtp_status.  Shape, pointer, dtype and workspace
 *     errors are detected on the host before anything is launched; mtp_last_error() then
 *     returns a message (thread-local).  Conditions only the device can see (a KV cache that
 *     would overflow, a token id >= vocab) are recorded in the workspace's status word and
 *     reported by mtp_check(); the affected rows are skipped, never written out of bounds.
 *   - Workspaces ("ws") are caller-allocated device memory of at least the size the matching
 *     *_workspace_size() call reports, zero-filled once before first use.  The library leaves
 *     its internal counters at zero after every call, so a workspace can be reused by any
 *     number of later calls on the same stream.  Two calls that run concurrently must not
 *     share a workspace.
 */
#ifndef MTP_HIP_H_
#define MTP_HIP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTP_OK = 0,
  MTP_ERR_ARG = -1,        /* NULL pointer, bad size, unsupported option */
  MTP_ERR_SHAPE = -2,      /* shape constraint violated (alignment of dims, head layout) */
  MTP_ERR_DTYPE = -3,      /* unknown dtype code */
  MTP_ERR_CAPACITY = -4,   /* device: appending rows would overflow the KV cache */
  MTP_ERR_WORKSPACE = -5,  /* workspace smaller than required */
  MTP_ERR_HIP = -6,        /* a HIP runtime call failed */
  MTP_ERR_TOKEN = -7       /* device: a token id outside [0, vocab) was given (the row is skipped) */
} mtp_status;

typedef enum { MTP_F32 = 0, MTP_BF16 = 1 } mtp_dtype;

/* Shape of the draft head.  [HB14 "The draft head"]: a 2H->H projection, RMSNorms of the
 * embedding and of the main model's hidden, one (or n_layers) full-attention decoder layers
 * with RoPE, a final RMSNorm and the shared lm_head.  Constraints: hidden, ffn and
 * n_heads*head_dim multiples of 8; head_dim 64 or 128; n_heads a multiple of n_kv_heads. */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, n_layers;
  float rope_theta, rms_eps;
  int32_t wdtype; /* mtp_dtype of weights and KV cache */
} mtp_config;

/* One pre-norm decoder block.  wq [nq*hd][H], wk/wv [nkv*hd][H], wo [H][nq*hd],
 * wgate/wup [F][H], wdown [H][F]; in_norm/post_norm [H] gains. */
typedef struct {
  const void *in_norm, *wq, *wk, *wv, *wo, *post_norm, *wgate, *wup, *wdown;
} mtp_layer_weights;

/* embed/lm_head [V][H] (shared with the main model, [HB14], [YL 一]); enorm/hnorm/final_norm
 * [H]; eh_proj [H][2H] whose input is [embedding half ; hidden half] ([HB14], [YL 二.2]).
 * `layers` is a HOST array of n_layers entries; every draft step runs all of them. */
typedef struct {
  const void *embed, *enorm, *hnorm, *eh_proj, *final_norm, *lm_head;
  const mtp_layer_weights* layers;
} mtp_weights;

/* The head's own KV cache ([HB14]: an attention state truncated along T on rollback).
 * k: [n_layers][batch][n_kv_heads][max_len][head_dim] in cfg->wdtype, keys stored after RoPE;
 * v: [n_layers][batch][n_kv_heads][head_dim][max_len] in cfg->wdtype: values are stored
 * transposed (each channel's positions contiguous), the layout the attention's value
 * contraction over positions reads.  max_len: a positive multiple of 8 (MTP_ERR_ARG
 * otherwise); a multiple of 64 puts every 64-position segment of a bf16 value row on one
 * 128-byte line, which the batched attention streams fastest (the binding rounds to 64).
 * len: device int32[batch], the number of valid positions per sequence;
 * position p lives in slot p.  Slots at or past len may hold anything. */
typedef struct {
  void *k, *v;
  int32_t* len;
  int32_t batch, max_len;
} mtp_kv;

/* Verification settings.  temperature <= 0 selects greedy verification.  Otherwise
 * temperature, top-k and top-p are applied in that order ([DLM "Why a hand-written decoding
 * loop"]); top_k <= 0 (or >= vocab) disables top-k, top_p >= 1 disables top-p.  top_k in
 * [1, 128] runs on a per-row candidate buffer; top-k off or larger runs over the whole
 * vocabulary (a radix search of each row's kept set: slower, for settings without a small k).
 * q_mode 0: the drafts are greedy, so the draft distribution is one-hot at the draft;
 * q_mode 1: the draft distribution is the same warp of draft_logits and the drafts were
 * sampled from it. */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
  int32_t q_mode;
} mtp_sampling;

/* Message of the last host-side error on this thread ("" if none). */
const char* mtp_last_error(void);

/* Bytes of workspace a drafter call needs for `batch` sequences of up to `rows_per_seq` rows
 * each with a cache of `max_len` positions.  mtp_draft_loop needs rows_per_seq >= 1 and D. */
int mtp_draft_workspace_size(const mtp_config* cfg, int32_t batch, int32_t rows_per_seq, int32_t D,
                             int32_t max_len, size_t* bytes);

/* One draft-head forward over a padded batch of rows.  [HB14 "The draft head"] (the head's
 * forward, its prompt-length prefill, the catch-up after a verification: two rows at pos-2 on
 * a hit, one row at pos-1 on a miss) and [YL 二.2, 三 stage 1].
 *   tokens     [B][rows_per_seq]     next-token ids; a negative id marks a padding row.  The
 *                                    valid rows of a sequence must be a prefix.
 *   hidden_in  [B][rows_per_seq][H]  the main model's (post-final-norm) hidden of each row.
 *   Row i of sequence b sits at position kv->len[b] + i: it appends its K/V there and attends
 *   to positions 0 .. kv->len[b] + i.  On return kv->len[b] has grown by the valid rows.
 *   hidden_out [B][rows_per_seq][H]  the head's post-final-norm output of every valid row.
 *   draft_out  [B]                   argmax of lm_head over each sequence's last valid row,
 *                                    lowest id on ties ([DLM]); -1 for a sequence without rows.
 *   logits_out [B][V] or NULL        that row's logits.
 * B = kv->batch.  hidden_in may not alias hidden_out. */
int mtp_draft_step(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* kv, int32_t rows_per_seq,
                   const int32_t* tokens, const float* hidden_in, float* hidden_out, int32_t* draft_out,
                   float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The serial D-step draft loop ([YL 三 stages 1-2]): one mtp_draft_step over the catch-up
 * rows (tokens/hidden_in as above), then D-1 single-row steps, step k fed the draft and the
 * output hidden of step k-1, one position after it.
 *   drafts       [B][D]        draft tokens (-1 for sequences without rows)
 *   hiddens      [B][D][H] or NULL   each step's output hidden (of the last row)
 *   draft_logits [B][D][V] or NULL   each step's logits
 * kv->len[b] grows by (valid catch-up rows) + D - 1. */
int mtp_draft_loop(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* kv, int32_t D,
                   int32_t rows_per_seq, const int32_t* tokens, const float* hidden_in, int32_t* drafts,
                   float* hiddens, float* draft_logits, void* ws, size_t ws_bytes, hipStream_t stream);

/* The D-step draft loop over M MTP modules ([YL 二.3]: the predictor holds several MTP layers; a
 * single module is reused for every step, chosen by the step index modulo the layer count, and
 * multi-module MTP gives each draft position its own layer; [YL 五]: that form needs a re-prefill
 * to repair the stale KV left by rejected tokens).  modules[m] and kvs[m] (HOST arrays of M) are
 * module m's weights and its own cache (all caches with the same batch B and max_len; the
 * embedding and lm_head may be the same tensors for every module).
 *   Catch-up: every module appends the catch-up rows (tokens / hidden_in as in mtp_draft_loop);
 *   module 0's last row gives draft 1.  Modules other than 0 skip the final norm and lm_head.
 *   Step k >= 2: module (k-1) mod M first appends the rows of this round's chain it has not seen
 *   (steps s+1 .. k-1 after the last step s it drafted, or after the catch-up), each row fed
 *   (draft, output hidden) of the step before it and placed one position after it, then its own
 *   row for step k; that row gives draft k.
 * With M = 1 this is mtp_draft_loop.  Outputs as in mtp_draft_loop.  Each kvs[m].len grows by the
 * rows module m appended; after verification the caller crops every module's cache to the same
 * length (kv_crop) and the next catch-up re-prefills the settled rows.
 * Workspace: mtp_draft_workspace_size(cfg, B, max(rows_per_seq, M > 1 ? D - 1 : 1), D, max_len). */
int mtp_draft_loop_multi(const mtp_config* cfg, const mtp_weights* modules, int32_t M, const mtp_kv* kvs, int32_t D,
                         int32_t rows_per_seq, const int32_t* tokens, const float* hidden_in, int32_t* drafts,
                         float* hiddens, float* draft_logits, void* ws, size_t ws_bytes, hipStream_t stream);

/* The D-step draft loop of a head that keeps no KV cache of its own and reads the main model's
 * keys and values ([DLM "MTP speculative decoding"] item 1: the drafter has no cache and reads the
 * model's keys and values directly; its input is the last token's embedding beside the model's
 * last hidden).  target_kv is the main model's cache: `target_layers` layers in the mtp_kv layout,
 * with cfg->n_kv_heads and cfg->head_dim, B = target_kv->batch.  Head layer l attends over layer
 * kv_layer[l] (HOST array of cfg->n_layers entries in [0, target_layers)) at positions
 * 0 .. target_kv->len[b] - 1.  The head projects q only (w->layers[l].wk / .wv are not read and
 * may be NULL), appends nothing, and leaves target_kv->len unchanged.
 *   tokens    [B]     the settled next token of each sequence; negative: no drafts.
 *   hidden_in [B][H]  the main model's post-final-norm hidden at its last cached position.
 * Step 1 is the row (tokens[b], hidden_in[b]) at position len[b] - 1; step k >= 2 the row
 * (draft k-1, output hidden k-1) at position len[b] + k - 2.  A sequence whose cache is empty
 * (len[b] == 0) gets no drafts.  No catch-up rows are needed: there is no head cache to fill.
 *   drafts [B][D], hiddens [B][D][H] or NULL, draft_logits [B][D][V] or NULL: as in
 *   mtp_draft_loop (-1 / untouched for sequences without drafts).
 * Workspace: mtp_draft_workspace_size(cfg, B, 1, D, target_kv->max_len).  A token id >= vocab is
 * reported through mtp_check (MTP_ERR_TOKEN); there is no capacity error. */
int mtp_draft_loop_shared_kv(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* target_kv,
                             int32_t target_layers, const int32_t* kv_layer, int32_t D, const int32_t* tokens,
                             const float* hidden_in, int32_t* drafts, float* hiddens, float* draft_logits, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace spec_verify needs. */
int spec_verify_workspace_size(int32_t B, int32_t D, int32_t V, const mtp_sampling* sp, size_t* bytes);

/* Verify D drafts per sequence against D+1 target rows ([HB14] loop steps 2-3, [DLM] items 2-3,
 * [YL 三 stages 3-4]).  Target row j judges draft j+1.
 *   target_logits [B][D+1][V]; drafts [B][D]; draft_logits [B][D][V] (q_mode 1 only, else NULL)
 *   u_accept [B][D], u_sample [B]: uniforms in [0,1) (sampling only, else NULL)
 *   ctx_len [B]: target positions before the round (those before the settled token's)
 * Greedy (sp NULL or temperature <= 0): a = length of the prefix where argmax(target[j]) ==
 * draft[j] (lowest id on ties); emitted drafts[0..a-1] then argmax(target[a]).
 * Sampling: draft j is kept when P_j(d) > 0 and u_accept[j] <= P_j(d)/Q_j(d); at the first
 * rejection one token is drawn from normalize(max(0, P_j - Q_j)) (P_j if that is empty); if all
 * hold, one token is drawn from P_D.  A draw takes the smallest id whose cumulative weight, in
 * ascending id order, exceeds u_sample * total.
 * Outputs: n_accept [B] = a; out_tokens [B][D+1] = the a+1 emitted tokens then -1;
 * crop_len [B] = ctx_len + 1 + a (the target's new length). */
int spec_verify(int32_t B, int32_t D, int32_t V, const float* target_logits, const int32_t* drafts,
                const float* draft_logits, const mtp_sampling* sp, const float* u_accept, const float* u_sample,
                const int32_t* ctx_len, int32_t* n_accept, int32_t* out_tokens, int32_t* crop_len, void* ws,
                size_t ws_bytes, hipStream_t stream);

/* spec_verify for callers that cannot allocate device memory or bring a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments (without
 * ws / ws_bytes), checks and results as spec_verify.  Its scratch (the greedy chunk partials or
 * the sampling top-k buffers) is a device array inside the library of MTP_VERIFY_SCRATCH_BYTES,
 * one per GPU the library runs on, held until the process ends; the call allocates and frees
 * nothing.  A call that would need more scratch than that (greedy: 8 bytes per target row and
 * logits chunk; sampling: 8 * top_k bytes per row, plus per-chunk candidates when there are fewer
 * than 128 rows) returns MTP_ERR_WORKSPACE and launches nothing.  Every call on a GPU uses the
 * same array, which keeps the last call's contents (nothing in it needs to start at zero): calls
 * that overlap in time on one GPU, from other streams or threads, race on it and must be
 * serialised by the caller. */
#define MTP_VERIFY_SCRATCH_BYTES (4u << 20)
int spec_verify_noalloc(int32_t B, int32_t D, int32_t V, const float* target_logits, const int32_t* drafts,
                        const float* draft_logits, const mtp_sampling* sp, const float* u_accept,
                        const float* u_sample, const int32_t* ctx_len, int32_t* n_accept, int32_t* out_tokens,
                        int32_t* crop_len, hipStream_t stream);

/* Truncate each sequence's cache: len[b] = min(len[b], max(new_len[b], 0)) ([HB14] rollback
 * keeps the first n positions; [DLM] item 2 crop()). new_len: device int32[batch]. */
int kv_crop(const mtp_kv* kv, const int32_t* new_len, hipStream_t stream);

/* Copy B recurrent states of bytes_per_seq bytes each (state [B][bytes_per_seq]) into snap,
 * before verification ([HB14], the paragraph after the loop: the memory tables and conv
 * windows are copied because they cannot be truncated).  bytes_per_seq multiple of 16. */
int mtp_state_snapshot(const void* state, void* snap, size_t bytes_per_seq, int32_t B, hipStream_t stream);

/* Copy snap back into state for every sequence b with n_accept[b] < D (a rejected draft): [HB14],
 * the paragraph after the loop -- on a miss the recurrent layers' memory tables and conv windows
 * are put back from the copy taken before verification, while attention caches are only cut. */
int mtp_state_restore(void* state, const void* snap, size_t bytes_per_seq, int32_t B, const int32_t* n_accept,
                      int32_t D, hipStream_t stream);

/* Synchronise `stream`, then read and clear the device status word of a drafter or verifier
 * workspace: MTP_OK, MTP_ERR_CAPACITY or MTP_ERR_TOKEN. */
int mtp_check(void* ws, hipStream_t stream);

/* Per-kernel timing with HIP events recorded around every launch of one kernel (a measurement
 * aid, not part of the method).  kernel: MTP_KERNEL_LM_HEAD (the lm_head's main kernel: the
 * GEMV or the MFMA GEMM with its per-workgroup argmax, without its activation preparation) or
 * MTP_KERNEL_VERIFY (the whole spec_verify call).  mtp_timer_start arms recording for up to
 * max_launches launches; mtp_timer_read synchronises on the last event and returns the summed
 * milliseconds and the launch count; mtp_timer_kernel_name names the kernel last timed (a
 * static string, "" before any). */
enum { MTP_KERNEL_LM_HEAD = 1, MTP_KERNEL_VERIFY = 2 };
int mtp_timer_start(int32_t kernel, int32_t max_launches);
int mtp_timer_read(int32_t kernel, float* total_ms, int32_t* launches);
const char* mtp_timer_kernel_name(int32_t kernel);

/* ---- The target's verify forward (a dense stand-in main model) ----
 * [HB14 "The draft head"]: the main model scores the settled token and the D drafts in one pass,
 * returns logits for each of those positions and hands the head its hidden states; the head
 * shares the main model's token embedding and output layer.  The pages do not describe the main
 * model's layers; this stand-in stacks the head's decoder block: x = E[tok]; cfg->n_layers
 * blocks over the target's own KV cache (RoPE, append, GQA attention, o_proj, SwiGLU MLP);
 * g = rms(x) * final_norm; logits = lm_head g.  cfg describes the target (n_layers = its layers).
 * embed / lm_head [V][H], final_norm [H], `layers` a HOST array of cfg->n_layers entries. */
typedef struct {
  const void *embed, *final_norm, *lm_head;
  const mtp_layer_weights* layers;
} mtp_target_weights;

/* Workspace bytes for mtp_target_forward on `batch` sequences of `rows_per_seq` rows with a
 * cache of `max_len` positions. */
int mtp_target_workspace_size(const mtp_config* cfg, int32_t batch, int32_t rows_per_seq, int32_t max_len,
                              size_t* bytes);

/* One target pass over tokens [B][rows_per_seq] (B = kv->batch): the valid rows of sequence b are
 * the prefix of non-negative tokens (inside the vocabulary and the cache, as in mtp_draft_step;
 * violations are reported through mtp_check); row i sits at position kv->len[b] + i, appends
 * its K/V there and attends to positions 0 .. kv->len[b] + i; kv->len[b] grows by the valid rows.
 *   hidden_out [B][rows_per_seq][H] or NULL: g of every valid row (what the head consumes).
 *   logits_out [B][rows_per_seq][V]: logits of every valid row; rows past the valid prefix are
 *                                   not written.
 * For verification, tokens[b] = [x_n, d_1 .. d_D] (rows_per_seq = D + 1) gives spec_verify's
 * target_logits directly; afterwards kv_crop(target kv, crop_len) drops the rejected positions. */
int mtp_target_forward(const mtp_config* cfg, const mtp_target_weights* w, const mtp_kv* kv, int32_t rows_per_seq,
                       const int32_t* tokens, float* hidden_out, float* logits_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MTP_HIP_H_ */
