/*
 * jl.h -- C ABI of the MI355X (gfx950) forward pass of the Julia-1 decision model.
 *
 * The model: an mmBERT-small encoder (ModernBERT block: 22 pre-norm layers of
 * width 384, 6 heads of 64, RoPE, a +-64-token window on two of every three
 * layers, GEGLU feed-forward of 1,152), a type row added to every position,
 * two pre-norm transformer layers (feed-forward 1,536, ReLU, biases), a gather
 * at the option markers and a LayerNorm -> Linear(384,384) -> GELU ->
 * Linear(384,1) scorer, one logit per option, then a softmax across each
 * question's options.  Sources: "Julia-1: one score per mask token ..." (The
 * decision head; Three modes through one head), "Julia-1 MLX" (Performance),
 * "julia1 - Rust runtime for Julia-1" (Use; Why it is faster).
 *
 * Conventions for every entry point:
 *   - Return value: JL_OK (0) or a negative jl_status; jl_last_error() then
 *     holds a message (thread-local, valid until the next call on the thread).
 *   - Validation runs on the host before anything is enqueued.  On an error
 *     nothing is enqueued and no output is touched.  Inputs are never
 *     truncated: an over-long or malformed batch is rejected.
 *   - Calls return once their work is enqueued on `stream` (a hipStream_t, or
 *     NULL for the default stream); the caller synchronizes that stream before
 *     reading outputs.  A handle owns one workspace: calls on one handle must
 *     be ordered (one stream, or the caller orders them), never concurrent.
 *   - "_dev" pointers are device memory on the handle's device, caller-owned.
 *     All other pointers are host memory, caller-owned, read only during the
 *     call.
 *   - Device faults: a HIP error that leaves the device unusable (memory
 *     fault, kernel exception, abort or timeout, uncorrectable ECC error),
 *     seen by any call on a handle -- at a launch, at the wait for an earlier
 *     call's metadata slot, or at a synchronization -- returns JL_ERR_DEVICE
 *     with the HIP error string and marks the handle poisoned: from then on
 *     every call that enqueues or waits on it returns JL_ERR_DEVICE naming the
 *     first fault, and only jl_free, jl_model_info and jl_set_debug accept it.
 *     Faults surface asynchronously (at a later call or the caller's own
 *     synchronization) unless JL_DEBUG_SYNC is on.
 */
#ifndef JL_H
#define JL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct jl_model jl_model; /* opaque: weights on the device + workspace */

enum jl_precision {
  JL_FP32 = 0, /* every product in FP32 (FP32 matrix cores)                    */
  JL_BF16 = 1, /* GEMM and attention operands in bf16 (round to nearest even),  */
               /* FP32 accumulation; residual stream, LayerNorms, embeddings,   */
               /* RoPE tables, scorer and softmax stay FP32 ("Julia-1 MLX",     */
               /* Performance: the residual carries outliers near 4,000)        */
  JL_FP8 = 2   /* as JL_BF16, but the encoder's QKV (layers 1-21) and W_i       */
               /* products take OCP e4m3 operands on the matrix cores: weights  */
               /* scaled per output row at load (row max -> 448), normalized    */
               /* activations per token row inside the product, FP32            */
               /* accumulation, both scales applied to the FP32 result; the     */
               /* reduced-precision projection mode of "Julia-1 MLX",           */
               /* Performance (precision), on gfx950's fp8 matrix cores, in     */
               /* both schedules                                                */
};

enum jl_status {
  JL_OK = 0,
  JL_ERR_ARG = -1,      /* null pointer, negative count, bad precision/stage   */
  JL_ERR_OPTIONS = -2,  /* a question with <2 or >20 options, noul without 2,  */
                        /* markers unsorted, duplicated or outside every seq  */
  JL_ERR_LENGTH = -3,   /* a sequence of length 0 or > 8,192, offsets not      */
                        /* increasing from 0                                   */
  JL_ERR_QTYPE = -4,    /* a question type outside {0,1,2}                     */
  JL_ERR_FILE = -5,     /* weight file missing, truncated, bad magic/checksum  */
  JL_ERR_DEVICE = -6,   /* a HIP runtime error (message holds its string); a   */
                        /* device fault also poisons the handle (see below)    */
  JL_ERR_OOM = -7,      /* device or pinned-host allocation failed at load     */
  JL_ERR_CAPACITY = -8, /* more tokens or markers than the handle was sized for */
  JL_ERR_GUARD = -9     /* jl_check_guards: a workspace guard band overwritten  */
};

enum jl_qtype { JL_CHOICE = 0, JL_SCORE = 1, JL_NOUL = 2 };

#define JL_MAX_SEQ_LEN 8192 /* tokens per sequence (explainer: 8,192 in all) */
#define JL_MIN_OPTIONS 2    /* options per question: 2-20 (all pages)          */
#define JL_MAX_OPTIONS 20

/*
 * Load a weight file written by the seeded generator (format "JLW1": header
 * with tensor names, shapes, offsets and per-tensor checksums, then FP32
 * data) onto `device`, convert it for `precision` and size a workspace for
 * batches of up to `max_tokens` packed tokens and `max_markers` options.
 * The tensors are those of the model the explainer page lays out ("Julia-1:
 * one score per mask token ...", The decision head: the mmBERT-small encoder,
 * the type table, two transformer layers with a 1,536-wide feed-forward and
 * the LayerNorm -> Linear -> GELU -> Linear scorer); the 256,000 x 384
 * embedding table stays resident in FP32, as do the norms and the head
 * ("Julia-1 MLX", Performance).  Checks every tensor's presence, shape and
 * checksum.  path: NUL-terminated, read during the call.  max_tokens in
 * 1..2^26, max_markers in 2..max_tokens.  On success *out holds a new handle
 * that the caller releases with jl_free; on error *out is NULL and nothing
 * stays allocated.  Errors: JL_ERR_ARG, JL_ERR_FILE, JL_ERR_DEVICE, JL_ERR_OOM.
 */
int jl_load_weights(const char *path, int precision, int64_t max_tokens,
                    int64_t max_markers, int device, jl_model **out);

/* Release a handle and all its device memory (NULL is allowed). */
void jl_free(jl_model *m);

/*
 * Host-only check of a packed batch; jl_forward and jl_probs call it first.
 * The limits are the pages' problem statement: each question carries 2 to
 * 20 options ("Julia-1: one score per mask token ...", Three modes through
 * one head; more go through the Router), a noul question exactly the two
 * options [false, true] (same section), and a sequence holds at most 8,192
 * tokens ("Julia-1 MLX", Performance); an over-long input is refused, never
 * truncated ("Julia-1 MLX", Quick start).
 *   seq_offsets  [n_seqs+1] cumulative lengths: seq_offsets[0] = 0, strictly
 *                increasing, every length in [1, 8192], total <= max_tokens.
 *   mask_positions [n_markers] absolute packed indices of the <mask> markers,
 *                strictly increasing; each sequence owns the markers inside
 *                [start, end), 2 to 20 of them, exactly 2 for a noul question
 *                (options [false, true]); n_markers <= max_markers.
 *   qtype        [n_seqs] 0 choice, 1 score, 2 noul.
 * n_seqs = 0 (an empty batch) is valid.
 */
int jl_validate(const int32_t *seq_offsets, int32_t n_seqs,
                const int32_t *mask_positions, int32_t n_markers,
                const int32_t *qtype, int64_t max_tokens, int64_t max_markers);

/*
 * Option logits of a packed batch: logits_dev[k] is the score of marker k
 * (FP32, [n_markers]), the scorer's output at the hidden state of the k-th
 * <mask> marker after the encoder, the type row and the two head layers
 * ("Julia-1: one score per mask token ...", From a state to one decision;
 * The decision head).  ids_dev: int32 token ids [seq_offsets[n_seqs]] on the
 * device, caller-owned; an id outside [0, 256000) makes its whole sequence's
 * logits NaN.  Sequences never attend to each other; ragged lengths need no
 * padding ("julia1 - Rust runtime for Julia-1", Why it is faster: unpadded
 * batches).  The other arguments are as jl_validate checks them; errors are
 * jl_validate's, JL_ERR_ARG for NULL device pointers and JL_ERR_DEVICE.
 */
int jl_forward(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets,
               int32_t n_seqs, const int32_t *mask_positions, int32_t n_markers,
               const int32_t *qtype, float *logits_dev, void *stream);

/*
 * jl_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and result as jl_forward, bitwise, with the activation
 * workspace and the batch metadata in the library's static device array
 * (30.4 MiB, one per GPU, taken at the first jl_load_weights on that GPU and
 * held until the process ends) instead of the handle's workspace.  Allocates
 * nothing, on the device or the host, and records no timer events.
 * Limits: at most 2,048 tokens and 256 markers (and the handle's own
 * capacity); larger batches are rejected with JL_ERR_CAPACITY before
 * anything is enqueued.  Every call on one GPU shares the array, which keeps
 * the previous call's contents (nothing in it needs to start at zero): calls
 * that overlap on one GPU, from any handle or stream, race -- order them.
 * Arguments and other errors as jl_forward; no graph replay.
 */
int jl_forward_static(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets,
                      int32_t n_seqs, const int32_t *mask_positions, int32_t n_markers,
                      const int32_t *qtype, float *logits_dev, void *stream);

/*
 * Softmax across each question's options (temperature 1) and the answers of
 * the three modes ("Julia-1: one score per mask token ...", Three modes
 * through one head):
 *   probs_dev   [n_markers] FP32 option probabilities;
 *   answer_dev  [n_seqs] FP32: choice -> index of the argmax option,
 *               score -> expected index sum_i i * p_i (0-based),
 *               noul -> p(true) = p_1;
 *   argmax_dev  [n_seqs] int32, the first maximum on ties;
 *   maxprob_dev [n_seqs] FP32, the largest probability.
 * Any output pointer may be NULL to skip it.
 */
int jl_probs(jl_model *m, const float *logits_dev, const int32_t *seq_offsets,
             int32_t n_seqs, const int32_t *mask_positions, int32_t n_markers,
             const int32_t *qtype, float *probs_dev, float *answer_dev,
             int32_t *argmax_dev, float *maxprob_dev, void *stream);

/*
 * Diagnostic: run the forward pass up to `stage` and copy a hidden state out
 * (FP32, row-major, width 384):
 *   0..22  the residual stream after the embedding and `stage` encoder
 *          layers, [T, 384];
 *   23     the head input: final encoder LayerNorm plus the type row, [T, 384];
 *   24     after the first head layer, [T, 384];
 *   25     after the second head layer, marker rows only, [n_markers, 384].
 */
int jl_debug_hidden(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets,
                    int32_t n_seqs, const int32_t *mask_positions, int32_t n_markers,
                    const int32_t *qtype, int32_t stage, float *out_dev, void *stream);

/*
 * Tuning: bf16 and FP8 batches of at least `min_tokens` packed tokens run
 * each encoder layer as one attention launch plus one row-block layer launch
 * (64 token rows per work-group: out-projection, LayerNorm, GEGLU MLP and the
 * next layer's QKV with the rows resident in LDS, weights streamed from L2);
 * smaller batches, and the FP32 mode, run one launch per GEMM.  Default 8,192; 0
 * forces the row-block path, INT64_MAX the per-GEMM path.  Both compute the
 * same function; their roundings differ in summation order only.
 */
int jl_set_row_block_min_tokens(jl_model *m, int64_t min_tokens);

/*
 * Graph mode: with max_graphs > 0, jl_forward captures its launch sequence
 * for each batch shape into a HIP graph on first use and replays it after
 * (per-launch host cost ~10 us becomes one graph launch; this matters for
 * small batches, whose forward pass is ~180 launches).  A shape is the token,
 * marker and sequence counts, the attention work-item counts, the schedule
 * and the ids_dev / logits_dev pointers; up to max_graphs shapes are kept,
 * least recently used evicted.  Each call still uploads its own batch
 * metadata first (to one graph-owned device buffer, ordered on the stream),
 * so any batch of a cached shape is computed exactly as eagerly.  Calls on
 * the NULL stream, calls while the per-kernel timer is on, and calls with a
 * debugging flag set (jl_set_debug) run eagerly.  0 (the default) turns
 * graphs off and releases the cached graphs; at most 64.  The launch count is
 * the cost "julia1 - Rust runtime for Julia-1" (Why it is faster) names for
 * its CUDA path: about 200 launches per forward with no interpreter between.
 */
int jl_set_graph_cache(jl_model *m, int max_graphs);

/*
 * Router: choice questions with more than 20 options ("Julia-1: one score per
 * mask token ...", More than 20 options: the Router).  Per question, the
 * candidates are split, in order, into consecutive groups of at most 20; every
 * group is scored as one choice question; a group keeps its winner alone when
 * the winner's probability is above 0.95 and every other option's is below
 * 0.045, else its top two; rounds repeat until at most 20 candidates remain,
 * then one final call scores them.  Readings where the page is silent: a group
 * of a single candidate passes it on unscored; survivors keep their order;
 * ties go to the earlier candidate.  All groups of all questions in a round
 * share one packed jl_forward call (several when the handle's capacity is
 * exceeded).
 *
 * Each question's scored sequence is
 *     prefix, then (mask_id, option tokens) for each of its candidates, then suffix
 * (the prefix holds everything before the first option marker, the suffix
 * everything after the last option), with question type choice.
 *   n_questions        number of questions (0 is valid).
 *   prefix_ids / prefix_offsets [n_questions+1]: concatenated prefixes.
 *   suffix_ids / suffix_offsets [n_questions+1]: concatenated suffixes.
 *   option_ids / option_offsets [n_options_total+1]: concatenated options of
 *              all questions, each 1 or more tokens.
 *   question_options [n_questions+1]: question q owns options
 *              question_options[q] .. question_options[q+1]-1; 2 to 4,096 each.
 * Outputs (host memory, caller-owned): pick[q] the chosen option's index
 * within its question, pick_prob[q] its final probability, n_final[q] the
 * final candidate count (<= 20), final_idx/final_prob [n_questions x 20] the
 * final candidates (question-local indices, in order) and their final
 * probabilities, calls[q] the groups scored for the question (final call
 * included), rounds[q] the rounds before the final call.  Any of calls,
 * rounds, final_idx, final_prob, n_final may be NULL.
 * Errors: JL_ERR_ARG for malformed inputs, JL_ERR_LENGTH when one group's
 * sequence is longer than 8,192 tokens or the handle's capacity; plus those of
 * jl_forward.  Synchronous: returns when the pick is known.
 */
int jl_route(jl_model *m, int32_t n_questions, const int32_t *prefix_ids, const int64_t *prefix_offsets,
             const int32_t *suffix_ids, const int64_t *suffix_offsets, const int32_t *option_ids,
             const int64_t *option_offsets, const int32_t *question_options, int32_t mask_id,
             int32_t *pick, float *pick_prob, int32_t *n_final, int32_t *final_idx, float *final_prob,
             int32_t *calls, int32_t *rounds, void *stream);

/*
 * The same tournament with a caller-supplied scorer instead of the model, for
 * other engines and for testing the rule on the host: `score` receives one
 * packed batch (host arrays; question type choice for every sequence) and
 * writes the option probabilities [n_markers] (softmax across each sequence's
 * markers), returning 0 or an error code, which aborts the routing.  Batches
 * hold at most max_tokens tokens and max_markers markers.
 */
typedef int (*jl_score_fn)(void *user, const int32_t *ids, const int32_t *seq_offsets, int32_t n_seqs,
                           const int32_t *mask_positions, int32_t n_markers, float *probs);
int jl_route_with_scorer(jl_score_fn score, void *user, int64_t max_tokens, int64_t max_markers,
                         int32_t n_questions, const int32_t *prefix_ids, const int64_t *prefix_offsets,
                         const int32_t *suffix_ids, const int64_t *suffix_offsets, const int32_t *option_ids,
                         const int64_t *option_offsets, const int32_t *question_options, int32_t mask_id,
                         int32_t *pick, float *pick_prob, int32_t *n_final, int32_t *final_idx,
                         float *final_prob, int32_t *calls, int32_t *rounds);

/*
 * A second handle over the weights of `src`, with a workspace of its own
 * (max_tokens, max_markers), metadata ring, graph cache and timer.  Handles
 * that share weights may run jl_forward / jl_probs concurrently on different
 * streams, as the concurrent requests of "Julia-1 MLX" (Performance) each run
 * on a stream of their own; the weights stay allocated until the last handle sharing them is
 * freed with jl_free.  Errors: JL_ERR_ARG (NULL or sizes out of range),
 * JL_ERR_OOM / JL_ERR_DEVICE.
 */
int jl_share(const jl_model *src, int64_t max_tokens, int64_t max_markers, jl_model **out);

/*
 * Micro-batch plan of a request queue, as jl_serve uses it ("Julia-1 MLX",
 * Performance: concurrent requests; the serving scenarios of "julia1 - Rust
 * runtime", Benchmarks).  Host only.  Request r has id_offsets[r+1] -
 * id_offsets[r] tokens and mask_offsets[r+1] - mask_offsets[r] markers.
 * Requests are ordered longest first (stable: equal lengths keep their
 * order) and packed greedily: a micro-batch closes when the next request
 * would exceed max_batch_tokens, max_batch_markers or max_batch_seqs.
 * Out: order[i] = the i-th request in execution order, batch_of[r] = its
 * micro-batch (0-based, non-decreasing along `order`), *n_batches.
 * Errors: JL_ERR_ARG (bad offsets or limits), JL_ERR_LENGTH (a request larger
 * than one micro-batch).
 */
int jl_serve_plan(int32_t n_requests, const int64_t *id_offsets, const int64_t *mask_offsets,
                  int64_t max_batch_tokens, int64_t max_batch_markers, int64_t max_batch_seqs,
                  int32_t *order, int32_t *batch_of, int32_t *n_batches);

/*
 * Serve n_requests independent requests held in host memory: request r is
 * ids[id_offsets[r] .. id_offsets[r+1]) with markers mask_positions[
 * mask_offsets[r] .. mask_offsets[r+1]) (positions inside the request) and
 * question type qtype[r].  The requests are planned as by jl_serve_plan
 * (token budget max_batch_tokens, capped by the handles' capacities) and the
 * micro-batches run round-robin on the n_models handles (1..16, normally
 * sharing weights through jl_share), each on a stream of its own with its own
 * device buffers and pinned staging (made on the handle's first jl_serve and
 * kept until jl_free); each micro-batch is jl_forward + jl_probs.  Outputs
 * (host, caller-owned): logits and probs [mask_offsets[n_requests]] in request
 * order; answer, argmax, maxprob [n_requests] as jl_probs defines them;
 * *n_batches (may be NULL).  Every request is validated as jl_validate
 * would a batch of that one request before any work starts, so a rejected
 * call leaves the outputs untouched.  Blocks until every result is in the
 * output arrays.  Calls that share a handle must not overlap.
 * With the graph cache on (jl_set_graph_cache on every handle), each
 * micro-batch is padded to a shape bucket and replays one captured graph per
 * bucket: B sequences become B_b = ceil((B + 2) / 8) * 8 by F = B_b - B filler
 * questions (choice type, token id 0, 2-20 markers each), M markers become
 * M_b = ceil((M + 2F) / 32) * 32 and T tokens T_b = ceil((T + 21F) / 2048) *
 * 2048; the fillers' results are discarded, and the micro-batch budget is
 * lowered by that headroom.  A request's results then depend on the bucket
 * (the schedule follows T_b), within the bf16 bounds of the two schedules.
 */
int jl_serve(jl_model *const *models, int32_t n_models, int32_t n_requests, const int32_t *ids,
             const int64_t *id_offsets, const int32_t *mask_positions, const int64_t *mask_offsets,
             const int32_t *qtype, int64_t max_batch_tokens, float *logits, float *probs, float *answer,
             int32_t *argmax, float *maxprob, int32_t *n_batches);

/* Kernel classes reported by the per-kernel timer: the per-operation timings
 * that "julia1 - Rust runtime for Julia-1" prints with JULIA_PROFILE=1
 * (Layout, after the list of what is not ported), taken on the device. */
enum jl_kernel_class {
  JL_K_EMBED = 0,      /* embedding gather + LayerNorm (row-block path: also   */
                       /* the first layer's QKV)                                */
  JL_K_QKV = 1,        /* encoder QKV GEMM (RoPE on store)                      */
  JL_K_ATTN_GLOBAL = 2,/* encoder attention, global layers                      */
  JL_K_ATTN_LOCAL = 3, /* encoder attention, +-64 window layers                 */
  JL_K_OUTPROJ = 4,    /* encoder out-projection GEMM + residual                */
  JL_K_MLP_IN = 5,     /* encoder Wi GEMM + GEGLU                               */
  JL_K_MLP_OUT = 6,    /* encoder Wo GEMM + residual                            */
  JL_K_HEAD_GEMM = 7,  /* decision-head GEMMs                                   */
  JL_K_HEAD_ATTN = 8,  /* decision-head attention                               */
  JL_K_MISC = 9,       /* final LayerNorm + type row, gathers, scorer, softmax  */
  JL_K_LN = 10,        /* LayerNorm rows -> GEMM operand                        */
  JL_K_LAYER = 11,     /* row-block layer kernel: out-proj, LayerNorm, GEGLU    */
                       /* MLP and the next layer's QKV (large bf16 batches)     */
  JL_K_HEAD_LAYER = 12,/* row-block head-layer kernel: the first head layer     */
                       /* after its attention + the second's keys and values    */
  JL_K_NCLASS = 13
};

/* Per-kernel timer: while on, every launch of the classes in `class_mask`
 * (bit i = class i) is bracketed by HIP events recorded on the launch stream.
 * enable = 1 turns it on and clears previous records, 2 turns it on and keeps
 * them (to time a sample of calls), 0 turns it off and keeps them. */
int jl_profile(jl_model *m, int enable, uint32_t class_mask);

/* Total device time (ms) and launch count of one class since jl_profile(1).
 * Synchronizes on the recorded events. */
int jl_profile_read(jl_model *m, int kernel_class, double *total_ms, int64_t *launches);

/* info[0..n), n <= 10: precision, max_tokens, max_markers, device, device
 * bytes of weights, device bytes of workspace, graphs captured and graph
 * replays so far (jl_set_graph_cache), 1 if the handle is poisoned, the
 * debugging flags (jl_set_debug). */
int jl_model_info(const jl_model *m, int64_t *info, int n);

/*
 * Debugging switches of a handle (replacing its previous flags; 0 = off).
 *   JL_DEBUG_SYNC            after every kernel launch, wait for the stream
 *                            and check hipGetLastError, so that an error or a
 *                            device fault is reported by the call and kernel
 *                            class that caused it; graph replay is off.  Also
 *                            set at load when the environment variable
 *                            JL_DEBUG_SYNC is set and not "0".
 *   JL_DEBUG_REVERSE_BLOCKS  every kernel whose work-groups own tiles, row
 *                            blocks, attention items or heads (the GEMMs, the
 *                            row-block kernels, attention, the scorer) takes
 *                            them in reversed order.  Each work-group computes
 *                            its outputs alone and the scorer adds its
 *                            partial sums in a fixed order, so the results
 *                            are the same bit for bit; a difference exposes a
 *                            race between work-groups.  Graph replay is off.
 *   JL_DEBUG_SIMULATE_FAULT  the next call that enqueues work reports a
 *                            memory fault after its launches, as a real one
 *                            would be reported (the work itself runs
 *                            normally), poisoning the handle; cleared when
 *                            used.  For testing callers' fault handling.
 * Errors: JL_ERR_ARG (NULL handle, unknown flag).
 */
enum jl_debug_flag { JL_DEBUG_SYNC = 1, JL_DEBUG_REVERSE_BLOCKS = 2, JL_DEBUG_SIMULATE_FAULT = 4 };
int jl_set_debug(jl_model *m, uint32_t flags);

/*
 * Workspace guard bands: every buffer of the handle's workspace (activations,
 * marker rows, scorer partials and counters, metadata blocks) is followed by
 * 256 bytes of 0xA5, written at load and never by a kernel.  Synchronizes the
 * device, reads the bands back and returns JL_OK, or JL_ERR_GUARD naming the
 * first buffer whose band was overwritten (a write past its end).  Errors:
 * JL_ERR_ARG, JL_ERR_DEVICE.
 */
int jl_check_guards(jl_model *m);

/* Message of the last failed call on this thread ("" if none). */
const char *jl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JL_H */
