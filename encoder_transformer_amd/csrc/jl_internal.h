// Internal declarations shared by the kernel and host translation units of
// libjl.  Nothing here is part of the public C ABI (include/jl.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <exception>
#include <new>

namespace jl {

// Model shape (mmBERT-small encoder + Julia-1 decision head).
constexpr int kVocab = 256000;
constexpr int kWidth = 384;
constexpr int kHeads = 6;
constexpr int kHeadDim = 64;
constexpr int kLayers = 22;
constexpr int kGeglu = 1152;        // GEGLU output width (projection is 2 x 1152)
constexpr int kHeadFfn = 1536;
constexpr int kHalfWindow = 64;     // local layers: |i - j| <= 64
constexpr int kMaxSeq = 8192;
constexpr double kThetaLocal = 10000.0;
constexpr double kThetaGlobal = 160000.0;
constexpr float kLnEps = 1e-5f;
constexpr int kLayerRows = 64;      // rows per work-group of the row-block layer kernel
// Factor on q (the q rows of every in-projection and the q bias, applied at
// load): 1 / sqrt(head dim) for the softmax and log2(e) for exp2 scores.
constexpr float kQScale = (float)(1.4426950408889634 / 8.0);

// A layer is global when its index is a multiple of 3 (layers 0, 3, ..., 21).
inline bool layer_is_global(int l) { return l % 3 == 0; }

enum EMode { E_STORE = 0, E_RESID = 1, E_GEGLU = 2, E_RELU = 3 };

// C[M, N] = A[M, K] . W[N, K]^T with a fused epilogue.
struct GemmArgs {
  const void *A;        // element matrix [M, lda]
  int lda;
  const void *W;        // element matrix [N, ldw] (GEGLU: rows interleaved by 16)
  int ldw;
  const float *bias;    // [N] or nullptr
  void *C;              // output (element type, or FP32 for E_RESID)
  int ldc;
  int M, N, K;
  const float *rope_cos;// E_STORE: [8192, 32] table or nullptr (no RoPE)
  const float *rope_sin;
  const int *pos;       // [M] position of each row inside its sequence (RoPE)
  int rope_cols;        // columns [0, rope_cols) are rotated (q and k: 768)
  // LayerNorm fused into the A operand (launch_ln_gemm): A = LN(ln_x) rows
  const float *ln_x;    // FP32 [M, 384]
  const float *ln_gain; // nullptr: A = ln_x converted, unnormalized (identity pre-norm)
  const float *ln_shift;// or nullptr
  // e4m3 products (launch_ln_gemm only): W holds e4m3 codes [N, ldw] and
  // w_scale[N] each row's scale; nullptr: W is bf16/FP32
  const float *w_scale;
  int rev;              // nonzero: work-groups take their tiles in reversed order
};

// One attention work item: up to 64 or 128 queries (the launch's tile size) of
// one sequence, one head per blockIdx.y.
struct AttnWork {
  int q_row0;   // first query row in the q buffer
  int n_q;      // queries in this item (1..tile size)
  int kv_row0;  // first key row of the sequence in the k/v buffers
  int kv_len;   // sequence length
  int q_pos0;   // position of the first query inside its sequence
  int pad0, pad1, pad2;
};

struct AttnArgs {
  const void *q; int q_stride;      // element strides between rows; head h at column 64h
  const void *k; const void *v; int kv_stride;
  void *o; int o_stride;
  const AttnWork *work;
  int half_window;                  // < 0: attend to the whole sequence
  int rev;                          // nonzero: work items and heads in reversed order
};

// Row-block layer kernel (bf16 only): out-projection + residual, LayerNorm,
// GEGLU MLP + residual, then the next layer's LayerNorm + QKV (+RoPE), or the
// final LayerNorm + type row after the last layer.  Weight matrices here are
// in matrix-core fragment order (see pack_fragments in jl_api.cpp).
struct LayerArgs {
  float *x;                     // [T, 384] residual stream (updated in place)
  const __bf16 *o;              // [T, 384] attention output of this layer
  const __bf16 *Wo;             // fragment-packed [384 x 384]
  const float *mlp_norm;        // [384]
  const __bf16 *Wi;             // fragment-packed [2304 x 384], GEGLU rows interleaved by 16
  const __bf16 *Wout;           // fragment-packed [384 x 1152]
  const float *attn_norm_next;  // next layer's attention pre-norm gain
  const __bf16 *Wqkv_next;      // fragment-packed [1152 x 384]; nullptr after the last layer
                                // (with final_norm == nullptr too: store the residual only)
  const float *rope_cos_next, *rope_sin_next;
  // After the last layer, with final_norm set: the first head layer's
  // attention input instead of a next encoder layer (Wqkv_next = its packed
  // in-projection, attn_norm_next / attn_shift_next its pre-norm, no RoPE).
  const float *attn_shift_next; // pre-norm shift, or nullptr
  const float *qkv_bias_next;   // [1152] in-projection bias; non-null selects the head mode
  const int *pos;               // [T] position inside the sequence
  __bf16 *qkv_out;              // [T, 1152]
  const float *final_norm;      // after the last layer: final LayerNorm gain,
  const float *type_rows;       //   type table [3, 384],
  const int *qtype;             //   question type per sequence,
  const int *tok_seq;           //   sequence of each token
  // e4m3 products (JL_FP8), or nullptr for bf16: W_i and the next encoder
  // layer's QKV as e4m3 codes in the 128-k fragment order of the fp8
  // matrix-core product, with one scale per (packed) weight row; the
  // LayerNorm rows that feed them are scaled and coded per row in the kernel
  const uint8_t *Wi8;           // [2304 x 384] codes, GEGLU rows interleaved by 16
  const float *si;              // [2304] row scales, same order
  const uint8_t *Wqkv8_next;    // [1152 x 384] codes of the next encoder layer
  const float *sqkv_next;       // [1152]
  int T;
  int rev;                      // nonzero: row blocks in reversed order
};

// Row-block head-layer kernel (bf16 only): everything of one head layer
// (torch pre-norm encoder layer) after its attention -- biased out-projection
// + residual, LayerNorm with shift, ReLU feed-forward with biases + residual
// -- then the next head layer's LayerNorm and biased key/value projection.
struct HeadArgs {
  float *x;                     // [T, 384] residual stream (updated in place)
  const __bf16 *o;              // [T, 384] attention output of this layer
  const __bf16 *Wo;             // fragment-packed [384 x 384]
  const float *bo;              // [384]
  const float *n2_w, *n2_b;     // feed-forward pre-norm gain and shift
  const __bf16 *W1;             // fragment-packed [1536 x 384]
  const float *b1;              // [1536]
  const __bf16 *W2;             // fragment-packed [384 x 1536]
  const float *b2;              // [384]
  const float *nk_w, *nk_b;     // next layer's attention pre-norm gain and shift
  const __bf16 *Wkv;            // fragment-packed [768 x 384]: the next layer's key and
                                // value rows; nullptr: store the residual only
  const float *bkv;             // [768]
  __bf16 *kv_out;               // [T, 768]: keys, then values
  int T;
  int rev;                      // nonzero: row blocks in reversed order
};

// Row-block embedding kernel (bf16 only): token embedding gather + its
// LayerNorm into x, each token's sequence and position, and the first
// layer's QKV with RoPE (that layer has no attention pre-norm).
struct EmbedArgs {
  const int32_t *ids;           // [T] token ids (out-of-range ids give NaN rows)
  const float *emb;             // [vocab, 384]
  const float *gain;            // embedding LayerNorm gain
  const int *seq_offsets;       // [n_seqs + 1]
  int n_seqs;
  float *x;                     // [T, 384] out: residual stream
  int *pos;                     // [T] out: position inside the sequence
  int *tok_seq;                 // [T] out: sequence of each token
  const __bf16 *Wqkv;           // first layer, fragment-packed [1152 x 384]
  const float *rope_cos, *rope_sin;  // the first layer's RoPE table [8192, 32]
  __bf16 *qkv_out;              // [T, 1152]
  int T;
  int rev;                      // nonzero: row blocks in reversed order
};

// Launchers (jl_kernels.hip, jl_layer.hip, jl_head.hip, jl_embed.hip).  `bf16` selects the bf16 instantiation, else FP32.
hipError_t launch_embed(const int32_t *ids, const float *emb, const float *gain, int T,
                        const int *seq_offsets, int n_seqs, float *x, int *pos, int *tok_seq,
                        hipStream_t s);
hipError_t launch_gemm(bool bf16, int emode, const GemmArgs &a, hipStream_t s);
// A = LayerNorm(ln_x; ln_gain, ln_shift) (K = 384), then launch_gemm's product.
// bf16 batches small enough for 64-row tiles normalize inside the GEMM's
// work-groups; otherwise the rows are normalized into a.A first.
hipError_t launch_ln_gemm(bool bf16, int emode, const GemmArgs &a, hipStream_t s);
hipError_t launch_ln_rows(bool bf16_out, const float *x, const float *gain, const float *shift, int n, void *out,
                          hipStream_t s);
hipError_t launch_attention(bool bf16, const AttnArgs &a, int n_work, int queries_per_block, hipStream_t s);
hipError_t launch_layer(const LayerArgs &a, hipStream_t s);
hipError_t launch_head_layer(const HeadArgs &a, hipStream_t s);
hipError_t launch_embed_qkv(const EmbedArgs &a, hipStream_t s);
hipError_t launch_final_ln_type(const float *x, const float *gain, const float *type_rows,
                                const int *qtype, const int *tok_seq, int T, float *h,
                                hipStream_t s);
// Row groups of the scorer (16 marker rows each).
constexpr int score_groups(int n) { return (n + 15) / 16; }
// dst = src rows `rows` (the marker rows); also clears the scorer's
// score_groups(n) counters for this pass.
hipError_t launch_gather_rows(const float *src, const int *rows, int n, float *dst, int *score_cnt, hipStream_t s);
// logits = w2 . GELU(W1 . LayerNorm(z; g, b) + b1) + b2 for the n rows of z
// (FP32, one launch): part [n, 6] holds partial sums, cnt the row groups'
// counters (cleared by the gather of the same pass, left cleared).  `rev`:
// work-groups in reversed order (the result is the same bit for bit).
hipError_t launch_score(const float *z, const float *g, const float *b, const float *W1, const float *b1,
                        const float *w2, const float *b2, int n, float *part, int *cnt, float *logits, int rev,
                        hipStream_t s);
hipError_t launch_probs(const float *logits, const int *marker_offsets, const int *qtype,
                        int n_seqs, float *probs, float *answer, int *argmax, float *maxprob,
                        hipStream_t s);

// Sets the calling thread's jl_last_error() message; returns `code`.
int set_error(int code, const char *msg);

// Body of an extern "C" entry point that uses C++ containers: no exception
// crosses the C ABI (an allocation failure becomes JL_ERR_OOM).
#define JL_CATCH_ALL(call)                                                  \
  try {                                                                     \
    return call;                                                            \
  } catch (const std::bad_alloc &) {                                        \
    return ::jl::set_error(JL_ERR_OOM, "host memory exhausted");            \
  } catch (const std::exception &e_) {                                      \
    return ::jl::set_error(JL_ERR_ARG, e_.what());                          \
  }

}  // namespace jl

struct jl_model;

namespace jl {

// jl_serve's per-handle stream and buffers (jl_serve.cpp), released by jl_free.
struct ServeState;
void free_serve_state(ServeState *st);
ServeState *&model_serve_state(jl_model *m);
// The handle's host-call buffers (made with its serving state on first use,
// kept until jl_free): device ids [max_tokens] and outputs [2 max_markers +
// 2 max_seqs] floats, with pinned host copies of each.
struct HandleBuffers {
  int32_t *d_ids, *h_ids;
  float *d_out, *h_out;
  int64_t max_tokens, max_markers;
};
int handle_buffers(jl_model *m, HandleBuffers *out);
// jl_forward for a batch already padded to its bucket's exact shape (jl_serve
// adds filler sequences): the attention work lists are padded with empty
// items to the capacity of (tokens, sequences), so that every batch of the
// bucket replays one captured graph.  Falls back to jl_forward when the
// handle's graph cache is off, on the NULL stream, or with the timer on.
int forward_bucketed(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets, int32_t n_seqs,
                     const int32_t *mask_positions, int32_t n_markers, const int32_t *qtype, float *logits_dev,
                     hipStream_t s);
int model_graph_cap(const jl_model *m);
// A HIP error seen on the handle's work: sets jl_last_error() to `what` and
// the HIP string and returns JL_ERR_DEVICE; an error that leaves the device
// context unusable (a memory fault, a kernel abort or timeout, an
// uncorrectable ECC error) also marks the handle poisoned, after which every
// call on it fails with JL_ERR_DEVICE until jl_free.
int device_error(jl_model *m, hipError_t e, const char *what);
// JL_OK, or the error (with its message) of a NULL or poisoned handle.
int model_check(const jl_model *m);
int model_device(const jl_model *m);
int64_t model_max_tokens(const jl_model *m);
int64_t model_max_markers(const jl_model *m);

}  // namespace jl
