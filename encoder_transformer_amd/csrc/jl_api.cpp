// Host side of libjl: weight loading, workspace, per-call planning and the C ABI.
//
// One call of jl_forward validates the packed batch on the host, uploads a few
// KB of metadata (offsets, marker lists, attention work items) through a
// pinned staging buffer, and enqueues about 120 kernels on the caller's
// stream.  No allocation happens per call.
#include "jl.h"
#include "jl_internal.h"

#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

using namespace jl;

namespace {

// Default: batches of at least this many tokens (bf16) take the row-block
// layer kernel (one work-group per 64 rows: 8,192 tokens give 128 of them).
constexpr int64_t kRowBlockMinTokens = 8192;

thread_local std::string g_err;

int fail(int code, const std::string &msg) {
  g_err = msg;
  return code;
}

// HIP errors after which the device context is unusable (later HIP calls in
// the process fail with the same error): memory faults, kernel exceptions,
// aborts and timeouts, uncorrectable ECC errors.
bool is_fault(hipError_t e) {
  switch (e) {
    case hipErrorIllegalAddress:
    case hipErrorLaunchFailure:
    case hipErrorLaunchTimeOut:
    case hipErrorAssert:
    case hipErrorECCNotCorrectable:
      return true;
    default:
      return false;
  }
}

#define JL_HIP(expr)                                                                      \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(JL_ERR_DEVICE, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

uint16_t f32_to_bf16(float f) {  // round to nearest even; NaN stays NaN
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP e4m3 (1 sign, 4 exponent bits biased by 7, 3 mantissa bits; no
// infinities, S.1111.111 is NaN, largest finite 448), round to nearest even.
// Normal codes hold (1 + m/8) 2^(e-7) for e = 1..15, subnormal ones m/8 2^-6;
// a magnitude that rounds above 448 becomes NaN, as the device conversion does.
uint8_t f32_to_e4m3(float f) {
  const uint8_t sign = std::signbit(f) ? 0x80 : 0x00;
  const float a = std::fabs(f);
  if (!(a == a)) return sign | 0x7f;
  if (a < 0x1p-6f) return sign | (uint8_t)std::nearbyint(a * 0x1p9f);  // 8 steps of 2^-9; 8 -> 2^-6 (0x08)
  int e;
  std::frexp(a, &e);  // a = f 2^e, f in [0.5, 1): a = (1 + m/8) 2^(e-1)
  int E = e - 1;
  int q = (int)std::nearbyint((std::ldexp(a, -E) - 1.0f) * 8.0f);  // exact in FP32
  if (q == 8) q = 0, ++E;
  const int code = ((E + 7) << 3) | q;
  return code > 0x7e ? (uint8_t)(sign | 0x7f) : (uint8_t)(sign | code);
}

// Matrix-core fragment order of a row-major W [N, K] (rows = output columns):
// block (gn, s) holds 64 lanes x 8 bf16, lane l element e = W[16 gn + l % 16]
// [32 s + 8 (l / 16) + e]; blocks are stored gn-major (index gn * K/32 + s), so a
// wave's B fragment for 16 output columns and 32 k is one contiguous 1 KB load.
// `row_of` maps packed row -> source row (GEGLU interleave), or nullptr;
// `row_scale` scales packed rows by powers of two (exact), or nullptr.
void pack_fragments(const float *W, int N, int K, const std::vector<int> *row_of, uint16_t *out,
                    const std::vector<float> *row_scale = nullptr) {
  const int ks = K / 32;
  for (int gn = 0; gn < N / 16; ++gn)
    for (int s = 0; s < ks; ++s) {
      uint16_t *blk = out + ((size_t)gn * ks + s) * 512;
      for (int l = 0; l < 64; ++l) {
        const int r = 16 * gn + (l & 15);
        const float *src = W + (size_t)(row_of ? (*row_of)[r] : r) * K + 32 * s + 8 * (l >> 4);
        const float sc = row_scale ? (*row_scale)[r] : 1.0f;
        for (int e = 0; e < 8; ++e) blk[l * 8 + e] = f32_to_bf16(sc * src[e]);
      }
    }
}

// e4m3 codes [N, 384] (row-major) in the row-block kernel's fp8 fragment
// order: block (gn, s) of 16 rows x 128 k is 2 KB, half h of it 1 KB in which
// lane l holds row 16 gn + l % 16, k = 128 s + 32 (l / 16) + 16 h + e at byte
// 16 l + e; blocks gn-major, so a wave's fragment is two contiguous 1 KB loads.
void pack_fragments8(const uint8_t *codes, int N, int K, uint8_t *out) {
  const int ks = K / 128;
  for (int gn = 0; gn < N / 16; ++gn)
    for (int s = 0; s < ks; ++s)
      for (int h = 0; h < 2; ++h) {
        uint8_t *blk = out + (((size_t)gn * ks + s) * 2 + h) * 1024;
        for (int l = 0; l < 64; ++l)
          std::memcpy(blk + 16 * l, codes + (size_t)(16 * gn + (l & 15)) * K + 128 * s + 32 * (l >> 4) + 16 * h, 16);
      }
}

struct LayerW {
  const float *attn_norm = nullptr;
  const void *Wqkv = nullptr, *Wo = nullptr, *Wi = nullptr, *Wout = nullptr;
  const float *mlp_norm = nullptr;
  // bf16 fragment-ordered copies for the row-block layer kernel
  const void *pWqkv = nullptr, *pWo = nullptr, *pWi = nullptr, *pWout = nullptr;
  // JL_FP8: e4m3 codes [N, 384] of the QKV (layers 1-21) and W_i rows and each row's scale
  const void *Wqkv8 = nullptr, *Wi8 = nullptr;
  const float *sqkv = nullptr, *si = nullptr;
  // the same codes in fp8 fragment order for the row-block layer kernel
  const void *pWqkv8 = nullptr, *pWi8 = nullptr;
};
struct HeadW {
  const void *in_w = nullptr, *out_w = nullptr, *l1_w = nullptr, *l2_w = nullptr;
  const float *in_b = nullptr, *out_b = nullptr, *l1_b = nullptr, *l2_b = nullptr;
  const float *n1_w = nullptr, *n1_b = nullptr, *n2_w = nullptr, *n2_b = nullptr;
  // bf16 fragment-ordered copies for the row-block kernels: the first layer's
  // in-projection, out-projection and feed-forward; the second layer's key
  // and value rows of the in-projection
  const void *pIn = nullptr, *pOut = nullptr, *pL1 = nullptr, *pL2 = nullptr, *pKV = nullptr;
};

struct ProfRec {
  int cls;
  hipEvent_t a, b;
};

// Activation buffers of one forward pass (device memory), laid out by
// layout_workspace:
//   x [T, 384] FP32 residual stream (the head's h from the final LayerNorm on);
//   qkv [T, 1152] (head layer 2: keys|values [T, 768]); o [T, 384] attention
//   output, also the normalized GEMM operand u; act [T, 1536] GEGLU output /
//   head FFN hidden; pos, tok_seq [T] int32; marker rows z [M, 384] FP32,
//   qm, om [M, 384], actm [M, 1536] (element type); the scorer's partial
//   sums score_part [M, 6] FP32 and counters score_cnt [M / 16] int32.
struct Workspace {
  float *x = nullptr, *z = nullptr, *score_part = nullptr;
  int *score_cnt = nullptr;
  char *qkv = nullptr, *o = nullptr, *act = nullptr, *qm = nullptr, *om = nullptr, *actm = nullptr;
  int *pos = nullptr, *tok_seq = nullptr;
};

// Metadata ints of one call for up to T tokens, Mm markers and Bm sequences:
// offsets, marker counts, types and positions, and work lists of 8-int items
// (attention items plus at most half as many empty ones, and 8 more).
constexpr size_t meta_ints_for(size_t T, size_t Mm, size_t Bm) {
  return 2 * (Bm + 1) + Bm + Mm + 12 * (T / 64 + Bm + 16) + 12 * (T / 128 + Bm + 16) + 8 * Bm + 64;
}

// Attention work items any batch of T tokens and B sequences can need with
// `tile`-query items: at most T / tile + B items, laid out per XCD with at
// most half again as many empty ones (and 8 more), rounded up to 8.  A
// bucketed call pads its lists to this count, so that its launch shape
// depends on (T, B) only.
constexpr int work_capacity(int64_t T, int64_t B, int tile) {
  return (int)(((T / tile + B) * 3 / 2 + 8 + 1 + 7) / 8 * 8);
}

constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Every workspace piece is followed by a guard band of kGuardBytes bytes of
// kGuardByte, written at load and never by a kernel; jl_check_guards reads
// them back (a write past the end of a piece lands there first).
constexpr size_t kGuardBytes = 256;
constexpr uint8_t kGuardByte = 0xA5;
constexpr int kWorkspacePieces = 12;
const char *const kPieceNames[kWorkspacePieces] = {"x",  "qkv", "o",     "act",  "pos",        "tok_seq",
                                                   "z",  "qm",  "om",    "actm", "score_part", "score_cnt"};

// Bytes of layout_workspace's layout (same pieces, same order).
constexpr size_t workspace_bytes(size_t T, size_t Mm, size_t es, size_t meta_ints, int n_meta) {
  const size_t D = kWidth;
  const size_t parts[kWorkspacePieces] = {T * D * 4,  T * 3 * D * es, T * D * es,  T * kHeadFfn * es,  T * 4,
                                          T * 4,      Mm * D * 4,     Mm * D * es, Mm * D * es,
                                          Mm * kHeadFfn * es,         Mm * (kWidth / 64) * 4,
                                          (Mm + 15) / 16 * 4};
  size_t off = 0;
  for (size_t p : parts) off = align256(off) + p + kGuardBytes;
  for (int k = 0; k < n_meta; ++k) off = align256(off) + meta_ints * 4 + kGuardBytes;
  return align256(off);
}

// Carve a workspace for T tokens and Mm markers (element size es) and n_meta
// metadata blocks of meta_ints ints out of `base` (256-byte aligned pieces,
// each followed by its guard band); with base == nullptr only the size is
// computed.  `guards` (or nullptr) receives each band's byte offset, pieces
// first, then the metadata blocks.  Returns the bytes used.
size_t layout_workspace(char *base, size_t T, size_t Mm, size_t es, size_t meta_ints, Workspace *w, int **meta,
                        int n_meta, std::vector<size_t> *guards = nullptr) {
  const size_t D = kWidth;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    off = (off + 255) & ~size_t(255);
    char *p = base ? base + off : nullptr;
    off += bytes;
    if (guards) guards->push_back(off);
    off += kGuardBytes;
    return p;
  };
  w->x = (float *)take(T * D * 4);
  w->qkv = take(T * 3 * D * es);
  w->o = take(T * D * es);
  w->act = take(T * kHeadFfn * es);
  w->pos = (int *)take(T * 4);
  w->tok_seq = (int *)take(T * 4);
  w->z = (float *)take(Mm * D * 4);
  w->qm = take(Mm * D * es);
  w->om = take(Mm * D * es);
  w->actm = take(Mm * kHeadFfn * es);
  w->score_part = (float *)take(Mm * (kWidth / 64) * 4);
  w->score_cnt = (int *)take((Mm + 15) / 16 * 4);
  for (int k = 0; k < n_meta; ++k) meta[k] = (int *)take(meta_ints * 4);
  return align256(off);  // == workspace_bytes(T, Mm, es, meta_ints, n_meta)
}

}  // namespace

struct jl_model {
  int device = 0;
  int precision = JL_BF16;
  bool bf16 = true;
  size_t esize = 2;
  int64_t max_tokens = 0, max_markers = 0, max_seqs = 0;
  int64_t row_block_min_tokens = 8192;

  char *warena = nullptr;  // weights; freed with the last handle that shares them
  std::shared_ptr<void> warena_owner;
  size_t wbytes = 0;
  ServeState *serve = nullptr;  // jl_serve's stream and buffers, made on first use
  char *ws = nullptr;
  size_t wsbytes = 0;

  // weights
  const float *emb = nullptr, *emb_norm = nullptr, *final_norm = nullptr, *type_rows = nullptr;
  LayerW L[kLayers];
  HeadW H[2];
  const float *sc_nw = nullptr, *sc_nb = nullptr, *sc_w1 = nullptr, *sc_b1 = nullptr, *sc_w2 = nullptr,
              *sc_b2 = nullptr;
  const float *rope_cos[2] = {nullptr, nullptr}, *rope_sin[2] = {nullptr, nullptr};  // [0] local, [1] global

  // workspace
  Workspace w;
  // Batch metadata ring: call i uses slot i % kMetaSlots (pinned staging +
  // device copy); slot_done[k] is recorded after the last kernel that reads
  // slot k, so the host may run up to kMetaSlots - 1 calls ahead of the GPU.
  static constexpr int kMetaSlots = 4;
  int *meta[kMetaSlots] = {};
  // Graph mode: jl_forward replays a captured HIP graph per batch shape; the
  // graphs read their metadata from this one device buffer, which each call
  // refills on the stream before its replay.
  int *gmeta = nullptr;
  struct GraphEntry {
    int T, B, M, n_work, n_work_wide;
    bool row_block;
    const void *ids, *out;
    hipGraph_t graph;
    hipGraphExec_t exec;
    uint64_t last_use;
  };
  std::vector<GraphEntry> graphs;
  int graph_cap = 0;
  uint64_t graph_clock = 0;
  int64_t graph_captures = 0, graph_replays = 0;

  // debugging (jl_set_debug; JL_DEBUG_SYNC=1 in the environment at load sets
  // JL_DEBUG_SYNC) and the poisoned state after a device fault
  uint32_t debug = 0;
  bool poisoned = false;
  std::string poison_msg;
  std::vector<size_t> guards;  // workspace guard band offsets (layout_workspace)
  int *host_meta[kMetaSlots] = {};
  hipEvent_t slot_done[kMetaSlots] = {};
  bool slot_pending[kMetaSlots] = {};
  int next_slot = 0;
  size_t meta_ints = 0;

  // Host-side planning buffers, reserved at load for max_tokens / max_seqs
  // so that planning a call allocates nothing: the longest-first sequence
  // order and the attention items of each of the 8 XCDs.
  std::vector<int> plan_order;
  std::vector<AttnWork> plan_per[8];

  // per-kernel timer (suspended inside jl_forward_static, which records no events)
  bool prof_suspended = false;
  bool prof = false;
  uint32_t prof_mask = 0;
  std::vector<ProfRec> prof_rec;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
};

namespace {

// ---------------------------------------------------------------------------
// weight file
// ---------------------------------------------------------------------------

struct TensorEntry {
  std::vector<uint32_t> shape;
  uint64_t offset = 0, checksum = 0;
};

struct MappedFile {
  void *base = MAP_FAILED;
  size_t size = 0;
  ~MappedFile() {
    if (base != MAP_FAILED) munmap(base, size);
  }
};

int parse_weight_file(const char *path, MappedFile &mf, std::map<std::string, TensorEntry> &tab) {
  const int fd = open(path, O_RDONLY);
  if (fd < 0) return fail(JL_ERR_FILE, std::string("cannot open weight file ") + path);
  struct stat st;
  if (fstat(fd, &st) != 0) {
    close(fd);
    return fail(JL_ERR_FILE, "cannot stat weight file");
  }
  mf.size = (size_t)st.st_size;
  if (mf.size < 16) {
    close(fd);
    return fail(JL_ERR_FILE, "weight file truncated (no header)");
  }
  mf.base = mmap(nullptr, mf.size, PROT_READ, MAP_PRIVATE, fd, 0);
  close(fd);
  if (mf.base == MAP_FAILED) return fail(JL_ERR_FILE, "cannot map weight file");
  const unsigned char *p = (const unsigned char *)mf.base;
  if (std::memcmp(p, "JLW1", 4) != 0) return fail(JL_ERR_FILE, "bad weight-file magic");
  uint32_t version, n, hdr;
  std::memcpy(&version, p + 4, 4);
  std::memcpy(&n, p + 8, 4);
  std::memcpy(&hdr, p + 12, 4);
  if (version != 1) return fail(JL_ERR_FILE, "unsupported weight-file version");
  if (hdr > mf.size) return fail(JL_ERR_FILE, "weight file truncated (header)");
  size_t off = 16;
  for (uint32_t i = 0; i < n; ++i) {
    if (off + 2 > hdr) return fail(JL_ERR_FILE, "corrupt weight-file header");
    uint16_t nl;
    std::memcpy(&nl, p + off, 2);
    off += 2;
    if (off + nl + 1 > hdr) return fail(JL_ERR_FILE, "corrupt weight-file header");
    std::string name((const char *)p + off, nl);
    off += nl;
    const uint8_t nd = p[off++];
    if (nd > 4 || off + 4 * nd + 16 > hdr) return fail(JL_ERR_FILE, "corrupt weight-file header");
    TensorEntry e;
    uint64_t count = 1;
    for (int d = 0; d < nd; ++d) {
      uint32_t v;
      std::memcpy(&v, p + off, 4);
      off += 4;
      e.shape.push_back(v);
      count *= v;
    }
    std::memcpy(&e.offset, p + off, 8);
    std::memcpy(&e.checksum, p + off + 8, 8);
    off += 16;
    if (e.offset % 4 != 0 || e.offset + count * 4 > mf.size)
      return fail(JL_ERR_FILE, "weight file truncated (tensor " + name + ")");
    tab[name] = e;
  }
  return JL_OK;
}

uint64_t checksum_words(const uint32_t *w, size_t n) {
  uint64_t s = 0;
  for (size_t i = 0; i < n; ++i) s += w[i];
  return s;
}

// Host staging of the converted weights (everything but the embedding table).
struct Arena {
  std::vector<char> buf;
  size_t add(size_t bytes) {
    const size_t off = (buf.size() + 255) & ~size_t(255);
    buf.resize(off + bytes);
    return off;
  }
};

}  // namespace

int jl::device_error(jl_model *m, hipError_t e, const char *what) {
  std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  if (is_fault(e) && m && !m->poisoned) {
    m->poisoned = true;
    m->poison_msg = msg;
  }
  return fail(JL_ERR_DEVICE, msg);
}

namespace {

// A HIP call on the handle `m`'s work: errors through device_error.
#define JL_HIPM(expr)                                                   \
  do {                                                                  \
    hipError_t e_ = (expr);                                             \
    if (e_ != hipSuccess) return ::jl::device_error(m, e_, #expr);     \
  } while (0)

// Entry check of every call that enqueues work on, or waits for, a handle.
int usable(const jl_model *m) {
  if (!m) return fail(JL_ERR_ARG, "model handle is NULL");
  if (m->poisoned)
    return fail(JL_ERR_DEVICE, "the handle is poisoned by an earlier device fault (" + m->poison_msg +
                                   "); free it with jl_free");
  return JL_OK;
}

uint32_t debug_from_env() {
  const char *v = std::getenv("JL_DEBUG_SYNC");
  return v && v[0] && std::strcmp(v, "0") != 0 ? (uint32_t)JL_DEBUG_SYNC : 0u;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" const char *jl_last_error(void) { return g_err.c_str(); }

extern "C" int jl_validate(const int32_t *seq_offsets, int32_t n_seqs, const int32_t *mask_positions,
                           int32_t n_markers, const int32_t *qtype, int64_t max_tokens,
                           int64_t max_markers) {
  if (n_seqs < 0 || n_markers < 0) return fail(JL_ERR_ARG, "negative sequence or marker count");
  if (!seq_offsets) return fail(JL_ERR_ARG, "seq_offsets is NULL");
  if (n_seqs > 0 && !qtype) return fail(JL_ERR_ARG, "qtype is NULL");
  if (n_markers > 0 && !mask_positions) return fail(JL_ERR_ARG, "mask_positions is NULL");
  if (seq_offsets[0] != 0) return fail(JL_ERR_LENGTH, "seq_offsets[0] must be 0");
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t len = (int64_t)seq_offsets[b + 1] - seq_offsets[b];
    if (len < 1 || len > JL_MAX_SEQ_LEN)
      return fail(JL_ERR_LENGTH, "sequence " + std::to_string(b) + " has length " + std::to_string(len) +
                                     " (must be 1.." + std::to_string(JL_MAX_SEQ_LEN) + ")");
    if (qtype[b] < 0 || qtype[b] > 2)
      return fail(JL_ERR_QTYPE, "sequence " + std::to_string(b) + " has question type " + std::to_string(qtype[b]));
  }
  const int64_t T = seq_offsets[n_seqs];
  if (T > max_tokens)
    return fail(JL_ERR_CAPACITY, std::to_string(T) + " tokens exceed the handle's " + std::to_string(max_tokens));
  if (n_markers > max_markers)
    return fail(JL_ERR_CAPACITY,
                std::to_string(n_markers) + " markers exceed the handle's " + std::to_string(max_markers));
  for (int32_t k = 0; k < n_markers; ++k) {
    if (mask_positions[k] < 0 || mask_positions[k] >= T)
      return fail(JL_ERR_OPTIONS, "marker " + std::to_string(k) + " lies outside every sequence");
    if (k > 0 && mask_positions[k] <= mask_positions[k - 1])
      return fail(JL_ERR_OPTIONS, "marker positions must be strictly increasing");
  }
  int32_t k = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    int32_t c = 0;
    while (k < n_markers && mask_positions[k] < seq_offsets[b + 1]) {
      ++k;
      ++c;
    }
    if (c < JL_MIN_OPTIONS || c > JL_MAX_OPTIONS)
      return fail(JL_ERR_OPTIONS, "sequence " + std::to_string(b) + " has " + std::to_string(c) +
                                      " options (must be 2..20)");
    if (qtype[b] == JL_NOUL && c != 2)
      return fail(JL_ERR_OPTIONS, "noul sequence " + std::to_string(b) + " must have exactly 2 options");
  }
  return JL_OK;
}

extern "C" void jl_free(jl_model *m) {
  if (!m) return;
  DeviceGuard dg(m->device);
  for (int k = 0; k < jl_model::kMetaSlots; ++k) {
    if (m->slot_done[k]) {
      (void)hipEventSynchronize(m->slot_done[k]);
      (void)hipEventDestroy(m->slot_done[k]);
    }
    if (m->host_meta[k]) (void)hipHostFree(m->host_meta[k]);
  }
  for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
  for (auto &g : m->graphs) {
    (void)hipGraphExecDestroy(g.exec);
    (void)hipGraphDestroy(g.graph);
  }
  if (m->serve) free_serve_state(m->serve);
  if (m->ws) (void)hipFree(m->ws);
  m->warena_owner.reset();  // frees the weights if no other handle shares them
  delete m;
}

namespace {
// Device workspace, metadata ring and pinned staging of a handle, sized by its
// max_tokens / max_markers (and precision).  On failure the caller frees m.
int alloc_workspace(jl_model *m) {
  const size_t T = (size_t)m->max_tokens, Mm = (size_t)m->max_markers, Bm = (size_t)m->max_seqs;
  m->meta_ints = meta_ints_for(T, Mm, Bm);
  int *meta[jl_model::kMetaSlots + 1];
  m->wsbytes = layout_workspace(nullptr, T, Mm, m->esize, m->meta_ints, &m->w, meta, jl_model::kMetaSlots + 1);
  if (hipMalloc((void **)&m->ws, m->wsbytes) != hipSuccess) return fail(JL_ERR_OOM, "cannot allocate the device workspace");
  m->guards.clear();
  layout_workspace(m->ws, T, Mm, m->esize, m->meta_ints, &m->w, meta, jl_model::kMetaSlots + 1, &m->guards);
  for (size_t g : m->guards)
    if (hipMemset(m->ws + g, kGuardByte, kGuardBytes) != hipSuccess)
      return fail(JL_ERR_DEVICE, "cannot write the workspace guard bands");
  if (hipDeviceSynchronize() != hipSuccess) return fail(JL_ERR_DEVICE, "cannot write the workspace guard bands");
  m->debug = debug_from_env();
  for (int k = 0; k < jl_model::kMetaSlots; ++k) m->meta[k] = meta[k];
  m->gmeta = meta[jl_model::kMetaSlots];
  m->plan_order.reserve(Bm);
  for (auto &v : m->plan_per) v.reserve(T / 64 + Bm + 8);
  for (int k = 0; k < jl_model::kMetaSlots; ++k) {
    if (hipHostMalloc((void **)&m->host_meta[k], m->meta_ints * 4, hipHostMallocDefault) != hipSuccess)
      return fail(JL_ERR_OOM, "cannot allocate pinned staging memory");
    if (hipEventCreateWithFlags(&m->slot_done[k], hipEventDisableTiming) != hipSuccess)
      return fail(JL_ERR_DEVICE, "cannot create an event");
  }
  return JL_OK;
}

}  // namespace

namespace {

// Largest batch of jl_forward_static: 2,048 tokens and 256 markers (so at
// most 128 sequences), in any precision; its workspace (FP32 mode: 31.3 MB)
// lives in `scratch`, one copy per GPU, held until the process ends.
constexpr int64_t kStaticMaxTokens = 2048, kStaticMaxMarkers = 256, kStaticMaxSeqs = kStaticMaxMarkers / 2;
constexpr size_t kStaticMetaInts = meta_ints_for(kStaticMaxTokens, kStaticMaxMarkers, kStaticMaxSeqs);
constexpr size_t kScratchBytes = workspace_bytes(kStaticMaxTokens, kStaticMaxMarkers, 4, kStaticMetaInts, 1);
static_assert(kScratchBytes <= ((size_t)32 << 20), "static workspace above 32 MiB");

static __device__ __align__(256) char scratch[kScratchBytes];

// The array's device address on each GPU (hipGetSymbolAddress, taken once
// per device at the first jl_load_weights there, with that device current).
// In host code `scratch` names a host-side stand-in, never device memory:
// only these addresses are passed to kernels and copies.
std::mutex g_scratch_mu;
void *g_scratch_dev[64] = {};

int scratch_init(int device) {
  if (device >= 64) return fail(JL_ERR_DEVICE, "device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[device]) return JL_OK;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != device) return fail(JL_ERR_DEVICE, "scratch: device not current");
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return fail(JL_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  g_scratch_dev[device] = p;
  return JL_OK;
}

}  // namespace

static int jl_load_weights_impl(const char *path, int precision, int64_t max_tokens, int64_t max_markers,
                               int device, jl_model **out) {
  if (!path || !out) return fail(JL_ERR_ARG, "path and out must not be NULL");
  *out = nullptr;
  if (precision != JL_FP32 && precision != JL_BF16 && precision != JL_FP8)
    return fail(JL_ERR_ARG, "precision must be JL_FP32, JL_BF16 or JL_FP8");
  if (max_tokens < 1 || max_tokens > (int64_t)1 << 26) return fail(JL_ERR_ARG, "max_tokens must be in 1..2^26");
  if (max_markers < 2 || max_markers > max_tokens) return fail(JL_ERR_ARG, "max_markers must be in 2..max_tokens");
  if (device < 0) return fail(JL_ERR_ARG, "device must be >= 0");

  // Parse, verify and convert on the host first: file errors never need a GPU.
  MappedFile mf;
  std::map<std::string, TensorEntry> tab;
  if (int rc = parse_weight_file(path, mf, tab)) return rc;

  const bool bf = precision != JL_FP32;  // JL_FP8: bf16 operands outside its e4m3 products
  const bool f8 = precision == JL_FP8;
  const size_t es = bf ? 2 : 4;
  const char *base = (const char *)mf.base;
  auto get = [&](const std::string &name, std::vector<uint32_t> shape, const float **data) -> int {
    auto it = tab.find(name);
    if (it == tab.end()) return fail(JL_ERR_FILE, "weight file lacks tensor " + name);
    if (it->second.shape != shape) return fail(JL_ERR_FILE, "tensor " + name + " has the wrong shape");
    size_t n = 1;
    for (uint32_t d : shape) n *= d;
    const uint32_t *w = (const uint32_t *)(base + it->second.offset);
    if (checksum_words(w, n) != it->second.checksum) return fail(JL_ERR_FILE, "checksum mismatch in tensor " + name);
    *data = (const float *)w;
    return JL_OK;
  };

  Arena ar;
  // Offsets are resolved to device pointers after the upload.
  struct Pending {
    const void **dst;
    size_t off;
  };
  std::vector<Pending> pend;
  auto put_f32 = [&](const float *src, size_t n, const float **dst) {
    const size_t off = ar.add(n * 4);
    std::memcpy(ar.buf.data() + off, src, n * 4);
    pend.push_back({(const void **)dst, off});
  };
  // element matrix [rows, cols]; `row_of` maps destination row -> source row
  auto put_elem = [&](const float *src, size_t rows, size_t cols, const void **dst, const std::vector<int> *row_of) {
    const size_t off = ar.add(rows * cols * es);
    char *d = ar.buf.data() + off;
    for (size_t r = 0; r < rows; ++r) {
      const float *s = src + (size_t)(row_of ? (*row_of)[r] : (int)r) * cols;
      if (bf) {
        uint16_t *o = (uint16_t *)d + r * cols;
        for (size_t c = 0; c < cols; ++c) o[c] = f32_to_bf16(s[c]);
      } else {
        std::memcpy((float *)d + r * cols, s, cols * 4);
      }
    }
    pend.push_back({dst, off});
  };

  // e4m3 codes of a matrix [rows, cols] (rows through `row_of`): each row
  // times 448 / max |row| (in FP32), and the row scales max |row| / 448
  auto put_e4m3 = [&](const float *src, size_t rows, size_t cols, const void **dst, const float **scale,
                      const std::vector<int> *row_of, const void **packed) {
    const size_t off = ar.add(rows * cols), soff = ar.add(rows * 4), poff = ar.add(rows * cols);
    uint8_t *d = (uint8_t *)(ar.buf.data() + off);
    float *sc = (float *)(ar.buf.data() + soff);
    for (size_t r = 0; r < rows; ++r) {
      const float *sr = src + (size_t)(row_of ? (*row_of)[r] : (int)r) * cols;
      float amax = 0.f;
      for (size_t c = 0; c < cols; ++c) amax = std::max(amax, std::fabs(sr[c]));
      const float rc = amax > 0.f ? 448.0f / amax : 1.0f;
      sc[r] = amax > 0.f ? amax / 448.0f : 1.0f;
      for (size_t c = 0; c < cols; ++c) d[r * cols + c] = f32_to_e4m3(sr[c] * rc);
    }
    pack_fragments8(d, (int)rows, (int)cols, (uint8_t *)(ar.buf.data() + poff));
    pend.push_back({dst, off});
    pend.push_back({(const void **)scale, soff});
    pend.push_back({packed, poff});
  };
  auto put_packed = [&](const float *src, int rows, int cols, const void **dst, const std::vector<int> *row_of,
                        const std::vector<float> *row_scale = nullptr) {
    const size_t off = ar.add((size_t)rows * cols * 2);
    pack_fragments(src, rows, cols, row_of, (uint16_t *)(ar.buf.data() + off), row_scale);
    pend.push_back({dst, off});
  };

  jl_model *m = new jl_model();
  m->device = device;
  m->precision = precision;
  m->bf16 = bf;
  m->esize = es;
  m->max_tokens = max_tokens;
  m->max_markers = max_markers;
  m->max_seqs = std::min<int64_t>(max_tokens, max_markers / 2);
  m->row_block_min_tokens = kRowBlockMinTokens;

  const uint32_t D = kWidth;
  const float *t = nullptr;
  int rc = JL_OK;
#define GET(name, ...)                                   \
  if ((rc = get(name, {__VA_ARGS__}, &t)) != JL_OK) {    \
    delete m;                                            \
    return rc;                                           \
  }
  const float *emb_host = nullptr;
  GET("embeddings.tok_embeddings.weight", (uint32_t)kVocab, D);
  emb_host = t;
  GET("embeddings.norm.weight", D);
  put_f32(t, D, &m->emb_norm);
  // GEGLU rows interleaved by 16: [a0..a15, g0..g15, a16..a31, g16..g31, ...]
  std::vector<int> geglu_rows(2 * kGeglu);
  // The row-block kernel's packed copy carries the gate rows halved (exact),
  // so its GEGLU computes gelu(z) g = (z + |z| erf(|z|/sqrt 2)) (g/2).
  std::vector<float> gate_half(2 * kGeglu);
  for (int o = 0; o < kGeglu; ++o) {
    geglu_rows[32 * (o / 16) + (o % 16)] = o;
    geglu_rows[32 * (o / 16) + 16 + (o % 16)] = kGeglu + o;
    gate_half[32 * (o / 16) + (o % 16)] = 1.0f;
    gate_half[32 * (o / 16) + 16 + (o % 16)] = 0.5f;
  }
  // Attention consumes q scaled by log2(e) / sqrt(64) (scores in the exp2
  // domain): the factor goes into the q rows of every in-projection (and the
  // q bias) here, in FP32 before the element conversion.
  std::vector<float> qscaled;
  auto scale_q_rows = [&](const float *w, size_t rows, size_t cols) -> const float * {
    qscaled.assign(w, w + rows * cols);
    for (size_t i = 0; i < (size_t)D * cols; ++i) qscaled[i] *= kQScale;
    return qscaled.data();
  };
  for (int l = 0; l < kLayers; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    if (l != 0) {
      GET(p + "attn_norm.weight", D);
      put_f32(t, D, &m->L[l].attn_norm);
    }
    GET(p + "attn.Wqkv.weight", 3 * D, D);
    t = scale_q_rows(t, 3 * D, D);
    put_elem(t, 3 * D, D, &m->L[l].Wqkv, nullptr);
    if (bf) put_packed(t, 3 * D, D, &m->L[l].pWqkv, nullptr);
    if (f8 && l != 0) put_e4m3(t, 3 * D, D, &m->L[l].Wqkv8, &m->L[l].sqkv, nullptr, &m->L[l].pWqkv8);
    GET(p + "attn.Wo.weight", D, D);
    put_elem(t, D, D, &m->L[l].Wo, nullptr);
    if (bf) put_packed(t, D, D, &m->L[l].pWo, nullptr);
    GET(p + "mlp_norm.weight", D);
    put_f32(t, D, &m->L[l].mlp_norm);
    GET(p + "mlp.Wi.weight", 2 * kGeglu, D);
    put_elem(t, 2 * kGeglu, D, &m->L[l].Wi, &geglu_rows);
    if (f8) put_e4m3(t, 2 * kGeglu, D, &m->L[l].Wi8, &m->L[l].si, &geglu_rows, &m->L[l].pWi8);
    if (bf) put_packed(t, 2 * kGeglu, D, &m->L[l].pWi, &geglu_rows, &gate_half);
    GET(p + "mlp.Wo.weight", D, kGeglu);
    put_elem(t, D, kGeglu, &m->L[l].Wout, nullptr);
    if (bf) put_packed(t, D, kGeglu, &m->L[l].pWout, nullptr);
  }
  GET("final_norm.weight", D);
  put_f32(t, D, &m->final_norm);
  GET("head.type_embedding.weight", 3, D);
  put_f32(t, 3 * D, &m->type_rows);
  for (int j = 0; j < 2; ++j) {
    const std::string p = "head.layers." + std::to_string(j) + ".";
    HeadW &h = m->H[j];
    GET(p + "self_attn.in_proj_weight", 3 * D, D);
    t = scale_q_rows(t, 3 * D, D);
    put_elem(t, 3 * D, D, &h.in_w, nullptr);
    if (bf && j == 0) put_packed(t, 3 * D, D, &h.pIn, nullptr);
    if (bf && j == 1) put_packed(t + (size_t)D * D, 2 * D, D, &h.pKV, nullptr);
    GET(p + "self_attn.in_proj_bias", 3 * D);
    t = scale_q_rows(t, 3 * D, 1);
    put_f32(t, 3 * D, &h.in_b);
    GET(p + "self_attn.out_proj.weight", D, D);
    put_elem(t, D, D, &h.out_w, nullptr);
    if (bf && j == 0) put_packed(t, D, D, &h.pOut, nullptr);
    GET(p + "self_attn.out_proj.bias", D);
    put_f32(t, D, &h.out_b);
    GET(p + "linear1.weight", (uint32_t)kHeadFfn, D);
    put_elem(t, kHeadFfn, D, &h.l1_w, nullptr);
    if (bf && j == 0) put_packed(t, kHeadFfn, D, &h.pL1, nullptr);
    GET(p + "linear1.bias", (uint32_t)kHeadFfn);
    put_f32(t, kHeadFfn, &h.l1_b);
    GET(p + "linear2.weight", D, (uint32_t)kHeadFfn);
    put_elem(t, D, kHeadFfn, &h.l2_w, nullptr);
    if (bf && j == 0) put_packed(t, D, kHeadFfn, &h.pL2, nullptr);
    GET(p + "linear2.bias", D);
    put_f32(t, D, &h.l2_b);
    GET(p + "norm1.weight", D);
    put_f32(t, D, &h.n1_w);
    GET(p + "norm1.bias", D);
    put_f32(t, D, &h.n1_b);
    GET(p + "norm2.weight", D);
    put_f32(t, D, &h.n2_w);
    GET(p + "norm2.bias", D);
    put_f32(t, D, &h.n2_b);
  }
  GET("head.scorer.norm.weight", D);
  put_f32(t, D, &m->sc_nw);
  GET("head.scorer.norm.bias", D);
  put_f32(t, D, &m->sc_nb);
  GET("head.scorer.fc1.weight", D, D);
  put_f32(t, (size_t)D * D, &m->sc_w1);
  GET("head.scorer.fc1.bias", D);
  put_f32(t, D, &m->sc_b1);
  GET("head.scorer.fc2.weight", 1, D);
  put_f32(t, D, &m->sc_w2);
  GET("head.scorer.fc2.bias", 1);
  put_f32(t, 1, &m->sc_b2);
#undef GET
  // RoPE tables: angle p * theta^(-2j/64) in double, cos/sin rounded to FP32
  for (int gl = 0; gl < 2; ++gl) {
    const double theta = gl ? kThetaGlobal : kThetaLocal;
    std::vector<float> c((size_t)kMaxSeq * 32), s((size_t)kMaxSeq * 32);
    for (int j = 0; j < 32; ++j) {
      const double omega = std::pow(theta, -2.0 * j / kHeadDim);
      for (int p = 0; p < kMaxSeq; ++p) {
        const double a = (double)p * omega;
        c[(size_t)p * 32 + j] = (float)std::cos(a);
        s[(size_t)p * 32 + j] = (float)std::sin(a);
      }
    }
    put_f32(c.data(), c.size(), &m->rope_cos[gl]);
    put_f32(s.data(), s.size(), &m->rope_sin[gl]);
  }

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device >= ndev) {
    delete m;
    return fail(JL_ERR_DEVICE, "no HIP device " + std::to_string(device));
  }
  DeviceGuard dg(device);
  if (int rc = scratch_init(device)) {
    delete m;
    return rc;
  }
  const size_t emb_bytes = (size_t)kVocab * D * 4;
  const size_t rest = (ar.buf.size() + 255) & ~size_t(255);
  m->wbytes = emb_bytes + rest;
  if (hipMalloc((void **)&m->warena, m->wbytes) != hipSuccess) {
    delete m;
    return fail(JL_ERR_OOM, "cannot allocate device memory for the weights");
  }
  m->warena_owner = std::shared_ptr<void>(m->warena, [dev = device](void *p) {
    DeviceGuard g(dev);
    (void)hipFree(p);
  });
  auto bail = [&](int code, const std::string &msg) {
    jl_free(m);
    return fail(code, msg);
  };
  if (hipMemcpy(m->warena, emb_host, emb_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(m->warena + emb_bytes, ar.buf.data(), ar.buf.size(), hipMemcpyHostToDevice) != hipSuccess)
    return bail(JL_ERR_DEVICE, "weight upload failed");
  m->emb = (const float *)m->warena;
  for (const Pending &pd : pend) *pd.dst = m->warena + emb_bytes + pd.off;

  if (int rc = alloc_workspace(m)) {
    jl_free(m);
    return rc;
  }
  *out = m;
  return JL_OK;
}

extern "C" int jl_load_weights(const char *path, int precision, int64_t max_tokens, int64_t max_markers,
                               int device, jl_model **out) {
  JL_CATCH_ALL(jl_load_weights_impl(path, precision, max_tokens, max_markers, device, out));
}

static int jl_share_impl(const jl_model *src, int64_t max_tokens, int64_t max_markers, jl_model **out) {
  if (!src || !out) return fail(JL_ERR_ARG, "src and out must not be NULL");
  if (max_tokens < 1 || max_tokens > (int64_t)1 << 26) return fail(JL_ERR_ARG, "max_tokens must be in 1..2^26");
  if (max_markers < 2 || max_markers > max_tokens) return fail(JL_ERR_ARG, "max_markers must be in 2..max_tokens");
  DeviceGuard dg(src->device);
  jl_model *m = new jl_model();
  m->device = src->device;
  m->precision = src->precision;
  m->bf16 = src->bf16;
  m->esize = src->esize;
  m->max_tokens = max_tokens;
  m->max_markers = max_markers;
  m->max_seqs = std::min<int64_t>(max_tokens, max_markers / 2);
  m->row_block_min_tokens = src->row_block_min_tokens;
  m->warena = src->warena;
  m->warena_owner = src->warena_owner;
  m->wbytes = src->wbytes;
  m->emb = src->emb;
  m->emb_norm = src->emb_norm;
  m->final_norm = src->final_norm;
  m->type_rows = src->type_rows;
  for (int l = 0; l < kLayers; ++l) m->L[l] = src->L[l];
  for (int j = 0; j < 2; ++j) m->H[j] = src->H[j];
  m->sc_nw = src->sc_nw;
  m->sc_nb = src->sc_nb;
  m->sc_w1 = src->sc_w1;
  m->sc_b1 = src->sc_b1;
  m->sc_w2 = src->sc_w2;
  m->sc_b2 = src->sc_b2;
  for (int k = 0; k < 2; ++k) {
    m->rope_cos[k] = src->rope_cos[k];
    m->rope_sin[k] = src->rope_sin[k];
  }
  if (int rc = alloc_workspace(m)) {
    jl_free(m);
    return rc;
  }
  *out = m;
  return JL_OK;
}

extern "C" int jl_share(const jl_model *src, int64_t max_tokens, int64_t max_markers, jl_model **out) {
  JL_CATCH_ALL(jl_share_impl(src, max_tokens, max_markers, out));
}

ServeState *&jl::model_serve_state(jl_model *m) { return m->serve; }
int jl::model_check(const jl_model *m) { return usable(m); }
int jl::model_device(const jl_model *m) { return m->device; }
int64_t jl::model_max_tokens(const jl_model *m) { return m->max_tokens; }
int64_t jl::model_max_markers(const jl_model *m) { return m->max_markers; }

extern "C" int jl_set_row_block_min_tokens(jl_model *m, int64_t min_tokens) {
  if (!m) return fail(JL_ERR_ARG, "model handle is NULL");
  if (min_tokens < 0) return fail(JL_ERR_ARG, "min_tokens must be >= 0");
  m->row_block_min_tokens = min_tokens;
  return JL_OK;
}

extern "C" int jl_model_info(const jl_model *m, int64_t *info, int n) {
  if (!m || !info) return fail(JL_ERR_ARG, "NULL argument");
  const int64_t v[10] = {m->precision, m->max_tokens,     m->max_markers,  m->device, (int64_t)m->wbytes,
                         (int64_t)m->wsbytes, m->graph_captures, m->graph_replays, m->poisoned ? 1 : 0,
                         (int64_t)m->debug};
  for (int i = 0; i < n && i < 10; ++i) info[i] = v[i];
  return JL_OK;
}

extern "C" int jl_set_debug(jl_model *m, uint32_t flags) {
  if (!m) return fail(JL_ERR_ARG, "model handle is NULL");
  if (flags & ~(uint32_t)(JL_DEBUG_SYNC | JL_DEBUG_REVERSE_BLOCKS | JL_DEBUG_SIMULATE_FAULT))
    return fail(JL_ERR_ARG, "unknown debug flag");
  m->debug = flags;
  return JL_OK;
}

extern "C" int jl_check_guards(jl_model *m) {
  if (int rc = usable(m)) return rc;
  DeviceGuard dg(m->device);
  JL_HIPM(hipDeviceSynchronize());
  uint8_t band[kGuardBytes];
  for (size_t i = 0; i < m->guards.size(); ++i) {
    JL_HIPM(hipMemcpy(band, m->ws + m->guards[i], kGuardBytes, hipMemcpyDeviceToHost));
    for (size_t k = 0; k < kGuardBytes; ++k)
      if (band[k] != kGuardByte) {
        const std::string piece = i < (size_t)kWorkspacePieces ? std::string("workspace buffer ") + kPieceNames[i]
                                                               : "metadata block " + std::to_string(i - kWorkspacePieces);
        return fail(JL_ERR_GUARD, "guard band after " + piece + " overwritten at byte " + std::to_string(k));
      }
  }
  return JL_OK;
}

// ---------------------------------------------------------------------------
// per-call planning and launch sequence
// ---------------------------------------------------------------------------

namespace {

struct Plan {
  int slot = 0;
  int B = 0, M = 0, T = 0;
  int n_work = 0, n_work_wide = 0;  // 64-query and 128-query attention items
  const int *d_so = nullptr, *d_mo = nullptr, *d_qt = nullptr, *d_mp = nullptr;
  const AttnWork *d_aw = nullptr, *d_aw_wide = nullptr, *d_mw = nullptr;
};

// Build the metadata in pinned memory and enqueue its upload.
// `dmeta_override`: device block to upload to instead of the handle's own
// (the allocation-free entry point's, in its static scratch).  Allocates
// nothing: the host-side vectors are the handle's, reserved at load.
// `pad64` / `pad128` > 0: pad the 64- and 128-query attention lists with empty
// items to exactly that many (a bucketed call; see work_capacity).
int upload_plan(jl_model *m, const int32_t *so, int32_t B, const int32_t *mp, int32_t M, const int32_t *qt,
                hipStream_t s, Plan &pl, bool to_graph_buffer = false, int *dmeta_override = nullptr, int pad64 = 0,
                int pad128 = 0) {
  pl.B = B;
  pl.M = M;
  pl.T = so[B];
  const int slot = m->next_slot;
  m->next_slot = (slot + 1) % jl_model::kMetaSlots;
  if (m->slot_pending[slot]) {
    JL_HIPM(hipEventSynchronize(m->slot_done[slot]));
    m->slot_pending[slot] = false;
  }
  pl.slot = slot;
  // Size of what follows, checked before anything is written: offsets,
  // marker counts, types and positions, then three lists of 8-int items --
  // 64- and 128-query attention items (each list at most half again its
  // item count plus 8 of empty padding) and one marker item per sequence.
  {
    size_t items64 = 0, items128 = 0;
    for (int b = 0; b < B; ++b) {
      const size_t len = (size_t)(so[b + 1] - so[b]);
      items64 += (len + 63) / 64;
      items128 += (len + 127) / 128;
    }
    const size_t need = (((size_t)(B + 1) * 2 + B + M + 7) & ~size_t(7)) +
                        8 * std::max(items64 + items64 / 2 + 8, (size_t)pad64) +
                        8 * std::max(items128 + items128 / 2 + 8, (size_t)pad128) + 8 * (size_t)B;
    if (need > m->meta_ints) return fail(JL_ERR_CAPACITY, "batch metadata exceeds the staging buffer");
  }
  int *h = m->host_meta[slot];
  int *dmeta = dmeta_override ? dmeta_override : to_graph_buffer ? m->gmeta : m->meta[slot];
  size_t o = 0;
  const size_t o_so = o;
  for (int b = 0; b <= B; ++b) h[o++] = so[b];
  const size_t o_mo = o;
  {
    int k = 0;
    for (int b = 0; b <= B; ++b) {
      while (k < M && mp[k] < so[b]) ++k;
      h[o++] = k;
    }
  }
  const size_t o_qt = o;
  for (int b = 0; b < B; ++b) h[o++] = qt[b];
  const size_t o_mp = o;
  for (int k = 0; k < M; ++k) h[o++] = mp[k];
  o = (o + 7) & ~size_t(7);
  // encoder / head-layer-1 work items, longest sequences first
  std::vector<int> &order = m->plan_order;  // capacity max_seqs >= B (reserved at load)
  order.resize(B);
  for (int b = 0; b < B; ++b) order[b] = b;
  std::sort(order.begin(), order.end(), [&](int a, int b) {  // stable: equal lengths keep their order
    const int la = so[a + 1] - so[a], lb = so[b + 1] - so[b];
    return la > lb || (la == lb && a < b);
  });
  // Work-groups go to the 8 XCDs round-robin by flattened index, and the
  // grid's x extent is a multiple of 8, so item x runs on XCD x % 8 for every
  // head.  Items are laid out per XCD: sequences, longest first, go whole to
  // the least loaded XCD (cost = keys read per item), a sequence costing more
  // than an eighth of the total in contiguous runs of about that cost; XCD c's
  // items sit at x = 8 k + c in order.  The query tiles of a sequence, which
  // read the same keys and values, then share one XCD's L2.  Shorter lists
  // are padded with empty items (n_q = 0); if padding would exceed half the
  // items, the plain order is used instead.
  auto work_list = [&](int tile, bool whole_seq, int &count) {
    auto cost_of = [&](int len) {
      return (double)(whole_seq ? len : std::min(len, tile + 2 * kHalfWindow));
    };
    double total = 0.0;
    int n_items = 0;
    for (int b = 0; b < B; ++b) {
      const int len = so[b + 1] - so[b];
      n_items += (len + tile - 1) / tile;
      total += ((len + tile - 1) / tile) * cost_of(len);
    }
    std::vector<AttnWork> *per = m->plan_per;  // each reserved for every item of a batch
    for (int c = 0; c < 8; ++c) per[c].clear();
    double load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const double cap = total / 8.0;
    auto least = [&]() {
      int c = 0;
      for (int i = 1; i < 8; ++i)
        if (load[i] < load[c]) c = i;
      return c;
    };
    for (int b : order) {
      const int start = so[b], len = so[b + 1] - so[b];
      const double item_cost = cost_of(len);
      const int items = (len + tile - 1) / tile;
      const int run = item_cost * items > cap ? std::max(1, (int)std::ceil(cap / item_cost)) : items;
      int c = least();
      for (int i = 0; i < items; ++i) {
        if (i % run == 0) c = least();
        const int q0 = i * tile;
        per[c].push_back(AttnWork{start + q0, std::min(tile, len - q0), start, len, q0, 0, 0, 0});
        load[c] += item_cost;
      }
    }
    size_t kmax = 0;
    for (int c = 0; c < 8; ++c) kmax = std::max(kmax, per[c].size());
    count = 0;
    if (8 * kmax <= (size_t)n_items + n_items / 2 + 8) {
      for (size_t k = 0; k < kmax; ++k)
        for (int c = 0; c < 8; ++c) {
          const AttnWork w = k < per[c].size() ? per[c][k] : AttnWork{0, 0, 0, 0, 0, 0, 0, 0};
          std::memcpy(h + o, &w, sizeof(w));
          o += 8;
          ++count;
        }
    } else {
      for (int b : order) {
        const int start = so[b], len = so[b + 1] - so[b];
        for (int q0 = 0; q0 < len; q0 += tile) {
          AttnWork w{start + q0, std::min(tile, len - q0), start, len, q0, 0, 0, 0};
          std::memcpy(h + o, &w, sizeof(w));
          o += 8;
          ++count;
        }
      }
    }
  };
  const size_t o_aw = o;
  int nw = 0, nw_wide = 0;
  auto pad_to = [&](int &count, int target) -> int {
    if (target <= 0) return JL_OK;
    if (count > target) return fail(JL_ERR_CAPACITY, "attention work list longer than its bucket's capacity");
    const AttnWork empty{0, 0, 0, 0, 0, 0, 0, 0};
    for (; count < target; ++count, o += 8) std::memcpy(h + o, &empty, sizeof(empty));
    return JL_OK;
  };
  work_list(64, false, nw);
  if (int rc = pad_to(nw, pad64)) return rc;
  const size_t o_aw_wide = o;
  work_list(128, true, nw_wide);
  if (int rc = pad_to(nw_wide, pad128)) return rc;
  const size_t o_mw = o;
  for (int b = 0; b < B; ++b) {
    const int first = h[o_mo + b], cnt = h[o_mo + b + 1] - first;
    AttnWork w{first, cnt, so[b], so[b + 1] - so[b], 0, 0, 0, 0};
    std::memcpy(h + o, &w, sizeof(w));
    o += 8;
  }
  JL_HIPM(hipMemcpyAsync(dmeta, h, o * 4, hipMemcpyHostToDevice, s));
  pl.n_work = nw;
  pl.n_work_wide = nw_wide;
  pl.d_aw_wide = (const AttnWork *)(dmeta + o_aw_wide);
  pl.d_so = dmeta + o_so;
  pl.d_mo = dmeta + o_mo;
  pl.d_qt = dmeta + o_qt;
  pl.d_mp = dmeta + o_mp;
  pl.d_aw = (const AttnWork *)(dmeta + o_aw);
  pl.d_mw = (const AttnWork *)(dmeta + o_mw);
  return JL_OK;
}

// After the last launch that reads the slot's metadata (always, even after an
// error, so that the slot is never left without a completion marker).
// JL_DEBUG_SIMULATE_FAULT: the call reports a memory fault here, as if the
// device had raised one (the enqueued work itself runs normally).
int finish_plan(jl_model *m, const Plan &pl, hipStream_t s, int rc) {
  const hipError_t e = hipEventRecord(m->slot_done[pl.slot], s);
  if (e == hipSuccess) {
    m->slot_pending[pl.slot] = true;
  } else if (rc == JL_OK) {
    rc = ::jl::device_error(m, e, "hipEventRecord(slot_done)");
    if (hipStreamSynchronize(s) != hipSuccess) return rc;
  }
  if (rc == JL_OK && (m->debug & JL_DEBUG_SIMULATE_FAULT)) {
    m->debug &= ~(uint32_t)JL_DEBUG_SIMULATE_FAULT;
    return ::jl::device_error(m, hipErrorIllegalAddress, "simulated device fault (JL_DEBUG_SIMULATE_FAULT)");
  }
  return rc;
}

hipEvent_t prof_event(jl_model *m) {
  if (m->ev_used == m->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    m->ev_pool.push_back(e);
  }
  return m->ev_pool[m->ev_used++];
}

struct Launch {
  jl_model *m;
  hipStream_t s;
  int cls;
  hipEvent_t a = nullptr;
  Launch(jl_model *m_, hipStream_t s_, int c) : m(m_), s(s_), cls(c) {
    if (m->prof && !m->prof_suspended && (m->prof_mask >> c & 1u)) {
      a = prof_event(m);
      if (a) (void)hipEventRecord(a, s);
    }
  }
  void done() {
    if (a) {
      hipEvent_t b = prof_event(m);
      if (b) {
        (void)hipEventRecord(b, s);
        m->prof_rec.push_back({cls, a, b});
      }
    }
  }
};

// One launch of kernel class `cls`.  JL_DEBUG_SYNC: wait for it and check
// the stream, so that an error is reported by the launch that caused it.
int after_launch(jl_model *m, hipStream_t s, int cls, hipError_t e) {
  static const char *const names[JL_K_NCLASS] = {"embed",   "qkv",       "attn_global", "attn_local", "outproj",
                                                 "mlp_in",  "mlp_out",   "head_gemm",   "head_attn",  "misc",
                                                 "ln",      "layer",     "head_layer"};
  if (e == hipSuccess && (m->debug & JL_DEBUG_SYNC)) {
    e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e == hipSuccess) return JL_OK;
  const std::string what = std::string("kernel class ") + names[cls];
  return ::jl::device_error(m, e, what.c_str());
}

#define JL_LAUNCH(cls, call)                                                          \
  do {                                                                                \
    Launch L_(m, s, cls);                                                             \
    hipError_t e_ = (call);                                                           \
    L_.done();                                                                        \
    if (int rc_ = after_launch(m, s, cls, e_)) return rc_;                            \
  } while (0)

// Sequence-wide attention takes 128-query work items (two 16-query sub-tiles
// per wave reuse every K/V fragment read from LDS) when they give at least
// one work-group per CU; fewer (short batches) leave CUs idle, and the
// 64-query items, each half the chain, finish sooner.  The +-64 window takes
// 64-query items: 3 key tiles per item, a shorter chain per work-group than
// the 4 of a 128-query item (measured no faster).
hipError_t attention(bool bf, AttnArgs at, const Plan &pl, bool whole_sequence, hipStream_t s) {
  constexpr int kCUs = 256;
  const bool wide = whole_sequence && (long)pl.n_work_wide * kHeads >= kCUs;
  at.work = wide ? pl.d_aw_wide : pl.d_aw;
  return launch_attention(bf, at, wide ? pl.n_work_wide : pl.n_work, wide ? 128 : 64, s);
}

// A = LayerNorm(x; gain, shift) for launch_ln_gemm (a.A: the fallback's bf16/FP32 rows).
GemmArgs with_ln(GemmArgs a, const float *x, const float *gain, const float *shift) {
  a.ln_x = x;
  a.ln_gain = gain;
  a.ln_shift = shift;
  return a;
}

GemmArgs gemm(const void *A, int lda, const void *W, int ldw, const float *bias, void *C, int ldc, int M, int N,
              int K) {
  GemmArgs a{};
  a.A = A;
  a.lda = lda;
  a.W = W;
  a.ldw = ldw;
  a.bias = bias;
  a.C = C;
  a.ldc = ldc;
  a.M = M;
  a.N = N;
  a.K = K;
  return a;
}

// Enqueue the forward pass up to `stop` (see jl_debug_hidden; 26 = logits).
//   x   FP32 residual stream [T, 384] (the head's h from the final LayerNorm on)
//   u   normalized GEMM operand [T, 384] (shares the attention-output buffer o)
//   qkv [T, 1152]; head layer 2 keeps keys|values there as [T, 768]
//   act [T, 1152] GEGLU output / [T, 1536] head FFN hidden
int run_forward(jl_model *m, const Workspace &w, const int32_t *ids, const Plan &pl, int stop, float *out,
                hipStream_t s) {
  const bool bf = m->bf16;
  const size_t es = m->esize;
  const int T = pl.T, M = pl.M, D = kWidth;
  char *u = w.o;
  // JL_DEBUG_REVERSE_BLOCKS: every kernel whose work-groups own tiles, row
  // blocks or work items takes them in reversed order
  const int rev = (m->debug & JL_DEBUG_REVERSE_BLOCKS) ? 1 : 0;
  auto launch_gemm_r = [rev](bool b, int e, GemmArgs a, hipStream_t st) {
    a.rev = rev;
    return launch_gemm(b, e, a, st);
  };
  auto launch_ln_gemm_r = [rev](bool b, int e, GemmArgs a, hipStream_t st) {
    a.rev = rev;
    return launch_ln_gemm(b, e, a, st);
  };
  auto copy_out = [&](const float *src, size_t rows) -> int {
    JL_HIPM(hipMemcpyAsync(out, src, rows * D * 4, hipMemcpyDeviceToDevice, s));
    return JL_OK;
  };
  const bool row_block = m->precision != JL_FP32 && T >= m->row_block_min_tokens;
  if (row_block) {  // the embedding kernel also computes the first layer's QKV
    EmbedArgs ea{};
    ea.ids = ids;
    ea.emb = m->emb;
    ea.gain = m->emb_norm;
    ea.seq_offsets = pl.d_so;
    ea.n_seqs = pl.B;
    ea.x = w.x;
    ea.pos = w.pos;
    ea.tok_seq = w.tok_seq;
    ea.Wqkv = (const __bf16 *)m->L[0].pWqkv;
    ea.rope_cos = m->rope_cos[layer_is_global(0)];
    ea.rope_sin = m->rope_sin[layer_is_global(0)];
    ea.qkv_out = (__bf16 *)w.qkv;
    ea.T = T;
    ea.rev = rev;
    JL_LAUNCH(JL_K_EMBED, launch_embed_qkv(ea, s));
  } else {
    JL_LAUNCH(JL_K_EMBED, launch_embed(ids, m->emb, m->emb_norm, T, pl.d_so, pl.B, w.x, w.pos, w.tok_seq, s));
  }
  if (stop == 0) return copy_out(w.x, T);

  AttnArgs at{};
  at.q = w.qkv;
  at.q_stride = 3 * D;
  at.k = w.qkv + D * es;
  at.v = w.qkv + 2 * D * es;
  at.kv_stride = 3 * D;
  at.o = w.o;
  at.o_stride = D;
  at.work = pl.d_aw;
  at.rev = rev;
  if (row_block) {
    // Row-block path: one attention launch and one layer launch per layer.
    for (int l = 0; l < kLayers; ++l) {
      const bool glob = layer_is_global(l);
      at.half_window = glob ? -1 : kHalfWindow;
      JL_LAUNCH(glob ? JL_K_ATTN_GLOBAL : JL_K_ATTN_LOCAL, attention(bf, at, pl, glob, s));
      LayerArgs la{};
      const LayerW &W = m->L[l];
      la.x = w.x;
      la.o = (const __bf16 *)w.o;
      la.Wo = (const __bf16 *)W.pWo;
      la.mlp_norm = W.mlp_norm;
      la.Wi = (const __bf16 *)W.pWi;
      la.Wout = (const __bf16 *)W.pWout;
      la.pos = w.pos;
      la.qkv_out = (__bf16 *)w.qkv;
      la.T = T;
      la.rev = rev;
      if (W.pWi8) {  // JL_FP8: e4m3 W_i and next QKV
        la.Wi8 = (const uint8_t *)W.pWi8;
        la.si = W.si;
      }
      if (l + 1 < kLayers && stop != l + 1) {
        const LayerW &N = m->L[l + 1];
        la.attn_norm_next = N.attn_norm;
        la.Wqkv_next = (const __bf16 *)N.pWqkv;
        la.Wqkv8_next = (const uint8_t *)N.pWqkv8;
        la.sqkv_next = N.sqkv;
        la.rope_cos_next = m->rope_cos[layer_is_global(l + 1)];
        la.rope_sin_next = m->rope_sin[layer_is_global(l + 1)];
      } else if (l + 1 == kLayers && stop != kLayers) {
        la.final_norm = m->final_norm;
        la.type_rows = m->type_rows;
        la.qtype = pl.d_qt;
        la.tok_seq = w.tok_seq;
        if (stop != kLayers + 1) {  // continue into the head's first attention input
          const HeadW &H = m->H[0];
          la.attn_norm_next = H.n1_w;
          la.attn_shift_next = H.n1_b;
          la.Wqkv_next = (const __bf16 *)H.pIn;
          la.qkv_bias_next = H.in_b;
        }
      }
      JL_LAUNCH(JL_K_LAYER, launch_layer(la, s));
      if (stop == l + 1) return copy_out(w.x, T);
    }
  } else {
  for (int l = 0; l < kLayers; ++l) {
    const LayerW &W = m->L[l];
    const bool glob = layer_is_global(l);
    GemmArgs q = with_ln(gemm(u, D, W.Wqkv8 ? W.Wqkv8 : W.Wqkv, D, nullptr, w.qkv, 3 * D, T, 3 * D, D), w.x,
                         W.attn_norm, nullptr);
    q.w_scale = W.sqkv;  // e4m3 products (JL_FP8), else nullptr
    q.rope_cos = m->rope_cos[glob];
    q.rope_sin = m->rope_sin[glob];
    q.pos = w.pos;
    q.rope_cols = 2 * D;
    JL_LAUNCH(JL_K_QKV, launch_ln_gemm_r(bf, E_STORE, q, s));
    at.half_window = glob ? -1 : kHalfWindow;
    JL_LAUNCH(glob ? JL_K_ATTN_GLOBAL : JL_K_ATTN_LOCAL, attention(bf, at, pl, glob, s));
    JL_LAUNCH(JL_K_OUTPROJ, launch_gemm_r(bf, E_RESID, gemm(w.o, D, W.Wo, D, nullptr, w.x, D, T, D, D), s));
    GemmArgs wi = with_ln(gemm(u, D, W.Wi8 ? W.Wi8 : W.Wi, D, nullptr, w.act, kGeglu, T, 2 * kGeglu, D), w.x,
                          W.mlp_norm, nullptr);
    wi.w_scale = W.si;
    JL_LAUNCH(JL_K_MLP_IN, launch_ln_gemm_r(bf, E_GEGLU, wi, s));
    JL_LAUNCH(JL_K_MLP_OUT,
              launch_gemm_r(bf, E_RESID, gemm(w.act, kGeglu, W.Wout, kGeglu, nullptr, w.x, D, T, D, kGeglu), s));
    if (stop == l + 1) return copy_out(w.x, T);
  }
  // head input: final LayerNorm + type row (in place)
  JL_LAUNCH(JL_K_MISC, launch_final_ln_type(w.x, m->final_norm, m->type_rows, pl.d_qt, w.tok_seq, T, w.x, s));
  }
  if (stop == 23) return copy_out(w.x, T);

  // head layer 1 over every token (row-block path: its LayerNorm and
  // in-projection ran in the last encoder layer's kernel; everything after
  // its attention, with the second layer's keys and values, in one kernel)
  char *kv = w.qkv;  // head layer 2's keys and values, [T, 768]: k then v
  {
    const HeadW &H = m->H[0];
    if (!row_block) {
      JL_LAUNCH(JL_K_HEAD_GEMM,
                launch_ln_gemm_r(bf, E_STORE,
                               with_ln(gemm(u, D, H.in_w, D, H.in_b, w.qkv, 3 * D, T, 3 * D, D), w.x, H.n1_w, H.n1_b),
                               s));
    }
    at.half_window = -1;
    JL_LAUNCH(JL_K_HEAD_ATTN, attention(bf, at, pl, true, s));
    if (row_block) {
      const HeadW &N = m->H[1];
      HeadArgs ha{};
      ha.x = w.x;
      ha.o = (const __bf16 *)w.o;
      ha.Wo = (const __bf16 *)H.pOut;
      ha.bo = H.out_b;
      ha.n2_w = H.n2_w;
      ha.n2_b = H.n2_b;
      ha.W1 = (const __bf16 *)H.pL1;
      ha.b1 = H.l1_b;
      ha.W2 = (const __bf16 *)H.pL2;
      ha.b2 = H.l2_b;
      if (stop != 24) {
        ha.nk_w = N.n1_w;
        ha.nk_b = N.n1_b;
        ha.Wkv = (const __bf16 *)N.pKV;
        ha.bkv = N.in_b + D;
        ha.kv_out = (__bf16 *)kv;
      }
      ha.T = T;
      ha.rev = rev;
      JL_LAUNCH(JL_K_HEAD_LAYER, launch_head_layer(ha, s));
    } else {
      JL_LAUNCH(JL_K_HEAD_GEMM, launch_gemm_r(bf, E_RESID, gemm(w.o, D, H.out_w, D, H.out_b, w.x, D, T, D, D), s));
      JL_LAUNCH(JL_K_HEAD_GEMM,
                launch_ln_gemm_r(bf, E_RELU,
                               with_ln(gemm(u, D, H.l1_w, D, H.l1_b, w.act, kHeadFfn, T, kHeadFfn, D), w.x, H.n2_w,
                                       H.n2_b),
                               s));
      JL_LAUNCH(JL_K_HEAD_GEMM, launch_gemm_r(bf, E_RESID,
                                            gemm(w.act, kHeadFfn, H.l2_w, kHeadFfn, H.l2_b, w.x, D, T, D, kHeadFfn),
                                            s));
    }
  }
  if (stop == 24) return copy_out(w.x, T);

  // head layer 2: keys and values for every token, the rest at marker rows only
  {
    const HeadW &H = m->H[1];
    if (!row_block) {
      JL_LAUNCH(JL_K_HEAD_GEMM,
                launch_ln_gemm_r(bf, E_STORE,
                               with_ln(gemm(u, D, (const char *)H.in_w + (size_t)D * D * es, D, H.in_b + D, kv, 2 * D,
                                            T, 2 * D, D),
                                       w.x, H.n1_w, H.n1_b),
                               s));
    }
    JL_LAUNCH(JL_K_MISC, launch_gather_rows(w.x, pl.d_mp, M, w.z, w.score_cnt, s));
    char *um = w.om;  // normalized marker rows, then the marker attention output
    JL_LAUNCH(JL_K_HEAD_GEMM,
              launch_ln_gemm_r(bf, E_STORE, with_ln(gemm(um, D, H.in_w, D, H.in_b, w.qm, D, M, D, D), w.z, H.n1_w, H.n1_b),
                             s));
    AttnArgs mk{};
    mk.q = w.qm;
    mk.q_stride = D;
    mk.k = kv;
    mk.v = kv + D * es;
    mk.kv_stride = 2 * D;
    mk.o = w.om;
    mk.o_stride = D;
    mk.work = pl.d_mw;
    mk.half_window = -1;
    mk.rev = rev;
    JL_LAUNCH(JL_K_HEAD_ATTN, launch_attention(bf, mk, pl.B, 64, s));
    JL_LAUNCH(JL_K_HEAD_GEMM, launch_gemm_r(bf, E_RESID, gemm(w.om, D, H.out_w, D, H.out_b, w.z, D, M, D, D), s));
    JL_LAUNCH(JL_K_HEAD_GEMM,
              launch_ln_gemm_r(bf, E_RELU,
                             with_ln(gemm(um, D, H.l1_w, D, H.l1_b, w.actm, kHeadFfn, M, kHeadFfn, D), w.z, H.n2_w,
                                     H.n2_b),
                             s));
    JL_LAUNCH(JL_K_HEAD_GEMM, launch_gemm_r(bf, E_RESID,
                                          gemm(w.actm, kHeadFfn, H.l2_w, kHeadFfn, H.l2_b, w.z, D, M, D, kHeadFfn),
                                          s));
  }
  if (stop == 25) return copy_out(w.z, M);

  // scorer (FP32 in every mode), one launch
  JL_LAUNCH(JL_K_MISC, launch_score(w.z, m->sc_nw, m->sc_nb, m->sc_w1, m->sc_b1, m->sc_w2, m->sc_b2, M, w.score_part,
                                    w.score_cnt, out, rev, s));
  return JL_OK;
}

// Replay (capturing on first use) the forward pass of this batch shape.
int forward_graph(jl_model *m, const int32_t *ids, const Plan &pl, float *out, hipStream_t s) {
  const bool row_block = m->precision != JL_FP32 && pl.T >= m->row_block_min_tokens;
  jl_model::GraphEntry *hit = nullptr;
  for (auto &g : m->graphs)
    if (g.T == pl.T && g.B == pl.B && g.M == pl.M && g.n_work == pl.n_work && g.n_work_wide == pl.n_work_wide &&
        g.row_block == row_block && g.ids == ids && g.out == out) {
      hit = &g;
      break;
    }
  if (!hit) {
    if ((int)m->graphs.size() >= m->graph_cap) {  // evict the least recently used
      size_t lru = 0;
      for (size_t i = 1; i < m->graphs.size(); ++i)
        if (m->graphs[i].last_use < m->graphs[lru].last_use) lru = i;
      (void)hipGraphExecDestroy(m->graphs[lru].exec);
      (void)hipGraphDestroy(m->graphs[lru].graph);
      m->graphs.erase(m->graphs.begin() + lru);
    }
    JL_HIPM(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    const int rc = run_forward(m, m->w, ids, pl, 26, out, s);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (rc != JL_OK) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess) return ::jl::device_error(m, e, "graph capture");
    hipGraphExec_t ge = nullptr;
    const hipError_t ei = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
      (void)hipGraphDestroy(g);
      return ::jl::device_error(m, ei, "graph instantiation");
    }
    m->graphs.push_back({pl.T, pl.B, pl.M, pl.n_work, pl.n_work_wide, row_block, ids, out, g, ge, 0});
    hit = &m->graphs.back();
    ++m->graph_captures;
  } else {
    ++m->graph_replays;
  }
  hit->last_use = ++m->graph_clock;
  JL_HIPM(hipGraphLaunch(hit->exec, s));
  return JL_OK;
}

}  // namespace

int jl::set_error(int code, const char *msg) { return fail(code, msg); }

extern "C" int jl_set_graph_cache(jl_model *m, int max_graphs) {
  if (!m) return fail(JL_ERR_ARG, "model handle is NULL");
  if (max_graphs < 0 || max_graphs > 64) return fail(JL_ERR_ARG, "max_graphs must be in 0..64");
  DeviceGuard dg(m->device);
  for (auto &g : m->graphs) {
    (void)hipGraphExecDestroy(g.exec);
    (void)hipGraphDestroy(g.graph);
  }
  m->graphs.clear();
  m->graph_cap = max_graphs;
  return JL_OK;
}

extern "C" int jl_forward(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets, int32_t n_seqs,
                          const int32_t *mask_positions, int32_t n_markers, const int32_t *qtype, float *logits_dev,
                          void *stream) {
  if (int rc = usable(m)) return rc;
  if (int rc = jl_validate(seq_offsets, n_seqs, mask_positions, n_markers, qtype, m->max_tokens, m->max_markers))
    return rc;
  if (n_seqs == 0) return JL_OK;
  if (!ids_dev || !logits_dev) return fail(JL_ERR_ARG, "ids_dev and logits_dev must not be NULL");
  DeviceGuard dg(m->device);
  hipStream_t s = (hipStream_t)stream;
  Plan pl;
  // graphs need a capturable stream, no per-launch timer events and no
  // debugging switches (per-launch synchronization cannot be captured)
  const bool use_graph = m->graph_cap > 0 && s != nullptr && !m->prof && !m->debug;
  if (int rc = upload_plan(m, seq_offsets, n_seqs, mask_positions, n_markers, qtype, s, pl, use_graph)) return rc;
  if (!use_graph) return finish_plan(m, pl, s, run_forward(m, m->w, ids_dev, pl, 26, logits_dev, s));
  return finish_plan(m, pl, s, forward_graph(m, ids_dev, pl, logits_dev, s));
}

// ---------------------------------------------------------------------------
// allocation-free forward: the workspace in a static device array
// ---------------------------------------------------------------------------

extern "C" int jl_forward_static(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets, int32_t n_seqs,
                                 const int32_t *mask_positions, int32_t n_markers, const int32_t *qtype,
                                 float *logits_dev, void *stream) {
  if (int rc = usable(m)) return rc;
  const int64_t max_t = std::min(m->max_tokens, kStaticMaxTokens), max_m = std::min(m->max_markers, kStaticMaxMarkers);
  if (int rc = jl_validate(seq_offsets, n_seqs, mask_positions, n_markers, qtype, max_t, max_m)) {
    if (rc == JL_ERR_CAPACITY)
      g_err = "jl_forward_static takes at most " + std::to_string(max_t) + " tokens and " + std::to_string(max_m) +
              " markers (static workspace of 2,048 tokens / 256 markers, and the handle's capacity): " + g_err;
    return rc;
  }
  if (n_seqs == 0) return JL_OK;
  if (!ids_dev || !logits_dev) return fail(JL_ERR_ARG, "ids_dev and logits_dev must not be NULL");
  char *base = m->device < 64 ? (char *)g_scratch_dev[m->device] : nullptr;
  if (!base) return fail(JL_ERR_DEVICE, "no static workspace on this device");
  DeviceGuard dg(m->device);
  Workspace w;
  int *dmeta = nullptr;
  layout_workspace(base, kStaticMaxTokens, kStaticMaxMarkers, m->esize, kStaticMetaInts, &w, &dmeta, 1);
  hipStream_t s = (hipStream_t)stream;
  Plan pl;
  if (int rc = upload_plan(m, seq_offsets, n_seqs, mask_positions, n_markers, qtype, s, pl, false, dmeta)) return rc;
  m->prof_suspended = true;  // timer events would have to be created on demand
  const int rc = run_forward(m, w, ids_dev, pl, 26, logits_dev, s);
  m->prof_suspended = false;
  return finish_plan(m, pl, s, rc);
}

int jl::forward_bucketed(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets, int32_t n_seqs,
                         const int32_t *mask_positions, int32_t n_markers, const int32_t *qtype, float *logits_dev,
                         hipStream_t s) {
  if (m->graph_cap <= 0 || s == nullptr || m->prof || m->debug || m->poisoned)
    return jl_forward(m, ids_dev, seq_offsets, n_seqs, mask_positions, n_markers, qtype, logits_dev, s);
  if (int rc = jl_validate(seq_offsets, n_seqs, mask_positions, n_markers, qtype, m->max_tokens, m->max_markers))
    return rc;
  if (n_seqs == 0) return JL_OK;
  DeviceGuard dg(m->device);
  const int64_t T = seq_offsets[n_seqs];
  Plan pl;
  if (int rc = upload_plan(m, seq_offsets, n_seqs, mask_positions, n_markers, qtype, s, pl, true, nullptr,
                           work_capacity(T, n_seqs, 64), work_capacity(T, n_seqs, 128)))
    return rc;
  return finish_plan(m, pl, s, forward_graph(m, ids_dev, pl, logits_dev, s));
}

int jl::model_graph_cap(const jl_model *m) { return m->graph_cap; }

extern "C" int jl_debug_hidden(jl_model *m, const int32_t *ids_dev, const int32_t *seq_offsets, int32_t n_seqs,
                               const int32_t *mask_positions, int32_t n_markers, const int32_t *qtype, int32_t stage,
                               float *out_dev, void *stream) {
  if (int rc = usable(m)) return rc;
  if (stage < 0 || stage > 25) return fail(JL_ERR_ARG, "stage must be in 0..25");
  if (int rc = jl_validate(seq_offsets, n_seqs, mask_positions, n_markers, qtype, m->max_tokens, m->max_markers))
    return rc;
  if (n_seqs == 0) return JL_OK;
  if (!ids_dev || !out_dev) return fail(JL_ERR_ARG, "ids_dev and out_dev must not be NULL");
  DeviceGuard dg(m->device);
  hipStream_t s = (hipStream_t)stream;
  Plan pl;
  if (int rc = upload_plan(m, seq_offsets, n_seqs, mask_positions, n_markers, qtype, s, pl)) return rc;
  return finish_plan(m, pl, s, run_forward(m, m->w, ids_dev, pl, stage, out_dev, s));
}

extern "C" int jl_probs(jl_model *m, const float *logits_dev, const int32_t *seq_offsets, int32_t n_seqs,
                        const int32_t *mask_positions, int32_t n_markers, const int32_t *qtype, float *probs_dev,
                        float *answer_dev, int32_t *argmax_dev, float *maxprob_dev, void *stream) {
  if (int rc = usable(m)) return rc;
  if (int rc = jl_validate(seq_offsets, n_seqs, mask_positions, n_markers, qtype, m->max_tokens, m->max_markers))
    return rc;
  if (n_seqs == 0) return JL_OK;
  if (!logits_dev) return fail(JL_ERR_ARG, "logits_dev must not be NULL");
  DeviceGuard dg(m->device);
  hipStream_t s = (hipStream_t)stream;
  Plan pl;
  if (int rc = upload_plan(m, seq_offsets, n_seqs, mask_positions, n_markers, qtype, s, pl)) return rc;
  auto launch = [&]() -> int {
    JL_LAUNCH(JL_K_MISC, launch_probs(logits_dev, pl.d_mo, pl.d_qt, n_seqs, probs_dev, answer_dev, argmax_dev,
                                      maxprob_dev, s));
    return JL_OK;
  };
  return finish_plan(m, pl, s, launch());
}

extern "C" int jl_profile(jl_model *m, int enable, uint32_t class_mask) {
  if (!m) return fail(JL_ERR_ARG, "model handle is NULL");
  if (enable < 0 || enable > 2) return fail(JL_ERR_ARG, "enable must be 0, 1 or 2");
  m->prof = enable != 0;
  m->prof_mask = class_mask;
  if (enable == 1) {
    m->prof_rec.clear();
    m->ev_used = 0;
  }
  return JL_OK;
}

extern "C" int jl_profile_read(jl_model *m, int kernel_class, double *total_ms, int64_t *launches) {
  if (int rc = usable(m)) return rc;
  if (!total_ms || !launches) return fail(JL_ERR_ARG, "NULL argument");
  if (kernel_class < 0 || kernel_class >= JL_K_NCLASS) return fail(JL_ERR_ARG, "bad kernel class");
  DeviceGuard dg(m->device);
  double tot = 0.0;
  int64_t n = 0;
  for (const ProfRec &r : m->prof_rec) {
    if (r.cls != kernel_class) continue;
    JL_HIPM(hipEventSynchronize(r.b));
    float ms = 0.f;
    JL_HIPM(hipEventElapsedTime(&ms, r.a, r.b));
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return JL_OK;
}
