// Serving front of libjl: many independent requests in, their answers out.
//
// The pages' runtimes serve single requests or small batches; here a host
// thread packs a queue of ragged requests into micro-batches and keeps
// several of them in flight on one GPU:
//  * requests are ordered by length, longest first (a stable sort), and
//    packed greedily into micro-batches under a token budget and each
//    handle's marker and sequence capacity, so a micro-batch holds requests
//    of similar length;
//  * micro-batches go round-robin to one or more model handles that share
//    the weights (jl_share), each with its own workspace, stream, device
//    buffers and pinned staging, so one batch's upload, compute and
//    download overlap the next batch's packing and the other streams'
//    compute;
//  * results land in the caller's arrays in request order.
// Every step of a micro-batch is jl_forward + jl_probs, so a request's logits
// equal those of a jl_forward over a batch packed the same way.
#include "jl.h"
#include "jl_internal.h"

#include <algorithm>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

namespace jl {

// One handle's serving resources, made on the first jl_serve that uses it.
struct ServeState {
  jl_model *model = nullptr;     // the handle this state belongs to
  int device = 0;
  hipStream_t stream = nullptr;
  hipEvent_t done = nullptr;
  int32_t *d_ids = nullptr;      // [max_tokens]
  float *d_out = nullptr;        // logits, probs [max_markers]; answer, maxprob [max_seqs]
  int32_t *d_argmax = nullptr;   // [max_seqs]
  int32_t *h_ids = nullptr;      // pinned [max_tokens]
  float *h_out = nullptr;        // pinned, as d_out
  int32_t *h_argmax = nullptr;   // pinned [max_seqs]
  int64_t max_tokens = 0, max_markers = 0, max_seqs = 0;
  // the micro-batch in flight (scattered into the caller's arrays on completion)
  bool busy = false;
  std::vector<int32_t> reqs;     // requests of the batch, in batch order
};

void free_serve_state(ServeState *st) {
  if (!st) return;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(st->device);
  if (st->stream) (void)hipStreamSynchronize(st->stream);
  if (st->done) (void)hipEventDestroy(st->done);
  if (st->stream) (void)hipStreamDestroy(st->stream);
  if (st->d_ids) (void)hipFree(st->d_ids);
  if (st->d_out) (void)hipFree(st->d_out);
  if (st->d_argmax) (void)hipFree(st->d_argmax);
  if (st->h_ids) (void)hipHostFree(st->h_ids);
  if (st->h_out) (void)hipHostFree(st->h_out);
  if (st->h_argmax) (void)hipHostFree(st->h_argmax);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete st;
}

}  // namespace jl

using namespace jl;

namespace {

int serve_fail(int code, const std::string &msg) { return set_error(code, msg.c_str()); }

ServeState *serve_state(jl_model *m, int *rc) {
  ServeState *&st = model_serve_state(m);
  if (st) return st;
  ServeState *s = new ServeState();
  s->model = m;
  s->device = model_device(m);
  s->max_tokens = model_max_tokens(m);
  s->max_markers = model_max_markers(m);
  s->max_seqs = std::min<int64_t>(s->max_tokens, s->max_markers / 2);
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(s->device);
  const size_t out_floats = 2 * (size_t)s->max_markers + 2 * (size_t)s->max_seqs;
  bool ok = hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&s->done, hipEventDisableTiming) == hipSuccess &&
            hipMalloc((void **)&s->d_ids, s->max_tokens * 4) == hipSuccess &&
            hipMalloc((void **)&s->d_out, out_floats * 4) == hipSuccess &&
            hipMalloc((void **)&s->d_argmax, s->max_seqs * 4) == hipSuccess &&
            hipHostMalloc((void **)&s->h_ids, s->max_tokens * 4, hipHostMallocDefault) == hipSuccess &&
            hipHostMalloc((void **)&s->h_out, out_floats * 4, hipHostMallocDefault) == hipSuccess &&
            hipHostMalloc((void **)&s->h_argmax, s->max_seqs * 4, hipHostMallocDefault) == hipSuccess;
  if (prev >= 0) (void)hipSetDevice(prev);
  if (!ok) {
    free_serve_state(s);
    *rc = serve_fail(JL_ERR_OOM, "cannot allocate the serving stream and buffers");
    return nullptr;
  }
  st = s;
  return s;
}

// Pad a micro-batch (ids in `h_ids`, offsets `so`, marker positions `mp`,
// types `qt`) to its shape bucket with filler questions: B sequences to
// B_b = ceil((B + 2) / 8) * 8 (F = B_b - B fillers, 2..9), M markers to
// M_b = ceil((M + 2F) / 32) * 32 (each filler 2..20 of them), T tokens to
// T_b = ceil((T + 21F) / 2048) * 2048 (each filler at least one token more
// than its markers).  Filler tokens are id 0, its markers its first
// positions after the first, its type choice.
void bucket_pad(int32_t *h_ids, std::vector<int32_t> &so, std::vector<int32_t> &mp, std::vector<int32_t> &qt) {
  const int64_t B = (int64_t)qt.size(), M = (int64_t)mp.size(), T = so.back();
  const int64_t Bb = (B + 2 + 7) / 8 * 8, F = Bb - B;
  const int64_t Mb = (M + 2 * F + 31) / 32 * 32, Tb = (T + 21 * F + 2047) / 2048 * 2048;
  const int64_t E = Mb - M, R = Tb - T;
  for (int64_t f = 0; f < F; ++f) {
    // markers: 2 each, the rest dealt one by one (E - 2F <= 31 <= 18 F)
    const int64_t extra = E - 2 * F;
    const int64_t k = 2 + extra / F + (f < extra % F ? 1 : 0);
    const int64_t len = R / F + (f < R % F ? 1 : 0);  // >= 21 > k
    const int32_t start = so.back();
    for (int64_t i = 0; i < len; ++i) h_ids[start + i] = 0;
    for (int64_t i = 0; i < k; ++i) mp.push_back(start + 1 + (int32_t)i);
    qt.push_back(JL_CHOICE);
    so.push_back(start + (int32_t)len);
  }
}

}  // namespace

int jl::handle_buffers(jl_model *m, HandleBuffers *out) {
  int rc = JL_OK;
  ServeState *st = serve_state(m, &rc);
  if (!st) return rc;
  *out = HandleBuffers{st->d_ids, st->h_ids, st->d_out, st->h_out, st->max_tokens, st->max_markers};
  return JL_OK;
}

static int jl_serve_plan_impl(int32_t n_requests, const int64_t *id_offsets, const int64_t *mask_offsets,
                             int64_t max_batch_tokens, int64_t max_batch_markers, int64_t max_batch_seqs,
                             int32_t *order, int32_t *batch_of, int32_t *n_batches) {
  if (n_requests < 0 || (n_requests > 0 && (!id_offsets || !mask_offsets || !order || !batch_of)) || !n_batches)
    return serve_fail(JL_ERR_ARG, "NULL argument or negative request count");
  if (max_batch_tokens < 1 || max_batch_markers < 2 || max_batch_seqs < 1)
    return serve_fail(JL_ERR_ARG, "batch limits must be positive (at least 2 markers)");
  std::vector<int64_t> len(n_requests), mk(n_requests);
  for (int32_t r = 0; r < n_requests; ++r) {
    len[r] = id_offsets[r + 1] - id_offsets[r];
    mk[r] = mask_offsets[r + 1] - mask_offsets[r];
    if (len[r] < 1 || mk[r] < 0) return serve_fail(JL_ERR_ARG, "request " + std::to_string(r) + ": bad offsets");
    if (len[r] > max_batch_tokens || mk[r] > max_batch_markers)
      return serve_fail(JL_ERR_LENGTH, "request " + std::to_string(r) + " exceeds the micro-batch capacity");
  }
  std::vector<int32_t> idx(n_requests);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return len[a] > len[b]; });
  int32_t nb = 0;
  int64_t bt = 0, bm = 0, bs = 0;
  for (int32_t i = 0; i < n_requests; ++i) {
    const int32_t r = idx[i];
    if (bs > 0 && (bt + len[r] > max_batch_tokens || bm + mk[r] > max_batch_markers || bs + 1 > max_batch_seqs)) {
      ++nb;
      bt = bm = bs = 0;
    }
    bt += len[r];
    bm += mk[r];
    ++bs;
    order[i] = r;
    batch_of[r] = nb;
  }
  *n_batches = n_requests > 0 ? nb + 1 : 0;
  return JL_OK;
}

extern "C" int jl_serve_plan(int32_t n_requests, const int64_t *id_offsets, const int64_t *mask_offsets,
                             int64_t max_batch_tokens, int64_t max_batch_markers, int64_t max_batch_seqs,
                             int32_t *order, int32_t *batch_of, int32_t *n_batches) {
  JL_CATCH_ALL(jl_serve_plan_impl(n_requests, id_offsets, mask_offsets, max_batch_tokens, max_batch_markers, max_batch_seqs, order,
               batch_of, n_batches));
}

static int jl_serve_impl(jl_model *const *models, int32_t n_models, int32_t n_requests, const int32_t *ids,
                        const int64_t *id_offsets, const int32_t *mask_positions, const int64_t *mask_offsets,
                        const int32_t *qtype, int64_t max_batch_tokens, float *logits, float *probs, float *answer,
                        int32_t *argmax, float *maxprob, int32_t *n_batches) {
  if (!models || n_models < 1 || n_models > 16) return serve_fail(JL_ERR_ARG, "need 1..16 model handles");
  for (int32_t k = 0; k < n_models; ++k)
    if (int rc = model_check(models[k])) return rc;
  if (n_requests < 0) return serve_fail(JL_ERR_ARG, "negative request count");
  if (n_requests == 0) {
    if (n_batches) *n_batches = 0;
    return JL_OK;
  }
  if (!ids || !id_offsets || !mask_positions || !mask_offsets || !qtype || !logits || !probs || !answer || !argmax ||
      !maxprob)
    return serve_fail(JL_ERR_ARG, "NULL argument");
  if (id_offsets[0] != 0 || mask_offsets[0] != 0) return serve_fail(JL_ERR_ARG, "offsets must start at 0");
  // every request on its own first: a rejected call computes nothing
  int64_t cap_t = max_batch_tokens, cap_m = INT64_MAX, cap_s = INT64_MAX;
  for (int32_t k = 0; k < n_models; ++k) {
    cap_t = std::min(cap_t, model_max_tokens(models[k]));
    cap_m = std::min(cap_m, model_max_markers(models[k]));
    cap_s = std::min(cap_s, std::min(model_max_tokens(models[k]), model_max_markers(models[k]) / 2));
  }
  for (int32_t r = 0; r < n_requests; ++r) {
    const int64_t L = id_offsets[r + 1] - id_offsets[r], M = mask_offsets[r + 1] - mask_offsets[r];
    if (L < 1 || L > kMaxSeq || M < 0 || M > 64)
      return serve_fail(JL_ERR_LENGTH, "request " + std::to_string(r) + ": length or marker count out of range");
    const int32_t so[2] = {0, (int32_t)L};
    if (int rc = jl_validate(so, 1, mask_positions + mask_offsets[r], (int32_t)M, qtype + r, L, M > 1 ? M : 2))
      return serve_fail(rc, "request " + std::to_string(r) + ": " + jl_last_error());
  }
  // Graph mode: micro-batches padded to shape buckets (bucket_pad below), so
  // the plan leaves the padding's headroom: at most 9 fillers, 2,047 + 189
  // tokens and 18 + 31 markers.
  bool bucketed = true;
  for (int32_t k = 0; k < n_models; ++k) bucketed = bucketed && model_graph_cap(models[k]) > 0;
  constexpr int64_t kFill = 9, kPadTokens = 2047 + 21 * kFill, kPadMarkers = 2 * kFill + 31;
  if (bucketed && (cap_t <= kPadTokens + kMaxSeq || cap_m <= kPadMarkers + 64 || cap_s <= kFill + 1))
    bucketed = false;  // too small a handle to leave the headroom
  const int64_t plan_t = bucketed ? cap_t - kPadTokens : cap_t, plan_m = bucketed ? cap_m - kPadMarkers : cap_m;
  const int64_t plan_s = bucketed ? cap_s - kFill : cap_s;
  std::vector<int32_t> order(n_requests), batch_of(n_requests);
  int32_t nb = 0;
  if (int rc = jl_serve_plan(n_requests, id_offsets, mask_offsets, plan_t, plan_m, plan_s, order.data(),
                             batch_of.data(), &nb))
    return rc;
  std::vector<ServeState *> st(n_models);
  for (int32_t k = 0; k < n_models; ++k) {
    int rc = JL_OK;
    st[k] = serve_state(models[k], &rc);
    if (!st[k]) return rc;
  }
  int prev = -1;
  (void)hipGetDevice(&prev);
  // a finished micro-batch into the caller's arrays
  auto retire = [&](ServeState *s) -> int {
    if (!s->busy) return JL_OK;
    s->busy = false;
    hipError_t e = hipSetDevice(s->device);
    if (e == hipSuccess) e = hipEventSynchronize(s->done);
    if (e != hipSuccess) return device_error(s->model, e, "serving stream");
    const float *h_logits = s->h_out, *h_probs = s->h_out + s->max_markers;
    const float *h_answer = s->h_out + 2 * s->max_markers, *h_maxp = h_answer + s->max_seqs;
    int64_t k = 0;
    for (size_t b = 0; b < s->reqs.size(); ++b) {
      const int32_t r = s->reqs[b];
      const int64_t m0 = mask_offsets[r], M = mask_offsets[r + 1] - m0;
      std::memcpy(logits + m0, h_logits + k, M * 4);
      std::memcpy(probs + m0, h_probs + k, M * 4);
      k += M;
      answer[r] = h_answer[b];
      maxprob[r] = h_maxp[b];
      argmax[r] = s->h_argmax[b];
    }
    return JL_OK;
  };
  int rc = JL_OK;
  std::vector<int32_t> so, mp, qt;
  size_t next = 0;
  for (int32_t bi = 0; bi < nb && rc == JL_OK; ++bi) {
    ServeState *s = st[bi % n_models];
    jl_model *m = models[bi % n_models];
    if ((rc = retire(s)) != JL_OK) break;  // its staging buffers are ours again
    // pack this micro-batch
    s->reqs.clear();
    so.assign(1, 0);
    mp.clear();
    qt.clear();
    while (next < order.size() && batch_of[order[next]] == bi) {
      const int32_t r = order[next++];
      const int64_t i0 = id_offsets[r], L = id_offsets[r + 1] - i0;
      std::memcpy(s->h_ids + so.back(), ids + i0, L * 4);
      for (int64_t j = mask_offsets[r]; j < mask_offsets[r + 1]; ++j) mp.push_back(so.back() + mask_positions[j]);
      qt.push_back(qtype[r]);
      so.push_back(so.back() + (int32_t)L);
      s->reqs.push_back(r);
    }
    const int32_t B = (int32_t)qt.size(), M = (int32_t)mp.size(), T = so.back();
    if (bucketed) bucket_pad(s->h_ids, so, mp, qt);  // fillers after the requests
    const int32_t Tp = so.back();
    {
      hipError_t e = hipSetDevice(s->device);
      if (e == hipSuccess) e = hipMemcpyAsync(s->d_ids, s->h_ids, (size_t)Tp * 4, hipMemcpyHostToDevice, s->stream);
      if (e != hipSuccess) {
        rc = device_error(m, e, "id upload");
        break;
      }
    }
    float *d_logits = s->d_out, *d_probs = s->d_out + s->max_markers;
    float *d_answer = s->d_out + 2 * s->max_markers, *d_maxp = d_answer + s->max_seqs;
    if (bucketed) {
      rc = forward_bucketed(m, s->d_ids, so.data(), (int32_t)qt.size(), mp.data(), (int32_t)mp.size(), qt.data(),
                            d_logits, s->stream);
      // the read-offs of the requests only (the fillers come after them)
      so.resize(B + 1);
      mp.resize(M);
      qt.resize(B);
    } else {
      rc = jl_forward(m, s->d_ids, so.data(), B, mp.data(), M, qt.data(), d_logits, s->stream);
    }
    (void)T;
    if (rc != JL_OK) break;
    if ((rc = jl_probs(m, d_logits, so.data(), B, mp.data(), M, qt.data(), d_probs, d_answer, s->d_argmax, d_maxp,
                       s->stream)) != JL_OK)
      break;
    {
      hipError_t e = hipMemcpyAsync(s->h_out, s->d_out, (size_t)M * 4, hipMemcpyDeviceToHost, s->stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(s->h_out + s->max_markers, d_probs, (size_t)M * 4, hipMemcpyDeviceToHost, s->stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(s->h_out + 2 * s->max_markers, d_answer, (size_t)B * 4, hipMemcpyDeviceToHost, s->stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(s->h_out + 2 * s->max_markers + s->max_seqs, d_maxp, (size_t)B * 4, hipMemcpyDeviceToHost,
                           s->stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(s->h_argmax, s->d_argmax, (size_t)B * 4, hipMemcpyDeviceToHost, s->stream);
      if (e == hipSuccess) e = hipEventRecord(s->done, s->stream);
      if (e != hipSuccess) {
        rc = device_error(m, e, "result download");
        break;
      }
    }
    s->busy = true;
  }
  for (ServeState *s : st) {
    const int r2 = retire(s);
    if (rc == JL_OK) rc = r2;
  }
  if (prev >= 0) (void)hipSetDevice(prev);
  if (rc == JL_OK && n_batches) *n_batches = nb;
  return rc;
}

extern "C" int jl_serve(jl_model *const *models, int32_t n_models, int32_t n_requests, const int32_t *ids,
                        const int64_t *id_offsets, const int32_t *mask_positions, const int64_t *mask_offsets,
                        const int32_t *qtype, int64_t max_batch_tokens, float *logits, float *probs, float *answer,
                        int32_t *argmax, float *maxprob, int32_t *n_batches) {
  JL_CATCH_ALL(jl_serve_impl(models, n_models, n_requests, ids, id_offsets, mask_positions, mask_offsets, qtype, max_batch_tokens,
               logits, probs, answer, argmax, maxprob, n_batches));
}
