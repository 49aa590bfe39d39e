// Router tournament for choice questions with more than 20 options
// ("Julia-1: one score per mask token ...", More than 20 options: the Router).
//
// Host-side driver: each round packs the groups of every unfinished question
// into batches, scores them (the model through jl_forward + jl_probs, or a
// caller's scorer), and applies the survivor rule.  The arithmetic all runs
// on the device; this file only lays out sequences and selects survivors.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "jl.h"
#include "jl_internal.h"

namespace {

constexpr int kGroup = 20;           // options per scored group (the head's maximum)
constexpr int kMaxOptions = 4096;    // per question
constexpr float kWinAlone = 0.95f;   // a winner above this ...
constexpr float kOthersBelow = 0.045f;  // ... with every other option below this survives alone

struct Inputs {
  int32_t nq;
  const int32_t *prefix, *suffix, *opts;
  const int64_t *prefix_off, *suffix_off, *opt_off;
  const int32_t *q_opts;
  int32_t mask_id;
};

// One scored group: question q, candidate indices (question-local), final?
struct Group {
  int q;
  std::vector<int> cand;
  bool final_call;
};

using Scorer = int (*)(void *, const int32_t *, const int32_t *, int32_t, const int32_t *, int32_t, float *);

int64_t group_len(const Inputs &in, const Group &g) {
  int64_t n = (in.prefix_off[g.q + 1] - in.prefix_off[g.q]) + (in.suffix_off[g.q + 1] - in.suffix_off[g.q]);
  const int64_t o0 = in.q_opts[g.q];
  for (int c : g.cand) n += 1 + (in.opt_off[o0 + c + 1] - in.opt_off[o0 + c]);
  return n;
}

int check_inputs(const Inputs &in) {
  using jl::set_error;
  if (in.nq < 0) return set_error(JL_ERR_ARG, "n_questions must be >= 0");
  if (in.nq == 0) return JL_OK;
  if (!in.prefix || !in.suffix || !in.opts || !in.prefix_off || !in.suffix_off || !in.opt_off || !in.q_opts)
    return set_error(JL_ERR_ARG, "router input arrays must not be NULL");
  if (in.q_opts[0] != 0 || in.prefix_off[0] != 0 || in.suffix_off[0] != 0 || in.opt_off[0] != 0)
    return set_error(JL_ERR_ARG, "offset arrays must start at 0");
  for (int q = 0; q < in.nq; ++q) {
    const int n = in.q_opts[q + 1] - in.q_opts[q];
    if (n < 2 || n > kMaxOptions) return set_error(JL_ERR_ARG, "each question needs 2 to 4,096 options");
    if (in.prefix_off[q + 1] < in.prefix_off[q] || in.suffix_off[q + 1] < in.suffix_off[q])
      return set_error(JL_ERR_ARG, "prefix and suffix offsets must not decrease");
  }
  const int total = in.q_opts[in.nq];
  for (int k = 0; k < total; ++k)
    if (in.opt_off[k + 1] <= in.opt_off[k]) return set_error(JL_ERR_ARG, "every option needs at least one token");
  return JL_OK;
}

// Survivors of one scored group (question-local indices, in order).
std::vector<int> survivors(const std::vector<int> &cand, const float *p) {
  const int n = (int)cand.size();
  int w = 0;
  for (int i = 1; i < n; ++i)
    if (p[i] > p[w]) w = i;  // first maximum on ties
  bool alone = p[w] > kWinAlone;
  for (int i = 0; i < n && alone; ++i)
    if (i != w && !(p[i] < kOthersBelow)) alone = false;
  if (alone) return {cand[w]};
  int s = -1;
  for (int i = 0; i < n; ++i)
    if (i != w && (s < 0 || p[i] > p[s])) s = i;
  return w < s ? std::vector<int>{cand[w], cand[s]} : std::vector<int>{cand[s], cand[w]};
}

int route(Scorer score, void *user, int64_t max_tokens, int64_t max_markers, const Inputs &in, int32_t *pick,
          float *pick_prob, int32_t *n_final, int32_t *final_idx, float *final_prob, int32_t *calls,
          int32_t *rounds) {
  using jl::set_error;
  if (int rc = check_inputs(in)) return rc;
  if (in.nq == 0) return JL_OK;
  if (!pick || !pick_prob) return set_error(JL_ERR_ARG, "pick and pick_prob must not be NULL");
  std::vector<std::vector<int>> alive(in.nq);
  std::vector<int> n_calls(in.nq, 0), n_rounds(in.nq, 0);
  std::vector<bool> done(in.nq, false);
  for (int q = 0; q < in.nq; ++q) {
    const int n = in.q_opts[q + 1] - in.q_opts[q];
    alive[q].resize(n);
    for (int i = 0; i < n; ++i) alive[q][i] = i;
  }
  std::vector<int32_t> ids, so, mp, qt;
  std::vector<float> probs;
  for (;;) {
    // this round's groups: consecutive runs of at most 20 alive candidates,
    // or the final call of a question with 20 or fewer left
    std::vector<Group> groups;
    std::vector<std::vector<int>> next(in.nq);
    bool any = false;
    for (int q = 0; q < in.nq; ++q) {
      if (done[q]) continue;
      any = true;
      const auto &a = alive[q];
      if ((int)a.size() <= kGroup) {
        groups.push_back({q, a, true});
        continue;
      }
      for (size_t i = 0; i < a.size(); i += kGroup) {
        std::vector<int> g(a.begin() + i, a.begin() + std::min(a.size(), i + kGroup));
        if (g.size() == 1)
          next[q].push_back(g[0]);  // a single candidate passes on unscored
        else
          groups.push_back({q, std::move(g), false});
      }
    }
    if (!any) break;
    // pack the groups into batches within the capacity and score them
    size_t gi = 0;
    while (gi < groups.size()) {
      ids.clear();
      so.assign(1, 0);
      mp.clear();
      qt.clear();
      const size_t g0 = gi;
      while (gi < groups.size()) {
        const Group &g = groups[gi];
        const int64_t len = group_len(in, g);
        if (len > JL_MAX_SEQ_LEN || len > max_tokens || (int64_t)g.cand.size() > max_markers)
          return set_error(JL_ERR_LENGTH, "a router group's sequence exceeds 8,192 tokens or the capacity");
        if (gi > g0 && ((int64_t)ids.size() + len > max_tokens || (int64_t)(mp.size() + g.cand.size()) > max_markers))
          break;
        const int q = g.q;
        ids.insert(ids.end(), in.prefix + in.prefix_off[q], in.prefix + in.prefix_off[q + 1]);
        const int64_t o0 = in.q_opts[q];
        for (int c : g.cand) {
          mp.push_back((int32_t)ids.size());
          ids.push_back(in.mask_id);
          ids.insert(ids.end(), in.opts + in.opt_off[o0 + c], in.opts + in.opt_off[o0 + c + 1]);
        }
        ids.insert(ids.end(), in.suffix + in.suffix_off[q], in.suffix + in.suffix_off[q + 1]);
        so.push_back((int32_t)ids.size());
        qt.push_back(JL_CHOICE);
        ++gi;
      }
      probs.assign(mp.size(), 0.f);
      if (int rc = score(user, ids.data(), so.data(), (int32_t)qt.size(), mp.data(), (int32_t)mp.size(),
                         probs.data()))
        return rc;
      size_t k = 0;
      for (size_t j = g0; j < gi; ++j) {
        const Group &g = groups[j];
        const float *p = probs.data() + k;
        k += g.cand.size();
        ++n_calls[g.q];
        if (!g.final_call) {
          for (int c : survivors(g.cand, p)) next[g.q].push_back(c);
          continue;
        }
        int w = 0;
        for (size_t i = 1; i < g.cand.size(); ++i)
          if (p[i] > p[w]) w = (int)i;
        const int q = g.q;
        pick[q] = g.cand[w];
        pick_prob[q] = p[w];
        if (n_final) n_final[q] = (int32_t)g.cand.size();
        for (size_t i = 0; i < g.cand.size(); ++i) {
          if (final_idx) final_idx[q * kGroup + i] = g.cand[i];
          if (final_prob) final_prob[q * kGroup + i] = p[i];
        }
        done[q] = true;
      }
    }
    for (int q = 0; q < in.nq; ++q) {
      if (done[q]) continue;
      std::sort(next[q].begin(), next[q].end());  // survivors keep the candidates' order
      alive[q] = std::move(next[q]);
      ++n_rounds[q];
    }
  }
  for (int q = 0; q < in.nq; ++q) {
    if (calls) calls[q] = n_calls[q];
    if (rounds) rounds[q] = n_rounds[q];
  }
  return JL_OK;
}

// The model as a scorer: ids to the device, jl_forward + jl_probs, probabilities
// back.  The ids and probabilities pass through the handle's pinned staging
// and device buffers (jl_serve's, made on the handle's first host-side call
// and kept until jl_free), so routing allocates nothing per call.
struct ModelScorer {
  jl_model *m;
  hipStream_t s;
  int device;
  jl::HandleBuffers hb;
  static int call(void *self, const int32_t *ids, const int32_t *so, int32_t n_seqs, const int32_t *mp, int32_t M,
                  float *probs) {
    auto &ms = *static_cast<ModelScorer *>(self);
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != ms.device && hipSetDevice(ms.device) != hipSuccess)
      return jl::set_error(JL_ERR_DEVICE, "cannot select the model's device");
    const int rc = ms.score(ids, so, n_seqs, mp, M, probs);
    if (prev >= 0 && prev != ms.device) (void)hipSetDevice(prev);
    return rc;
  }
  int score(const int32_t *ids, const int32_t *so, int32_t n_seqs, const int32_t *mp, int32_t M, float *probs) {
    const size_t T = (size_t)so[n_seqs];
    // the router cuts its batches to the handle's capacity
    if ((int64_t)T > hb.max_tokens || M > hb.max_markers)
      return jl::set_error(JL_ERR_CAPACITY, "router batch exceeds the handle's capacity");
    std::vector<int32_t> qt(n_seqs, JL_CHOICE);
    float *logits_dev = hb.d_out, *probs_dev = hb.d_out + hb.max_markers;
    std::memcpy(hb.h_ids, ids, T * sizeof(int32_t));
    if (hipError_t e = hipMemcpyAsync(hb.d_ids, hb.h_ids, T * sizeof(int32_t), hipMemcpyHostToDevice, s))
      return jl::device_error(m, e, "router ids upload");
    if (int rc = jl_forward(m, hb.d_ids, so, n_seqs, mp, M, qt.data(), logits_dev, s)) return rc;
    if (int rc = jl_probs(m, logits_dev, so, n_seqs, mp, M, qt.data(), probs_dev, nullptr, nullptr, nullptr, s))
      return rc;
    hipError_t e = hipMemcpyAsync(hb.h_out, probs_dev, M * sizeof(float), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return jl::device_error(m, e, "router probabilities download");
    std::memcpy(probs, hb.h_out, M * sizeof(float));
    return JL_OK;
  }
};

}  // namespace

static int jl_route_with_scorer_impl(jl_score_fn score, void *user, int64_t max_tokens, int64_t max_markers,
                                    int32_t n_questions, const int32_t *prefix_ids, const int64_t *prefix_offsets,
                                    const int32_t *suffix_ids, const int64_t *suffix_offsets,
                                    const int32_t *option_ids, const int64_t *option_offsets,
                                    const int32_t *question_options, int32_t mask_id, int32_t *pick,
                                    float *pick_prob, int32_t *n_final, int32_t *final_idx, float *final_prob,
                                    int32_t *calls, int32_t *rounds) {
  if (!score) return jl::set_error(JL_ERR_ARG, "score must not be NULL");
  if (max_tokens < 1 || max_markers < 2) return jl::set_error(JL_ERR_ARG, "bad batch capacity");
  const Inputs in{n_questions, prefix_ids, suffix_ids, option_ids, prefix_offsets, suffix_offsets,
                  option_offsets, question_options, mask_id};
  return route(score, user, max_tokens, max_markers, in, pick, pick_prob, n_final, final_idx, final_prob, calls,
               rounds);
}

extern "C" int jl_route_with_scorer(jl_score_fn score, void *user, int64_t max_tokens, int64_t max_markers,
                                    int32_t n_questions, const int32_t *prefix_ids, const int64_t *prefix_offsets,
                                    const int32_t *suffix_ids, const int64_t *suffix_offsets,
                                    const int32_t *option_ids, const int64_t *option_offsets,
                                    const int32_t *question_options, int32_t mask_id, int32_t *pick,
                                    float *pick_prob, int32_t *n_final, int32_t *final_idx, float *final_prob,
                                    int32_t *calls, int32_t *rounds) {
  JL_CATCH_ALL(jl_route_with_scorer_impl(score, user, max_tokens, max_markers, n_questions, prefix_ids, prefix_offsets, suffix_ids,
               suffix_offsets, option_ids, option_offsets, question_options, mask_id, pick, pick_prob, n_final,
               final_idx, final_prob, calls, rounds));
}

static int jl_route_impl(jl_model *m, int32_t n_questions, const int32_t *prefix_ids, const int64_t *prefix_offsets,
                        const int32_t *suffix_ids, const int64_t *suffix_offsets, const int32_t *option_ids,
                        const int64_t *option_offsets, const int32_t *question_options, int32_t mask_id,
                        int32_t *pick, float *pick_prob, int32_t *n_final, int32_t *final_idx, float *final_prob,
                        int32_t *calls, int32_t *rounds, void *stream) {
  if (int rc = jl::model_check(m)) return rc;
  int64_t info[4];
  if (int rc = jl_model_info(m, info, 4)) return rc;
  ModelScorer ms{m, (hipStream_t)stream, (int)info[3], {}};
  if (int rc = jl::handle_buffers(m, &ms.hb)) return rc;
  const Inputs in{n_questions, prefix_ids, suffix_ids, option_ids, prefix_offsets, suffix_offsets,
                  option_offsets, question_options, mask_id};
  return route(&ModelScorer::call, &ms, info[1], info[2], in, pick, pick_prob, n_final, final_idx, final_prob,
               calls, rounds);
}

extern "C" int jl_route(jl_model *m, int32_t n_questions, const int32_t *prefix_ids, const int64_t *prefix_offsets,
                        const int32_t *suffix_ids, const int64_t *suffix_offsets, const int32_t *option_ids,
                        const int64_t *option_offsets, const int32_t *question_options, int32_t mask_id,
                        int32_t *pick, float *pick_prob, int32_t *n_final, int32_t *final_idx, float *final_prob,
                        int32_t *calls, int32_t *rounds, void *stream) {
  JL_CATCH_ALL(jl_route_impl(m, n_questions, prefix_ids, prefix_offsets, suffix_ids, suffix_offsets, option_ids, option_offsets,
               question_options, mask_id, pick, pick_prob, n_final, final_idx, final_prob, calls, rounds, stream));
}
