// Seeded fuzz of libjl's host-side code through its C ABI, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host pass
// (tests/test_host_sanitizers.py builds and runs it; no GPU is used).
//
//   jl_host_fuzz <seed> <iterations> <weight-file header>
//
// Parts, each stopping the program at its first failure (exit 1, a message
// naming the part, seed and iteration):
//   validate  random packed batches, most valid, some with one planted
//             defect, against an independent check of the rules include/jl.h
//             states for jl_validate (the return code must be the same);
//   parser    jl_load_weights on the given JLW1 header with random byte
//             mutations and truncations: every call must return an error
//             code (the file holds no tensor data) with a message, and leave
//             *out NULL;
//   plan      jl_serve_plan on random request queues: a permutation, batches
//             numbered in order, every batch within its limits;
//   router    jl_route_with_scorer with a random host scorer: every pick is
//             one of its question's options, counts within their ranges.
// The sanitizers turn any out-of-bounds access, use after free, leak or
// undefined behaviour on these paths into a failure of the run.
#include "jl.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <random>
#include <string>
#include <vector>

namespace {

std::mt19937_64 rng;
uint64_t seed_g = 0;

int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

[[noreturn]] void die(const char *part, long it, const std::string &msg) {
  std::fprintf(stderr, "FAIL %s seed %llu iteration %ld: %s\n", part, (unsigned long long)seed_g, it, msg.c_str());
  std::exit(1);
}

// The rules of jl_validate as include/jl.h states them, checked in the same
// order: arguments, offsets and lengths with the question types, capacity,
// marker positions, options per question.
int ref_validate(const std::vector<int32_t> &so, int32_t B, const std::vector<int32_t> &mp, int32_t M,
                 const std::vector<int32_t> &qt, int64_t max_tokens, int64_t max_markers) {
  if (B < 0 || M < 0) return JL_ERR_ARG;
  if (so[0] != 0) return JL_ERR_LENGTH;
  for (int b = 0; b < B; ++b) {
    const int64_t len = (int64_t)so[b + 1] - so[b];
    if (len < 1 || len > JL_MAX_SEQ_LEN) return JL_ERR_LENGTH;
    if (qt[b] < 0 || qt[b] > 2) return JL_ERR_QTYPE;
  }
  const int64_t T = so[B];
  if (T > max_tokens || M > max_markers) return JL_ERR_CAPACITY;
  for (int k = 0; k < M; ++k) {
    if (mp[k] < 0 || mp[k] >= T) return JL_ERR_OPTIONS;
    if (k > 0 && mp[k] <= mp[k - 1]) return JL_ERR_OPTIONS;
  }
  for (int b = 0; b < B; ++b) {
    int c = 0;
    for (int k = 0; k < M; ++k) c += mp[k] >= so[b] && mp[k] < so[b + 1];
    if (c < JL_MIN_OPTIONS || c > JL_MAX_OPTIONS) return JL_ERR_OPTIONS;
    if (qt[b] == JL_NOUL && c != 2) return JL_ERR_OPTIONS;
  }
  return JL_OK;
}

void fuzz_validate(long iters) {
  for (long it = 0; it < iters; ++it) {
    const int B = uni(0, 12);
    std::vector<int32_t> so(B + 1, 0), qt(B), mp;
    for (int b = 0; b < B; ++b) {
      const int len = uni(0, 9) == 0 ? uni(2, 8200) : uni(2, 300);
      so[b + 1] = so[b] + len;
      qt[b] = uni(0, 2);
      const int n = qt[b] == JL_NOUL ? 2 : uni(2, std::min(20, len));
      std::vector<int32_t> pos(len);
      for (int i = 0; i < len; ++i) pos[i] = so[b] + i;
      std::shuffle(pos.begin(), pos.end(), rng);
      std::vector<int32_t> pick(pos.begin(), pos.begin() + std::min(n, len));
      std::sort(pick.begin(), pick.end());
      mp.insert(mp.end(), pick.begin(), pick.end());
    }
    // one planted defect in about half the cases
    switch (uni(0, 13)) {
      case 0: if (!mp.empty()) std::swap(mp[0], mp[mp.size() - 1]); break;
      case 1: if (!mp.empty()) mp.push_back(mp.back()); break;
      case 2: if (!mp.empty()) mp[uni(0, (int)mp.size() - 1)] = uni(-5, so[B] + 5); break;
      case 3: if (B > 0) so[uni(1, B)] -= uni(1, 3); break;
      case 4: if (B > 0) qt[uni(0, B - 1)] = uni(-2, 5); break;
      case 5: so[0] = uni(-2, 2); break;
      case 6: if (!mp.empty()) mp.erase(mp.begin() + uni(0, (int)mp.size() - 1)); break;
      default: break;
    }
    const int M = (int)mp.size();
    if (mp.empty()) mp.push_back(0);  // keep .data() valid; M stays 0
    const int64_t T = so[B];
    const int64_t max_tokens = std::max<int64_t>(1, T + uni(-3, 3));
    const int64_t max_markers = std::max<int64_t>(2, M + uni(-2, 2));
    const int got = jl_validate(so.data(), B, mp.data(), M, qt.data(), max_tokens, max_markers);
    const int want = ref_validate(so, B, mp, M, qt, max_tokens, max_markers);
    if (got != want)
      die("validate", it, "jl_validate returned " + std::to_string(got) + ", the rules give " + std::to_string(want));
    if (got != JL_OK && std::strlen(jl_last_error()) == 0) die("validate", it, "error without a message");
  }
  // NULL arrays with non-zero counts
  int32_t so[2] = {0, 10}, mp[2] = {3, 5}, qt[1] = {0};
  if (jl_validate(nullptr, 1, mp, 2, qt, 100, 100) != JL_ERR_ARG ||
      jl_validate(so, 1, nullptr, 2, qt, 100, 100) != JL_ERR_ARG ||
      jl_validate(so, 1, mp, 2, nullptr, 100, 100) != JL_ERR_ARG)
    die("validate", -1, "NULL arrays not rejected with JL_ERR_ARG");
}

void fuzz_parser(long iters, const char *header_path) {
  std::vector<unsigned char> hdr;
  if (FILE *f = std::fopen(header_path, "rb")) {
    unsigned char buf[4096];
    size_t n;
    while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) hdr.insert(hdr.end(), buf, buf + n);
    std::fclose(f);
  }
  if (hdr.size() < 16) die("parser", -1, "cannot read the header file");
  const std::string path = "/tmp/jl_host_fuzz_" + std::to_string(seed_g) + ".bin";
  for (long it = 0; it < iters; ++it) {
    std::vector<unsigned char> h = hdr;
    const int edits = uni(1, 8);
    for (int e = 0; e < edits; ++e) {
      const size_t at = (size_t)uni(0, (int)h.size() - 1);
      switch (uni(0, 3)) {
        case 0: h[at] = (unsigned char)uni(0, 255); break;            // a random byte
        case 1: h[at] ^= (unsigned char)(1u << uni(0, 7)); break;     // a flipped bit
        case 2: h.resize(std::max<size_t>(1, at)); break;             // truncation
        default: if (at + 4 <= h.size()) std::memset(&h[at], 0xff, 4); break;  // a huge count
      }
    }
    if (uni(0, 9) == 0) h.insert(h.end(), (size_t)uni(1, 5000), 0);  // some data bytes
    FILE *f = std::fopen(path.c_str(), "wb");
    if (!f) die("parser", it, "cannot write " + path);
    std::fwrite(h.data(), 1, h.size(), f);
    std::fclose(f);
    jl_model *m = reinterpret_cast<jl_model *>(0x1);
    const int rc = jl_load_weights(path.c_str(), JL_BF16, 4096, 256, 0, &m);
    if (rc == JL_OK) die("parser", it, "a file without tensor data was accepted");
    if (m != nullptr) die("parser", it, "*out not NULL after an error");
    if (std::strlen(jl_last_error()) == 0) die("parser", it, "error without a message");
  }
  std::remove(path.c_str());
  jl_model *m = nullptr;
  if (jl_load_weights("/nonexistent/jl.bin", JL_BF16, 4096, 256, 0, &m) != JL_ERR_FILE || m)
    die("parser", -1, "a missing file is not JL_ERR_FILE");
}

void fuzz_plan(long iters) {
  for (long it = 0; it < iters; ++it) {
    const int R = uni(0, 60);
    std::vector<int64_t> io(R + 1, 0), mo(R + 1, 0);
    for (int r = 0; r < R; ++r) {
      io[r + 1] = io[r] + uni(1, 3000);
      mo[r + 1] = mo[r] + uni(0, 20);
    }
    const int64_t bt = uni(1, 9000), bm = uni(2, 300), bs = uni(1, 40);
    std::vector<int32_t> order(R + 1, -1), batch_of(R + 1, -1);
    int32_t nb = -1;
    const int rc = jl_serve_plan(R, io.data(), mo.data(), bt, bm, bs, order.data(), batch_of.data(), &nb);
    bool fits = true;
    for (int r = 0; r < R; ++r) fits = fits && io[r + 1] - io[r] <= bt && mo[r + 1] - mo[r] <= bm;
    if (!fits) {
      if (rc != JL_ERR_LENGTH) die("plan", it, "an oversized request not rejected");
      continue;
    }
    if (rc != JL_OK) die("plan", it, std::string("rejected: ") + jl_last_error());
    std::vector<int> seen(R, 0);
    std::vector<int64_t> tok, mk, sq;
    for (int i = 0; i < R; ++i) {
      const int r = order[i];
      if (r < 0 || r >= R || seen[r]++) die("plan", it, "order is not a permutation");
      const int b = batch_of[r];
      if (b < 0 || b >= nb || (i > 0 && b < batch_of[order[i - 1]])) die("plan", it, "batches out of order");
      if ((int)tok.size() <= b) tok.resize(b + 1, 0), mk.resize(b + 1, 0), sq.resize(b + 1, 0);
      tok[b] += io[r + 1] - io[r];
      mk[b] += mo[r + 1] - mo[r];
      sq[b] += 1;
    }
    for (size_t b = 0; b < tok.size(); ++b)
      if (tok[b] > bt || mk[b] > bm || sq[b] > bs) die("plan", it, "a micro-batch exceeds its limits");
  }
}

struct ScorerState {
  long calls = 0;
};

int random_scorer(void *user, const int32_t *ids, const int32_t *so, int32_t n_seqs, const int32_t *mp, int32_t M,
                  float *probs) {
  static_cast<ScorerState *>(user)->calls++;
  (void)ids;
  int k = 0;
  for (int b = 0; b < n_seqs; ++b) {
    int k0 = k;
    while (k < M && mp[k] < so[b + 1]) ++k;
    float s = 0.f;
    const bool peaked = uni(0, 2) == 0;
    for (int j = k0; j < k; ++j) s += probs[j] = peaked && j == k0 ? 1000.f : (float)uni(1, 100);
    for (int j = k0; j < k; ++j) probs[j] /= s;
  }
  return 0;
}

void fuzz_router(long iters) {
  for (long it = 0; it < iters; ++it) {
    const int Q = uni(0, 4);
    std::vector<int64_t> po(Q + 1, 0), su(Q + 1, 0), oo(1, 0);
    std::vector<int32_t> pid, sid, oid, qo(Q + 1, 0);
    for (int q = 0; q < Q; ++q) {
      const int pl = uni(1, 20), sl = uni(0, 30), n = uni(2, 90);
      for (int i = 0; i < pl; ++i) pid.push_back(uni(5, 255999));
      for (int i = 0; i < sl; ++i) sid.push_back(uni(5, 255999));
      po[q + 1] = po[q] + pl;
      su[q + 1] = su[q] + sl;
      for (int o = 0; o < n; ++o) {
        const int ol = uni(1, 12);
        for (int i = 0; i < ol; ++i) oid.push_back(uni(5, 255999));
        oo.push_back(oo.back() + ol);
      }
      qo[q + 1] = qo[q] + n;
    }
    if (pid.empty()) pid.push_back(0);
    if (sid.empty()) sid.push_back(0);
    if (oid.empty()) oid.push_back(0);
    std::vector<int32_t> pick(Q + 1, -1), nfin(Q + 1), fidx(20 * (Q + 1)), calls(Q + 1), rounds(Q + 1);
    std::vector<float> pp(Q + 1), fprob(20 * (Q + 1));
    ScorerState st;
    const int64_t cap_t = uni(2000, 20000), cap_m = uni(40, 400);
    const int rc = jl_route_with_scorer(random_scorer, &st, cap_t, cap_m, Q, pid.data(), po.data(), sid.data(),
                                        su.data(), oid.data(), oo.data(), qo.data(), 4, pick.data(), pp.data(),
                                        nfin.data(), fidx.data(), fprob.data(), calls.data(), rounds.data());
    if (rc != JL_OK) die("router", it, std::string("rejected: ") + jl_last_error());
    for (int q = 0; q < Q; ++q) {
      const int n = qo[q + 1] - qo[q];
      if (pick[q] < 0 || pick[q] >= n) die("router", it, "pick outside the question's options");
      if (nfin[q] < 1 || nfin[q] > 20 || calls[q] < 1 || rounds[q] < 0) die("router", it, "counts out of range");
      if (!(pp[q] >= 0.f && pp[q] <= 1.f)) die("router", it, "pick probability outside [0, 1]");
    }
  }
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s <seed> <iterations> <weight-file header>\n", argv[0]);
    return 2;
  }
  seed_g = std::strtoull(argv[1], nullptr, 10);
  const long iters = std::strtol(argv[2], nullptr, 10);
  rng.seed(seed_g);
  const char *part = "validate";
  try {
    fuzz_validate(iters);
    part = "parser";
    fuzz_parser(iters / 10 + 1, argv[3]);
    part = "plan";
    fuzz_plan(iters / 4 + 1);
    part = "router";
    fuzz_router(iters / 50 + 1);
  } catch (const std::exception &e) {  // the C ABI must never let an exception out
    die(part, -1, std::string("exception escaped: ") + e.what());
  }
  std::printf("ok: seed %llu, %ld iterations\n", (unsigned long long)seed_g, iters);
  return 0;
}
