"""The router on the GPU (jl_route): the model scores every group.

* jl_route against the same tournament driven from Python with the model as
  scorer (jl_route_with_scorer + jl_forward/jl_probs per packed batch): the
  batches are identical and the kernels batch-invariant, so picks, final sets
  and probabilities match bitwise;
* the oracle router replaying the model's recorded group probabilities makes
  the same decisions (the rule, on real model outputs);
* final-call probabilities against the float64 oracle forward.
"""
import numpy as np
import pytest

from encoder_transformer_amd import synth

from gpu_common import BF16_PROB_BOUND, MAX_MARKERS

pytestmark = pytest.mark.gpu

MASK = synth.MASK


def _questions():
    rng = np.random.default_rng(77)
    out = []
    for q, n in enumerate((45, 25, 12, 61)):
        prefix = [2, 1001, 1010, 1003] + list(rng.integers(5, synth.VOCAB, 8)) + [1]
        suffix = [1] + list(rng.integers(5, synth.VOCAB, 40)) + [1]
        options = [list(rng.integers(5, synth.VOCAB, int(rng.integers(1, 5)))) for _ in range(n)]
        out.append((prefix, suffix, options))
    return out


@pytest.fixture(scope="module")
def model():
    import torch
    from encoder_transformer_amd import lib
    assert torch.cuda.is_available()
    m = lib.Model(synth.cached_weight_file(), lib.BF16, 20000, MAX_MARKERS)
    yield m
    m.close()


def _gpu_scorer(model, record):
    import torch

    def score(ids, so, mp):
        qt = np.zeros(len(so) - 1, np.int32)
        ids_dev = torch.from_numpy(ids.astype(np.int32)).cuda()
        logits = model.forward(ids_dev, so, mp, qt)
        probs = model.probs(logits, so, mp, qt)[0]
        torch.cuda.synchronize()
        p = probs.cpu().numpy()
        for b in range(len(so) - 1):
            sel = (mp >= so[b]) & (mp < so[b + 1])
            record[tuple(ids[so[b]:so[b + 1]])] = p[sel].copy()
        return p
    return score


def test_router_matches_scripted_tournament_and_rule(model):
    import torch
    from encoder_transformer_amd import lib
    from oracle import router as orc
    qs = _questions()
    r = model.route(qs, MASK)
    torch.cuda.synchronize()
    record = {}
    ref = lib.route_with_scorer(_gpu_scorer(model, record), qs, MASK, max_tokens=20000, max_markers=MAX_MARKERS)
    assert np.array_equal(r.pick, ref.pick) and np.array_equal(r.pick_prob, ref.pick_prob)
    assert np.array_equal(r.calls, ref.calls) and np.array_equal(r.rounds, ref.rounds)
    for q in range(len(qs)):
        assert r.final[q] == ref.final[q] and np.array_equal(r.final_prob[q], ref.final_prob[q])
    # the oracle's rule on the model's own group probabilities
    for q, (prefix, suffix, options) in enumerate(qs):
        def replay(cands):
            ids, _ = orc.group_sequence(prefix, suffix, options, cands, MASK)
            return [float(v) for v in record[tuple(ids)]]
        o = orc.route(replay, len(options))
        assert o["pick"] == int(r.pick[q]) and o["final"] == r.final[q]
        assert o["calls"] == int(r.calls[q]) and o["rounds"] == int(r.rounds[q])
    # 45 options: 3 groups + final; 12: one call; 61: groups 20, 20, 20 and a
    # lone candidate that passes unscored, + final
    assert int(r.calls[0]) == 4 and int(r.calls[2]) == 1 and int(r.calls[3]) == 4


def test_router_final_probabilities_against_oracle(model):
    from oracle import julia_oracle as jo
    from oracle import router as orc
    qs = _questions()[1:3]
    r = model.route(qs, MASK)
    W = jo.OracleWeights(synth.make_weights())
    for q, (prefix, suffix, options) in enumerate(qs):
        ids, marks = orc.group_sequence(prefix, suffix, options, r.final[q], MASK)
        batch = synth.Batch(ids=np.asarray(ids, np.int32), seq_offsets=np.array([0, len(ids)], np.int32),
                            mask_positions=np.asarray(marks, np.int32), qtype=np.zeros(1, np.int32))
        logits = jo.forward(W, batch)
        p = jo.read_offs(logits, batch.seq_offsets, batch.mask_positions, batch.qtype)["probs"]
        assert np.max(np.abs(np.asarray(r.final_prob[q], np.float64) - p)) <= BF16_PROB_BOUND
