"""Router tournament on the CPU: the oracle pinned to the page's worked
figures and to the survivor rule's edges, and the library's router
(jl_route_with_scorer, through the C ABI with a host scorer) against the
oracle on the same scores, including the layout of every scored sequence and
batches split by capacity.  No GPU is used."""
import numpy as np
import pytest

from encoder_transformer_amd import lib

from oracle import router as orc

MASK = 4


def _hidden_scores(n, seed):
    return np.random.default_rng(seed).normal(0.0, 1.5, n)


def _softmax32(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return (e / e.sum()).astype(np.float32)


def _question(seed, n_options, q_len=6, s_len=9):
    rng = np.random.default_rng(seed)
    prefix = [2] + list(rng.integers(1000, 2000, q_len)) + [1]
    suffix = [1] + list(rng.integers(2000, 3000, s_len)) + [1]
    # distinct first tokens identify question and option inside scored sequences
    options = [[10000 + 5000 * (seed % 40) + k] + list(rng.integers(10, 900, int(rng.integers(0, 4))))
               for k in range(n_options)]
    return prefix, suffix, options


def _oracle(question, scores):
    prefix, suffix, options = question
    return orc.route(lambda cands: [float(v) for v in _softmax32(scores[cands])], len(options))


def _library_scorer(questions, scores, batches):
    """Scores packed batches like the model would see them, checking that every
    sequence is prefix + (mask, option)* + suffix of one question."""
    first_tok = {}
    for q, (prefix, suffix, options) in enumerate(questions):
        for k, o in enumerate(options):
            first_tok[o[0]] = (q, k)

    def score(ids, so, mp):
        batches.append((len(ids), len(mp)))
        out = np.zeros(len(mp), np.float32)
        k = 0
        for b in range(len(so) - 1):
            seq = ids[so[b]:so[b + 1]]
            marks = [m - so[b] for m in mp if so[b] <= m < so[b + 1]]
            q, _ = first_tok[int(seq[marks[0] + 1])]
            prefix, suffix, options = questions[q]
            cands = [first_tok[int(seq[m + 1])][1] for m in marks]
            ids_ref, marks_ref = orc.group_sequence(prefix, suffix, options, cands, MASK)
            assert list(seq) == ids_ref and marks == marks_ref
            out[k:k + len(marks)] = _softmax32(scores[q][cands])
            k += len(marks)
        return out
    return score


@pytest.mark.parametrize("n,calls", [(60, 4), (72, 5)])
def test_oracle_call_counts_from_the_page(n, calls):
    # The page: 60 options cost 3 calls in the first round and 1 final call;
    # the 72-label list costs 4 plus 1.  With near-uniform scores every group
    # keeps two survivors.
    r = orc.route(lambda c: [1.0 / len(c) + 1e-3 * i for i in range(len(c))], n)
    assert r["calls"] == calls and r["rounds"] == 1


def test_oracle_survivor_rule_edges():
    cands = list(range(5))
    assert orc.group_survivors(cands, [0.96, 0.01, 0.01, 0.01, 0.01]) == [0]
    assert orc.group_survivors(cands, [0.01, 0.01, 0.96, 0.01, 0.01]) == [2]
    # the winner must be above 0.95 and every other below 0.045, strictly
    assert orc.group_survivors(cands, [0.95, 0.0125, 0.0125, 0.0125, 0.0125]) == [0, 1]
    assert orc.group_survivors(cands, [0.955, 0.045, 0.0, 0.0, 0.0]) == [0, 1]
    # two survivors in candidate order; ties go to the earlier candidate
    assert orc.group_survivors([3, 8, 9], [0.2, 0.3, 0.5]) == [8, 9]
    assert orc.group_survivors([3, 8, 9], [0.4, 0.3, 0.3]) == [3, 8]
    assert orc.group_survivors([3, 8, 9], [0.3, 0.4, 0.3]) == [3, 8]


def test_oracle_rounds_and_singletons():
    near_uniform = lambda c: [1.0 / len(c) + 1e-4 * (i % 7) for i in range(len(c))]
    # 41 = 20 + 20 + 1: the lone candidate passes unscored
    r = orc.route(near_uniform, 41)
    assert r["calls"] == 3 and r["rounds"] == 1 and len(r["final"]) == 5
    # 4,096: 205 groups -> 410, 21 groups -> 42, 3 groups -> 6, final call
    r = orc.route(near_uniform, 4096)
    assert r["rounds"] == 3 and r["calls"] == 205 + 21 + 3 + 1
    # 20 or fewer: one call
    r = orc.route(near_uniform, 20)
    assert r["calls"] == 1 and r["rounds"] == 0 and r["final"] == list(range(20))


def test_oracle_winner_alone_narrows_to_group_winners():
    def dominant(c):  # the lowest candidate index of each group dominates
        p = [0.01 / (len(c) - 1)] * len(c)
        p[0] = 0.99
        return p
    r = orc.route(dominant, 100)
    assert r["final"] == [0, 20, 40, 60, 80] and r["pick"] == 0 and r["calls"] == 6


@pytest.mark.parametrize("seed,sizes", [(0, [60]), (1, [72, 25, 5]), (2, [130, 41, 2]), (3, [401])])
def test_library_router_matches_oracle(seed, sizes):
    questions = [_question(100 * seed + i, n) for i, n in enumerate(sizes)]
    scores = [_hidden_scores(n, 1000 * seed + i) for i, n in enumerate(sizes)]
    # make some groups decisive, so both survivor branches occur
    for s in scores:
        s[::17] += 9.0
    batches = []
    r = lib.route_with_scorer(_library_scorer(questions, scores, batches), questions, MASK)
    for q, question in enumerate(questions):
        ref = _oracle(question, scores[q])
        assert int(r.pick[q]) == ref["pick"] and float(r.pick_prob[q]) == ref["pick_prob"]
        assert r.final[q] == ref["final"]
        assert [float(v) for v in r.final_prob[q]] == ref["final_prob"]
        assert int(r.calls[q]) == ref["calls"] and int(r.rounds[q]) == ref["rounds"]
    # every round of every question is one packed call when capacity allows
    assert len(batches) == max(int(v) for v in r.rounds) + 1


def test_library_router_splits_batches_by_capacity():
    questions = [_question(7, 90), _question(8, 45)]
    scores = [_hidden_scores(90, 70), _hidden_scores(45, 80)]
    big, small = [], []
    r1 = lib.route_with_scorer(_library_scorer(questions, scores, big), questions, MASK)
    r2 = lib.route_with_scorer(_library_scorer(questions, scores, small), questions, MASK, max_tokens=200,
                               max_markers=30)
    assert len(small) > len(big)
    assert all(t <= 200 and m <= 30 for t, m in small)
    assert np.array_equal(r1.pick, r2.pick) and np.array_equal(r1.calls, r2.calls)
    assert all(a == b for a, b in zip(r1.final, r2.final))


def test_library_router_errors():
    ok = _question(1, 30)
    sc = lambda ids, so, mp: np.full(len(mp), 0.5, np.float32)
    for bad, code in [([(ok[0], ok[1], ok[2][:1])], lib.ERR_ARG),          # one option
                      ([(ok[0], ok[1], [[5]] * 4097)], lib.ERR_ARG),        # too many options
                      ([(ok[0], ok[1], ok[2][:5] + [[]])], lib.ERR_ARG)]:   # an empty option
        with pytest.raises(lib.JLError) as e:
            lib.route_with_scorer(sc, bad, MASK)
        assert e.value.code == code
    with pytest.raises(lib.JLError) as e:  # one group longer than the batch capacity
        lib.route_with_scorer(sc, [ok], MASK, max_tokens=40)
    assert e.value.code == lib.ERR_LENGTH
    with pytest.raises(ZeroDivisionError):  # a scorer failure aborts the routing
        lib.route_with_scorer(lambda ids, so, mp: 1 / 0, [ok], MASK)
    r = lib.route_with_scorer(sc, [], MASK)
    assert len(r.pick) == 0
