"""Serving front on the GPU (jl_share, jl_serve): a queue of ragged requests
served in micro-batches over handles that share the weights, each on its own
stream, against each request run alone through jl_forward / jl_probs.

Micro-batches below the row-block threshold take the per-GEMM schedule, which
is batch invariant, so logits and read-offs match bitwise; with larger
micro-batches (row-block schedule) they match within the bf16 agreement bound
of the two schedules."""
import numpy as np
import pytest

from encoder_transformer_amd import synth

from gpu_common import MAX_MARKERS, device_ids

pytestmark = pytest.mark.gpu

BF16_LOGIT_TIGHT = 3e-3


@pytest.fixture(scope="module")
def models():
    import torch
    from encoder_transformer_amd import lib
    assert torch.cuda.is_available()
    m = lib.Model(synth.cached_weight_file(), lib.BF16, 20000, MAX_MARKERS)
    shared = [m.share(), m.share(12000, 2048)]
    yield m, shared
    for s in shared:
        s.close()
    m.close()


def _requests(n, seed):
    from encoder_transformer_amd import lib
    b = synth.make_batch(4)
    rng = np.random.default_rng(seed)
    pick = rng.choice(b.n_seqs, n, replace=False)
    items = []
    for k in pick:
        ids, marks, qt = b.sequence(int(k))
        items.append((ids, marks, qt))
    return lib.Requests(items), items


def _alone(m, item):
    import torch
    ids, marks, qt = item
    so = [0, len(ids)]
    logits = m.forward(device_ids(synth.Batch(np.asarray(ids, np.int32), np.array(so, np.int32),
                                              np.asarray(marks, np.int32), np.array([qt], np.int32))),
                       so, marks, [qt])
    probs, answer, argmax, maxprob = m.probs(logits, so, marks, [qt])
    torch.cuda.synchronize()
    return (logits.cpu().numpy(), probs.cpu().numpy(), float(answer.cpu()[0]), int(argmax.cpu()[0]),
            float(maxprob.cpu()[0]))


@pytest.mark.parametrize("n_handles", [1, 3])
def test_serve_matches_requests_alone(models, n_handles):
    from encoder_transformer_amd import lib
    m, shared = models
    handles = ([m] + shared)[:n_handles]
    req, items = _requests(40, 5 + n_handles)
    res = lib.serve(handles, req, max_batch_tokens=6000)
    assert res.n_batches > n_handles  # several micro-batches per handle
    for r, item in enumerate(items):
        lg, pr, ans, am, mp = _alone(m, item)
        assert np.array_equal(res.request_logits(r), lg), r
        assert np.array_equal(res.probs[req.mask_offsets[r]:req.mask_offsets[r + 1]], pr), r
        assert res.answer[r] == np.float32(ans) and res.argmax[r] == am and res.maxprob[r] == np.float32(mp), r


def test_serve_row_block_micro_batches(models):
    from encoder_transformer_amd import lib
    m, shared = models
    req, items = _requests(60, 11)
    res = lib.serve([m, shared[0]], req, max_batch_tokens=20000)  # micro-batches above 8,192 tokens
    err = max(float(np.max(np.abs(res.request_logits(r) - _alone(m, it)[0]))) for r, it in enumerate(items))
    print("serve row-block vs alone max |dlogit|", err)
    assert err <= BF16_LOGIT_TIGHT


def test_serve_rejects_before_any_work(models):
    from encoder_transformer_amd import lib
    m, _ = models
    req, items = _requests(6, 3)
    bad = list(items)
    ids, marks, _ = bad[4]
    bad[4] = (ids, marks, 7)  # no such question type
    breq = lib.Requests(bad)
    M = int(breq.mask_offsets[-1])
    import ctypes
    L = lib.load_library()
    logits = np.full(M, 7.0, np.float32)
    hs = (ctypes.c_void_p * 1)(m._h)
    f = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    i = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    l64 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    other = [np.full(M, 7.0, np.float32), np.full(6, 7.0, np.float32), np.zeros(6, np.int32),
             np.full(6, 7.0, np.float32)]
    rc = L.jl_serve(hs, 1, 6, i(breq.ids), l64(breq.id_offsets), i(breq.mask_positions), l64(breq.mask_offsets),
                    i(breq.qtype), 8192, f(logits), f(other[0]), f(other[1]), i(other[2]), f(other[3]), None)
    assert rc == lib.ERR_QTYPE and "request 4" in L.jl_last_error().decode()
    assert np.all(logits == 7.0) and np.all(other[0] == 7.0)


@pytest.mark.parametrize("name", ["standard", "wide"])
def test_serve_against_the_oracle(name):
    """jl_serve on the requests of the 256-sequence ragged mix against the
    oracle: logits against the stored oracle logits (wide weights: all 256
    requests, logits of order one; published init: the 8 stored ones), the
    probabilities and answers against the oracle's read-offs of those logits.
    Micro-batches of up to 32,768 tokens on two handles, so both schedules run."""
    from encoder_transformer_amd import lib
    from gpu_common import BF16_PROB_BOUND, LOGIT_TOL, golden_for, weight_file
    from oracle import julia_oracle as jo
    batch, seqs, ref_logits = golden_for(4, wide=name == "wide")
    items = [batch.sequence(b) for b in seqs]
    req = lib.Requests(items)
    m = lib.Model(weight_file(name), lib.BF16, 32768, 4096)
    h2 = m.share()
    try:
        res = lib.serve([m, h2], req, max_batch_tokens=32768)
    finally:
        h2.close()
        m.close()
    bound = LOGIT_TOL[(name, "bf16")]
    worst = {"logit": 0.0, "prob": 0.0}
    for r, (ids, marks, qt) in enumerate(items):
        ref = np.asarray(ref_logits[r])
        got = res.request_logits(r)
        worst["logit"] = max(worst["logit"], float(np.max(np.abs(got - ref))))
        ro = jo.read_offs(ref, np.array([0, len(ids)]), np.asarray(marks), np.array([qt]))
        dp = float(np.max(np.abs(res.probs[req.mask_offsets[r]:req.mask_offsets[r + 1]] - ro["probs"])))
        worst["prob"] = max(worst["prob"], dp)
        n = len(marks)
        if qt == 1:  # expected index: sum_i i * dp_i
            assert abs(res.answer[r] - ro["answer"][0]) <= dp * n * (n - 1) / 2 + 1e-6, r
        elif qt == 2:  # p(true)
            assert abs(res.answer[r] - ro["answer"][0]) <= dp + 1e-6, r
        srt = np.sort(ref)[::-1]
        if srt[0] - srt[1] > 2 * bound:  # a clear question: the same argmax (and the choice answer)
            assert res.argmax[r] == ro["argmax"][0], r
            if qt == 0:
                assert res.answer[r] == ro["answer"][0], r
    print(name, "serve vs oracle", worst, "micro-batches", res.n_batches)
    assert worst["logit"] <= bound
    assert worst["prob"] <= BF16_PROB_BOUND


def test_serve_graph_buckets_against_the_oracle():
    """With the graph cache on, jl_serve pads each micro-batch to a shape
    bucket with filler questions and replays one graph per bucket: a second
    pass over the same queue replays every micro-batch and gives the same
    results bitwise; both against the oracle (wide weights, all 256
    requests of the ragged mix)."""
    from encoder_transformer_amd import lib
    from gpu_common import BF16_PROB_BOUND, LOGIT_TOL, golden_for, weight_file
    from oracle import julia_oracle as jo
    batch, seqs, ref_logits = golden_for(4, wide=True)
    items = [batch.sequence(b) for b in seqs]
    req = lib.Requests(items)
    m = lib.Model(weight_file("wide"), lib.BF16, 32768, 4096)
    h2 = m.share()
    try:
        for h in (m, h2):
            h.set_graph_cache(16)
        first = lib.serve([m, h2], req, max_batch_tokens=32768)
        info1 = [h.info() for h in (m, h2)]
        second = lib.serve([m, h2], req, max_batch_tokens=32768)
        info2 = [h.info() for h in (m, h2)]
    finally:
        h2.close()
        m.close()
    caps1 = sum(i["graph_captures"] for i in info1)
    caps2 = sum(i["graph_captures"] for i in info2)
    reps2 = sum(i["graph_replays"] for i in info2) - sum(i["graph_replays"] for i in info1)
    print("micro-batches", first.n_batches, "captured", caps1, "then", caps2, "replays in the second pass", reps2)
    if info1[0]["debug"] == 0:  # debugging switches (JL_DEBUG_SYNC at load) turn graph replay off
        assert caps1 >= 1 and caps2 == caps1 and reps2 == second.n_batches
    assert np.array_equal(first.logits, second.logits) and np.array_equal(first.probs, second.probs)
    bound = LOGIT_TOL[("wide", "bf16")]
    worst = {"logit": 0.0, "prob": 0.0}
    for r, (ids, marks, qt) in enumerate(items):
        ref = np.asarray(ref_logits[r])
        worst["logit"] = max(worst["logit"], float(np.max(np.abs(first.request_logits(r) - ref))))
        ro = jo.read_offs(ref, np.array([0, len(ids)]), np.asarray(marks), np.array([qt]))
        dp = float(np.max(np.abs(first.probs[req.mask_offsets[r]:req.mask_offsets[r + 1]] - ro["probs"])))
        worst["prob"] = max(worst["prob"], dp)
    print("bucketed serve vs oracle", worst)
    assert worst["logit"] <= bound and worst["prob"] <= BF16_PROB_BOUND
