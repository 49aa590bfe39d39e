"""Micro-batch planning of the serving front (jl_serve_plan, host only):
the documented rule -- requests longest first, equal lengths in request
order, a micro-batch closes when the next request would exceed the token,
marker or sequence budget -- written out here and compared with the
library on random queues, plus the budget invariants and the errors."""
import numpy as np
import pytest

from encoder_transformer_amd import lib


def _queue(seed, n, lo=1, hi=3000):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, n)
    lens[::7] = lens[0]  # some equal lengths, to pin the stable order
    marks = rng.integers(2, 21, n)
    return lib.Requests([([5] * int(L), list(range(int(m))), 0) for L, m in zip(lens, marks)])


def _rule(req, max_t, max_m, max_s):
    lens = np.diff(req.id_offsets)
    mk = np.diff(req.mask_offsets)
    order = sorted(range(req.n), key=lambda r: -lens[r])  # sorted() is stable
    batch_of = [0] * req.n
    b, t, m, s = 0, 0, 0, 0
    for r in order:
        if s and (t + lens[r] > max_t or m + mk[r] > max_m or s + 1 > max_s):
            b, t, m, s = b + 1, 0, 0, 0
        t, m, s = t + lens[r], m + mk[r], s + 1
        batch_of[r] = b
    return order, batch_of, (b + 1 if req.n else 0)


@pytest.mark.parametrize("seed,n,max_t,max_m,max_s", [(0, 50, 8192, 4096, 4096), (1, 300, 4096, 200, 64),
                                                      (2, 17, 3000, 40, 3), (3, 1, 5000, 30, 1)])
def test_plan_matches_the_rule(seed, n, max_t, max_m, max_s):
    req = _queue(seed, n)
    order, batch_of, nb = lib.serve_plan(req, max_t, max_m, max_s)
    ref_order, ref_batch, ref_nb = _rule(req, max_t, max_m, max_s)
    assert list(order) == ref_order and list(batch_of) == ref_batch and nb == ref_nb
    lens, mk = np.diff(req.id_offsets), np.diff(req.mask_offsets)
    assert sorted(order) == list(range(n))
    assert list(batch_of[order]) == sorted(batch_of[order])  # batches are contiguous along the order
    for b in range(nb):
        sel = batch_of == b
        assert sel.any() and lens[sel].sum() <= max_t and mk[sel].sum() <= max_m and sel.sum() <= max_s


def test_plan_empty_and_errors():
    assert lib.serve_plan(lib.Requests([]), 100, 10, 10)[2] == 0
    req = lib.Requests([([5] * 50, [0, 1], 0), ([5] * 150, [0, 1], 0)])
    with pytest.raises(lib.JLError) as e:
        lib.serve_plan(req, 100, 10, 10)
    assert e.value.code == lib.ERR_LENGTH
    with pytest.raises(lib.JLError) as e:
        lib.serve_plan(req, 0, 10, 10)
    assert e.value.code == lib.ERR_ARG
