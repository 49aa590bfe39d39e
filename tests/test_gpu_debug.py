"""Race and fault tooling of the C ABI (jl_set_debug, jl_check_guards, poisoned handles).

* Reversed work-group order (JL_DEBUG_REVERSE_BLOCKS): every GEMM, row-block,
  attention and scorer launch takes its tiles, row blocks, work items and
  heads last to first.  Each work-group computes its outputs alone and the
  scorer adds its partial sums in a fixed order, so logits and hidden states
  must equal the normal order's bit for bit, in every precision and both
  schedules; a difference would expose a race between work-groups.
* Per-launch synchronization (JL_DEBUG_SYNC, or the JL_DEBUG_SYNC environment
  variable at load) changes no result.
* Guard bands: caller-owned outputs sit between canary bands that no call may
  touch, and the handle's own workspace bands (jl_check_guards) stay intact,
  with the handle sized exactly to the batch so that a write one row past any
  buffer lands in a band.
* A device fault poisons the handle: forced from the host with
  JL_DEBUG_SIMULATE_FAULT (no kernel misbehaves); afterwards every call on the
  handle is refused with JL_ERR_DEVICE, while another handle over the same
  weights keeps working.
"""
import numpy as np
import pytest

from encoder_transformer_amd import synth

from gpu_common import device_ids, stage_batch

pytestmark = pytest.mark.gpu

CANARY = np.int32(0x7FA5A5A5)  # a NaN: any read of it would also show
BAND = 64                      # canary elements on each side of an output


@pytest.fixture(scope="module")
def models():
    import torch
    from encoder_transformer_amd import lib
    assert torch.cuda.is_available()
    path = synth.cached_weight_file()
    m = {"bf16": lib.Model(path, lib.BF16, 20000, 2048), "fp8": lib.Model(path, lib.FP8, 20000, 2048),
         "fp32": lib.Model(path, lib.FP32, 20000, 2048)}
    yield m
    for v in m.values():
        v.close()


def _schedule(model, name):
    model.set_row_block_min_tokens(0 if name == "row-block" else 2 ** 62)


def _run(model, batch, stages=(23, 25)):
    import torch
    ids = device_ids(batch)
    out = {"logits": model.forward(ids, batch.seq_offsets, batch.mask_positions, batch.qtype)}
    for s in stages:
        out[s] = model.debug_hidden(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, s)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _bitwise_equal(a, b):
    assert a.keys() == b.keys()
    for k in a:
        assert a[k].shape == b[k].shape, k
        diff = np.flatnonzero(a[k].view(np.int32).ravel() != b[k].view(np.int32).ravel())
        assert diff.size == 0, f"{k}: {diff.size} values differ, first at flat index {diff[0]}"


CASES = [("bf16", "per-gemm"), ("bf16", "row-block"), ("fp8", "per-gemm"), ("fp8", "row-block"),
         ("fp32", "per-gemm")]


@pytest.mark.parametrize("prec,sched", CASES)
def test_reversed_block_order_is_bitwise_identical(models, prec, sched):
    from encoder_transformer_amd import lib
    m = models[prec]
    _schedule(m, sched)
    # ragged tails (9, 1 and 63 rows past a 64-row tile) and the 16 x 1,024
    # configuration (many tiles and work items per launch)
    for batch in (stage_batch(), synth.make_batch(2)):
        m.set_debug(0)
        ref = _run(m, batch)
        m.set_debug(lib.DEBUG_REVERSE_BLOCKS)
        try:
            got = _run(m, batch)
        finally:
            m.set_debug(0)
        _bitwise_equal(ref, got)
    m.set_row_block_min_tokens(8192)


@pytest.mark.parametrize("prec,sched", [("bf16", "per-gemm"), ("bf16", "row-block"), ("fp32", "per-gemm")])
def test_debug_sync_changes_nothing(models, prec, sched):
    from encoder_transformer_amd import lib
    m = models[prec]
    _schedule(m, sched)
    batch = stage_batch()
    ref = _run(m, batch)
    m.set_debug(lib.DEBUG_SYNC)
    try:
        assert m.info()["debug"] == lib.DEBUG_SYNC
        got = _run(m, batch)
    finally:
        m.set_debug(0)
    _bitwise_equal(ref, got)
    m.set_row_block_min_tokens(8192)


def test_debug_sync_from_environment(models, monkeypatch):
    from encoder_transformer_amd import lib
    monkeypatch.setenv("JL_DEBUG_SYNC", "1")
    a = models["bf16"].share(4096, 512)
    monkeypatch.setenv("JL_DEBUG_SYNC", "0")
    b = models["bf16"].share(4096, 512)
    try:
        assert a.info()["debug"] == lib.DEBUG_SYNC
        assert b.info()["debug"] == 0
        batch = stage_batch()
        _bitwise_equal(_run(a, batch, ()), _run(b, batch, ()))
    finally:
        a.close()
        b.close()


def test_unknown_debug_flag_rejected(models):
    from encoder_transformer_amd import lib
    with pytest.raises(lib.JLError) as e:
        models["bf16"].set_debug(8)
    assert e.value.code == lib.ERR_ARG


def _guarded(torch, n, dtype=None, shape=None):
    """An output of n elements (rows of `shape`) between two canary bands:
    (whole buffer, interior view of `dtype`, float32 by default)."""
    dtype = dtype or torch.float32
    per = int(np.prod(shape[1:])) if shape else 1
    buf = torch.full((n * per + 2 * BAND,), 0, dtype=torch.int32, device="cuda:0")
    buf.fill_(int(CANARY))
    inner = buf[BAND:BAND + n * per]
    inner = inner.view(dtype) if dtype != torch.int32 else inner
    return buf, (inner.view(shape) if shape else inner)


def _bands_intact(buf):
    h = buf.cpu().numpy()
    assert np.all(h[:BAND] == CANARY), "canary band before the output overwritten"
    assert np.all(h[-BAND:] == CANARY), "canary band after the output overwritten"


@pytest.mark.parametrize("prec,sched", CASES)
def test_outputs_and_workspace_stay_inside_their_bounds(models, prec, sched):
    import torch
    batch = stage_batch()
    T, M, B = int(batch.seq_offsets[-1]), batch.n_markers, batch.n_seqs
    m = models[prec].share(T, M)  # buffers sized exactly to this batch
    try:
        _schedule(m, sched)
        ids = device_ids(batch)
        lb, logits = _guarded(torch, M)
        m.forward(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, out=logits)
        pb, probs = _guarded(torch, M)
        ab, answer = _guarded(torch, B)
        gb, argmax = _guarded(torch, B, torch.int32)
        xb, maxprob = _guarded(torch, B)
        m.probs(logits, batch.seq_offsets, batch.mask_positions, batch.qtype, out=(probs, answer, argmax, maxprob))
        hb, hidden = _guarded(torch, T, shape=(T, 384))
        m.debug_hidden(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, 23, out=hidden)
        kb, marks = _guarded(torch, M, shape=(M, 384))
        m.debug_hidden(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, 25, out=marks)
        torch.cuda.synchronize()
        for buf in (lb, pb, ab, gb, xb, hb, kb):
            _bands_intact(buf)
        assert np.isfinite(logits.cpu().numpy()).all()
        assert np.isfinite(hidden.cpu().numpy()).all()
        m.check_guards()
    finally:
        m.close()


def test_static_entry_point_outputs_stay_inside_their_bounds(models):
    import torch
    batch = stage_batch()
    m = models["bf16"]
    lb, logits = _guarded(torch, batch.n_markers)
    m.forward_static(device_ids(batch), batch.seq_offsets, batch.mask_positions, batch.qtype, logits)
    torch.cuda.synchronize()
    _bands_intact(lb)
    assert np.isfinite(logits.cpu().numpy()).all()


def test_device_fault_poisons_the_handle(models):
    import torch
    from encoder_transformer_amd import lib
    batch = stage_batch()
    ids = device_ids(batch)
    bad = models["bf16"].share(4096, 512)
    good = models["bf16"].share(4096, 512)
    try:
        ref = _run(good, batch, ())["logits"]
        bad.set_debug(lib.DEBUG_SIMULATE_FAULT)
        with pytest.raises(lib.JLError) as e:
            bad.forward(ids, batch.seq_offsets, batch.mask_positions, batch.qtype)
        assert e.value.code == lib.ERR_DEVICE and "simulated device fault" in e.value.message
        torch.cuda.synchronize()  # the enqueued work itself ran normally
        info = bad.info()
        assert info["poisoned"] == 1 and info["debug"] == 0  # the flag is used up
        logits = torch.zeros(batch.n_markers, dtype=torch.float32, device="cuda:0")
        calls = [
            lambda: bad.forward(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, out=logits),
            lambda: bad.forward_static(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, logits),
            lambda: bad.probs(logits, batch.seq_offsets, batch.mask_positions, batch.qtype),
            lambda: bad.debug_hidden(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, 1),
            lambda: bad.profile_read(lib.K_MISC),
            lambda: bad.check_guards(),
            lambda: bad.route([([1, 2, 3], [2], [[7], [8], [9]])]),
            lambda: lib.serve([bad], lib.Requests([batch.sequence(0)]), 4096),
        ]
        for i, call in enumerate(calls):
            with pytest.raises(lib.JLError) as e:
                call()
            assert e.value.code == lib.ERR_DEVICE and "poisoned" in e.value.message, (i, e.value.message)
        torch.cuda.synchronize()
        assert np.all(logits.cpu().numpy() == 0), "a refused call wrote its output"
        # the device and the other handle over the same weights are unaffected
        _bitwise_equal({"logits": ref}, _run(good, batch, ()))
        assert good.info()["poisoned"] == 0
    finally:
        bad.close()
        good.close()
