"""Graph mode of jl_forward (jl_set_graph_cache) against eager execution.

Each captured graph is replayed several times, with eager work and
synchronizations of the program in between, and every replay must match the
eager logits bitwise: the kernels are the same and batch metadata is uploaded
per call.  Also covers a batch of an already cached shape with different
content, eviction when the cache is full, both schedules, and the NULL stream
(which always runs eagerly).
"""
import numpy as np
import pytest

from encoder_transformer_amd import synth

from gpu_common import MAX_MARKERS, device_ids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def model():
    import torch
    from encoder_transformer_amd import lib
    assert torch.cuda.is_available()
    m = lib.Model(synth.cached_weight_file(), lib.BF16, 20000, MAX_MARKERS)
    yield m
    m.close()


def _same_shape_other_content(batch, seed):
    """Same lengths and marker counts, different token ids and marker positions."""
    rng = np.random.default_rng(seed)
    ids = batch.ids.copy()
    special = ids < 5
    ids[~special] = rng.integers(5, synth.VOCAB, size=int((~special).sum()), dtype=np.int32)
    return synth.Batch(ids=ids, seq_offsets=batch.seq_offsets.copy(), mask_positions=batch.mask_positions.copy(),
                       qtype=batch.qtype.copy())


def _logits(model, batch, ids_dev, out, stream):
    import torch
    torch.cuda.synchronize()  # inputs and output fills were written on the default stream
    with torch.cuda.stream(stream):
        model.forward(ids_dev, batch.seq_offsets, batch.mask_positions, batch.qtype, out=out)
    stream.synchronize()
    return out.cpu().numpy().copy()


def test_graph_replays_match_eager(model):
    import torch
    stream = torch.cuda.Stream()
    a = synth.concat([synth.make_batch(0), synth.make_ragged_batch(11, 3, 40, 300)])
    b = synth.make_batch(1)
    a2 = _same_shape_other_content(a, 5)
    runs = {}
    for name, batch in (("a", a), ("b", b), ("a2", a2)):
        ids = device_ids(batch)
        out = torch.empty(batch.n_markers, dtype=torch.float32, device="cuda:0")
        model.set_graph_cache(0)
        eager = _logits(model, batch, ids, out, stream)
        runs[name] = (batch, ids, out, eager)
    model.set_graph_cache(4)
    try:
        for rep in range(3):
            for name in ("a", "b", "a", "a2"):
                batch, ids, out, eager = runs[name]
                out.fill_(float("nan"))
                got = _logits(model, batch, ids, out, stream)
                assert np.array_equal(got, eager), (name, rep)
                # the program's own eager work between replays
                x = torch.randn(1 << 16, device="cuda:0")
                torch.cuda.synchronize()
                assert torch.isfinite((x * 2).sum())
    finally:
        model.set_graph_cache(0)


def test_one_graph_serves_batches_of_one_shape(model):
    """The same sequences in another order: equal token, marker and work-item
    counts, other offsets, markers and types, through the same device buffers,
    so the cached graph is reused with the new call's metadata."""
    import torch
    stream = torch.cuda.Stream()
    parts = [synth.make_batch(0), synth.make_ragged_batch(12, 1, 90, 90), synth.make_ragged_batch(13, 1, 300, 300)]
    a = synth.concat(parts)
    b = synth.concat(parts[::-1])
    assert a.n_tokens == b.n_tokens and a.n_markers == b.n_markers
    assert not np.array_equal(a.seq_offsets, b.seq_offsets)
    ids = torch.empty(a.n_tokens, dtype=torch.int32, device="cuda:0")
    out = torch.empty(a.n_markers, dtype=torch.float32, device="cuda:0")
    eager = {}
    model.set_graph_cache(0)
    for name, batch in (("a", a), ("b", b)):
        ids.copy_(device_ids(batch))
        eager[name] = _logits(model, batch, ids, out, stream)
    model.set_graph_cache(2)
    try:
        for rep in range(3):
            for name, batch in (("a", a), ("b", b)):
                ids.copy_(device_ids(batch))
                torch.cuda.synchronize()
                out.fill_(float("nan"))
                assert np.array_equal(_logits(model, batch, ids, out, stream), eager[name]), (name, rep)
    finally:
        model.set_graph_cache(0)


def test_graph_cache_eviction_and_row_block(model):
    import torch
    stream = torch.cuda.Stream()
    small = synth.make_batch(0)
    big = synth.concat([synth.make_batch(0), synth.make_batch(2).subset(range(8))])  # row-block schedule
    assert big.n_tokens >= 8192
    data = []
    for batch in (small, big):
        ids = device_ids(batch)
        out = torch.empty(batch.n_markers, dtype=torch.float32, device="cuda:0")
        model.set_graph_cache(0)
        data.append((batch, ids, out, _logits(model, batch, ids, out, stream)))
    model.set_graph_cache(1)  # every switch of shape evicts the other graph
    try:
        for _ in range(2):
            for batch, ids, out, eager in data:
                out.zero_()
                assert np.array_equal(_logits(model, batch, ids, out, stream), eager)
    finally:
        model.set_graph_cache(0)


def test_null_stream_runs_eagerly(model):
    import torch
    batch = synth.make_batch(0)
    ids = device_ids(batch)
    model.set_graph_cache(0)
    eager = model.forward(ids, batch.seq_offsets, batch.mask_positions, batch.qtype).cpu().numpy()
    model.set_graph_cache(2)
    try:
        # torch's default stream is the NULL stream: this call cannot be captured
        got = model.forward(ids, batch.seq_offsets, batch.mask_positions, batch.qtype)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), eager)
    finally:
        model.set_graph_cache(0)
