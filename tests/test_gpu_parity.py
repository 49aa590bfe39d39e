"""GPU parity of the HIP forward pass against the CPU oracle (needs an MI355X).

All calls go through the C ABI (libjl.so) via the ctypes binding.
* stage parity: hidden states after encoder layers, the head input and both
  head layers, both precisions and both bf16 schedules, on two weight sets
  with jittered LayerNorm gains (std 0.02 and 0.05), at per-stage bounds;
* logits: configurations 0 and 1 against the live oracle, configurations 2-4
  (full batches, the benchmark's launch shapes) against stored oracle logits
  of sampled sequences (tests/golden/make_oracle_expected.py) at the tight
  bounds; the wide weight set (std 0.05, logits of order one) on every
  configuration, with argmax agreement over the 256-question mix;
* long sequences: hidden rows at positions up to 8,191 of the 16 x 8,192
  batch against stored oracle rows, both precisions and both bf16 schedules;
* read-offs: jl_probs against the oracle's read-offs;
* invariances: batch composition, sequence order, run-to-run determinism;
* edge cases: empty batch, 2-token sequences, ragged tails, bad ids, errors.
"""
import os

import numpy as np
import pytest

from encoder_transformer_amd import synth

from gpu_common import (BF16_ARGMAX_AGREEMENT, BF16_LOGIT_BOUND, BF16_PROB_BOUND, FP32_LOGIT_BOUND, GOLDEN,
                        BF16_LOGIT_TIGHT, FP32_LOGIT_TIGHT, LOGIT_TOL, LONG_TOL, MAX_MARKERS, MAX_TOKENS,
                        STAGE_TOL, STAGES, argmax_report, device_ids, golden,
                        golden_for, marker_slices, oracle_stages, run_logits, run_stage, stage_batch,
                        weight_file, weights_of)

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def models():
    import torch
    from encoder_transformer_amd import lib
    assert torch.cuda.is_available()
    path = synth.cached_weight_file()
    m = {"bf16": lib.Model(path, lib.BF16, MAX_TOKENS, MAX_MARKERS),
         "fp32": lib.Model(path, lib.FP32, MAX_TOKENS, MAX_MARKERS)}
    yield m
    for v in m.values():
        v.close()


@pytest.fixture(scope="module")
def set_models():
    """bf16 and FP32 handles per weight set, loaded on first use."""
    from encoder_transformer_amd import lib
    cache = {}

    def get(name, prec):
        if (name, prec) not in cache:
            cache[(name, prec)] = lib.Model(weight_file(name), lib.BF16 if prec == "bf16" else lib.FP32,
                                            MAX_TOKENS, MAX_MARKERS)
        return cache[(name, prec)]
    yield get
    for v in cache.values():
        v.close()


def small_ragged():
    """Three sequences with ragged lengths (tails of 9, 1 and 63 tokens past a 64-tile)."""
    return synth.make_ragged_batch(seed=77, n_seqs=3, min_len=70, max_len=200)


_STAGE_REF = {}


def stage_reference(name):
    """Oracle hidden states of the stage batch at STAGES (computed once per weight set)."""
    if name not in _STAGE_REF:
        from oracle import julia_oracle as jo
        _STAGE_REF[name] = oracle_stages(jo.OracleWeights(weights_of(name)), stage_batch(), STAGES)
    return _STAGE_REF[name]


def check_stages(errs, name, prec):
    tol = STAGE_TOL[(name, prec)]
    print(name, prec, {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {s: (e, tol[s]) for s, e in errs.items() if not (np.isfinite(e) and e <= tol[s])}
    assert not bad, bad


@pytest.mark.parametrize("name", ["jit02", "jit05"])
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_stage_parity(set_models, name, prec):
    """Hidden states after encoder layers 1-4, 12, 22, the head input and both
    head layers (per-GEMM schedule: 506 tokens), against the oracle."""
    batch = stage_batch()
    ref = stage_reference(name)
    errs = {}
    for s in STAGES:
        got = run_stage(set_models(name, prec), batch, s)
        assert got.shape == ref[s].shape
        errs[s] = float(np.max(np.abs(got - ref[s])))
    check_stages(errs, name, prec)


def rowblock_batch():
    """The stage batch packed in front of eight 1,024-token sequences: over
    8,192 tokens, so a bf16 forward takes the row-block layer kernel."""
    return synth.concat([stage_batch(), synth.make_batch(2).subset(range(8))])


@pytest.mark.parametrize("name", ["jit02", "jit05"])
def test_stage_parity_rowblock_path(set_models, name):
    """Hidden states of the row-block path (bf16, >= 8,192 tokens) against the
    oracle, on the rows of the stage batch at the front (the oracle runs only
    those), at the stage-parity bounds."""
    from oracle import julia_oracle as jo
    batch = rowblock_batch()
    assert batch.n_tokens >= 8192
    head = stage_batch()
    rows = head.n_tokens
    ref = stage_reference(name)
    m = set_models(name, "bf16")
    errs = {}
    for st in STAGES:
        got = run_stage(m, batch, st)
        sub = got[:head.n_markers] if st == 25 else got[:rows]
        errs[st] = float(np.max(np.abs(sub - ref[st])))
    check_stages(errs, name, "bf16")
    got = run_logits(m, batch)
    ref_l = jo.forward(jo.OracleWeights(weights_of(name)), head)
    err = float(np.max(np.abs(got[:head.n_markers] - ref_l)))
    print("row-block bf16 max |dlogit|", err)
    assert err <= LOGIT_TOL[(name, "bf16")]


@pytest.mark.parametrize("name", ["jit02", "jit05"])
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_logits_stage_batch(set_models, name, prec):
    from oracle import julia_oracle as jo
    W = jo.OracleWeights(weights_of(name))
    batch = stage_batch()
    ref = jo.forward(W, batch)
    got = run_logits(set_models(name, prec), batch)
    err = float(np.max(np.abs(got - ref)))
    print(name, prec, "max |dlogit|", err)
    assert err <= LOGIT_TOL[(name, prec)]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_logits_random_ragged_batches(models, oracle_weights, seed, prec):
    """Seeded random packs of 1-6 sequences of 24-300 tokens (question types,
    option counts and lengths drawn as in the serving mix): every length
    class against the 64-key tiles, window edges and item boundaries."""
    from oracle import julia_oracle as jo
    batch = synth.make_ragged_batch(seed, 1 + seed, 24, 300)
    ref = jo.forward(oracle_weights, batch)
    got = run_logits(models[prec], batch)
    err = float(np.max(np.abs(got - ref)))
    print(prec, seed, np.diff(batch.seq_offsets).tolist(), "max |dlogit|", err)
    assert err <= (FP32_LOGIT_TIGHT if prec == "fp32" else BF16_LOGIT_TIGHT)


@pytest.mark.parametrize("config", [0, 1])
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_logits_small_configs(models, oracle_weights, config, prec):
    from oracle import julia_oracle as jo
    batch = synth.make_batch(config)
    ref = jo.forward(oracle_weights, batch)
    got = run_logits(models[prec], batch)
    err = float(np.max(np.abs(got - ref)))
    rep = argmax_report(ref, got, batch.seq_offsets, batch.mask_positions, LOGIT_TOL[("standard", prec)])
    print(prec, config, "max |dlogit|", err, rep)
    if prec == "fp32":
        assert err <= FP32_LOGIT_BOUND and err <= FP32_LOGIT_TIGHT
        assert rep["clear_agree"] == rep["clear"]
    else:
        assert err <= BF16_LOGIT_BOUND and err <= BF16_LOGIT_TIGHT
        assert rep["clear_agree"] == rep["clear"]


def compare_golden(got, batch, seqs, ref_logits, name, prec, config):
    """max |dlogit| over the stored sequences, and argmax agreement: a question
    is a tie when the oracle's top-2 gap is within twice the logit bound
    (either answer is then correct); every other question must agree in FP32,
    >= 99.5% of them in bf16 (the benchmark spec)."""
    assert got.shape == (batch.n_markers,) and np.all(np.isfinite(got))
    sl = marker_slices(batch)
    ref = np.concatenate([np.asarray(r) for r in ref_logits])
    sub = np.concatenate([got[sl[s]] for s in seqs])
    err = float(np.max(np.abs(sub - ref)))
    so = np.concatenate([[0], np.cumsum([len(r) for r in ref_logits])])
    bound = LOGIT_TOL[(name, prec)]
    rep = argmax_report(ref, sub, so, np.arange(len(ref)), bound)
    print(name, prec, config, "sampled seqs", len(seqs), "max |dlogit|", err, rep)
    assert err <= bound
    if prec == "fp32":
        assert rep["clear_agree"] == rep["clear"]
    else:
        assert rep["clear_agree"] >= BF16_ARGMAX_AGREEMENT * rep["clear"]
    return rep


@pytest.mark.parametrize("config", [2, 3, 4])
@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_logits_golden_full_batches(models, config, prec):
    """The full batches in the benchmark's launch shapes (published init)
    against stored oracle logits of sampled sequences, at the tight bounds."""
    batch, seqs, ref_logits = golden_for(config)
    compare_golden(run_logits(models[prec], batch), batch, seqs, ref_logits, "standard", prec, config)


@pytest.mark.parametrize("config", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_logits_golden_wide(set_models, config, prec):
    """The wide weight set (std 0.05), whose option logits spread to order
    one: every question of configurations 0-2 and of the 256-sequence mix,
    two of the 16 x 8,192 batch; argmax agreement is meaningful here."""
    batch, seqs, ref_logits = golden_for(config, wide=True)
    rep = compare_golden(run_logits(set_models("wide", prec), batch), batch, seqs, ref_logits, "wide", prec,
                         config)
    # FP32: the same argmax on every question, near-ties included.  bf16:
    # compare_golden requires it on every question whose oracle top-2 gap
    # exceeds twice the bound; the agreement over all questions is printed
    # (on the 256-question mix 249 of 256 measured: the 7 others are
    # near-ties that bf16 rounding reorders)
    if prec == "fp32":
        assert rep["agree"] == rep["questions"]
    print("wide", prec, config, "argmax agreement over all questions", rep["agree"], "/", rep["questions"])
    if config == 4:
        assert rep["questions"] == 256


def long_rows():
    d = np.load(os.path.join(GOLDEN, "oracle_rows_long.npz"))
    return {k: d[k] for k in d.files}


@pytest.mark.parametrize("name", ["standard", "wide"])
@pytest.mark.parametrize("path", ["fp32", "bf16-row-block", "bf16-per-gemm"])
def test_long_sequence_rows(set_models, name, path):
    """Hidden rows of two 8,192-token sequences of the 16 x 8,192 batch at
    positions up to 8,191 (RoPE table ends, tile and window edges), run as the
    whole batch, against stored oracle rows."""
    import hashlib
    import torch
    d = long_rows()
    batch = synth.make_batch(3)
    h = hashlib.sha256()
    for a in (batch.ids, batch.seq_offsets, batch.mask_positions, batch.qtype):
        h.update(np.ascontiguousarray(a, np.int32).tobytes())
    assert h.hexdigest().encode() == d["batch_digest"].tobytes()
    prec = "fp32" if path == "fp32" else "bf16"
    m = set_models(name, prec)
    if path == "bf16-per-gemm":
        m.set_row_block_min_tokens(1 << 62)
    try:
        ids = device_ids(batch)
        pos = d["positions"].astype(np.int64)
        sl = marker_slices(batch)
        errs = {}
        for st in (1, 2, 22, 24, 25):
            out = m.debug_hidden(ids, batch.seq_offsets, batch.mask_positions, batch.qtype, st)
            for s in d["seqs"]:
                s = int(s)
                rows = pos + int(batch.seq_offsets[s]) if st != 25 else np.arange(sl[s].start, sl[s].stop)
                got = out[torch.from_numpy(rows).to(out.device)].cpu().numpy().astype(np.float64)
                ref = d[f"{name}_s{s}_stage{st}"].astype(np.float64)
                errs[st] = max(errs.get(st, 0.0), float(np.max(np.abs(got - ref))))
        lg = run_logits(m, batch)
        errs["logits"] = max(float(np.max(np.abs(lg[sl[int(s)]] - d[f"{name}_s{int(s)}_logits"])))
                             for s in d["seqs"])
    finally:
        m.set_row_block_min_tokens(8192)
    tol = LONG_TOL[(name, prec)]
    print(name, path, {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: (e, tol[k]) for k, e in errs.items() if not (np.isfinite(e) and e <= tol[k])}
    assert not bad, bad


@pytest.mark.parametrize("wide", [False, True])
def test_golden_inputs_unchanged(wide):
    """The stored oracle logits belong to today's generator output."""
    import hashlib
    g = golden(wide)
    for c, entry in g["configs"].items():
        b = synth.make_batch(int(c))
        h = hashlib.sha256()
        for a in (b.ids, b.seq_offsets, b.mask_positions, b.qtype):
            h.update(np.ascontiguousarray(a, np.int32).tobytes())
        assert h.hexdigest() == entry["batch_digest"], c


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_probs_and_read_offs(models, oracle_weights, prec):
    import torch
    from oracle import julia_oracle as jo
    batch = synth.make_batch(2)
    logits_t = models[prec].forward(device_ids(batch), batch.seq_offsets, batch.mask_positions, batch.qtype)
    probs, answer, argmax, maxprob = models[prec].probs(logits_t, batch.seq_offsets, batch.mask_positions,
                                                        batch.qtype)
    torch.cuda.synchronize()
    lg = logits_t.cpu().numpy().astype(np.float64)
    # the same logits through the oracle's read-offs
    r = jo.read_offs(lg, batch.seq_offsets, batch.mask_positions, batch.qtype)
    assert np.max(np.abs(probs.cpu().numpy() - r["probs"])) <= 1e-6
    assert np.array_equal(argmax.cpu().numpy(), r["argmax"])
    assert np.max(np.abs(maxprob.cpu().numpy() - r["maxprob"])) <= 1e-6
    assert np.max(np.abs(answer.cpu().numpy() - r["answer"])) <= 1e-5
    # and against the oracle's own logits for the sampled sequences
    b2, seqs, ref_logits = golden_for(2)
    ref = np.concatenate([np.asarray(x) for x in ref_logits])
    rr = jo.read_offs(ref, batch.seq_offsets, batch.mask_positions, batch.qtype)
    dp = float(np.max(np.abs(probs.cpu().numpy() - rr["probs"])))
    print(prec, "max |dprob|", dp)
    assert dp <= BF16_PROB_BOUND


@pytest.mark.parametrize("path", ["fp32", "bf16-per-gemm", "bf16-row-block"])
def test_batch_composition_and_order(models, path):
    """A sequence's logits do not depend on its neighbours or its place in the
    batch: bitwise, within one code path."""
    m = models["fp32" if path == "fp32" else "bf16"]
    if path == "bf16-row-block":
        m.set_row_block_min_tokens(0)
    elif path == "bf16-per-gemm":
        m.set_row_block_min_tokens(1 << 62)
    try:
        batch = synth.make_batch(4).subset(list(range(12)))
        packed = run_logits(m, batch)
        sl = marker_slices(batch)
        for b in (0, 5, 11):
            alone = run_logits(m, batch.subset([b]))
            assert np.array_equal(alone, packed[sl[b]]), b
        perm = [7, 2, 11, 0, 9, 4, 1, 10, 3, 8, 6, 5]
        got = run_logits(m, batch.subset(perm))
        expect = np.concatenate([packed[sl[b]] for b in perm])
        assert np.array_equal(got, expect)
    finally:
        m.set_row_block_min_tokens(8192)


def test_per_gemm_tile_regimes_bitwise(models):
    """The per-GEMM schedule picks its tiles and pipeline depth from the packed
    token count T: for the N = 384 residual updates 32 x 64 tiles (up to 42
    row blocks of 32), 64 x 64 (up to 42 of 64), 6-stage 64 x 128 (up to 85
    of 64) and the 2-stage tiles of larger grids.  Each output element still
    sums over K in the same order, so a sequence's logits are bitwise the same
    in every regime."""
    def regime(t):
        if -(-t // 32) * 6 <= 256:
            return "32x64"
        if -(-t // 64) * 6 <= 256:
            return "64x64"
        return "64x128/6" if -(-t // 64) * 3 <= 256 else "64x128/2"

    m = models["bf16"]
    base = synth.make_batch(4)
    lens = np.diff(base.seq_offsets)
    s0 = int(np.argmax(lens < 1300))
    others = [b for b in range(base.n_seqs) if b != s0]
    totals = lens[s0] + np.cumsum(lens[others])
    m.set_row_block_min_tokens(1 << 62)
    try:
        ref = run_logits(m, base.subset([s0]))
        regimes = {regime(int(lens[s0]))}
        for target in (2000, 4000, 6200):
            k = int(np.searchsorted(totals, target)) + 1
            batch = base.subset([s0] + others[:k])
            regimes.add(regime(batch.n_tokens))
            got = run_logits(m, batch)
            assert np.array_equal(got[:len(ref)], ref), (target, batch.n_tokens)
        assert len(regimes) == 4, regimes
    finally:
        m.set_row_block_min_tokens(8192)


def test_row_block_and_per_gemm_paths_agree(models):
    """The two bf16 schedules compute the same function (rounding aside)."""
    m = models["bf16"]
    batch = synth.make_batch(2)
    try:
        m.set_row_block_min_tokens(0)
        a = run_logits(m, batch)
        m.set_row_block_min_tokens(1 << 62)
        b = run_logits(m, batch)
    finally:
        m.set_row_block_min_tokens(8192)
    err = float(np.max(np.abs(a - b)))
    print("row-block vs per-GEMM max |dlogit|", err)
    assert err <= BF16_LOGIT_TIGHT


def test_determinism(models):
    batch = synth.make_batch(2)
    a = run_logits(models["bf16"], batch)
    b = run_logits(models["bf16"], batch)
    assert np.array_equal(a, b)


def test_edge_cases(models, oracle_weights):
    import torch
    from encoder_transformer_amd import lib
    from oracle import julia_oracle as jo
    m = models["fp32"]
    # empty batch: nothing to do, no error
    out = torch.full((1,), 7.0, device="cuda:0")
    m.forward(torch.zeros(1, dtype=torch.int32, device="cuda:0"), [0], [], [], out=out)
    torch.cuda.synchronize()
    assert out.item() == 7.0
    # two-token sequences (both tokens are markers) next to a longer one
    tiny = synth.pack([np.array([synth.MASK, synth.MASK], np.int32),
                       synth.make_batch(0).ids, np.array([synth.MASK, 9, synth.MASK], np.int32)],
                      [np.array([0, 1]), synth.make_batch(0).mask_positions, np.array([0, 2])], [2, 0, 1])
    got = run_logits(m, tiny)
    ref = jo.forward(oracle_weights, tiny)
    assert np.max(np.abs(got - ref)) <= FP32_LOGIT_TIGHT
    # an out-of-range id poisons its own sequence only
    bad = synth.make_batch(4).subset([0, 1, 2])
    ids = bad.ids.copy()
    ids[bad.seq_offsets[1] + 3] = synth.VOCAB
    poisoned = synth.Batch(ids, bad.seq_offsets, bad.mask_positions, bad.qtype)
    got = run_logits(m, poisoned)
    sl = marker_slices(bad)
    clean = run_logits(m, bad)
    assert np.all(np.isnan(got[sl[1]]))
    assert np.array_equal(got[sl[0]], clean[sl[0]]) and np.array_equal(got[sl[2]], clean[sl[2]])
    # validation errors leave the output untouched
    b0 = synth.make_batch(0)
    out = torch.full((3,), 7.0, device="cuda:0")
    for so, mp, qt, code in [([0, 128], [15, 22, 29], [3], lib.ERR_QTYPE),
                             ([0, 128], [15], [0], lib.ERR_OPTIONS),
                             ([0, 128], [15, 22, 29], [2], lib.ERR_OPTIONS),
                             ([0, 0], [15, 22], [0], lib.ERR_LENGTH)]:
        with pytest.raises(lib.JLError) as e:
            m.forward(device_ids(b0), so, mp, qt, out=out)
        assert e.value.code == code
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("path", ["fp32", "bf16-per-gemm", "bf16-row-block"])
def test_out_of_range_id_poisons_its_sequence_only(models, path):
    m = models["fp32" if path == "fp32" else "bf16"]
    if path == "bf16-row-block":
        m.set_row_block_min_tokens(0)
    elif path == "bf16-per-gemm":
        m.set_row_block_min_tokens(1 << 62)
    try:
        bad = synth.make_batch(4).subset([0, 1, 2])
        for pos, val in ((bad.seq_offsets[1] + 3, synth.VOCAB), (bad.seq_offsets[2] + 70, -1)):
            ids = bad.ids.copy()
            ids[pos] = val
            got = run_logits(m, synth.Batch(ids, bad.seq_offsets, bad.mask_positions, bad.qtype))
            clean = run_logits(m, bad)
            sl = marker_slices(bad)
            hit = int(np.searchsorted(bad.seq_offsets, pos, side="right") - 1)
            assert np.all(np.isnan(got[sl[hit]])), (path, pos)
            for b in range(3):
                if b != hit:
                    assert np.array_equal(got[sl[b]], clean[sl[b]]), (path, pos, b)
    finally:
        m.set_row_block_min_tokens(8192)


def test_capacity_error():
    import torch
    from encoder_transformer_amd import lib
    m = lib.Model(synth.cached_weight_file(), lib.BF16, max_tokens=512, max_markers=64)
    try:
        b = synth.make_batch(1)  # 1,024 tokens
        with pytest.raises(lib.JLError) as e:
            m.forward(device_ids(b), b.seq_offsets, b.mask_positions, b.qtype)
        assert e.value.code == lib.ERR_CAPACITY
        b0 = synth.make_batch(0)
        assert np.all(np.isfinite(run_logits(m, b0)))
    finally:
        m.close()
