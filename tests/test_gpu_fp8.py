"""FP8 mode (JL_FP8): the e4m3 QKV and W_i products against the oracle.

The oracle's FP8 variant rounds the same operands to e4m3 from the format's
definition (pinned to torch's float8_e4m3fn on the CPU): each normalized
activation row and each weight row scaled so that its largest magnitude is
448. The bf16 roundings elsewhere in the pass (attention operands, the GEGLU
output, the other products) move a normalized value across an e4m3 rounding
boundary now and then, one step of 2^-3 on that element, so the two sides are
compared at the bf16 mode's tight bound, not closer.
"""
import numpy as np
import pytest

from encoder_transformer_amd import synth
from gpu_common import marker_slices, run_logits, run_stage, stage_batch, weight_file, weights_of

pytestmark = pytest.mark.gpu

FP8_LOGIT_TIGHT = 3e-3


@pytest.fixture(scope="module")
def models8():
    from encoder_transformer_amd import lib
    path = synth.cached_weight_file()
    m = {"fp8": lib.Model(path, lib.FP8, 20000, 1024), "bf16": lib.Model(path, lib.BF16, 20000, 1024)}
    yield m
    for v in m.values():
        v.close()


def make(kind, n):
    return synth.make_batch(n) if kind == "config" else synth.make_ragged_batch(n, 2 + n, 24, 300)


@pytest.mark.parametrize("kind,n", [("config", 0), ("config", 1), ("ragged", 0), ("ragged", 1), ("ragged", 2)])
def test_fp8_logits_against_the_e4m3_oracle(models8, oracle_weights, kind, n):
    from oracle import julia_oracle as jo
    batch = make(kind, n)
    ref8 = jo.forward(oracle_weights, batch, fp8=True)
    got = run_logits(models8["fp8"], batch)
    err = float(np.max(np.abs(got - ref8)))
    print(kind, n, "max |dlogit| against the e4m3 oracle", err)
    assert err <= FP8_LOGIT_TIGHT
    # the e4m3 products ran: the logits differ from the bf16 mode's
    assert not np.array_equal(got, run_logits(models8["bf16"], batch))


def test_fp8_sequence_alone_equals_packed(models8):
    """The e4m3 products scale per row: a sequence's logits do not depend on the batch."""
    batch = synth.make_ragged_batch(7, 4, 24, 300)
    packed = run_logits(models8["fp8"], batch)
    sl = marker_slices(batch)
    for b in range(batch.n_seqs):
        assert np.array_equal(run_logits(models8["fp8"], batch.subset([b])), packed[sl[b]]), b



def test_fp8_multi_round_grids(models8, oracle_weights):
    """4,288 tokens: the e4m3 products run 64 x 128 tiles over several rounds
    of work-groups (two per CU), beyond the one-round grids of the cases above."""
    from oracle import julia_oracle as jo
    batch = synth.make_ragged_batch(300, 3, 1300, 1700)
    assert ((int(batch.seq_offsets[-1]) + 63) // 64) * (2304 // 128) > 256
    ref8 = jo.forward(oracle_weights, batch, fp8=True)
    err = float(np.max(np.abs(run_logits(models8["fp8"], batch) - ref8)))
    print("max |dlogit| against the e4m3 oracle", err)
    assert err <= FP8_LOGIT_TIGHT


@pytest.fixture(scope="module")
def jit8():
    from encoder_transformer_amd import lib
    m = {name: lib.Model(weight_file(name), lib.FP8, 20000, 1024) for name in ("jit02", "jit05")}
    yield m
    for v in m.values():
        v.close()


def rowblock_batch():
    """The stage batch packed in front of eight 1,024-token sequences: over
    8,192 tokens, so the forward takes the row-block layer kernel."""
    return synth.concat([stage_batch(), synth.make_batch(2).subset(range(8))])


_STAGE_REFS = {}


def stage_refs(name):
    """The oracle's hidden states of the stage batch after layers 1-4, with
    e4m3 products and exact ones."""
    if name not in _STAGE_REFS:
        from oracle import julia_oracle as jo
        W = jo.OracleWeights(weights_of(name))
        batch = stage_batch()
        per8, per = {s: [] for s in (1, 2, 3, 4)}, {s: [] for s in (1, 2, 3, 4)}
        for b in range(batch.n_seqs):
            ids, _, _ = batch.sequence(b)
            x8 = x = jo.embed(W, ids)
            for l in range(4):
                x8 = jo.encoder_layer(W, l, x8, fp8=True)
                x = jo.encoder_layer(W, l, x)
                per8[l + 1].append(x8)
                per[l + 1].append(x)
        _STAGE_REFS[name] = ({s: np.concatenate(v) for s, v in per8.items()},
                             {s: np.concatenate(v) for s, v in per.items()})
    return _STAGE_REFS[name]


def check_fp8_stages(model, name, batch):
    """Hidden states of the stage batch's rows (at the front of `batch`) after
    the first four layers (jittered weights at std 0.02 and 0.05): the e4m3
    rounding moves the oracle's states by 13x the bf16 mode's error there
    (1.6e-2 against 1.2e-3 after layer 1 at std 0.02), so the FP8 mode must
    stay within a quarter of that gap of the oracle's e4m3 forward -- not
    near its exact forward, and not off by a scale.  Further on, bf16-level
    differences ahead of each quantization flip a few e4m3 codes (steps of
    2^-3) and the flips compound: after 22 layers at std 0.05 the logits are
    0.064 from the e4m3 oracle and 0.056 from the exact one, which are 0.086
    apart."""
    per8, per = stage_refs(name)
    n = stage_batch().n_tokens
    # Measured at std 0.02: 0.18-0.20 of the gap from the e4m3 oracle and
    # 0.99-1.01 of it from the exact one.  At std 0.05 the bf16 attention
    # ahead of layer 0's W_i already leaves differences of ~2e-2 in its
    # input, which flip some e4m3 codes, and the flips compound: 0.35, 0.47,
    # 0.54, 0.51 of the gap after layers 1-4 (0.98-1.06 from the exact one);
    # there the e4m3 oracle is matched after layer 1 only, and the exact
    # oracle must be missed at every stage.
    frac = {"jit02": 0.3, "jit05": 0.5}[name]
    check_upto = {"jit02": 4, "jit05": 1}[name]  # stages up to this one held to frac
    rows = []
    for st in (1, 2, 3, 4):
        got = run_stage(model, batch, st)[:n]
        e8 = float(np.max(np.abs(got - per8[st])))
        ex = float(np.max(np.abs(got - per[st])))
        gap = float(np.max(np.abs(per8[st] - per[st])))
        print(name, "stage", st, "max |d| vs e4m3 oracle", e8, "vs exact oracle", ex, "e4m3 gap", gap)
        rows.append((st, e8, ex, gap))
    for st, e8, ex, gap in rows:
        assert ex >= 0.75 * gap, (st, e8, ex, gap)  # not the exact products
        if st <= check_upto:
            assert e8 <= frac * gap, (st, e8, ex, gap)  # the e4m3 products, scaled as the oracle scales them


@pytest.mark.parametrize("name", ["jit02", "jit05"])
def test_fp8_stages_follow_the_e4m3_products(jit8, name):
    """The per-GEMM schedule (the stage batch alone, 506 tokens)."""
    check_fp8_stages(jit8[name], name, stage_batch())


@pytest.mark.parametrize("name", ["jit02", "jit05"])
def test_fp8_rowblock_stages_follow_the_e4m3_products(jit8, name):
    """The row-block schedule: W_i and the next layer's QKV on e4m3 codes of
    the LayerNorm rows inside the layer kernel (the stage batch in front of
    eight 1,024-token sequences)."""
    batch = rowblock_batch()
    assert batch.n_tokens >= 8192
    check_fp8_stages(jit8[name], name, batch)

