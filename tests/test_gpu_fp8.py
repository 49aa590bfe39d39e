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
from gpu_common import marker_slices, run_logits

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
