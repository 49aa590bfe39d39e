"""Shared helpers of the GPU tests: models, device batches, oracle stages, metrics."""
import json
import os

import numpy as np

from encoder_transformer_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Bounds on the option logits (the benchmark spec): FP32 mode max |dlogit| <= 2e-3 with
# the same argmax; bf16 mode max |dlogit| <= 5e-2, max |dprob| <= 1e-2, argmax
# agreement >= 99.5% of questions.
FP32_LOGIT_BOUND = 2e-3
BF16_LOGIT_BOUND = 5e-2
BF16_PROB_BOUND = 1e-2
BF16_ARGMAX_AGREEMENT = 0.995

MAX_TOKENS = 300_000
MAX_MARKERS = 4_096

# Weight sets of the parity tests (synth.make_weights arguments):
#   standard  the published init: std 0.02, LayerNorm gains 1 and shifts 0;
#   wide      std 0.05: attention peaked, option logits spread to order one;
#   jit02     std 0.02 with LayerNorm gains 1 + N(0, 0.1^2), shifts N(0, 0.1^2);
#   jit05     std 0.05, jittered likewise.
WEIGHT_SETS = {
    "standard": dict(seed=0, norm_jitter=False, std=synth.INIT_STD),
    "wide": dict(seed=0, norm_jitter=False, std=synth.WIDE_STD),
    "jit02": dict(seed=3, norm_jitter=True, std=synth.INIT_STD),
    "jit05": dict(seed=3, norm_jitter=True, std=synth.WIDE_STD),
}
_WEIGHTS = {}


def weights_of(name):
    if name not in _WEIGHTS:
        _WEIGHTS[name] = synth.make_weights(**WEIGHT_SETS[name])
    return _WEIGHTS[name]


def weight_file(name):
    return synth.cached_weight_file(weights=weights_of(name), **WEIGHT_SETS[name])


# Hidden-state stages compared by the stage-parity tests (jl_debug_hidden):
# after encoder layers 1-4, 12 and 22, the head input (23), after the first
# head layer (24) and after the second at the markers (25).
STAGES = [1, 2, 3, 4, 12, 22, 23, 24, 25]


def stage_batch():
    """The 1 x 128 configuration and three ragged sequences of 70-200 tokens
    (tails of 9, 1 and 63 tokens past a 64-row tile), 506 tokens."""
    return synth.concat([synth.make_batch(0), synth.make_ragged_batch(seed=77, n_seqs=3, min_len=70, max_len=200)])


# Bounds on max |hidden - oracle| over the stage batch's rows, per weight set,
# precision and stage.  bf16: every GEMM and attention operand carries a
# relative rounding of up to 2^-9 (R22), so the error grows with depth and
# with the weights' scale; each bound is about twice the error measured on
# the MI355X for that stage.  FP32: products in FP32 against the float64
# oracle, ~1e-7 relative per layer.  A CPU test (test_parity_mutations.py)
# shows that each plausible mistake in the method moves some compared stage
# by at least 3x its bound.  Measured (per-GEMM and row-block schedules):
# jit02 bf16 1.2e-3 (stage 1) .. 7.2e-3 (23); jit05 bf16 2.2e-2 .. 0.45 (22);
# FP32 8e-7 .. 2.2e-6 (jit02) and 7.7e-6 .. 8.5e-5 (jit05).
STAGE_TOL = {
    ("jit02", "bf16"): {1: 2.5e-3, 2: 3.6e-3, 3: 4e-3, 4: 5e-3, 12: 9e-3, 22: 1.2e-2, 23: 1.45e-2, 24: 1.4e-2,
                        25: 1.3e-2},
    ("jit05", "bf16"): {1: 4.5e-2, 2: 8.5e-2, 3: 0.12, 4: 0.175, 12: 0.45, 22: 0.9, 23: 0.21, 24: 0.32, 25: 0.32},
    ("jit02", "fp32"): {1: 2e-6, 2: 2e-6, 3: 2e-6, 4: 2.5e-6, 12: 3.2e-6, 22: 4e-6, 23: 4.5e-6, 24: 4.5e-6,
                        25: 3.2e-6},
    ("jit05", "fp32"): {1: 1.6e-5, 2: 1.9e-5, 3: 2.5e-5, 4: 3.1e-5, 12: 8.7e-5, 22: 1.7e-4, 23: 3.8e-5, 24: 5.6e-5,
                        25: 4.9e-5},
}

# Logit bounds, about twice the largest error measured on the MI355X for
# that weight set and precision and inside the benchmark spec's bounds (FP32 2e-3,
# bf16 5e-2).  Published init: FP32 products against the float64 oracle
# drift by ~1e-7 relative per layer (measured: 1.4e-7 on the logits at full
# size); bf16 operands carry a relative rounding of up to 2^-9 on every GEMM
# and attention input (measured: 4.7e-4).  Wide weights (std 0.05): the
# hidden states grow to |x| ~ 25 and the logits spread to ~0.3 (measured:
# FP32 5.1e-6, bf16 2.6e-2).
FP32_LOGIT_TIGHT = 3e-7
BF16_LOGIT_TIGHT = 1e-3
LOGIT_TOL = {("standard", "fp32"): FP32_LOGIT_TIGHT, ("standard", "bf16"): BF16_LOGIT_TIGHT,
             ("jit02", "fp32"): FP32_LOGIT_TIGHT, ("jit02", "bf16"): BF16_LOGIT_TIGHT,
             ("wide", "fp32"): 1e-5, ("wide", "bf16"): 5e-2,
             ("jit05", "fp32"): 1e-5, ("jit05", "bf16"): 5e-2}

# Bounds on max |hidden - oracle| for the stored long-sequence rows (two
# 8,192-token sequences of the 16 x 8,192 batch), per weight set and
# precision: stages 1, 2 (a global and a window layer), 22, 24, 25 (markers)
# and the logits; about twice the measured error (the largest of the two
# bf16 schedules).
LONG_TOL = {
    ("standard", "bf16"): {1: 2e-3, 2: 2.6e-3, 22: 1.2e-2, 24: 1.3e-2, 25: 1.45e-2, "logits": 1e-3},
    ("standard", "fp32"): {1: 1e-6, 2: 1e-6, 22: 3.5e-6, 24: 4e-6, 25: 3.2e-6, "logits": 3e-7},
    ("wide", "bf16"): {1: 4e-2, 2: 6.2e-2, 22: 0.75, 24: 0.24, 25: 0.25, "logits": 3e-2},
    ("wide", "fp32"): {1: 1.3e-5, 2: 1.6e-5, 22: 1.5e-4, 24: 5e-5, 25: 5.2e-5, "logits": 7e-6},
}


def device_ids(batch, device=0):
    import torch
    return torch.from_numpy(np.ascontiguousarray(batch.ids, np.int32)).to(f"cuda:{device}")


def run_logits(model, batch):
    import torch
    out = model.forward(device_ids(batch), batch.seq_offsets, batch.mask_positions, batch.qtype)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def run_stage(model, batch, stage):
    import torch
    out = model.debug_hidden(device_ids(batch), batch.seq_offsets, batch.mask_positions, batch.qtype, stage)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_stages(W, batch, stages):
    """Oracle hidden states at the library's diagnostic stages, packed like the batch."""
    from oracle import julia_oracle as jo
    res = {s: [] for s in stages}
    for b in range(batch.n_seqs):
        ids, marks, qt = batch.sequence(b)
        x = jo.embed(W, ids)
        if 0 in res:
            res[0].append(x)
        for l in range(22):
            x = jo.encoder_layer(W, l, x)
            if l + 1 in res:
                res[l + 1].append(x)
        h = jo.head_input(W, x, qt)
        if 23 in res:
            res[23].append(h)
        h = jo.head_layer(W, 0, h)
        if 24 in res:
            res[24].append(h)
        if 25 in res:
            res[25].append(jo.head_layer(W, 1, h)[marks])
    return {s: np.concatenate(v) for s, v in res.items()}


def argmax_report(ref, got, seq_offsets, mask_positions, err_bound):
    """Argmax agreement per question; a question is a tie when the oracle's top-2
    gap is within 2 x `err_bound`, where either answer is correct."""
    agree = ties = clear = clear_agree = 0
    for b in range(len(seq_offsets) - 1):
        sel = (mask_positions >= seq_offsets[b]) & (mask_positions < seq_offsets[b + 1])
        r, g = ref[sel], got[sel]
        same = int(np.argmax(r)) == int(np.argmax(g))
        agree += same
        srt = np.sort(r)[::-1]
        if srt[0] - srt[1] <= 2 * err_bound:
            ties += 1
        else:
            clear += 1
            clear_agree += same
    return {"questions": len(seq_offsets) - 1, "agree": agree, "ties": ties, "clear": clear,
            "clear_agree": clear_agree}


def golden(wide=False):
    with open(os.path.join(GOLDEN, "oracle_logits_wide.json" if wide else "oracle_logits.json")) as f:
        return json.load(f)


def golden_for(config, wide=False):
    g = golden(wide)["configs"][str(config)]
    b = synth.make_batch(config)
    return b, g["seqs"], g["logits"]


def marker_slices(batch):
    out, o = [], 0
    for b in range(batch.n_seqs):
        n = len(batch.sequence(b)[1])
        out.append(slice(o, o + n))
        o += n
    return out
