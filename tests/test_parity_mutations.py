"""Every plausible mistake in the method fails some GPU parity test (CPU only).

Each mistake is planted in the oracle, never in the library: the oracle's
module attributes are patched (or a weight matrix is permuted) for the
duration of one run, on the inputs of a GPU parity test, and the test here
asserts that some quantity that GPU test compares moves by at least 3x that
test's bound, in the bf16 mode and in the FP32 mode.  A GPU path that made the
mistake would then fail its parity test with room to spare.

Quantities compared (tests/test_gpu_parity.py):
* the stage batch's hidden states after encoder layers 1-4, 12, 22, the head
  input and both head layers, and its logits, on the jittered weight sets
  with std 0.02 and 0.05 (STAGE_TOL, LOGIT_TOL);
* rows of an 8,192-token sequence after the first two layers, at
  positions up to 8,191, on the wide weight set (LONG_TOL).

Two mistakes change the pass by less than bf16 rounding does and are caught
in the FP32 mode only: the tanh approximation of GELU (at most ~1e-3 on a
value that bf16 rounds by 2^-9 relative) and the unbiased variance in
LayerNorm (a factor 1 + 1/766 on rstd).
"""
import contextlib

import numpy as np
import pytest

from encoder_transformer_amd import synth
from gpu_common import LOGIT_TOL, LONG_TOL, STAGE_TOL, STAGES, stage_batch, weights_of
from oracle import julia_oracle as jo

SETS = ["jit02", "jit05"]
MARGIN = 3.0


@contextlib.contextmanager
def patched(**attrs):
    old = {k: getattr(jo, k) for k in attrs}
    for k, v in attrs.items():
        setattr(jo, k, v)
    try:
        yield
    finally:
        for k, v in old.items():
            setattr(jo, k, v)


_rope = jo.rope
_head_input = jo.head_input
_head_layer = jo.head_layer
_attention_global = jo.attention_global
_attention_band = jo.attention_band


def rope_interleaved(x, cos, sin):
    """Rotation of adjacent pairs (2j, 2j+1) instead of (j, j+32)."""
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = cos[:, None, :], sin[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def head_layer_variant(window=None, rotate=False):
    """The head layer computed with a window or with RoPE (both absent in the method)."""
    def f(W, j, h):
        P = W.head[j]
        L = h.shape[0]
        qkv = jo.layer_norm(h, P["n1_w"], P["n1_b"]) @ P["in_w"].T + P["in_b"]
        q, k, v = (jo.split_heads(qkv[:, i * 384:(i + 1) * 384]) for i in range(3))
        if rotate:
            c, s = jo.rope_angles(np.arange(L), jo.THETA_LOCAL)
            q, k = jo.rope(q, c, s), jo.rope(k, c, s)
        o = _attention_band(q, k, v, window) if window else _attention_global(q, k, v)
        h = h + (o.reshape(L, 384) @ P["out_w"].T + P["out_b"])
        f_ = np.maximum(jo.layer_norm(h, P["n2_w"], P["n2_b"]) @ P["l1_w"].T + P["l1_b"], 0.0)
        return h + (f_ @ P["l2_w"].T + P["l2_b"])
    return f


def gelu_tanh(z):
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def ln_unbiased(x, gain, shift=None):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    y = (x - mu) / np.sqrt(var + jo.LN_EPS) * gain
    return y + shift if shift is not None else y


def scaled_q(fn, factor):
    return lambda q, k, v, *a: fn(q * factor, k, v, *a)


def swap_geglu_halves(W):
    for P in W.layers:
        P["Wi"] = np.concatenate([P["Wi"][jo.GEGLU_HALF:], P["Wi"][:jo.GEGLU_HALF]])


def score_relu(W, z):
    """The scorer with ReLU in place of its GELU."""
    S = W.scorer
    t = np.maximum(jo.layer_norm(z, S["n_w"], S["n_b"]) @ S["fc1_w"].T + S["fc1_b"], 0.0)
    return (t @ S["fc2_w"].T + S["fc2_b"])[:, 0]


# name -> (context factory, weight transform or None, first stage it can touch, FP32 only)
MUTATIONS = {
    "every layer windowed": (lambda: patched(is_global=lambda l: False), None, 1, False),
    "every layer global": (lambda: patched(is_global=lambda l: True), None, 2, False),
    "global layers at l % 3 == 2": (lambda: patched(is_global=lambda l: l % 3 == 2), None, 1, False),
    "window +-32": (lambda: patched(HALF_WINDOW=32), None, 2, False),
    "window +-63 (exclusive edge)": (lambda: patched(HALF_WINDOW=63), None, 2, False),
    "window +-65": (lambda: patched(HALF_WINDOW=65), None, 2, False),
    "no RoPE": (lambda: patched(rope=lambda x, c, s: x), None, 1, False),
    "RoPE sign flipped": (lambda: patched(rope=lambda x, c, s: _rope(x, c, -s)), None, 1, False),
    "RoPE on adjacent pairs": (lambda: patched(rope=rope_interleaved), None, 1, False),
    "RoPE thetas swapped": (lambda: patched(THETA_GLOBAL=jo.THETA_LOCAL, THETA_LOCAL=jo.THETA_GLOBAL), None, 1,
                            False),
    "RoPE theta 10k everywhere": (lambda: patched(THETA_GLOBAL=jo.THETA_LOCAL), None, 1, False),
    "attention scale 1/64": (lambda: patched(attention_global=scaled_q(_attention_global, 0.125),
                                             attention_band=scaled_q(_attention_band, 0.125)), None, 1, False),
    "GELU on the gate half": (contextlib.nullcontext, swap_geglu_halves, 1, False),
    "wrong type row": (lambda: patched(head_input=lambda W, x, qt: _head_input(W, x, (qt + 1) % 3)), None, 23,
                       False),
    "no final LayerNorm": (lambda: patched(head_input=lambda W, x, qt: x + W.type_rows[qt]), None, 23, False),
    "first head layer skipped": (lambda: patched(head_layer=lambda W, j, h: h if j == 0 else _head_layer(W, j, h)),
                                 None, 24, False),
    "second head layer skipped": (lambda: patched(head_layer=lambda W, j, h: h if j == 1 else _head_layer(W, j, h)),
                                  None, 25, False),
    "head attention windowed": (lambda: patched(head_layer=head_layer_variant(window=64)), None, 24, False),
    "RoPE in the head layers": (lambda: patched(head_layer=head_layer_variant(rotate=True)), None, 24, False),
    "scorer GELU as ReLU": (lambda: patched(score=score_relu), None, 26, False),
    "tanh GELU": (lambda: patched(gelu=gelu_tanh), None, 1, True),
    "unbiased LayerNorm variance": (lambda: patched(layer_norm=ln_unbiased), None, 1, True),
}


def stage_values(W, batch, first, encoder_out=None):
    """Yield (stage, packed value) in order; stage 26 = logits.  Stages
    before `first` are not yielded (a mistake cannot touch them);
    `encoder_out` (the sequences' encoder outputs) skips the encoder."""
    per = [batch.sequence(b) for b in range(batch.n_seqs)]
    if encoder_out is None:
        xs = [jo.embed(W, ids) for ids, _, _ in per]
        for l in range(jo.N_LAYERS):
            xs = [jo.encoder_layer(W, l, x) for x in xs]
            if l + 1 in STAGES and l + 1 >= first:
                yield l + 1, np.concatenate(xs)
        encoder_out = xs
    hs = [jo.head_input(W, x, qt) for x, (_, _, qt) in zip(encoder_out, per)]
    if first <= 23:
        yield 23, np.concatenate(hs)
    hs = [jo.head_layer(W, 0, h) for h in hs]
    if first <= 24:
        yield 24, np.concatenate(hs)
    zs = [jo.head_layer(W, 1, h)[marks] for h, (_, marks, _) in zip(hs, per)]
    yield 25, np.concatenate(zs)
    yield 26, np.concatenate([jo.score(W, z) for z in zs])


_REF = {}


def reference(name):
    """Unplanted stage values and encoder outputs of the stage batch."""
    if name not in _REF:
        W = jo.OracleWeights(weights_of(name))
        batch = stage_batch()
        vals = dict(stage_values(W, batch, 1))
        _REF[name] = (vals, np.split(vals[22], batch.seq_offsets[1:-1]))
    return _REF[name]


def bound(name, prec, stage):
    return LOGIT_TOL[(name, prec)] if stage == 26 else STAGE_TOL[(name, prec)][stage]


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_mutation_fails_a_gpu_parity_test(mutation):
    ctx, transform, first, fp32_only = MUTATIONS[mutation]
    best = {"bf16": 0.0, "fp32": 0.0}
    where = {}
    for name in SETS:
        ref, enc = reference(name)
        W = jo.OracleWeights(weights_of(name))
        if transform is not None:
            transform(W)
        with ctx():
            for stage, val in stage_values(W, stage_batch(), first, enc if first > 22 else None):
                d = float(np.max(np.abs(val - ref[stage])))
                for prec in best:
                    r = d / bound(name, prec, stage)
                    if r > best[prec]:
                        best[prec], where[prec] = r, (name, stage, d)
                if best["fp32"] >= MARGIN and (fp32_only or best["bf16"] >= MARGIN):
                    break
        if best["fp32"] >= MARGIN and (fp32_only or best["bf16"] >= MARGIN):
            break
    print(mutation, {p: (round(best[p], 1), where.get(p)) for p in best})
    assert best["fp32"] >= MARGIN, where.get("fp32")
    if not fp32_only:
        assert best["bf16"] >= MARGIN, where.get("bf16")


def test_long_position_mistake_fails_the_long_row_test():
    """A RoPE table of 4,096 rows (positions wrapping at 4,096) moves the rows
    after the first two layers (a global and a window layer) at the stored
    positions past 4,095 of an 8,192-token sequence by more than 3x the
    long-row bound (wide weights: peaked attention)."""
    b = synth.make_batch(3)
    ids, _, _ = b.sequence(0)
    W = jo.OracleWeights(weights_of("wide"))
    pos = np.array([4096, 4097, 6000, 8063, 8064, 8127, 8128, 8190, 8191])

    def two_layers():
        return jo.encoder_layer(W, 1, jo.encoder_layer(W, 0, jo.embed(W, ids)))[pos]
    ref = two_layers()
    angles = jo.rope_angles
    with patched(rope_angles=lambda p, theta: angles(np.asarray(p) % 4096, theta)):
        got = two_layers()
    d = float(np.max(np.abs(got - ref)))
    print("positions wrapped at 4,096: stage-2 max |d|", d)
    for prec in ("bf16", "fp32"):
        assert d >= MARGIN * LONG_TOL[("wide", prec)][2], prec
