"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one part of the oracle to a library routine, a closed form, an
invariant, brute force on tiny inputs, or a value printed on the pages:

* encoder: HuggingFace `ModernBertModel` (the published ModernBERT block the
  explainer page names for mmBERT-small), same weights, float64;
* head layers: `torch.nn.TransformerEncoderLayer(norm_first=True, relu)`, the
  module the Julia-1 MLX page names;
* the whole forward: HF encoder + type row + two torch layers + a torch scorer,
  composed independently of the oracle;
* sliding-window attention: brute force with an explicit boolean mask, torch
  SDPA with that mask, window locality, window >= L equals global;
* RoPE: norm preservation and the relative-position property;
* read-offs: probabilities sum to 1, score = sum_i i p_i, noul = p_1;
* shapes: parameter counts against the pages' 98M / 42M / 3.7M / 144.3M;
* layout: the explainer's card example puts its markers at 12, 17 and 21.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from encoder_transformer_amd import synth
from oracle import julia_oracle as jo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
torch.set_num_threads(min(8, os.cpu_count() or 1))


def small_weights(seed=7, vocab=2000):
    """Full-architecture weights with a reduced vocabulary and jittered norms."""
    return synth.make_weights(seed=seed, norm_jitter=True, vocab=vocab)


@pytest.fixture(scope="module")
def wsmall():
    return small_weights()


def rand_qkv(L, H=2, d=8, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((L, H, d)), r.standard_normal((L, H, d)), r.standard_normal((L, H, d)))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def brute_force_attention(q, k, v, allowed):
    """Pure-Python loops over an explicit boolean mask [L, L]."""
    L, H, d = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for p in range(L):
            keys = [r for r in range(L) if allowed[p, r]]
            s = [sum(q[p, h, i] * k[r, h, i] for i in range(d)) / math.sqrt(d) for r in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for wgt, r in zip(e, keys):
                out[p, h] += (wgt / z) * v[r, h]
    return out


@pytest.mark.parametrize("L", [7, 130, 200])
def test_band_attention_equals_masked_bruteforce(L):
    q, k, v = rand_qkv(L, seed=L)
    idx = np.arange(L)
    allowed = np.abs(idx[:, None] - idx[None, :]) <= 64
    got = jo.attention_band(q, k, v, 64)
    ref = brute_force_attention(q, k, v, allowed)
    assert np.max(np.abs(got - ref)) <= 1e-6
    # and the library routine with the same explicit mask
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(allowed)[None, None])
    assert np.max(np.abs(got - sdpa[0].permute(1, 0, 2).numpy())) <= 1e-10


def test_global_attention_equals_sdpa():
    q, k, v = rand_qkv(300, H=3, d=16, seed=3)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    sdpa = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    got = jo.attention_global(q, k, v)
    assert np.max(np.abs(got - sdpa[0].permute(1, 0, 2).numpy())) <= 1e-10


def test_window_locality_attention():
    q, k, v = rand_qkv(400, seed=11)
    base = jo.attention_band(q, k, v, 64)
    k2, v2 = k.copy(), v.copy()
    r = np.random.default_rng(5)
    # keys 165.. are more than 64 away from every query 0..99
    k2[165:] += r.standard_normal(k2[165:].shape) * 10
    v2[165:] += r.standard_normal(v2[165:].shape) * 10
    pert = jo.attention_band(q, k2, v2, 64)
    assert np.array_equal(base[:100], pert[:100])
    assert not np.array_equal(base[100:], pert[100:])


def test_window_locality_layer(wsmall):
    W = jo.OracleWeights(wsmall)
    r = np.random.default_rng(2)
    x = r.standard_normal((300, 384))
    x2 = x.copy()
    x2[200:] += r.standard_normal((100, 384))
    for l in (1, 2, 4):  # local layers
        assert not jo.is_global(l)
        a = jo.encoder_layer(W, l, x)
        b = jo.encoder_layer(W, l, x2)
        # rows 0..135 have no key at 200.. within +-64
        assert np.array_equal(a[:136], b[:136])
        assert not np.array_equal(a[136:200], b[136:200])


@pytest.mark.parametrize("L", [5, 64, 150])
def test_window_at_least_length_equals_global(L):
    q, k, v = rand_qkv(L, H=2, d=16, seed=L + 1)
    g = jo.attention_global(q, k, v)
    for w in (L - 1, L, 2 * L):
        assert np.max(np.abs(jo.attention_band(q, k, v, w) - g)) <= 1e-12


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_preserves_norm():
    r = np.random.default_rng(0)
    x = r.standard_normal((8192, 6, 64))
    for theta in (jo.THETA_LOCAL, jo.THETA_GLOBAL):
        c, s = jo.rope_angles(np.arange(8192), theta)
        y = jo.rope(x, c, s)
        rel = np.abs(np.linalg.norm(y, axis=-1) / np.linalg.norm(x, axis=-1) - 1)
        assert rel.max() <= 1e-6


def test_rope_relative_position():
    r = np.random.default_rng(1)
    qv = r.standard_normal((1, 1, 64))
    kv = r.standard_normal((1, 1, 64))
    for theta in (jo.THETA_LOCAL, jo.THETA_GLOBAL):
        def dot(p, q_):
            cq, sq = jo.rope_angles(np.array([p]), theta)
            ck, sk = jo.rope_angles(np.array([q_]), theta)
            return float(np.sum(jo.rope(qv, cq, sq) * jo.rope(kv, ck, sk)))
        for p, q_ in [(3, 10), (100, 37), (5000, 4990)]:
            for shift in (1, 17, 2000):
                assert abs(dot(p + shift, q_ + shift) - dot(p, q_)) <= 1e-9 * (1 + abs(dot(p, q_)))
        # at equal positions the rotation cancels exactly in the dot product
        assert abs(dot(777, 777) - float(np.sum(qv * kv))) <= 1e-9


# ---------------------------------------------------------------------------
# elementary ops against torch
# ---------------------------------------------------------------------------

def test_layer_norm_and_gelu_and_softmax_match_torch():
    r = np.random.default_rng(4)
    x = r.standard_normal((50, 384)) * 3 + 1
    g = r.standard_normal(384)
    b = r.standard_normal(384)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (384,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    assert np.max(np.abs(jo.layer_norm(x, g, b) - ref)) <= 1e-12
    z = np.linspace(-8, 8, 2001)
    refg = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    assert np.max(np.abs(jo.gelu(z) - refg)) <= 1e-14
    # the tanh approximation differs visibly: the pin separates the two forms
    tanh_g = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.max(np.abs(jo.gelu(z) - tanh_g)) > 1e-4
    s = r.standard_normal((7, 20)) * 10
    assert np.max(np.abs(jo.softmax(s) - torch.softmax(torch.from_numpy(s), -1).numpy())) <= 1e-15


# ---------------------------------------------------------------------------
# encoder vs HuggingFace ModernBERT
# ---------------------------------------------------------------------------

def hf_encoder(w, vocab):
    from transformers import ModernBertConfig, ModernBertModel
    cfg = ModernBertConfig(
        vocab_size=vocab, hidden_size=384, intermediate_size=1152, num_hidden_layers=22,
        num_attention_heads=6, local_attention=128, norm_eps=1e-5, norm_bias=False,
        attention_bias=False, mlp_bias=False, hidden_activation="gelu",
        layer_types=["full_attention" if i % 3 == 0 else "sliding_attention" for i in range(22)],
        rope_parameters={"sliding_attention": {"rope_type": "default", "rope_theta": 10000.0},
                         "full_attention": {"rope_type": "default", "rope_theta": 160000.0}},
        max_position_embeddings=8192, pad_token_id=0, bos_token_id=2, eos_token_id=1,
        cls_token_id=2, sep_token_id=1, attn_implementation="eager")
    m = ModernBertModel(cfg)
    sd = {k: torch.from_numpy(np.ascontiguousarray(w[k])) for k in m.state_dict().keys()}
    m.load_state_dict(sd, strict=True)
    return m.double().eval()


@pytest.mark.parametrize("L", [40, 300])
def test_encoder_matches_hf_modernbert(wsmall, L):
    W = jo.OracleWeights(wsmall)
    ids = np.random.default_rng(L).integers(5, 2000, size=L).astype(np.int64)
    m = hf_encoder(wsmall, 2000)
    with torch.no_grad():
        ref = m(input_ids=torch.from_numpy(ids)[None]).last_hidden_state[0].numpy()
    got = jo.layer_norm(jo.encoder(W, ids), W.final_norm)
    # HF rotates q and k in float32 even in a float64 model (~1e-7 here); a
    # window of 63, a flipped rotation, the wrong theta or tanh-GELU all move
    # the result by 2e-4 or more
    assert np.max(np.abs(got - ref)) <= 2e-6


# ---------------------------------------------------------------------------
# head layers and scorer vs torch modules
# ---------------------------------------------------------------------------

def torch_head_layer(w, j):
    layer = torch.nn.TransformerEncoderLayer(384, 6, 1536, dropout=0.0, activation="relu",
                                             norm_first=True, batch_first=True)
    p = f"head.layers.{j}."
    sd = {k: torch.from_numpy(np.ascontiguousarray(w[p + k])) for k in layer.state_dict().keys()}
    layer.load_state_dict(sd, strict=True)
    return layer.double().eval()


def torch_scorer(w):
    seq = torch.nn.Sequential(torch.nn.LayerNorm(384), torch.nn.Linear(384, 384),
                              torch.nn.GELU(), torch.nn.Linear(384, 1))
    names = ["norm.weight", "norm.bias", "fc1.weight", "fc1.bias", "fc2.weight", "fc2.bias"]
    sd = dict(zip(seq.state_dict().keys(),
                  [torch.from_numpy(np.ascontiguousarray(w["head.scorer." + n])) for n in names]))
    seq.load_state_dict(sd, strict=True)
    return seq.double().eval()


def test_head_layers_match_torch(wsmall):
    W = jo.OracleWeights(wsmall)
    h = np.random.default_rng(9).standard_normal((230, 384))
    for j in range(2):
        with torch.no_grad():
            ref = torch_head_layer(wsmall, j)(torch.from_numpy(h)[None])[0].numpy()
        assert np.max(np.abs(jo.head_layer(W, j, h) - ref)) <= 1e-10


def test_scorer_matches_torch(wsmall):
    W = jo.OracleWeights(wsmall)
    z = np.random.default_rng(10).standard_normal((25, 384))
    with torch.no_grad():
        ref = torch_scorer(wsmall)(torch.from_numpy(z))[:, 0].numpy()
    assert np.max(np.abs(jo.score(W, z) - ref)) <= 1e-12


def test_whole_forward_matches_library_composition(wsmall):
    """HF encoder + type row + two torch layers + marker gather + torch scorer."""
    W = jo.OracleWeights(wsmall)
    rng = np.random.default_rng(21)
    L, marks = 260, np.array([20, 31, 45, 60, 61], np.int32)
    ids = rng.integers(5, 2000, size=L).astype(np.int64)
    enc = hf_encoder(wsmall, 2000)
    for qtype in (0, 1, 2):
        with torch.no_grad():
            h = enc(input_ids=torch.from_numpy(ids)[None]).last_hidden_state
            h = h + torch.from_numpy(wsmall["head.type_embedding.weight"][qtype].astype(np.float64))
            h = torch_head_layer(wsmall, 0)(h)
            h = torch_head_layer(wsmall, 1)(h)
            ref = torch_scorer(wsmall)(h[0, torch.from_numpy(marks).long()])[:, 0].numpy()
        got = jo.forward_sequence(W, ids, marks, qtype)
        assert np.max(np.abs(got - ref)) <= 2e-6


# ---------------------------------------------------------------------------
# read-offs
# ---------------------------------------------------------------------------

def test_read_offs():
    rng = np.random.default_rng(3)
    offs = np.array([0, 50, 90, 200, 260])
    marks = np.array([5, 9, 13, 55, 60, 100, 110, 120, 130, 140, 150, 161, 170, 181, 192, 210, 230])
    qtype = np.array([0, 2, 1, 0])
    logits = rng.standard_normal(len(marks)) * 3
    r = jo.read_offs(logits, offs, marks, qtype)
    for b in range(4):
        sel = (marks >= offs[b]) & (marks < offs[b + 1])
        p = r["probs"][sel]
        ref = torch.softmax(torch.from_numpy(logits[sel]), 0).numpy()
        assert abs(p.sum() - 1) <= 1e-6 and np.max(np.abs(p - ref)) <= 1e-15
        assert r["argmax"][b] == int(np.argmax(logits[sel]))
        assert r["maxprob"][b] == p.max()
    assert r["answer"][0] == r["argmax"][0]
    assert r["answer"][1] == r["probs"][4]                           # noul: p(true) = p_1
    p2 = r["probs"][5:15]
    assert abs(r["answer"][2] - sum(i * p2[i] for i in range(10))) <= 1e-12   # expected index
    # ties go to the first maximum
    t = jo.read_offs(np.array([1.0, 3.0, 3.0]), np.array([0, 10]), np.array([1, 2, 3]), np.array([0]))
    assert t["argmax"][0] == 1 and t["answer"][0] == 1


# ---------------------------------------------------------------------------
# shapes and layout against the pages
# ---------------------------------------------------------------------------

def test_parameter_counts_match_pages():
    spec = synth.weight_spec()
    size = lambda pred: sum(int(np.prod(s)) for n, s, _ in spec if pred(n))
    emb = size(lambda n: n.startswith("embeddings.tok"))
    encoder = size(lambda n: not n.startswith("head."))
    head = size(lambda n: n.startswith("head."))
    # "98M of the 144M parameters" (Julia-1 MLX, Performance: Embedding)
    assert round(emb / 1e6) == 98
    # mmBERT-small: 140M total, 42M non-embedding (explainer, The decision head)
    assert round(encoder / 1e6) == 140 and round((encoder - emb) / 1e6) == 42
    # "3.7M parameters of head" (explainer, The ledger); a scorer without its
    # hidden Linear(384,384) would give 3.55M
    assert round(head / 1e5) == 37
    # 144.3M in all (launch page); the undocumented act_head makes up the rest
    assert 0 < 144.3e6 - (encoder + head) < 0.2e6
    # non-embedding weights in FP32: "175 MiB of weights instead of 550 MiB"
    assert round((encoder - emb + head) * 4 / 2**20) == 175


def test_card_example_marker_positions():
    with open(os.path.join(GOLDEN, "card_example_layout.json")) as f:
        g = json.load(f)
    got = synth.marker_positions(g["question_tokens"], g["option_tokens"])
    assert got == g["markers"]
    rng = np.random.default_rng(0)
    ids, marks = synth.layout_sequence(rng, 0, g["question_tokens"], g["option_tokens"], 9)
    assert marks.tolist() == g["markers"] and all(ids[m] == synth.MASK for m in marks)


def test_config_layouts():
    b0 = synth.make_batch(0)
    assert b0.n_tokens == 128 and b0.mask_positions.tolist() == [15, 22, 29]
    b1 = synth.make_batch(1)
    assert b1.n_tokens == 1024 and b1.mask_positions.tolist() == [35 + 21 * k for k in range(20)]
    b2 = synth.make_batch(2)
    assert b2.n_tokens == 16384 and np.all(np.diff(b2.seq_offsets) == 1024)
    b3 = synth.make_batch(3)
    assert b3.n_tokens == 131072 and b3.n_markers == 80
    assert b3.mask_positions[:5].tolist() == [50 + 41 * k for k in range(5)]
    b4 = synth.make_batch(4)
    lens = np.diff(b4.seq_offsets)
    assert b4.n_seqs == 256 and lens.min() >= 64 and lens.max() <= 2048
    for b in (b0, b1, b2, b3, b4):
        for s in range(b.n_seqs):
            ids, marks, qt = b.sequence(s)
            assert 2 <= len(marks) <= 20 and (qt != 2 or len(marks) == 2)
            assert ids[0] == synth.BOS and ids[-1] == synth.EOS and np.all(ids[marks] == synth.MASK)
            assert np.all((ids >= 0) & (ids < synth.VOCAB))
    # the same seed gives the same batch
    again = synth.make_batch(2)
    assert np.array_equal(again.ids, b2.ids) and np.array_equal(again.mask_positions, b2.mask_positions)


def test_batch_composition_oracle(oracle_weights):
    batch = synth.make_ragged_batch(seed=5, n_seqs=3, min_len=70, max_len=160)
    packed = jo.forward(oracle_weights, batch)
    sizes = [len(batch.sequence(b)[1]) for b in range(3)]
    o = 0
    for b in range(3):
        alone = jo.forward(oracle_weights, batch.subset([b]))
        assert np.array_equal(alone, packed[o:o + sizes[b]])
        o += sizes[b]


# ---------------------------------------------------------------------------
# e4m3 rounding and per-row quantization (the FP8 mode's reference)
# ---------------------------------------------------------------------------

def test_e4m3_round_matches_torch_float8_e4m3fn():
    import torch
    from oracle import julia_oracle as jo
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 60,
                        rng.uniform(-0.03, 0.03, 50_000).astype(np.float32),
                        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11],
                                 np.float32)])
    x = x[np.abs(x) < 464]  # 464 and above round past the largest code
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(jo.e4m3_round(x).view(np.uint32), ref.view(np.uint32))


def test_e4m3_round_ties_and_codes():
    import torch
    from oracle import julia_oracle as jo
    # ties go to the even mantissa: 1.0625 lies between 1 (m = 0) and 1.125
    # (m = 1); 1.1875 between 1.125 and 1.25 (m = 2); 2^-10 between 0 and 2^-9
    got = jo.e4m3_round(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 456.0], np.float32))
    assert np.array_equal(got, np.array([1.0, 1.25, 0.0, 2.0 ** -8, 448.0], np.float32))
    # 464 is the tie between 448 (m = 6) and 480 (m = 7, the NaN code): even
    # wins; anything above it has no code
    assert jo.e4m3_round(np.array([464.0], np.float32))[0] == 448.0
    assert np.isnan(jo.e4m3_round(np.array([470.0], np.float32))[0])
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    fin = codes[np.isfinite(codes)]
    assert fin.size == 254 and np.max(fin) == 448.0
    assert np.array_equal(jo.e4m3_round(fin), fin)  # every code is a fixed point


def test_quantize_rows_e4m3():
    from oracle import julia_oracle as jo
    rng = np.random.default_rng(6)
    m = rng.standard_normal((40, 384)) * np.exp(rng.uniform(-6, 6, (40, 1)))
    m[3] = 0.0
    dq = jo.quantize_rows_e4m3(m)
    m32 = m.astype(np.float32).astype(np.float64)
    s = np.max(np.abs(m32), axis=1) / 448.0
    s[3] = 1.0
    q = dq / s[:, None]
    nz = np.arange(40) != 3
    assert np.allclose(np.max(np.abs(q[nz]), axis=1), 448.0, rtol=1e-6)  # the row maximum maps to 448
    assert np.all(dq[3] == 0.0)
    normal = np.abs(q) >= 2.0 ** -6
    rel = np.abs(dq - m32)[normal] / np.abs(m32)[normal]
    assert np.max(rel) <= 2.0 ** -4 * (1 + 1e-6)  # half a step of 3 mantissa bits


def test_fp8_forward_is_a_small_perturbation(oracle_weights):
    from oracle import julia_oracle as jo
    batch = synth.make_batch(0)
    ref = jo.forward(oracle_weights, batch)
    q = jo.forward(oracle_weights, batch, fp8=True)
    d = np.max(np.abs(q - ref))
    assert 0.0 < d < 0.05 * np.max(np.abs(ref)) + 1e-3
