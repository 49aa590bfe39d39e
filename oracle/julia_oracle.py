"""Plain CPU oracle of the Julia-1 decision-model forward pass (test infrastructure).

This module is test infrastructure. Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code with the GPU library: it reads the same seeded weights and
packed batches and nothing else.

Every step is the plain definition, evaluated in float64 with NumPy (a BLAS
matmul and `scipy.special.erf` serve as library primitives), one sequence at a
time, with no blocking or fusion beyond what the definition states. Sources,
by page title and section:

* "Julia-1 MLX" (PyPI), Performance: every third layer attends globally, the
  other 14 within +-64 tokens (local_attention=128); the residual stream,
  norms, embeddings and decision head are FP32, FP32 is the parity mode.
* "julia1 - Rust runtime for Julia-1", Why it is faster: GEGLU feed-forward
  with a [T, 2304] intermediate, RoPE, sliding-window layers that only need
  their band, packed sequences with no padding; the last head layer is only
  needed at option markers.
* "Julia-1: one score per mask token ...", The decision head: mmBERT-small
  (ModernBERT block, 22 layers, width 384, 6 heads); the four head steps (type
  row, two pre-norm transformer layers with feed-forward 1,536, marker gather,
  LayerNorm -> Linear(384,384) -> GELU -> Linear(384,1) and a softmax across
  the options); Three modes through one head: choice -> argmax, score ->
  expected index sum_i i*p_i, noul -> p(true) with options [false, true].

Readings taken where the pages are silent (each is listed in the design doc):
embedding LayerNorm present and the first layer's attention pre-norm the
identity; global layers are those with index % 3 == 0; the window is
|i - j| <= 64 inclusive; rotate-half RoPE over all 64 dims with
omega_j = theta^(-2j/64), theta 160k on global and 10k on local layers;
LayerNorm eps 1e-5 with biased variance; encoder linears bias-free, head and
scorer linears with bias; exact (erf) GELU, applied to the first half of the
GEGLU projection; attention scale 1/sqrt(64); score index 0-based; argmax ties
go to the lowest index.

Parity: pinned (see tests/test_oracle_pins.py) except the embedding-norm /
layer-0 pre-norm reading, which no test can separate from its alternative at
the published init (parity unpinned for that reading alone).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

WIDTH = 384
N_HEADS = 6
HEAD_DIM = 64
N_LAYERS = 22
GEGLU_HALF = 1152
LN_EPS = 1e-5
HALF_WINDOW = 64              # local layers: |i - j| <= 64
THETA_LOCAL = 10_000.0
THETA_GLOBAL = 160_000.0
QUERY_CHUNK = 1024            # rows per attention block (memory only, not arithmetic)


# ---------------------------------------------------------------------------
# elementary steps
# ---------------------------------------------------------------------------

def layer_norm(x: np.ndarray, gain: np.ndarray, shift: Optional[np.ndarray] = None) -> np.ndarray:
    """LayerNorm over the last axis: gain * (x - mean) / sqrt(var + eps) (+ shift), biased var."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + LN_EPS) * gain
    if shift is not None:
        y = y + shift
    return y


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def rope_angles(positions: np.ndarray, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of p * theta^(-2j/64), j = 0..31, for each position p."""
    j = np.arange(HEAD_DIM // 2, dtype=np.float64)
    omega = theta ** (-2.0 * j / HEAD_DIM)
    ang = positions.astype(np.float64)[:, None] * omega[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (j, j+32) of every head: x [L, H, 64], cos/sin [L, 32]."""
    a, b = x[..., : HEAD_DIM // 2], x[..., HEAD_DIM // 2:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention_global(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Softmax(q k^T / sqrt d) v over all keys of the sequence; q,k,v [L, H, d]."""
    L, H, d = q.shape
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    for h in range(H):
        kh, vh = k[:, h, :], v[:, h, :]
        for s0 in range(0, L, QUERY_CHUNK):
            s = (q[s0:s0 + QUERY_CHUNK, h, :] @ kh.T) * scale
            out[s0:s0 + QUERY_CHUNK, h, :] = softmax(s) @ vh
    return out


def attention_band(q: np.ndarray, k: np.ndarray, v: np.ndarray, half_window: int) -> np.ndarray:
    """Attention where query p sees keys r with |p - r| <= half_window.

    Only the band is computed: for query p the candidate keys are
    p - w .. p + w (2w+1 of them); those outside the sequence are excluded.
    """
    L, H, d = q.shape
    w = int(half_window)
    width = 2 * w + 1
    scale = 1.0 / np.sqrt(d)
    pad_k = np.zeros((L + 2 * w, H, d))
    pad_v = np.zeros((L + 2 * w, H, d))
    pad_k[w:w + L] = k
    pad_v[w:w + L] = v
    out = np.empty_like(q)
    chunk = max(1, min(QUERY_CHUNK, (1 << 24) // max(1, width * d)))
    for s0 in range(0, L, chunk):
        p = np.arange(s0, min(L, s0 + chunk))
        # band slot t of query p holds key r = p - w + t
        slots = p[:, None] + np.arange(width)[None, :]
        r = slots - w
        valid = (r >= 0) & (r < L)
        for h in range(H):
            kb = pad_k[slots, h, :]          # [n, width, d]
            vb = pad_v[slots, h, :]
            s = np.einsum("nd,ntd->nt", q[p, h, :], kb) * scale
            s = np.where(valid, s, -np.inf)
            pr = softmax(s, axis=-1)
            out[p, h, :] = np.einsum("nt,ntd->nd", pr, vb)
    return out


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest OCP e4m3 value (ties to even).

    e4m3 (the OCP 8-bit floating-point format E4M3): sign, 4 exponent bits
    with bias 7, 3 mantissa bits; normal values (1 + m/8) 2^(e-7), e = 1..15,
    subnormal ones (m/8) 2^-6; no infinities, the largest finite value 448.
    A magnitude that rounds above 448 has no code and becomes NaN.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    out = np.empty_like(a)
    sub = a < 2.0 ** -6
    out[sub] = np.round(a[sub] * 2.0 ** 9) * 2.0 ** -9  # np.round: ties to even
    nz = ~sub
    e = np.floor(np.log2(a[nz]))
    step = 2.0 ** (e - 3)  # 8 steps per binade
    out[nz] = np.round(a[nz] / step) * step
    out[out > 448.0] = np.nan
    return np.copysign(out, x).astype(np.float32)


def quantize_rows_e4m3(m: np.ndarray) -> np.ndarray:
    """Per-row e4m3 quantization, returned dequantized (float64).

    Each row, in float32, is multiplied by r = 448 / max |row| and rounded to
    e4m3; the codes stand for code * s with the row's scale s = max |row| / 448
    (r = s = 1 for an all-zero row).
    """
    m32 = np.asarray(m, dtype=np.float32)
    amax = np.max(np.abs(m32), axis=1)
    safe = np.where(amax > 0, amax, np.float32(448.0)).astype(np.float32)
    r = (np.float32(448.0) / safe).astype(np.float32)
    s = (safe / np.float32(448.0)).astype(np.float32)
    q = e4m3_round((m32 * r[:, None]).astype(np.float32))
    return q.astype(np.float64) * s.astype(np.float64)[:, None]


class OracleWeights:
    """float64 view of the weights; the embedding table stays float32 and rows are gathered."""

    def __init__(self, w: Dict[str, np.ndarray]):
        self.emb = w["embeddings.tok_embeddings.weight"]
        f = lambda n: np.asarray(w[n], dtype=np.float64)
        self.emb_norm = f("embeddings.norm.weight")
        self.layers = []
        for l in range(N_LAYERS):
            p = f"layers.{l}."
            self.layers.append({
                "attn_norm": f(p + "attn_norm.weight") if l != 0 else None,
                "Wqkv": f(p + "attn.Wqkv.weight"),
                "Wo": f(p + "attn.Wo.weight"),
                "mlp_norm": f(p + "mlp_norm.weight"),
                "Wi": f(p + "mlp.Wi.weight"),
                "Wout": f(p + "mlp.Wo.weight"),
            })
        self.final_norm = f("final_norm.weight")
        self.type_rows = f("head.type_embedding.weight")
        self.head = []
        for j in range(2):
            p = f"head.layers.{j}."
            self.head.append({k: f(p + n) for k, n in [
                ("in_w", "self_attn.in_proj_weight"), ("in_b", "self_attn.in_proj_bias"),
                ("out_w", "self_attn.out_proj.weight"), ("out_b", "self_attn.out_proj.bias"),
                ("l1_w", "linear1.weight"), ("l1_b", "linear1.bias"),
                ("l2_w", "linear2.weight"), ("l2_b", "linear2.bias"),
                ("n1_w", "norm1.weight"), ("n1_b", "norm1.bias"),
                ("n2_w", "norm2.weight"), ("n2_b", "norm2.bias")]})
        self.scorer = {k: f("head.scorer." + n) for k, n in [
            ("n_w", "norm.weight"), ("n_b", "norm.bias"), ("fc1_w", "fc1.weight"),
            ("fc1_b", "fc1.bias"), ("fc2_w", "fc2.weight"), ("fc2_b", "fc2.bias")]}


# ---------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------

def is_global(layer: int) -> bool:
    return layer % 3 == 0


def split_heads(t: np.ndarray) -> np.ndarray:
    return t.reshape(t.shape[0], N_HEADS, HEAD_DIM)


def embed(W: OracleWeights, ids: np.ndarray) -> np.ndarray:
    """Gather the token rows and apply the embedding LayerNorm (gain only)."""
    return layer_norm(W.emb[ids].astype(np.float64), W.emb_norm)


def e4m3_weights(P: dict, name: str) -> np.ndarray:
    """A weight matrix quantized per row to e4m3 (cached beside it)."""
    if name + "_e4m3" not in P:
        P[name + "_e4m3"] = quantize_rows_e4m3(P[name])
    return P[name + "_e4m3"]


def encoder_layer(W: OracleWeights, l: int, x: np.ndarray, half_window: Optional[int] = None,
                  fp8: bool = False) -> np.ndarray:
    """One pre-norm ModernBERT layer: x += Attn(LN x); x += GEGLU-MLP(LN x).

    ``half_window`` overrides the local band (used by the window pins).
    ``fp8``: the QKV product (layers after the first, whose input has no
    pre-norm) and the W_i product take both operands quantized per row to e4m3.
    """
    P = W.layers[l]
    L = x.shape[0]
    glob = is_global(l)
    u = x if P["attn_norm"] is None else layer_norm(x, P["attn_norm"])
    if fp8 and P["attn_norm"] is not None:
        qkv = quantize_rows_e4m3(u) @ e4m3_weights(P, "Wqkv").T
    else:
        qkv = u @ P["Wqkv"].T
    q = split_heads(qkv[:, :WIDTH])
    k = split_heads(qkv[:, WIDTH:2 * WIDTH])
    v = split_heads(qkv[:, 2 * WIDTH:])
    cos, sin = rope_angles(np.arange(L), THETA_GLOBAL if glob else THETA_LOCAL)
    q, k = rope(q, cos, sin), rope(k, cos, sin)
    if glob:
        o = attention_global(q, k, v)
    else:
        o = attention_band(q, k, v, HALF_WINDOW if half_window is None else half_window)
    x = x + o.reshape(L, WIDTH) @ P["Wo"].T
    if fp8:
        ab = quantize_rows_e4m3(layer_norm(x, P["mlp_norm"])) @ e4m3_weights(P, "Wi").T
    else:
        ab = layer_norm(x, P["mlp_norm"]) @ P["Wi"].T
    a, g = ab[:, :GEGLU_HALF], ab[:, GEGLU_HALF:]
    return x + (gelu(a) * g) @ P["Wout"].T


def encoder(W: OracleWeights, ids: np.ndarray, n_layers: int = N_LAYERS, fp8: bool = False) -> np.ndarray:
    x = embed(W, ids)
    for l in range(n_layers):
        x = encoder_layer(W, l, x, fp8=fp8)
    return x


def head_layer(W: OracleWeights, j: int, h: np.ndarray) -> np.ndarray:
    """PyTorch TransformerEncoderLayer, norm_first, 6 heads, ReLU FFN 1,536, no dropout."""
    P = W.head[j]
    L = h.shape[0]
    qkv = layer_norm(h, P["n1_w"], P["n1_b"]) @ P["in_w"].T + P["in_b"]
    q = split_heads(qkv[:, :WIDTH])
    k = split_heads(qkv[:, WIDTH:2 * WIDTH])
    v = split_heads(qkv[:, 2 * WIDTH:])
    o = attention_global(q, k, v).reshape(L, WIDTH)
    h = h + (o @ P["out_w"].T + P["out_b"])
    f = np.maximum(layer_norm(h, P["n2_w"], P["n2_b"]) @ P["l1_w"].T + P["l1_b"], 0.0)
    return h + (f @ P["l2_w"].T + P["l2_b"])


def head_input(W: OracleWeights, x: np.ndarray, qtype: int) -> np.ndarray:
    """Final encoder LayerNorm, then the decision type's row added to every position."""
    return layer_norm(x, W.final_norm) + W.type_rows[qtype]


def score(W: OracleWeights, z: np.ndarray) -> np.ndarray:
    """LayerNorm -> Linear(384,384) -> GELU -> Linear(384,1), one logit per row."""
    S = W.scorer
    t = gelu(layer_norm(z, S["n_w"], S["n_b"]) @ S["fc1_w"].T + S["fc1_b"])
    return (t @ S["fc2_w"].T + S["fc2_b"])[:, 0]


def forward_sequence(W: OracleWeights, ids: np.ndarray, marks: np.ndarray, qtype: int,
                     fp8: bool = False) -> np.ndarray:
    """Option logits of one sequence (markers given relative to the sequence)."""
    x = encoder(W, ids, fp8=fp8)
    h = head_input(W, x, qtype)
    h = head_layer(W, 0, h)
    h = head_layer(W, 1, h)
    return score(W, h[marks])


def forward(W: OracleWeights, batch, seqs: Optional[Sequence[int]] = None, fp8: bool = False) -> np.ndarray:
    """Logits of every marker of the packed batch, in marker order.

    Sequences never see each other, so each is evaluated on its own.
    ``seqs`` restricts the evaluation to some sequences (their logits, concatenated).
    """
    out: List[np.ndarray] = []
    for b in (range(batch.n_seqs) if seqs is None else seqs):
        ids, marks, qt = batch.sequence(b)
        out.append(forward_sequence(W, ids, marks, qt, fp8=fp8))
    return np.concatenate(out) if out else np.zeros(0)


def read_offs(logits: np.ndarray, seq_offsets: np.ndarray, mask_positions: np.ndarray,
              qtype: np.ndarray) -> Dict[str, np.ndarray]:
    """Softmax across each sequence's options and the three modes' answers.

    choice -> index of the first maximum; score -> sum_i i * p_i (0-based);
    noul -> p_1 (options are [false, true]).
    """
    B = len(qtype)
    probs = np.zeros(len(logits))
    answer = np.zeros(B)
    argmax = np.zeros(B, np.int64)
    maxprob = np.zeros(B)
    for b in range(B):
        sel = np.nonzero((mask_positions >= seq_offsets[b]) & (mask_positions < seq_offsets[b + 1]))[0]
        p = softmax(np.asarray(logits[sel], np.float64))
        probs[sel] = p
        a = int(np.argmax(p))
        argmax[b] = a
        maxprob[b] = p[a]
        if qtype[b] == 0:
            answer[b] = a
        elif qtype[b] == 1:
            answer[b] = float(np.sum(np.arange(len(p)) * p))
        else:
            answer[b] = p[1]
    return {"probs": probs, "answer": answer, "argmax": argmax, "maxprob": maxprob}
