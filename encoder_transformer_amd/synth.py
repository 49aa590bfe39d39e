"""Seeded synthetic inputs for the Julia-1 decision-model forward pass.

This module only draws random numbers and lays out token sequences. It holds
none of the model's arithmetic, so both the CPU oracle and the GPU library can
take their inputs from it without sharing any computation.

Two kinds of input are produced:

* weights -- every tensor of the model at its published shape (mmBERT-small
  encoder: vocabulary 256,000, width 384, 22 layers, GEGLU intermediate 1,152;
  the decision head: a 3-row type table, two PyTorch-style transformer layers
  with a 1,536-wide feed-forward, and a LayerNorm -> Linear -> GELU -> Linear
  scorer), drawn N(0, 0.02^2), LayerNorm gains 1 and shifts 0 (Julia-1 MLX page,
  "Performance"; explainer page, "The decision head"). `write_weight_file`
  stores them in the library's weight-file format.
* batches -- packed, unpadded token sequences laid out by the marker
  serialization of the explainer page ("From a state to one decision"):
  ``<bos> type(3) question <eos> (<mask> option)*n <eos> state <eos>``.

Token ids of special tokens are a reading (the tokenizer is not available):
PAD 0, EOS 1, BOS 2, UNK 3, MASK 4; ordinary ids are uniform in [5, 256000).
"""
from __future__ import annotations

import dataclasses
import os
import struct
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

VOCAB = 256_000
WIDTH = 384
N_LAYERS = 22
INTERMEDIATE = 1_152
HEAD_FFN = 1_536
N_TYPES = 3
N_HEAD_LAYERS = 2

PAD, EOS, BOS, UNK, MASK = 0, 1, 2, 3, 4
FIRST_ORDINARY_ID = 5
# the three-token prefix "<type> question :" of each decision type, fixed ids
TYPE_WORDS = {0: (1_001, 1_010, 1_003), 1: (1_011, 1_010, 1_003), 2: (1_021, 1_010, 1_003)}

CHOICE, SCORE, NOUL = 0, 1, 2
INIT_STD = 0.02
WIDE_STD = 0.05   # the "wide" weight set of the parity tests (see make_weights)
WEIGHT_SEED = 0


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def weight_spec(vocab: int = VOCAB) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Every tensor in draw order: (name, shape, kind).

    kind is "normal" (N(0, 0.02^2)), "ones" (LayerNorm gain) or "zeros"
    (LayerNorm shift). The names follow the upstream PyTorch module names.
    """
    D = WIDTH
    spec: List[Tuple[str, Tuple[int, ...], str]] = []
    spec.append(("embeddings.tok_embeddings.weight", (vocab, D), "normal"))
    spec.append(("embeddings.norm.weight", (D,), "ones"))
    for l in range(N_LAYERS):
        p = f"layers.{l}."
        if l != 0:  # the first layer's attention pre-norm is the identity
            spec.append((p + "attn_norm.weight", (D,), "ones"))
        spec.append((p + "attn.Wqkv.weight", (3 * D, D), "normal"))
        spec.append((p + "attn.Wo.weight", (D, D), "normal"))
        spec.append((p + "mlp_norm.weight", (D,), "ones"))
        spec.append((p + "mlp.Wi.weight", (2 * INTERMEDIATE, D), "normal"))
        spec.append((p + "mlp.Wo.weight", (D, INTERMEDIATE), "normal"))
    spec.append(("final_norm.weight", (D,), "ones"))
    spec.append(("head.type_embedding.weight", (N_TYPES, D), "normal"))
    for j in range(N_HEAD_LAYERS):
        p = f"head.layers.{j}."
        spec.append((p + "self_attn.in_proj_weight", (3 * D, D), "normal"))
        spec.append((p + "self_attn.in_proj_bias", (3 * D,), "normal"))
        spec.append((p + "self_attn.out_proj.weight", (D, D), "normal"))
        spec.append((p + "self_attn.out_proj.bias", (D,), "normal"))
        spec.append((p + "linear1.weight", (HEAD_FFN, D), "normal"))
        spec.append((p + "linear1.bias", (HEAD_FFN,), "normal"))
        spec.append((p + "linear2.weight", (D, HEAD_FFN), "normal"))
        spec.append((p + "linear2.bias", (D,), "normal"))
        spec.append((p + "norm1.weight", (D,), "ones"))
        spec.append((p + "norm1.bias", (D,), "zeros"))
        spec.append((p + "norm2.weight", (D,), "ones"))
        spec.append((p + "norm2.bias", (D,), "zeros"))
    spec.append(("head.scorer.norm.weight", (D,), "ones"))
    spec.append(("head.scorer.norm.bias", (D,), "zeros"))
    spec.append(("head.scorer.fc1.weight", (D, D), "normal"))
    spec.append(("head.scorer.fc1.bias", (D,), "normal"))
    spec.append(("head.scorer.fc2.weight", (1, D), "normal"))
    spec.append(("head.scorer.fc2.bias", (1,), "normal"))
    return spec


def make_weights(seed: int = WEIGHT_SEED, norm_jitter: bool = False,
                 vocab: int = VOCAB, std: float = INIT_STD) -> Dict[str, np.ndarray]:
    """Draw all weights with NumPy PCG64 (`default_rng(seed)`), float32.

    One `standard_normal` call per "normal" tensor, in `weight_spec` order,
    scaled by ``std`` (0.02, the published init). A larger ``std`` (the
    "wide" weight set, 0.05) makes attention peaked and spreads the option
    logits to order one, so that a wrong window, rotation or head step moves
    the logits far more than bf16 rounding does. With ``norm_jitter`` the LayerNorm gains become
    1 + N(0, 0.1^2) and the shifts N(0, 0.1^2), drawn after all other tensors,
    so that the gain and shift paths are exercised (the published init leaves
    them at 1 and 0, where a wrong gain index would go unnoticed).
    ``vocab`` shrinks the embedding table for small CPU-side checks.
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, np.ndarray] = {}
    for name, shape, kind in weight_spec(vocab):
        if kind == "normal":
            a = rng.standard_normal(shape, dtype=np.float32)
            a *= np.float32(std)
        elif kind == "ones":
            a = np.ones(shape, np.float32)
        else:
            a = np.zeros(shape, np.float32)
        out[name] = a
    if norm_jitter:
        for name, shape, kind in weight_spec(vocab):
            if kind == "ones":
                out[name] = (1.0 + 0.1 * rng.standard_normal(shape)).astype(np.float32)
            elif kind == "zeros":
                out[name] = (0.1 * rng.standard_normal(shape)).astype(np.float32)
    return out


# weight file: little-endian
#   magic "JLW1" | u32 version (1) | u32 n_tensors | u32 header_bytes
#   n_tensors x entry: u16 name_len | name bytes | u8 ndim | ndim x u32 dims |
#                      u64 data_offset | u64 checksum
#   data: float32 tensors, each starting at a 256-byte aligned offset
# checksum = sum of the tensor's little-endian uint32 words modulo 2^64
WEIGHT_FILE_MAGIC = b"JLW1"
WEIGHT_FILE_VERSION = 1
_ALIGN = 256


def tensor_checksum(a: np.ndarray) -> int:
    w = np.ascontiguousarray(a, dtype="<f4").view("<u4").ravel()
    total = 0
    step = 1 << 24
    for i in range(0, w.size, step):
        total += int(w[i:i + step].sum(dtype=np.uint64))
    return total % (1 << 64)


def weight_file_header(tensors: Sequence[Tuple[str, Tuple[int, ...], int]]) -> Tuple[bytes, List[int], int]:
    """Header bytes of a weight file holding `tensors` ((name, shape,
    checksum) in file order), each tensor's data offset and the file size."""
    hdr_size = 16
    for n, shape, _ in tensors:
        hdr_size += 2 + len(n.encode()) + 1 + 4 * len(shape) + 16
    off = (hdr_size + _ALIGN - 1) // _ALIGN * _ALIGN
    layout = []
    for _, shape, _ in tensors:
        layout.append(off)
        off += int(np.prod(shape)) * 4
        off = (off + _ALIGN - 1) // _ALIGN * _ALIGN
    hdr = bytearray()
    hdr += WEIGHT_FILE_MAGIC
    hdr += struct.pack("<III", WEIGHT_FILE_VERSION, len(tensors), hdr_size)
    for (n, shape, checksum), o in zip(tensors, layout):
        nb = n.encode()
        hdr += struct.pack("<H", len(nb)) + nb + struct.pack("<B", len(shape))
        hdr += struct.pack("<" + "I" * len(shape), *shape)
        hdr += struct.pack("<QQ", o, checksum)
    assert len(hdr) == hdr_size
    return bytes(hdr), layout, off


def write_weight_file(path: str, weights: Dict[str, np.ndarray]) -> None:
    names = [n for n, _, _ in weight_spec(weights["embeddings.tok_embeddings.weight"].shape[0])]
    hdr, layout, total = weight_file_header([(n, weights[n].shape, tensor_checksum(weights[n])) for n in names])
    tmp = path + ".tmp%d" % os.getpid()
    with open(tmp, "wb") as f:
        f.write(hdr)
        for n, o in zip(names, layout):
            f.seek(o)
            f.write(np.ascontiguousarray(weights[n], dtype="<f4").tobytes())
        f.truncate(total)
    os.replace(tmp, path)


def cached_weight_file(seed: int = WEIGHT_SEED, norm_jitter: bool = False,
                       directory: Optional[str] = None,
                       weights: Optional[Dict[str, np.ndarray]] = None, std: float = INIT_STD) -> str:
    """Path of the weight file for (``seed``, ``norm_jitter``, ``std``), written once per directory."""
    directory = directory or os.environ.get("JL_WEIGHT_DIR") or "/tmp"
    tag = "" if std == INIT_STD else "_std%g" % std
    path = os.path.join(directory, "jl_weights_s%d%s%s.bin" % (seed, "_jit" if norm_jitter else "", tag))
    if not os.path.exists(path):
        write_weight_file(path, weights if weights is not None else make_weights(seed, norm_jitter, std=std))
    return path


# ---------------------------------------------------------------------------
# batches
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Batch:
    """A packed, unpadded batch: what the forward pass consumes."""
    ids: np.ndarray             # int32 [T]
    seq_offsets: np.ndarray     # int32 [B+1], cumulative lengths
    mask_positions: np.ndarray  # int32 [M], absolute indices, increasing
    qtype: np.ndarray           # int32 [B]: 0 choice, 1 score, 2 noul

    @property
    def n_tokens(self) -> int:
        return int(self.seq_offsets[-1])

    @property
    def n_seqs(self) -> int:
        return int(self.qtype.shape[0])

    @property
    def n_markers(self) -> int:
        return int(self.mask_positions.shape[0])

    def sequence(self, b: int) -> Tuple[np.ndarray, np.ndarray, int]:
        """(ids, marker positions relative to the sequence, qtype) of sequence b."""
        s, e = int(self.seq_offsets[b]), int(self.seq_offsets[b + 1])
        m = self.mask_positions
        sel = m[(m >= s) & (m < e)] - s
        return self.ids[s:e], sel.astype(np.int32), int(self.qtype[b])

    def subset(self, seqs: Sequence[int]) -> "Batch":
        parts = [self.sequence(b) for b in seqs]
        return pack([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])


def head_length(q: int, option_lengths: Sequence[int]) -> int:
    """Tokens from <bos> through the <eos> that closes the options."""
    return 6 + q + sum(1 + l for l in option_lengths)


def layout_sequence(rng: np.random.Generator, qtype: int, q: int,
                    option_lengths: Sequence[int], state: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token ids and marker positions of one serialized decision."""
    def words(n):
        return rng.integers(FIRST_ORDINARY_ID, VOCAB, size=n, dtype=np.int64).tolist()
    toks = [BOS] + list(TYPE_WORDS[qtype]) + words(q) + [EOS]
    marks = []
    for l in option_lengths:
        marks.append(len(toks))
        toks += [MASK] + words(l)
    toks += [EOS] + words(state) + [EOS]
    return np.asarray(toks, np.int32), np.asarray(marks, np.int32)


def marker_positions(q: int, option_lengths: Sequence[int]) -> List[int]:
    """Marker positions of a layout without drawing any token (for layout checks)."""
    pos, out = 1 + 3 + q + 1, []
    for l in option_lengths:
        out.append(pos)
        pos += 1 + l
    return out


def pack(seq_ids: Sequence[np.ndarray], seq_marks: Sequence[np.ndarray], qtypes: Sequence[int]) -> Batch:
    lens = [len(s) for s in seq_ids]
    offs = np.zeros(len(lens) + 1, np.int32)
    offs[1:] = np.cumsum(lens)
    ids = np.concatenate(seq_ids).astype(np.int32) if seq_ids else np.zeros(0, np.int32)
    marks = (np.concatenate([m + offs[i] for i, m in enumerate(seq_marks)]).astype(np.int32)
             if seq_marks else np.zeros(0, np.int32))
    return Batch(ids, offs, marks, np.asarray(qtypes, np.int32))


def _draw_head(rng, qtype: int, limit: int):
    """(q, option lengths) of a random decision whose head fits ``limit``."""
    while True:
        n = 2 if qtype == NOUL else int(rng.integers(2, 21))
        lens = rng.integers(1, 49, size=n).tolist()
        q = int(rng.integers(4, 33))
        if head_length(q, lens) <= limit:
            return q, lens


CONFIG_NAMES = {
    0: "smoke 1x128 choice, 3 options",
    1: "latency 1x1024 score, 20 options",
    2: "throughput 16x1024 mixed types",
    3: "long-context 16x8192, 5 options",
    4: "ragged serving mix, 256 seqs of 64-2048",
}


def concat(batches: Sequence[Batch]) -> Batch:
    """One packed batch holding every sequence of ``batches`` in order."""
    parts = [b.sequence(i) for b in batches for i in range(b.n_seqs)]
    return pack([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])


def make_batch(config: int, seed: Optional[int] = None) -> Batch:
    """The packed batch of one of the five workload configurations."""
    rng = np.random.default_rng(1000 + config if seed is None else seed)
    ids, marks, types = [], [], []
    if config == 0:
        t, m = layout_sequence(rng, CHOICE, 10, [6, 6, 6], 128 - head_length(10, [6] * 3) - 1)
        ids.append(t); marks.append(m); types.append(CHOICE)
    elif config == 1:
        lens = [20] * 20
        t, m = layout_sequence(rng, SCORE, 30, lens, 1024 - head_length(30, lens) - 1)
        ids.append(t); marks.append(m); types.append(SCORE)
    elif config == 2:
        for r in range(16):
            qt = r % 3
            q, lens = _draw_head(rng, qt, 512)
            t, m = layout_sequence(rng, qt, q, lens, 1024 - head_length(q, lens) - 1)
            ids.append(t); marks.append(m); types.append(qt)
    elif config == 3:
        lens = [40] * 5
        for r in range(16):
            qt = CHOICE if r % 2 == 0 else SCORE
            t, m = layout_sequence(rng, qt, 45, lens, 8192 - head_length(45, lens) - 1)
            ids.append(t); marks.append(m); types.append(qt)
    elif config == 4:
        for r in range(256):
            L = int(rng.integers(64, 2049))
            qt = int(rng.integers(0, 3))
            q, lens = _draw_head(rng, qt, min(512, L - 2))
            t, m = layout_sequence(rng, qt, q, lens, L - head_length(q, lens) - 1)
            ids.append(t); marks.append(m); types.append(qt)
    else:
        raise ValueError("unknown configuration %r" % (config,))
    return pack(ids, marks, types)


def make_ragged_batch(seed: int, n_seqs: int, min_len: int, max_len: int) -> Batch:
    """A ragged batch like the serving mix, with lengths uniform in [min_len, max_len]."""
    rng = np.random.default_rng(seed)
    ids, marks, types = [], [], []
    for _ in range(n_seqs):
        L = int(rng.integers(min_len, max_len + 1))
        qt = int(rng.integers(0, 3))
        limit = min(512, L - 2)
        q, lens = _draw_head(rng, qt, limit)
        t, m = layout_sequence(rng, qt, q, lens, L - head_length(q, lens) - 1)
        ids.append(t); marks.append(m); types.append(qt)
    return pack(ids, marks, types)
