"""The benchmark's algorithmic work counts (host only).

Every roofline and utilization figure `bench.py` reports divides these counts
by a measured time, so they are pinned here against figures derived from the
model's shapes and by brute force, not against the counting code itself.
"""
import numpy as np
import pytest

import bench
from encoder_transformer_amd import synth

D, HEADS, HD = 384, 6, 64
GEMM_CLASSES = ("embed", "qkv", "outproj", "mlp_in", "mlp_out", "layer", "head_layer", "head_gemm", "misc")


def window_pairs_brute(L, w=64):
    """(query, key) pairs of one sequence with |i - j| <= w, by enumeration."""
    return sum(1 for i in range(L) for j in range(L) if abs(i - j) <= w)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 128, 129, 130, 200, 300])
def test_band_pairs_brute_force(L):
    assert bench.band_pairs(L) == window_pairs_brute(L)


@pytest.mark.parametrize("L", [129, 1024, 2048, 8192])
def test_band_pairs_closed_form(L):
    # every query sees 129 keys except the 64 at each end, which lose
    # 64 + 63 + ... + 1 = 2,080 keys per end
    assert bench.band_pairs(L) == 129 * L - 2 * 2080


def per_token_gemm_flops():
    """2 x multiply-adds per token, from the layer shapes (no shared code)."""
    encoder_layer = D * 3 * D + D * D + D * 2 * 1152 + 1152 * D  # QKV, out, W_i (GELU + gate halves), W_out
    head_layer1 = D * 3 * D + D * D + D * 1536 + 1536 * D  # in-projection, out-projection, FFN
    head_layer2_kv = D * 2 * D  # keys and values of every token
    return 2 * (22 * encoder_layer + head_layer1 + head_layer2_kv)


def per_marker_flops():
    head_layer2_rest = D * D + D * D + D * 1536 + 1536 * D  # query, out-projection, FFN
    scorer = D * D + D  # Linear(384, 384), then Linear(384, 1)
    return 2 * (head_layer2_rest + scorer)


def test_per_token_count_matches_the_model_shapes():
    assert per_token_gemm_flops() == 88_473_600  # encoder 84,344,832 + head 3,538,944 + 589,824


@pytest.mark.parametrize("config", [0, 1])
@pytest.mark.parametrize("row_block", [False, True])
def test_class_flops_totals(config, row_block):
    batch = synth.make_batch(config)
    f = bench.class_flops(batch, row_block)
    T, M = int(batch.seq_offsets[-1]), batch.n_markers
    gemm = sum(f.get(k, 0) for k in GEMM_CLASSES)
    assert gemm == per_token_gemm_flops() * T + per_marker_flops() * M
    lens = np.diff(batch.seq_offsets)
    pair = 2 * 2 * HD * HEADS  # QK^T and PV per (query, key) pair over the heads
    assert f["attn_global"] == 8 * pair * int(np.sum(lens.astype(np.int64) ** 2))
    assert f["attn_local"] == 14 * pair * sum(window_pairs_brute(int(L)) for L in lens)
    markers = [len(batch.sequence(b)[1]) for b in range(batch.n_seqs)]
    assert f["head_attn"] == pair * int(sum(int(L) * (int(L) + m) for L, m in zip(lens, markers)))


def test_class_split_does_not_change_the_total():
    batch = synth.make_batch(0)
    a, b = bench.class_flops(batch, False), bench.class_flops(batch, True)
    assert sum(a.values()) == sum(b.values())
