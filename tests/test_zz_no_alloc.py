"""jl_forward_static, the allocation-free forward pass, against jl_forward.

The entry point runs the same kernels as jl_forward on a workspace held in
the library's static device array (one per GPU) instead of the handle's.
Checked through the C ABI on two calls in a row, the second smaller than the
first (the array keeps the previous call's contents), in each precision,
bitwise against jl_forward on the same batch; and its size limit.
"""
import ctypes

import numpy as np
import pytest

from encoder_transformer_amd import synth
from gpu_common import device_ids, run_logits

pytestmark = pytest.mark.gpu


def _static_logits(m, batch):
    import torch
    from encoder_transformer_amd import lib
    L = lib.load_library()
    out = torch.full((batch.n_markers,), float("nan"), dtype=torch.float32, device="cuda:0")
    ids = device_ids(batch)
    so = np.ascontiguousarray(batch.seq_offsets, np.int32)
    mp = np.ascontiguousarray(batch.mask_positions, np.int32)
    qt = np.ascontiguousarray(batch.qtype, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = L.jl_forward_static(m._h, ctypes.c_void_p(ids.data_ptr()), p(so), len(qt), p(mp), len(mp), p(qt),
                             ctypes.c_void_p(out.data_ptr()), None)
    torch.cuda.synchronize()
    assert rc == 0, L.jl_last_error().decode()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("prec", ["bf16", "fp32", "fp8"])
def test_forward_static_matches_forward(prec):
    from encoder_transformer_amd import lib
    m = lib.Model(synth.cached_weight_file(), {"bf16": lib.BF16, "fp32": lib.FP32, "fp8": lib.FP8}[prec],
                  4096, 512)
    try:
        big = synth.concat([synth.make_batch(1), synth.make_ragged_batch(5, 4, 100, 300)])  # near 2,048 tokens
        small = synth.make_batch(0)
        assert 1024 < big.n_tokens <= 2048
        for batch in (big, small, big):
            got = _static_logits(m, batch)
            ref = run_logits(m, batch)
            assert np.all(np.isfinite(got)) and np.array_equal(got, ref), (prec, batch.n_tokens)
    finally:
        m.close()


def test_forward_static_size_limit():
    import torch
    from encoder_transformer_amd import lib
    m = lib.Model(synth.cached_weight_file(), lib.BF16, 8192, 512)
    try:
        b = synth.make_batch(2).subset([0, 1, 2])  # 3,072 tokens
        out = torch.full((b.n_markers,), 7.0, device="cuda:0")
        with pytest.raises(lib.JLError) as e:
            m.forward_static(device_ids(b), b.seq_offsets, b.mask_positions, b.qtype, out)
        assert e.value.code == lib.ERR_CAPACITY and "2,048 tokens" in e.value.message
        torch.cuda.synchronize()
        assert torch.all(out == 7.0)
    finally:
        m.close()
