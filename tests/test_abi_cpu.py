"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, validates batches on the host and rejects bad weight files before
touching a device."""
import ctypes
import os
import struct

import numpy as np
import pytest

from encoder_transformer_amd import lib, synth


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        from encoder_transformer_amd import build
        build.build()
    return lib.load_library()


def test_exports_every_declared_symbol(L):
    names = lib.declared_symbols()
    assert {"jl_load_weights", "jl_forward", "jl_probs", "jl_validate", "jl_free", "jl_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def validate_code(so, mp, qt, max_tokens=100_000, max_markers=10_000):
    try:
        lib.validate(so, mp, qt, max_tokens, max_markers)
        return lib.OK
    except lib.JLError as e:
        assert e.message
        return e.code


def test_validate_accepts_the_configurations(L):
    for c in range(5):
        b = synth.make_batch(c)
        assert validate_code(b.seq_offsets, b.mask_positions, b.qtype, 300_000, 4096) == lib.OK
    assert validate_code([0], [], []) == lib.OK  # empty batch


@pytest.mark.parametrize("so,mp,qt,code", [
    ([0, 10], [3], [0], lib.ERR_OPTIONS),                     # one option
    ([0, 100], list(range(0, 42, 2)), [0], lib.ERR_OPTIONS),  # 21 options
    ([0, 10], [3, 5, 7], [2], lib.ERR_OPTIONS),               # noul with 3 options
    ([0, 10], [5, 3], [0], lib.ERR_OPTIONS),                  # unsorted
    ([0, 10], [3, 3], [0], lib.ERR_OPTIONS),                  # duplicated
    ([0, 10], [3, 10], [0], lib.ERR_OPTIONS),                 # outside every sequence
    ([0, 10], [-1, 3], [0], lib.ERR_OPTIONS),
    ([0, 10, 20], [2, 4, 12, 14, 15], [0, 0], lib.OK),
    ([0, 10, 20], [2, 4, 6, 12], [0, 0], lib.ERR_OPTIONS),    # second sequence has 1
    ([0, 10], [3, 5], [3], lib.ERR_QTYPE),
    ([0, 10], [3, 5], [-1], lib.ERR_QTYPE),
    ([1, 10], [3, 5], [0], lib.ERR_LENGTH),                   # offsets must start at 0
    ([0, 10, 10], [3, 5, 7, 8], [0, 0], lib.ERR_LENGTH),      # empty sequence
    ([0, 8193], [3, 5], [0], lib.ERR_LENGTH),                 # longer than 8,192
    ([0, 8192], [3, 5], [1], lib.OK),
])
def test_validate_errors(L, so, mp, qt, code):
    assert validate_code(so, mp, qt) == code


def test_validate_capacity(L):
    assert validate_code([0, 100], [3, 5], [0], max_tokens=99) == lib.ERR_CAPACITY
    assert validate_code([0, 100], [3, 5], [0], max_markers=1) == lib.ERR_CAPACITY


def test_null_and_negative_arguments(L):
    so = np.array([0, 10], np.int32)
    mp = np.array([3, 5], np.int32)
    qt = np.array([0], np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    null = ctypes.POINTER(ctypes.c_int32)()
    assert L.jl_validate(null, 1, p(mp), 2, p(qt), 100, 100) == lib.ERR_ARG
    assert L.jl_validate(p(so), 1, null, 2, p(qt), 100, 100) == lib.ERR_ARG
    assert L.jl_validate(p(so), 1, p(mp), 2, null, 100, 100) == lib.ERR_ARG
    assert L.jl_validate(p(so), -1, p(mp), 2, p(qt), 100, 100) == lib.ERR_ARG
    # entry points reject a NULL handle before anything else
    vp = ctypes.c_void_p
    assert L.jl_forward(None, None, p(so), 1, p(mp), 2, p(qt), None, None) == lib.ERR_ARG
    assert L.jl_probs(None, None, p(so), 1, p(mp), 2, p(qt), None, None, None, None, None) == lib.ERR_ARG
    assert L.jl_debug_hidden(None, None, p(so), 1, p(mp), 2, p(qt), 0, None, None) == lib.ERR_ARG
    assert L.jl_set_debug(None, lib.DEBUG_SYNC) == lib.ERR_ARG
    assert L.jl_check_guards(None) == lib.ERR_ARG
    L.jl_free(None)


def _header_enum(name):
    """{member: value} of `enum name { ... }` in include/jl.h."""
    import re
    with open(lib.HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    body = re.search(r"enum\s+" + name + r"\s*\{(.*?)\}", text, re.S).group(1)
    return {k: int(v) for k, v in re.findall(r"(JL_\w+)\s*=\s*(-?\d+)", body)}


def test_binding_constants_match_the_header():
    status = _header_enum("jl_status")
    assert {k[len("JL_"):]: v for k, v in status.items()} == {
        ("OK" if v == 0 else "ERR_" + lib.STATUS_NAMES[v]): v for v in lib.STATUS_NAMES}
    for k, v in status.items():
        assert getattr(lib, k[len("JL_"):]) == v, k
    debug = _header_enum("jl_debug_flag")
    assert debug == {"JL_DEBUG_SYNC": lib.DEBUG_SYNC, "JL_DEBUG_REVERSE_BLOCKS": lib.DEBUG_REVERSE_BLOCKS,
                     "JL_DEBUG_SIMULATE_FAULT": lib.DEBUG_SIMULATE_FAULT}
    assert _header_enum("jl_precision") == {"JL_FP32": lib.FP32, "JL_BF16": lib.BF16, "JL_FP8": lib.FP8}


def load_code(L, path, precision=lib.BF16, max_tokens=1024, max_markers=64):
    h = ctypes.c_void_p()
    rc = L.jl_load_weights(path.encode() if path else None, precision, max_tokens, max_markers, 0, ctypes.byref(h))
    assert not h.value
    return rc, L.jl_last_error().decode()


def write_header_only(path, tensors, magic=b"JLW1", version=1, data_bytes=0, checksum=0):
    """A weight file whose header lists `tensors` [(name, shape)], data left sparse."""
    hdr = bytearray(magic + struct.pack("<III", version, len(tensors), 0))
    body = bytearray()
    size = 16 + sum(2 + len(n) + 1 + 4 * len(s) + 16 for n, s in tensors)
    off = (size + 255) // 256 * 256
    for n, s in tensors:
        body += struct.pack("<H", len(n)) + n.encode() + struct.pack("<B", len(s))
        body += struct.pack("<" + "I" * len(s), *s) + struct.pack("<QQ", off, checksum)
        off += int(np.prod(s)) * 4
    hdr[12:16] = struct.pack("<I", size)
    with open(path, "wb") as f:
        f.write(bytes(hdr) + bytes(body))
        f.truncate(off if data_bytes is None else max(size, data_bytes))


def test_load_rejects_bad_files(L, tmp_path):
    assert load_code(L, None)[0] == lib.ERR_ARG
    assert load_code(L, str(tmp_path / "missing.bin"))[0] == lib.ERR_FILE
    p = str(tmp_path / "w.bin")
    emb = ("embeddings.tok_embeddings.weight", (256000, 384))
    write_header_only(p, [emb], magic=b"XXXX", data_bytes=None)
    assert load_code(L, p)[0] == lib.ERR_FILE
    write_header_only(p, [emb], version=2, data_bytes=None)
    assert load_code(L, p)[0] == lib.ERR_FILE
    write_header_only(p, [emb], data_bytes=4096)             # data truncated
    rc, msg = load_code(L, p)
    assert rc == lib.ERR_FILE and "truncated" in msg
    write_header_only(p, [("embeddings.tok_embeddings.weight", (1000, 384))], data_bytes=None)
    rc, msg = load_code(L, p)
    assert rc == lib.ERR_FILE and "shape" in msg
    write_header_only(p, [("something.else", (4,))], data_bytes=None)
    rc, msg = load_code(L, p)
    assert rc == lib.ERR_FILE and "lacks" in msg
    write_header_only(p, [emb], data_bytes=None, checksum=12345)  # zeros sum to 0
    rc, msg = load_code(L, p)
    assert rc == lib.ERR_FILE and "checksum" in msg
    with open(p, "wb") as f:
        f.write(b"JLW")
    assert load_code(L, p)[0] == lib.ERR_FILE


def test_load_rejects_bad_arguments(L, tmp_path):
    p = str(tmp_path / "x.bin")
    assert load_code(L, p, precision=7)[0] == lib.ERR_ARG
    assert load_code(L, p, max_tokens=0)[0] == lib.ERR_ARG
    assert load_code(L, p, max_markers=1)[0] == lib.ERR_ARG
    assert load_code(L, p, max_tokens=10, max_markers=20)[0] == lib.ERR_ARG


def test_weight_file_roundtrip_header(tmp_path):
    """The generator's file lists every tensor at its shape with its checksum."""
    w = synth.make_weights(seed=1, vocab=64)
    p = str(tmp_path / "small.bin")
    synth.write_weight_file(p, w)
    raw = open(p, "rb").read()
    assert raw[:4] == b"JLW1"
    _, n, hdr = struct.unpack("<III", raw[4:16])
    assert n == len(synth.weight_spec(64))
    off = 16
    for name, shape, _ in synth.weight_spec(64):
        nl = struct.unpack("<H", raw[off:off + 2])[0]
        assert raw[off + 2:off + 2 + nl].decode() == name
        off += 2 + nl
        nd = raw[off]
        dims = struct.unpack("<" + "I" * nd, raw[off + 1:off + 1 + 4 * nd])
        assert tuple(dims) == shape
        off += 1 + 4 * nd
        o, cs = struct.unpack("<QQ", raw[off:off + 16])
        off += 16
        data = np.frombuffer(raw, "<f4", count=int(np.prod(shape)), offset=o)
        assert np.array_equal(data.reshape(shape), w[name])
        assert cs == int(data.view("<u4").astype(np.uint64).sum()) % (1 << 64)
