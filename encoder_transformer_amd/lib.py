"""Python binding of libjl (include/jl.h): argument marshalling only.

Every step of the forward pass runs in the library's HIP kernels. PyTorch
supplies device memory and streams; host-side batch metadata travels as
NumPy int32 arrays. The binding raises `JLError` on any non-zero status and
`RuntimeError` when the library has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjl.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "jl.h")

FP32, BF16, FP8 = 0, 1, 2  # jl_precision: FP32 products; bf16 operands; bf16 with e4m3 QKV and W_i products
OK, ERR_ARG, ERR_OPTIONS, ERR_LENGTH, ERR_QTYPE, ERR_FILE, ERR_DEVICE, ERR_OOM, ERR_CAPACITY, ERR_GUARD = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
STATUS_NAMES = {0: "OK", -1: "ARG", -2: "OPTIONS", -3: "LENGTH", -4: "QTYPE", -5: "FILE",
                -6: "DEVICE", -7: "OOM", -8: "CAPACITY", -9: "GUARD"}
DEBUG_SYNC, DEBUG_REVERSE_BLOCKS, DEBUG_SIMULATE_FAULT = 1, 2, 4  # jl_debug_flag
(K_EMBED, K_QKV, K_ATTN_GLOBAL, K_ATTN_LOCAL, K_OUTPROJ, K_MLP_IN, K_MLP_OUT, K_HEAD_GEMM, K_HEAD_ATTN,
 K_MISC, K_LN, K_LAYER, K_HEAD_LAYER) = range(13)
KERNEL_CLASS_NAMES = ["embed", "qkv", "attn_global", "attn_local", "outproj", "mlp_in", "mlp_out",
                      "head_gemm", "head_attn", "misc", "ln", "layer", "head_layer"]
N_KERNEL_CLASSES = len(KERNEL_CLASS_NAMES)

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
# int score(void *user, const int32_t *ids, const int32_t *seq_offsets, int32_t n_seqs,
#           const int32_t *mask_positions, int32_t n_markers, float *probs)
SCORE_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, _i32p, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32,
                            _f32p)
_lib = None


class JLError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"jl status {code} ({STATUS_NAMES.get(code, '?')}): {message}")
        self.code = code
        self.message = message


def load_library():
    """Load libjl.so (built by encoder_transformer_amd.build); raise if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m encoder_transformer_amd.build`")
    # PyTorch ships its own HIP runtime with the same soname (libamdhip64.so.7).
    # Loading torch first makes libjl bind to that one runtime instance, so the
    # streams and device pointers torch hands over are valid in libjl.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.jl_last_error.restype = ctypes.c_char_p
    L.jl_last_error.argtypes = []
    L.jl_load_weights.restype = ctypes.c_int
    L.jl_load_weights.argtypes = [ctypes.c_char_p, ctypes.c_int, i64, i64, ctypes.c_int, ctypes.POINTER(vp)]
    L.jl_free.restype = None
    L.jl_free.argtypes = [vp]
    L.jl_validate.restype = ctypes.c_int
    L.jl_validate.argtypes = [_i32p, i32, _i32p, i32, _i32p, i64, i64]
    L.jl_forward.restype = ctypes.c_int
    L.jl_forward.argtypes = [vp, vp, _i32p, i32, _i32p, i32, _i32p, vp, vp]
    L.jl_forward_static.restype = ctypes.c_int
    L.jl_forward_static.argtypes = [vp, vp, _i32p, i32, _i32p, i32, _i32p, vp, vp]
    L.jl_probs.restype = ctypes.c_int
    L.jl_probs.argtypes = [vp, vp, _i32p, i32, _i32p, i32, _i32p, vp, vp, vp, vp, vp]
    L.jl_debug_hidden.restype = ctypes.c_int
    L.jl_debug_hidden.argtypes = [vp, vp, _i32p, i32, _i32p, i32, _i32p, i32, vp, vp]
    L.jl_set_graph_cache.restype = ctypes.c_int
    L.jl_set_graph_cache.argtypes = [vp, ctypes.c_int]
    i64p = ctypes.POINTER(ctypes.c_int64)
    route_io = [i32, _i32p, i64p, _i32p, i64p, _i32p, i64p, _i32p, i32,
                _i32p, _f32p, _i32p, _i32p, _f32p, _i32p, _i32p]
    L.jl_route.restype = ctypes.c_int
    L.jl_route.argtypes = [vp] + route_io + [vp]
    L.jl_route_with_scorer.restype = ctypes.c_int
    L.jl_route_with_scorer.argtypes = [SCORE_FN, vp, i64, i64] + route_io
    L.jl_profile.restype = ctypes.c_int
    L.jl_profile.argtypes = [vp, ctypes.c_int, ctypes.c_uint32]
    L.jl_profile_read.restype = ctypes.c_int
    L.jl_profile_read.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.jl_set_row_block_min_tokens.restype = ctypes.c_int
    L.jl_set_row_block_min_tokens.argtypes = [vp, i64]
    L.jl_model_info.restype = ctypes.c_int
    L.jl_model_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.c_int]
    L.jl_set_debug.restype = ctypes.c_int
    L.jl_set_debug.argtypes = [vp, ctypes.c_uint32]
    L.jl_check_guards.restype = ctypes.c_int
    L.jl_check_guards.argtypes = [vp]
    L.jl_share.restype = ctypes.c_int
    L.jl_share.argtypes = [vp, i64, i64, ctypes.POINTER(vp)]
    L.jl_serve_plan.restype = ctypes.c_int
    L.jl_serve_plan.argtypes = [i32, i64p, i64p, i64, i64, i64, _i32p, _i32p, _i32p]
    L.jl_serve.restype = ctypes.c_int
    L.jl_serve.argtypes = [ctypes.POINTER(vp), i32, i32, _i32p, i64p, _i32p, i64p, _i32p, i64,
                           _f32p, _f32p, _f32p, _i32p, _f32p, _i32p]
    _lib = L
    return L


def declared_symbols() -> list:
    """Names of the functions include/jl.h declares."""
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(jl_[a-z_]+)\s*\(", text)))


def _check(rc: int):
    if rc != 0:
        raise JLError(rc, load_library().jl_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


class RouteResult:
    """Per question: pick (question-local option index), pick_prob, final
    candidates and their final probabilities, groups scored, rounds."""

    def __init__(self, pick, pick_prob, n_final, final_idx, final_prob, calls, rounds):
        self.pick, self.pick_prob, self.calls, self.rounds = pick, pick_prob, calls, rounds
        self.final = [list(final_idx[q, :n_final[q]]) for q in range(len(pick))]
        self.final_prob = [final_prob[q, :n_final[q]].copy() for q in range(len(pick))]


def _route_args(questions, mask_id):
    """questions: list of (prefix ids, suffix ids, [option ids, ...])."""
    nq = len(questions)
    cat = lambda parts: _i32(np.concatenate([np.asarray(p, np.int32) for p in parts])) if parts else _i32([])
    offs = lambda parts: np.ascontiguousarray(np.concatenate([[0], np.cumsum([len(p) for p in parts])]), np.int64)
    prefixes = [q[0] for q in questions]
    suffixes = [q[1] for q in questions]
    options = [o for q in questions for o in q[2]]
    q_opts = _i32(np.concatenate([[0], np.cumsum([len(q[2]) for q in questions])]))
    arrays = [cat(prefixes), offs(prefixes), cat(suffixes), offs(suffixes), cat(options), offs(options), q_opts]
    out = [np.zeros(nq, np.int32), np.zeros(nq, np.float32), np.zeros(nq, np.int32),
           np.zeros((nq, 20), np.int32), np.zeros((nq, 20), np.float32), np.zeros(nq, np.int32),
           np.zeros(nq, np.int32)]
    i64p = ctypes.POINTER(ctypes.c_int64)
    ptr = lambda a: a.ctypes.data_as(i64p if a.dtype == np.int64 else (_f32p if a.dtype == np.float32 else _i32p))
    args = [nq] + [ptr(a) for a in arrays] + [mask_id] + [ptr(a) for a in out]
    return args, arrays, out


def route_with_scorer(score, questions, mask_id: int = 4, max_tokens: int = 65536,
                      max_markers: int = 4096) -> RouteResult:
    """The router with a Python scorer: score(ids, seq_offsets, mask_positions)
    returns the option probabilities (NumPy, one per marker)."""
    failure = []

    def cb(_user, ids, so, n_seqs, mp, n_markers, probs):
        try:
            so_a = np.ctypeslib.as_array(so, (n_seqs + 1,)).copy()
            ids_a = np.ctypeslib.as_array(ids, (int(so_a[-1]),)).copy() if so_a[-1] > 0 else np.zeros(0, np.int32)
            mp_a = np.ctypeslib.as_array(mp, (n_markers,)).copy()
            p = np.asarray(score(ids_a, so_a, mp_a), np.float32)
            np.ctypeslib.as_array(probs, (n_markers,))[:] = p
            return 0
        except Exception as e:  # noqa: BLE001 - re-raised below
            failure.append(e)
            return ERR_ARG
    fn = SCORE_FN(cb)
    args, _keep, out = _route_args(questions, mask_id)
    rc = load_library().jl_route_with_scorer(fn, None, max_tokens, max_markers, *args)
    if rc != 0 and failure:
        raise failure[0]
    _check(rc)
    return RouteResult(*out)


def validate(seq_offsets, mask_positions, qtype, max_tokens: int, max_markers: int) -> None:
    so, mp, qt = _i32(seq_offsets), _i32(mask_positions), _i32(qtype)
    _check(load_library().jl_validate(_p(so), len(qt), _p(mp), len(mp), _p(qt), max_tokens, max_markers))


class Requests:
    """Independent requests for serve(): each (ids, marker positions inside
    the request, question type)."""

    def __init__(self, items):
        items = list(items)
        self.n = len(items)
        self.ids = _i32(np.concatenate([np.asarray(i, np.int32) for i, _, _ in items])) if items else _i32([])
        self.id_offsets = np.ascontiguousarray(np.concatenate([[0], np.cumsum([len(i) for i, _, _ in items])]),
                                               np.int64)
        self.mask_positions = (_i32(np.concatenate([np.asarray(m, np.int32) for _, m, _ in items]))
                               if items else _i32([]))
        self.mask_offsets = np.ascontiguousarray(np.concatenate([[0], np.cumsum([len(m) for _, m, _ in items])]),
                                                 np.int64)
        self.qtype = _i32([q for _, _, q in items])


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def serve_plan(requests: "Requests", max_batch_tokens: int, max_batch_markers: int, max_batch_seqs: int):
    """(order, batch_of, n_batches) of jl_serve_plan (host only)."""
    order = np.zeros(requests.n, np.int32)
    batch_of = np.zeros(requests.n, np.int32)
    nb = ctypes.c_int32()
    _check(load_library().jl_serve_plan(requests.n, _i64p(requests.id_offsets), _i64p(requests.mask_offsets),
                                        max_batch_tokens, max_batch_markers, max_batch_seqs, _p(order),
                                        _p(batch_of), ctypes.byref(nb)))
    return order, batch_of, nb.value


class ServeResult:
    """jl_serve outputs: per marker logits / probs (request order), per request
    answer, argmax and max probability, and the micro-batch count."""

    def __init__(self, requests, logits, probs, answer, argmax, maxprob, n_batches):
        self.logits, self.probs, self.answer, self.argmax, self.maxprob = logits, probs, answer, argmax, maxprob
        self.n_batches = n_batches
        self._mo = requests.mask_offsets

    def request_logits(self, r: int) -> np.ndarray:
        return self.logits[self._mo[r]:self._mo[r + 1]]


def serve(models, requests: "Requests", max_batch_tokens: int) -> ServeResult:
    """jl_serve over `models` (handles sharing weights, one stream each)."""
    L = load_library()
    hs = (ctypes.c_void_p * len(models))(*[m._h for m in models])
    M = int(requests.mask_offsets[-1])
    logits = np.zeros(M, np.float32)
    probs = np.zeros(M, np.float32)
    answer = np.zeros(requests.n, np.float32)
    argmax = np.zeros(requests.n, np.int32)
    maxprob = np.zeros(requests.n, np.float32)
    nb = ctypes.c_int32()
    f = lambda a: a.ctypes.data_as(_f32p)
    _check(L.jl_serve(hs, len(models), requests.n, _p(requests.ids), _i64p(requests.id_offsets),
                      _p(requests.mask_positions), _i64p(requests.mask_offsets), _p(requests.qtype),
                      int(max_batch_tokens), f(logits), f(probs), f(answer), _p(argmax), f(maxprob), ctypes.byref(nb)))
    return ServeResult(requests, logits, probs, answer, argmax, maxprob, nb.value)


class Model:
    """One loaded weight set on one device, with a workspace for `max_tokens` tokens."""

    def __init__(self, weight_path: Optional[str], precision: int = BF16, max_tokens: int = 16384,
                 max_markers: Optional[int] = None, device: int = 0, _share_from: Optional["Model"] = None):
        self._lib = load_library()
        self.device = device
        self.precision = precision
        self.max_tokens = int(max_tokens)
        self.max_markers = int(max_markers if max_markers is not None else max(2, min(max_tokens, 20 * 512)))
        h = ctypes.c_void_p()
        if _share_from is not None:
            _check(self._lib.jl_share(_share_from._h, self.max_tokens, self.max_markers, ctypes.byref(h)))
        else:
            _check(self._lib.jl_load_weights(weight_path.encode(), precision, self.max_tokens, self.max_markers,
                                             device, ctypes.byref(h)))
        self._h = h

    def share(self, max_tokens: Optional[int] = None, max_markers: Optional[int] = None) -> "Model":
        """A second handle over these weights with its own workspace (jl_share)."""
        return Model(None, self.precision, max_tokens or self.max_tokens, max_markers or self.max_markers,
                     self.device, _share_from=self)

    # -- helpers -----------------------------------------------------------
    def _stream(self, stream):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(s.cuda_stream)

    def _meta(self, seq_offsets, mask_positions, qtype):
        so, mp, qt = _i32(seq_offsets), _i32(mask_positions), _i32(qtype)
        return so, mp, qt

    def close(self):
        if getattr(self, "_h", None):
            self._lib.jl_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self) -> dict:
        buf = (ctypes.c_int64 * 10)()
        _check(self._lib.jl_model_info(self._h, buf, 10))
        keys = ["precision", "max_tokens", "max_markers", "device", "weight_bytes", "workspace_bytes",
                "graph_captures", "graph_replays", "poisoned", "debug"]
        return dict(zip(keys, list(buf)))

    def set_debug(self, flags: int):
        """jl_set_debug: DEBUG_SYNC | DEBUG_REVERSE_BLOCKS | DEBUG_SIMULATE_FAULT (0: off)."""
        _check(self._lib.jl_set_debug(self._h, int(flags)))

    def check_guards(self):
        """jl_check_guards: raise JLError (ERR_GUARD) if a workspace guard band was overwritten."""
        _check(self._lib.jl_check_guards(self._h))

    # -- entry points --------------------------------------------------------
    def forward(self, ids, seq_offsets, mask_positions, qtype, out=None, stream=None):
        """Option logits [n_markers] (torch float32 on the device)."""
        import torch
        so, mp, qt = self._meta(seq_offsets, mask_positions, qtype)
        if out is None:
            out = torch.empty(len(mp), dtype=torch.float32, device=f"cuda:{self.device}")
        _check(self._lib.jl_forward(self._h, ctypes.c_void_p(ids.data_ptr()), _p(so), len(qt), _p(mp), len(mp),
                                    _p(qt), ctypes.c_void_p(out.data_ptr()), self._stream(stream)))
        return out

    def forward_static(self, ids, seq_offsets, mask_positions, qtype, out, stream=None):
        """jl_forward_static: the forward pass on the library's static workspace
        (no allocation; at most 2,048 tokens and 256 markers)."""
        so, mp, qt = self._meta(seq_offsets, mask_positions, qtype)
        _check(self._lib.jl_forward_static(self._h, ctypes.c_void_p(ids.data_ptr()), _p(so), len(qt), _p(mp),
                                           len(mp), _p(qt), ctypes.c_void_p(out.data_ptr()), self._stream(stream)))
        return out

    def probs(self, logits, seq_offsets, mask_positions, qtype, stream=None, out=None):
        """(probs [M], answer [B], argmax [B] int32, maxprob [B]) as torch tensors on the device
        (written into `out`, such a 4-tuple, when given)."""
        import torch
        so, mp, qt = self._meta(seq_offsets, mask_positions, qtype)
        dev = f"cuda:{self.device}"
        if out is not None:
            probs, answer, argmax, maxprob = out
        else:
            probs = torch.empty(len(mp), dtype=torch.float32, device=dev)
            answer = torch.empty(len(qt), dtype=torch.float32, device=dev)
            argmax = torch.empty(len(qt), dtype=torch.int32, device=dev)
            maxprob = torch.empty(len(qt), dtype=torch.float32, device=dev)
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        _check(self._lib.jl_probs(self._h, ptr(logits), _p(so), len(qt), _p(mp), len(mp), _p(qt), ptr(probs),
                                  ptr(answer), ptr(argmax), ptr(maxprob), self._stream(stream)))
        return probs, answer, argmax, maxprob

    def debug_hidden(self, ids, seq_offsets, mask_positions, qtype, stage: int, stream=None, out=None):
        import torch
        so, mp, qt = self._meta(seq_offsets, mask_positions, qtype)
        rows = len(mp) if stage == 25 else int(so[-1])
        if out is None:
            out = torch.empty((rows, 384), dtype=torch.float32, device=f"cuda:{self.device}")
        _check(self._lib.jl_debug_hidden(self._h, ctypes.c_void_p(ids.data_ptr()), _p(so), len(qt), _p(mp),
                                         len(mp), _p(qt), stage, ctypes.c_void_p(out.data_ptr()),
                                         self._stream(stream)))
        return out

    def set_row_block_min_tokens(self, min_tokens: int):
        """bf16 batches with at least this many tokens use the row-block layer kernel."""
        _check(self._lib.jl_set_row_block_min_tokens(self._h, int(min_tokens)))

    def route(self, questions, mask_id: int = 4, stream=None) -> RouteResult:
        """The router (jl_route) over questions of (prefix ids, suffix ids, [option ids, ...])."""
        args, _keep, out = _route_args(questions, mask_id)
        _check(self._lib.jl_route(self._h, *args, self._stream(stream)))
        return RouteResult(*out)

    def set_graph_cache(self, max_graphs: int):
        """Replay jl_forward from captured HIP graphs, keeping up to max_graphs shapes (0: off)."""
        _check(self._lib.jl_set_graph_cache(self._h, int(max_graphs)))

    def profile(self, enable: int, class_mask: int = (1 << N_KERNEL_CLASSES) - 1):
        """1: on, clearing records; 2: on, keeping them; 0: off (records kept)."""
        _check(self._lib.jl_profile(self._h, int(enable), class_mask))

    def profile_read(self, kernel_class: int):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(self._lib.jl_profile_read(self._h, kernel_class, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value
