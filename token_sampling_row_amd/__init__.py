"""Python binding of libtsr.so, the gfx950 batched logits-to-token sampler.

Argument marshalling only: every step of the sampler runs in the HIP kernels
behind the C ABI declared in include/tsr.h. PyTorch supplies device memory and
the stream; tensors are passed as raw device pointers. There is no CPU
fallback: importing works without the library, but any call raises
``TsrUnavailable`` if libtsr.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "TsrError", "TsrUnavailable", "Params", "Sampler", "library_path", "load_library",
    "spec_verify_noalloc",
    "F32", "BF16", "JOINT", "SEQUENTIAL", "ROW_OK", "ROW_NONFINITE", "ROW_EMPTY",
    "ROW_BADTOKEN", "ROW_BADPARAM", "EXPORTED_SYMBOLS", "pack_row_params",
]

F32, BF16 = 0, 1
JOINT, SEQUENTIAL = 0, 1
ROW_OK, ROW_NONFINITE, ROW_EMPTY, ROW_BADTOKEN, ROW_BADPARAM = 0, 1, 2, 3, 4
EXPORTED_SYMBOLS = ("sampler_init", "sampler_destroy", "greedy_argmax", "sample_rows",
                    "sample_rows_masked", "sample_rows_ex", "spec_verify", "spec_verify_noalloc",
                    "tree_verify", "beam_step",
                    "sampler_philox", "sampler_strerror")

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("TSR_LIBRARY", os.path.join(_HERE, "libtsr.so"))


class TsrError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: error {code}")


class TsrUnavailable(RuntimeError):
    pass


class _Params(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_double), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_double), ("min_p", ctypes.c_double),
                ("filter_mode", ctypes.c_int32)]


class _Diag(ctypes.Structure):
    _fields_ = [("status", ctypes.c_void_p), ("kept_count", ctypes.c_void_p),
                ("threshold", ctypes.c_void_p), ("kept_mass", ctypes.c_void_p),
                ("probs", ctypes.c_void_p)]


class _Constraints(ctypes.Structure):
    _fields_ = [("allowed", ctypes.c_void_p), ("allowed_stride", ctypes.c_int64),
                ("history", ctypes.c_void_p), ("history_len", ctypes.c_int32),
                ("history_stride", ctypes.c_int64), ("repetition_penalty", ctypes.c_double),
                ("row_params", ctypes.c_void_p)]


_lib = None


def load_library():
    """Load libtsr.so once and declare its signatures. Raises TsrUnavailable."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise TsrUnavailable(f"{path} is not built; run token_sampling_row_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
    lib.sampler_init.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, u64]
    lib.sampler_destroy.argtypes = [vp]
    lib.greedy_argmax.argtypes = [vp, vp, i32, i32, i32, i64, vp, vp, vp]
    lib.sample_rows.argtypes = [vp, vp, i32, i32, i32, i64, ctypes.POINTER(_Params), u64, vp,
                                ctypes.POINTER(_Diag), vp]
    lib.sample_rows_masked.argtypes = [vp, vp, i32, i32, i32, i64, vp, i64,
                                       ctypes.POINTER(_Params), u64, vp, vp,
                                       ctypes.POINTER(_Diag), vp]
    lib.sample_rows_ex.argtypes = [vp, vp, i32, i32, i32, i64, ctypes.POINTER(_Constraints),
                                   ctypes.POINTER(_Params), u64, vp, vp, ctypes.POINTER(_Diag),
                                   vp]
    lib.spec_verify.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, ctypes.POINTER(_Params),
                                u64, vp, vp, vp, vp]
    lib.spec_verify_noalloc.argtypes = [i32, u64, vp, vp, i32, vp, i32, i32, i32,
                                        ctypes.POINTER(_Params), u64, vp, vp, vp, vp]
    lib.tree_verify.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, ctypes.POINTER(_Params),
                                u64, vp, vp, vp, vp, vp]
    lib.beam_step.argtypes = [vp, vp, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp]
    lib.sampler_philox.argtypes = [vp, vp, i32, vp, vp]
    lib.sampler_strerror.argtypes = [i32]
    lib.sampler_strerror.restype = ctypes.c_char_p
    for name in EXPORTED_SYMBOLS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(code: int, what: str):
    if code != 0:
        msg = load_library().sampler_strerror(code).decode()
        raise TsrError(code, f"{what}: {msg}")


@dataclass
class Params:
    """Sampling knobs (include/tsr.h, tsr_params). 0 / 1.0 / 0.0 switch a filter off."""

    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0
    mode: int = JOINT

    @staticmethod
    def of(p) -> "Params":
        if isinstance(p, Params):
            return p
        return Params(p.get("temperature", 1.0), p.get("top_k", 0), p.get("top_p", 1.0),
                      p.get("min_p", 0.0), p.get("mode", JOINT))

    def _c(self) -> _Params:
        return _Params(float(self.temperature), int(self.top_k), float(self.top_p),
                       float(self.min_p), int(self.mode))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"logits must be float32 or bfloat16, not {t.dtype}")


_raw_stream = None


def _current_stream_handle() -> int:
    """The current device's current stream as a raw handle. torch's C getter
    returns it without building a Stream object (a few microseconds a call,
    which bound small batches); the public API where that getter is absent."""
    global _raw_stream
    if _raw_stream is None:
        import torch
        getter = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        get_dev = getattr(torch._C, "_cuda_getDevice", None)
        if getter is not None and get_dev is not None:
            _raw_stream = lambda: getter(get_dev())
        else:
            _raw_stream = lambda: torch.cuda.current_stream().cuda_stream
    return _raw_stream()


def _stream_ptr(stream):
    return ctypes.c_void_p(_current_stream_handle() if stream is None else stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def pack_row_params(params_list):
    """Per-row parameters as the bytes of a tsr_params array (host uint8
    numpy array; copy it to the device for sample_rows_ex's row_params)."""
    import numpy as np
    arr = (_Params * len(params_list))(*[Params.of(p)._c() for p in params_list])
    return np.frombuffer(bytes(arr), dtype=np.uint8).copy()


def spec_verify_noalloc(device, seed, target, draft, draft_tokens, params, step: int,
                        out_tokens, out_accepted, out_status=None, stream=None):
    """spec_verify without a handle or any device allocation in the library
    (its workspace is a static device array; overlapping calls on one device
    race). Outputs must be preallocated: out_tokens [rows, K+1] and
    out_accepted [rows] int32 device tensors."""
    import torch
    rows, k1, vocab = target.shape
    assert target.is_contiguous() and (draft is None or draft.is_contiguous())
    assert draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous()
    cp = Params.of(params)._c()
    _check(load_library().spec_verify_noalloc(
        int(device), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)), _ptr(target), _ptr(draft),
        _dtype_code(target), _ptr(draft_tokens), rows, k1 - 1, vocab, ctypes.byref(cp),
        ctypes.c_uint64(int(step)), _ptr(out_tokens), _ptr(out_accepted), _ptr(out_status),
        _stream_ptr(stream)), "spec_verify_noalloc")
    return out_tokens, out_accepted


class Sampler:
    """A handle on one GPU: seed (the Philox key) and the verify workspace."""

    def __init__(self, device: int = 0, max_rows: int = 4096, max_vocab: int = 1 << 18,
                 max_k: int = 8, seed: int = 0):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.sampler_init(ctypes.byref(h), int(device), int(max_rows), int(max_vocab),
                                int(max_k), ctypes.c_uint64(int(seed) & (2 ** 64 - 1))),
               "sampler_init")
        self._h = h
        self.device = device
        self.seed = int(seed)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(load_library().sampler_destroy(self._h), "sampler_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ------------------------------------------------------------ calls
    def greedy_argmax(self, logits, out=None, status=None, stream=None):
        import torch
        rows, vocab = logits.shape
        assert logits.stride(1) == 1, "rows must be contiguous"
        out = torch.empty(rows, dtype=torch.int32, device=logits.device) if out is None else out
        _check(load_library().greedy_argmax(self._h, _ptr(logits), _dtype_code(logits), rows,
                                            vocab, logits.stride(0), _ptr(out), _ptr(status),
                                            _stream_ptr(stream)), "greedy_argmax")
        return out

    def sample_rows(self, logits, params, step: int, out=None, diag=None, stream=None):
        """Draw one token per row. ``diag`` may be a dict of preallocated tensors
        with keys status, kept_count, threshold, kept_mass, probs."""
        import torch
        rows, vocab = logits.shape
        assert logits.stride(1) == 1, "rows must be contiguous"
        out = torch.empty(rows, dtype=torch.int32, device=logits.device) if out is None else out
        cp = Params.of(params)._c()
        d = None
        if diag is not None:
            d = _Diag(*(ctypes.c_void_p(diag[k].data_ptr()) if diag.get(k) is not None else None
                        for k in ("status", "kept_count", "threshold", "kept_mass", "probs")))
        _check(load_library().sample_rows(self._h, _ptr(logits), _dtype_code(logits), rows,
                                          vocab, logits.stride(0), ctypes.byref(cp),
                                          ctypes.c_uint64(int(step)), _ptr(out),
                                          ctypes.byref(d) if d is not None else None,
                                          _stream_ptr(stream)), "sample_rows")
        return out

    def sample_rows_masked(self, logits, allowed, params, step: int, out=None, logprob=None,
                           diag=None, stream=None):
        """sample_rows over the allowed tokens only. ``allowed``: [rows, W] int32
        device tensor of bit words (token i = bit i % 32 of word i // 32,
        W >= ceil(vocab / 32)), or None (every token allowed). ``logprob``: a
        preallocated [rows] float32 tensor for log p~ of each drawn token, or
        None. Returns the tokens."""
        import torch
        rows, vocab = logits.shape
        assert logits.stride(1) == 1, "rows must be contiguous"
        if allowed is not None:
            assert allowed.dtype == torch.int32 and allowed.stride(1) == 1
            astride = allowed.stride(0)
        else:
            astride = 0
        out = torch.empty(rows, dtype=torch.int32, device=logits.device) if out is None else out
        cp = Params.of(params)._c()
        d = None
        if diag is not None:
            d = _Diag(*(ctypes.c_void_p(diag[k].data_ptr()) if diag.get(k) is not None else None
                        for k in ("status", "kept_count", "threshold", "kept_mass", "probs")))
        _check(load_library().sample_rows_masked(
            self._h, _ptr(logits), _dtype_code(logits), rows, vocab, logits.stride(0),
            _ptr(allowed), astride, ctypes.byref(cp), ctypes.c_uint64(int(step)), _ptr(out),
            _ptr(logprob), ctypes.byref(d) if d is not None else None, _stream_ptr(stream)),
            "sample_rows_masked")
        return out

    def sample_rows_ex(self, logits, params, step: int, allowed=None, history=None,
                       penalty: float = 1.0, out=None, logprob=None, diag=None, stream=None,
                       row_params=None):
        """sample_rows with an allowed-token mask (as in sample_rows_masked) and
        a repetition penalty: ``history`` is a [rows, H] int32 device tensor of
        each row's recent token ids (H <= 64, ids outside [0, vocab) ignored),
        ``penalty`` the factor r >= 1. Returns the tokens."""
        import torch
        rows, vocab = logits.shape
        assert logits.stride(1) == 1, "rows must be contiguous"
        cs = _Constraints(None, 0, None, 0, 0, float(penalty), None)
        if row_params is not None:   # a device tensor of packed tsr_params (see pack_row_params)
            cs.row_params = row_params.data_ptr()
        if allowed is not None:
            assert allowed.dtype == torch.int32 and allowed.stride(1) == 1
            cs.allowed, cs.allowed_stride = allowed.data_ptr(), allowed.stride(0)
        if history is not None:
            assert history.dtype == torch.int32 and history.stride(1) == 1
            cs.history, cs.history_len = history.data_ptr(), history.shape[1]
            cs.history_stride = history.stride(0)
        out = torch.empty(rows, dtype=torch.int32, device=logits.device) if out is None else out
        cp = Params.of(params)._c() if params is not None else None
        d = None
        if diag is not None:
            d = _Diag(*(ctypes.c_void_p(diag[k].data_ptr()) if diag.get(k) is not None else None
                        for k in ("status", "kept_count", "threshold", "kept_mass", "probs")))
        _check(load_library().sample_rows_ex(
            self._h, _ptr(logits), _dtype_code(logits), rows, vocab, logits.stride(0),
            ctypes.byref(cs), ctypes.byref(cp) if cp is not None else None, ctypes.c_uint64(int(step)), _ptr(out),
            _ptr(logprob), ctypes.byref(d) if d is not None else None, _stream_ptr(stream)),
            "sample_rows_ex")
        return out

    def spec_verify(self, target, draft, draft_tokens, params, step: int, out_tokens=None,
                    out_accepted=None, out_status=None, stream=None):
        """target [rows, K+1, V], draft [rows, K, V] (None for temperature 0),
        draft_tokens [rows, K] int32 -> (tokens [rows, K+1], accepted [rows])."""
        import torch
        rows, k1, vocab = target.shape
        K = k1 - 1
        assert target.is_contiguous() and (draft is None or draft.is_contiguous())
        assert draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous()
        dev = target.device
        if out_tokens is None:
            out_tokens = torch.empty(rows, K + 1, dtype=torch.int32, device=dev)
        if out_accepted is None:
            out_accepted = torch.empty(rows, dtype=torch.int32, device=dev)
        cp = Params.of(params)._c()
        _check(load_library().spec_verify(self._h, _ptr(target), _ptr(draft), _dtype_code(target),
                                          _ptr(draft_tokens), rows, K, vocab, ctypes.byref(cp),
                                          ctypes.c_uint64(int(step)), _ptr(out_tokens),
                                          _ptr(out_accepted), _ptr(out_status),
                                          _stream_ptr(stream)), "spec_verify")
        return out_tokens, out_accepted

    def tree_verify(self, target, draft, parent, tokens, params, step: int, status=None,
                    stream=None):
        """target, draft [rows, N, V] (draft None at temperature 0), parent and
        tokens [rows, N] int32 -> (tokens [rows, N], path [rows, N],
        accepted [rows])."""
        import torch
        rows, N, vocab = target.shape
        assert target.is_contiguous() and (draft is None or draft.is_contiguous())
        assert parent.dtype == torch.int32 and parent.is_contiguous()
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        dev = target.device
        out_t = torch.empty(rows, N, dtype=torch.int32, device=dev)
        out_p = torch.empty(rows, N, dtype=torch.int32, device=dev)
        acc = torch.empty(rows, dtype=torch.int32, device=dev)
        cp = Params.of(params)._c()
        _check(load_library().tree_verify(self._h, _ptr(target), _ptr(draft), _dtype_code(target),
                                          _ptr(parent), _ptr(tokens), rows, N, vocab,
                                          ctypes.byref(cp), ctypes.c_uint64(int(step)),
                                          _ptr(out_t), _ptr(out_p), _ptr(acc), _ptr(status),
                                          _stream_ptr(stream)), "tree_verify")
        return out_t, out_p, acc

    def beam_step(self, logits, beam_scores, beam: int, status=None, stream=None):
        """logits [groups * beam, V] device tensor (row g * beam + b: beam b
        of group g), beam_scores [groups * beam] float64 device tensor ->
        (parent, token, score), each [groups, beam], best first."""
        import torch
        rows, vocab = logits.shape
        assert logits.stride(1) == 1 and rows % beam == 0
        assert beam_scores.dtype == torch.float64 and beam_scores.is_contiguous()
        groups = rows // beam
        dev = logits.device
        parent = torch.empty(groups, beam, dtype=torch.int32, device=dev)
        token = torch.empty(groups, beam, dtype=torch.int32, device=dev)
        score = torch.empty(groups, beam, dtype=torch.float64, device=dev)
        _check(load_library().beam_step(self._h, _ptr(logits), _dtype_code(logits), groups, beam,
                                        vocab, logits.stride(0), _ptr(beam_scores), _ptr(parent),
                                        _ptr(token), _ptr(score), _ptr(status),
                                        _stream_ptr(stream)), "beam_step")
        return parent, token, score

    def philox(self, counters, stream=None):
        """counters: [n, 4] int32/uint32 device tensor -> [n, 4] words (int32 view)."""
        import torch
        n = counters.shape[0]
        out = torch.empty(n, 4, dtype=torch.int32, device=counters.device)
        _check(load_library().sampler_philox(self._h, _ptr(counters), n, _ptr(out),
                                             _stream_ptr(stream)), "sampler_philox")
        return out
