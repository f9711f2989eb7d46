"""Thin Python binding of libtq (include/tq.h).

Argument marshalling only: every step of the hot path runs in the HIP kernels
of libtq.so.  PyTorch supplies device memory and the current stream.  The
binding raises if the library is missing or a call fails; there is no other
code path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same library (the host-sanitizer
# build of build_lib.build_sanitized); there is no fallback when it is missing.
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "libtq.so")

MODE_PROD = 0
MODE_MSE = 1
F32 = 0
BF16 = 1

_STATUS = {0: "TQ_OK", 1: "TQ_ERR_INVALID_ARG", 2: "TQ_ERR_UNSUPPORTED",
           3: "TQ_ERR_ALIGNMENT", 4: "TQ_ERR_HIP", 5: "TQ_ERR_NO_MEMORY"}


class TQError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class _Params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("b", ctypes.c_int32), ("m", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("seed_pi", ctypes.c_uint64), ("seed_s", ctypes.c_uint64)]


class _PolarParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits1", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("seed_pi", ctypes.c_uint64)]


class _PolarCodes(ctypes.Structure):
    _fields_ = [("pq", ctypes.c_void_p), ("radius", ctypes.c_void_p)]


class _SplitParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("b_out", ctypes.c_int32), ("b_rest", ctypes.c_int32),
                ("n_out", ctypes.c_int32), ("seed_pi", ctypes.c_uint64), ("seed_s", ctypes.c_uint64),
                ("channels", ctypes.c_int32 * 128)]


class _SplitCodes(ctypes.Structure):
    _fields_ = [("words", ctypes.c_void_p), ("norms", ctypes.c_void_p)]


class _Codes(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("sgn", ctypes.c_void_p),
                ("knorm", ctypes.c_void_p), ("rnorm", ctypes.c_void_p)]


EXPORTS = ["tq_status_string", "tq_last_error", "tq_layout_version", "tq_make_codebook",
           "tq_codes_bytes", "tq_export_matrices", "tq_encode_workspace_bytes", "tq_encode",
           "tq_score_workspace_bytes",
           "tq_score", "tq_attend_workspace_bytes", "tq_attend", "tq_attend_noalloc", "tq_decode",
           "tq_search_workspace_bytes", "tq_search", "tq_encode_slots",
           "tq_attend_paged_workspace_bytes", "tq_attend_paged", "tq_polar_make_codebook", "tq_polar_encode",
           "tq_polar_score_workspace_bytes", "tq_polar_score", "tq_split_words", "tq_split_encode",
           "tq_split_score_workspace_bytes", "tq_split_score", "tq_release_cache"]

PAGE_POSITIONS = 512  # TQ_PAGE_POSITIONS

_lib = None


def lib():
    """Load libtq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, C, vp, i64 = ctypes.POINTER(_Params), _Codes, ctypes.c_void_p, ctypes.c_int64
        sz = ctypes.c_size_t
        PP, PC = ctypes.POINTER(_PolarParams), _PolarCodes
        SP, SC = ctypes.POINTER(_SplitParams), _SplitCodes
        sig = {
            "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "tq_last_error": (ctypes.c_char_p, []),
            "tq_layout_version": (ctypes.c_int32, []),
            "tq_make_codebook": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]),
            "tq_codes_bytes": (ctypes.c_int, [P, i64, ctypes.POINTER(sz)]),
            "tq_export_matrices": (ctypes.c_int, [P, vp, vp]),
            "tq_encode_workspace_bytes": (ctypes.c_int, [P, i64, ctypes.POINTER(sz)]),
            "tq_encode": (ctypes.c_int, [P, vp, ctypes.c_int32, i64, C, vp, sz, vp]),
            "tq_score_workspace_bytes": (ctypes.c_int, [P, i64, i64, ctypes.POINTER(sz)]),
            "tq_score": (ctypes.c_int, [P, vp, i64, i64, C, i64, vp, vp, sz, vp]),
            "tq_attend_workspace_bytes": (ctypes.c_int, [P, P, i64, i64, i64, i64, ctypes.POINTER(sz)]),
            "tq_attend": (ctypes.c_int, [P, P, vp, i64, i64, i64, C, C, i64, ctypes.c_float, vp, vp, sz, vp]),
            "tq_attend_noalloc": (ctypes.c_int, [P, P, vp, i64, i64, i64, C, C, i64, ctypes.c_float, vp, vp]),
            "tq_decode": (ctypes.c_int, [P, C, i64, vp, vp]),
            "tq_search_workspace_bytes": (ctypes.c_int, [P, i64, i64, ctypes.c_int32, ctypes.POINTER(sz)]),
            "tq_search": (ctypes.c_int, [P, vp, i64, C, i64, ctypes.c_int32, vp, vp, vp, sz, vp]),
            "tq_encode_slots": (ctypes.c_int, [P, vp, ctypes.c_int32, i64, vp, i64, C, vp]),
            "tq_attend_paged_workspace_bytes": (ctypes.c_int, [P, P, i64, i64, i64, i64, ctypes.POINTER(sz)]),
            "tq_attend_paged": (ctypes.c_int, [P, P, vp, i64, i64, i64, C, C, i64, vp, i64, vp, ctypes.c_float,
                                               vp, vp, sz, vp]),
            "tq_polar_make_codebook": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]),
            "tq_polar_encode": (ctypes.c_int, [PP, vp, ctypes.c_int32, i64, PC, vp]),
            "tq_polar_score_workspace_bytes": (ctypes.c_int, [PP, i64, i64, ctypes.POINTER(sz)]),
            "tq_polar_score": (ctypes.c_int, [PP, vp, i64, i64, PC, i64, vp, vp, sz, vp]),
            "tq_split_words": (ctypes.c_int, [SP, ctypes.POINTER(ctypes.c_int32)]),
            "tq_split_encode": (ctypes.c_int, [SP, vp, ctypes.c_int32, i64, SC, vp]),
            "tq_split_score_workspace_bytes": (ctypes.c_int, [SP, i64, i64, ctypes.POINTER(sz)]),
            "tq_split_score": (ctypes.c_int, [SP, vp, i64, i64, SC, i64, vp, vp, sz, vp]),
            "tq_release_cache": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise TQError(fn, status, lib().tq_last_error().decode())


@dataclass(frozen=True)
class Params:
    """The problem statement: d, total bits b, JL rows m, mode, seeds of Pi and S."""
    d: int
    b: int
    m: int = 128
    mode: int = MODE_PROD
    seed_pi: int = 2
    seed_s: int = 3

    @property
    def B(self) -> int:
        return self.b - 1 if self.mode == MODE_PROD else self.b

    @property
    def prod(self) -> bool:
        return self.mode == MODE_PROD

    def c(self) -> _Params:
        return _Params(self.d, self.b, self.m, self.mode, self.seed_pi, self.seed_s)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------- host calls
def make_codebook(d: int, b: int, mode: int = MODE_PROD):
    B = b - 1 if mode == MODE_PROD else b
    c = np.zeros(max(1, 1 << B), dtype=np.float32)
    t = np.zeros(max(1, (1 << B) - 1), dtype=np.float32)
    _check("tq_make_codebook", lib().tq_make_codebook(d, b, mode, c.ctypes.data, t.ctypes.data))
    return c[: (1 << B) if B else 0], t[: (1 << B) - 1 if B else 0]


def codes_bytes(p: Params, n: int):
    out = (ctypes.c_size_t * 4)()
    _check("tq_codes_bytes", lib().tq_codes_bytes(ctypes.byref(p.c()), n, out))
    return list(out)


def export_matrices(p: Params):
    pi = np.zeros((p.d, p.d), dtype=np.float32)
    s = np.zeros((p.m, p.d), dtype=np.float32) if p.prod else None
    _check("tq_export_matrices", lib().tq_export_matrices(
        ctypes.byref(p.c()), pi.ctypes.data, None if s is None else s.ctypes.data))
    return pi, s


def encode_workspace_bytes(p: Params, n: int) -> int:
    out = ctypes.c_size_t()
    _check("tq_encode_workspace_bytes", lib().tq_encode_workspace_bytes(ctypes.byref(p.c()), n, ctypes.byref(out)))
    return out.value


def score_workspace_bytes(p: Params, n_kv: int, g: int) -> int:
    out = ctypes.c_size_t()
    _check("tq_score_workspace_bytes", lib().tq_score_workspace_bytes(ctypes.byref(p.c()), n_kv, g, ctypes.byref(out)))
    return out.value


def attend_workspace_bytes(kp: Params, vp: Params, batch, n_kv, g, seq) -> int:
    out = ctypes.c_size_t()
    _check("tq_attend_workspace_bytes", lib().tq_attend_workspace_bytes(
        ctypes.byref(kp.c()), ctypes.byref(vp.c()), batch, n_kv, g, seq, ctypes.byref(out)))
    return out.value


def search_workspace_bytes(p: Params, nq: int, n: int, k: int) -> int:
    out = ctypes.c_size_t()
    _check("tq_search_workspace_bytes", lib().tq_search_workspace_bytes(ctypes.byref(p.c()), nq, n, k, ctypes.byref(out)))
    return out.value


def release_cache():
    _check("tq_release_cache", lib().tq_release_cache())


# ----------------------------------------------------------------- device memory
def alloc_codes(p: Params, n: int, device="cuda"):
    """Caller-owned code arrays (torch tensors) for n vectors."""
    import torch
    B = p.B
    return {
        "idx": torch.empty((n, p.d // 32, B), dtype=torch.int32, device=device) if B else None,
        "sgn": torch.empty((n, p.m // 32), dtype=torch.int32, device=device) if p.prod else None,
        "knorm": torch.empty((n,), dtype=torch.float32, device=device),
        "rnorm": torch.empty((n,), dtype=torch.float32, device=device) if p.prod else None,
    }


def _codes(c: dict) -> _Codes:
    return _Codes(*(None if c.get(k) is None else c[k].data_ptr() for k in ("idx", "sgn", "knorm", "rnorm")))


# ----------------------------------------------------------------- device calls
def alloc_workspace(nbytes: int, device="cuda"):
    """A device byte buffer (None for 0 bytes)."""
    import torch
    return torch.empty((nbytes,), dtype=torch.uint8, device=device) if nbytes else None


def encode(p: Params, x, codes: dict, workspace=None, stream=None):
    """x: cuda tensor [n, d] float32 or bfloat16, contiguous.  workspace: a
    device buffer of >= encode_workspace_bytes(p, n) bytes, allocated here if
    not given."""
    import torch
    assert x.is_contiguous() and x.dim() == 2 and x.shape[1] == p.d
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    if workspace is None:
        workspace = alloc_workspace(encode_workspace_bytes(p, x.shape[0]), x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tq_encode", lib().tq_encode(ctypes.byref(p.c()), _ptr(x), dt, x.shape[0],
                                        _codes(codes), _ptr(workspace), wsb, _stream(stream)))


def score(p: Params, q, codes: dict, n_kv: int, g: int, seq: int, logits, workspace, stream=None):
    """q: [n_kv*g, d] float32; logits: [n_kv*g, seq] float32 (written)."""
    assert q.is_contiguous() and logits.is_contiguous()
    _check("tq_score", lib().tq_score(ctypes.byref(p.c()), _ptr(q), n_kv, g, _codes(codes), seq,
                                      _ptr(logits), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


def attend(kp: Params, vp: Params, q, batch, n_kv, g, kcodes, vcodes, seq, out, workspace,
           scale: float = 0.0, stream=None):
    """q: [batch, n_kv*g, d] float32; out: [batch, n_kv*g, d] float32 (written)."""
    assert q.is_contiguous() and out.is_contiguous()
    _check("tq_attend", lib().tq_attend(ctypes.byref(kp.c()), ctypes.byref(vp.c()), _ptr(q), batch, n_kv, g,
                                        _codes(kcodes), _codes(vcodes), seq, scale, _ptr(out),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # TQ_NOALLOC_SCRATCH_BYTES


def attend_noalloc(kp: Params, vp: Params, q, batch, n_kv, g, kcodes, vcodes, seq, out,
                   scale: float = 0.0, stream=None):
    """tq_attend without a workspace (the library's per-GPU scratch array):
    q: [batch, n_kv*g, d] float32; out: [batch, n_kv*g, d] float32 (written)."""
    assert q.is_contiguous() and out.is_contiguous()
    _check("tq_attend_noalloc", lib().tq_attend_noalloc(ctypes.byref(kp.c()), ctypes.byref(vp.c()), _ptr(q),
                                                        batch, n_kv, g, _codes(kcodes), _codes(vcodes), seq,
                                                        scale, _ptr(out), _stream(stream)))


def decode(p: Params, codes: dict, n: int, out, stream=None):
    """out: [n, d] float32 (written) = ||x|| Pi^T c[idx]."""
    assert out.is_contiguous()
    _check("tq_decode", lib().tq_decode(ctypes.byref(p.c()), _codes(codes), n, _ptr(out), _stream(stream)))


def search(p: Params, q, codes: dict, n: int, k: int, out_idx, out_val, workspace, stream=None):
    """q: [nq, d] float32; out_idx: [nq, k] int64; out_val: [nq, k] float32 or None."""
    assert q.is_contiguous() and out_idx.is_contiguous()
    _check("tq_search", lib().tq_search(ctypes.byref(p.c()), _ptr(q), q.shape[0], _codes(codes), n, k,
                                        _ptr(out_idx), _ptr(out_val), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def encode_slots(p: Params, x, slots, capacity: int, codes: dict, stream=None):
    """x: [n, d] float32/bfloat16; slots: [n] int64 (device); vector i goes to
    slot slots[i] of a store of `capacity` vectors (codes sized for it)."""
    import torch
    assert x.is_contiguous() and slots.is_contiguous() and slots.dtype == torch.int64
    assert slots.numel() == x.shape[0]
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    _check("tq_encode_slots", lib().tq_encode_slots(ctypes.byref(p.c()), _ptr(x), dt, x.shape[0], _ptr(slots),
                                                    capacity, _codes(codes), _stream(stream)))


def attend_paged_workspace_bytes(kp: Params, vp: Params, batch: int, n_kv: int, g: int, max_pages: int) -> int:
    out = ctypes.c_size_t()
    _check("tq_attend_paged_workspace_bytes",
           lib().tq_attend_paged_workspace_bytes(ctypes.byref(kp.c()), ctypes.byref(vp.c()), batch, n_kv, g,
                                                 max_pages, ctypes.byref(out)))
    return out.value


def attend_paged(kp: Params, vp: Params, q, batch, n_kv, g, kcodes, vcodes, num_pages, block_table,
                 seq_lens, out, workspace, scale: float = 0.0, stream=None):
    """block_table: [batch, max_pages] int32; seq_lens: [batch] int32 (device);
    q, out: [batch, n_kv*g, d] float32."""
    import torch
    assert q.is_contiguous() and out.is_contiguous() and block_table.is_contiguous()
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    _check("tq_attend_paged", lib().tq_attend_paged(
        ctypes.byref(kp.c()), ctypes.byref(vp.c()), _ptr(q), batch, n_kv, g, _codes(kcodes), _codes(vcodes),
        num_pages, _ptr(block_table), block_table.shape[1], _ptr(seq_lens), scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


# ----------------------------------------------------------------- PolarQuant
@dataclass(frozen=True)
class PolarParams:
    """d, bits of a level-1 angle, bits of the later levels, seed of Pi."""
    d: int = 128
    bits1: int = 4
    bits: int = 2
    seed_pi: int = 2

    def c(self) -> _PolarParams:
        return _PolarParams(self.d, self.bits1, self.bits, 0, self.seed_pi)


POLAR_WORDS = 12  # uint32 words of a packed record at d = 128


def polar_make_codebook(d: int, level: int, nbits: int):
    c = np.zeros(1 << nbits, dtype=np.float32)
    t = np.zeros((1 << nbits) - 1, dtype=np.float32)
    _check("tq_polar_make_codebook", lib().tq_polar_make_codebook(d, level, nbits, c.ctypes.data, t.ctypes.data))
    return c, t


def alloc_polar_codes(n: int, device="cuda"):
    import torch
    return {"pq": torch.empty((n, POLAR_WORDS), dtype=torch.int32, device=device),
            "radius": torch.empty((n,), dtype=torch.float32, device=device)}


def _pcodes(c: dict) -> _PolarCodes:
    return _PolarCodes(c["pq"].data_ptr(), c["radius"].data_ptr())


def polar_encode(p: PolarParams, x, codes: dict, stream=None):
    """x: cuda tensor [n, d] float32 or bfloat16, contiguous."""
    import torch
    assert x.is_contiguous()
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    _check("tq_polar_encode", lib().tq_polar_encode(ctypes.byref(p.c()), _ptr(x), dt, x.shape[0], _pcodes(codes),
                                                    _stream(stream)))


def polar_score_workspace_bytes(p: PolarParams, n_kv: int, g: int) -> int:
    out = ctypes.c_size_t()
    _check("tq_polar_score_workspace_bytes",
           lib().tq_polar_score_workspace_bytes(ctypes.byref(p.c()), n_kv, g, ctypes.byref(out)))
    return out.value


def polar_score(p: PolarParams, q, codes: dict, n_kv: int, g: int, seq: int, logits, workspace, stream=None):
    """q: [n_kv*g, d] float32; logits: [n_kv*g, seq] float32 (written)."""
    assert q.is_contiguous() and logits.is_contiguous()
    _check("tq_polar_score", lib().tq_polar_score(ctypes.byref(p.c()), _ptr(q), n_kv, g, _pcodes(codes), seq,
                                                  _ptr(logits), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(), _stream(stream)))


# ----------------------------------------------------------------- mixed bit widths
class SplitParams:
    """Outlier-channel split of a d = 128 head: channels (a permutation of
    0..127, the first n_out are the outlier channels; n_out = 32, 64 or 96),
    b_out = b_rest + 1."""

    def __init__(self, channels, b_out: int = 3, b_rest: int = 2, seed_pi: int = 2, seed_s: int = 3,
                 n_out: int = 64):
        ch = [int(c) for c in channels]
        assert len(ch) == 128
        self.channels, self.b_out, self.b_rest, self.seed_pi, self.seed_s = ch, b_out, b_rest, seed_pi, seed_s
        self.n_out = n_out

    def c(self) -> _SplitParams:
        return _SplitParams(128, self.b_out, self.b_rest, self.n_out, self.seed_pi, self.seed_s,
                            (ctypes.c_int32 * 128)(*self.channels))


def split_words(p: SplitParams) -> int:
    out = ctypes.c_int32()
    _check("tq_split_words", lib().tq_split_words(ctypes.byref(p.c()), ctypes.byref(out)))
    return out.value


def alloc_split_codes(p: SplitParams, n: int, device="cuda"):
    import torch
    return {"words": torch.empty((n, split_words(p)), dtype=torch.int32, device=device),
            "norms": torch.empty((n, 4), dtype=torch.float32, device=device)}


def _scodes(c: dict) -> _SplitCodes:
    return _SplitCodes(c["words"].data_ptr(), c["norms"].data_ptr())


def split_encode(p: SplitParams, x, codes: dict, stream=None):
    import torch
    assert x.is_contiguous()
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    _check("tq_split_encode", lib().tq_split_encode(ctypes.byref(p.c()), _ptr(x), dt, x.shape[0], _scodes(codes),
                                                    _stream(stream)))


def split_score_workspace_bytes(p: SplitParams, n_kv: int, g: int) -> int:
    out = ctypes.c_size_t()
    _check("tq_split_score_workspace_bytes",
           lib().tq_split_score_workspace_bytes(ctypes.byref(p.c()), n_kv, g, ctypes.byref(out)))
    return out.value


def split_score(p: SplitParams, q, codes: dict, n_kv: int, g: int, seq: int, logits, workspace, stream=None):
    """q: [n_kv*g, 128] float32; logits: [n_kv*g, seq] float32 (written)."""
    assert q.is_contiguous() and logits.is_contiguous()
    _check("tq_split_score", lib().tq_split_score(ctypes.byref(p.c()), _ptr(q), n_kv, g, _scodes(codes), seq,
                                                  _ptr(logits), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(), _stream(stream)))
