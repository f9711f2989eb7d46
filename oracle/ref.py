"""ctypes binding of the C++ oracle (tq_oracle_ref.cpp).

TEST INFRASTRUCTURE ONLY: used by tests/ and by the cpu_baseline leg of
bench.py.  The library is built with g++ into oracle/libtqref.so (by
``build()``, which ``__graft_entry__.build()`` calls, or on first use here).
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq_oracle_ref.cpp")
LIB = os.path.join(HERE, "libtqref.so")
_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P, I64, I32, U64, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_double
        L.tqref_create.restype = P
        L.tqref_create.argtypes = [I32, I32, I32, I32, U64, U64]
        L.tqref_destroy.argtypes = [P]
        L.tqref_gaussian.argtypes = [U64, I64, I64, P]
        L.tqref_matrices.argtypes = [P, P, P, P, P]
        L.tqref_encode.argtypes = [P, P, I64, P, P, P, P, P, I32]
        L.tqref_score.argtypes = [P, P, I64, I64, P, P, P, P, I64, P, I32]
        L.tqref_attend.argtypes = [P, P, P, I64, I64, I64, I64, P, P, P, P, P, P, D, P, I32]
        L.tqref_search.argtypes = [P, P, I64, P, P, P, P, I64, I64, P, P, I32]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def gaussian(seed, rows, cols):
    out = np.empty((rows, cols), dtype=np.float64)
    lib().tqref_gaussian(seed, rows, cols, _ptr(out))
    return out


class Ref:
    """Parameters d, b, m, mode (0 prod, 1 mse) and the two seeds."""

    def __init__(self, d, b, m, mode=0, seed_pi=2, seed_s=3):
        self.d, self.b, self.m, self.mode = d, b, m, mode
        self.B = b - 1 if mode == 0 else b
        self.h = lib().tqref_create(d, b, m, mode, seed_pi, seed_s)
        if not self.h:
            raise ValueError("bad parameters")

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.tqref_destroy(self.h)

    def matrices(self):
        pi = np.empty((self.d, self.d))
        s = np.empty((self.m, self.d)) if self.mode == 0 else None
        L = 1 << self.B
        c = np.empty(L, dtype=np.float32) if self.B > 0 else None
        t = np.empty(L - 1, dtype=np.float32) if self.B > 0 else None
        lib().tqref_matrices(self.h, _ptr(pi), _ptr(s), _ptr(c), _ptr(t))
        return pi, s, c, t

    def encode(self, x, threads=1):
        x = np.ascontiguousarray(x, dtype=np.float64)
        n = x.shape[0]
        prod = self.mode == 0
        idx = np.empty((n, self.d), dtype=np.int32) if self.B > 0 else None
        sign = np.empty((n, self.m), dtype=np.uint8) if prod else None
        rnorm = np.empty(n, dtype=np.float32) if prod else None
        z = np.empty((n, self.m)) if prod else None
        knorm = np.empty(n, dtype=np.float32)
        lib().tqref_encode(self.h, _ptr(x), n, _ptr(idx), _ptr(sign), _ptr(knorm), _ptr(rnorm), _ptr(z), threads)
        out = {"knorm": knorm}
        if idx is not None:
            out["idx"] = idx.astype(np.int64)
        if prod:
            out["sign"] = sign.astype(bool)
            out["rnorm"] = rnorm
            out["z"] = z
        return out

    def score(self, q, codes, n_kv, g, seq, threads=1):
        q = np.ascontiguousarray(q, dtype=np.float64)
        idx = np.ascontiguousarray(codes["idx"], dtype=np.int32) if self.B > 0 else None
        sign = np.ascontiguousarray(codes["sign"], dtype=np.uint8) if self.mode == 0 else None
        rnorm = np.ascontiguousarray(codes["rnorm"], dtype=np.float32) if self.mode == 0 else None
        knorm = np.ascontiguousarray(codes["knorm"], dtype=np.float32)
        out = np.empty((n_kv * g, seq))
        lib().tqref_score(self.h, _ptr(q), n_kv, g, _ptr(idx), _ptr(sign), _ptr(knorm), _ptr(rnorm), seq,
                          _ptr(out), threads)
        return out

    def attend(self, vref, q, kcodes, vcodes, batch, n_kv, g, seq, scale=None, threads=1):
        """Attention of q [batch, n_kv g, d] over these K codes and the V codes
        of the mse-mode context ``vref``; scale None selects 1 / sqrt(d)."""
        q = np.ascontiguousarray(q, dtype=np.float64)
        kidx = np.ascontiguousarray(kcodes["idx"], dtype=np.int32) if self.B > 0 else None
        ksign = np.ascontiguousarray(kcodes["sign"], dtype=np.uint8) if self.mode == 0 else None
        krn = np.ascontiguousarray(kcodes["rnorm"], dtype=np.float32) if self.mode == 0 else None
        kn = np.ascontiguousarray(kcodes["knorm"], dtype=np.float32)
        vidx = np.ascontiguousarray(vcodes["idx"], dtype=np.int32)
        vn = np.ascontiguousarray(vcodes["knorm"], dtype=np.float32)
        out = np.empty((batch, n_kv * g, vref.d))
        lib().tqref_attend(self.h, vref.h, _ptr(q), batch, n_kv, g, seq, _ptr(kidx), _ptr(ksign), _ptr(kn),
                           _ptr(krn), _ptr(vidx), _ptr(vn), -1.0 if scale is None else float(scale), _ptr(out),
                           threads)
        return out

    def search(self, q, codes, n, k, threads=1):
        """Top-k (indices, logits) of each query over the n coded vectors."""
        q = np.ascontiguousarray(q, dtype=np.float64)
        nq = q.shape[0]
        idx = np.ascontiguousarray(codes["idx"], dtype=np.int32) if self.B > 0 else None
        sign = np.ascontiguousarray(codes["sign"], dtype=np.uint8) if self.mode == 0 else None
        rnorm = np.ascontiguousarray(codes["rnorm"], dtype=np.float32) if self.mode == 0 else None
        knorm = np.ascontiguousarray(codes["knorm"], dtype=np.float32)
        oi = np.empty((nq, k), dtype=np.int64)
        ov = np.empty((nq, k))
        lib().tqref_search(self.h, _ptr(q), nq, _ptr(idx), _ptr(sign), _ptr(knorm), _ptr(rnorm), n, k, _ptr(oi),
                           _ptr(ov), threads)
        return oi, ov
