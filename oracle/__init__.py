"""The oracle: a plain, slow, float64 CPU implementation of MLA attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and imports nothing from it.

The numerical functions live in ``mla_oracle.c`` (plain C loops in double,
OpenMP over the outer independent loop); this module compiles it with gcc and
calls it through ctypes.  The path threshold lives in ``threshold.py``, the
draft-cap cost model in ``draft_cap.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import threshold  # noqa: F401  (re-exported)
from . import draft_cap  # noqa: F401  (re-exported)
from . import fp8  # noqa: F401  (re-exported)
from . import sparse  # noqa: F401  (re-exported)
from . import indexer  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile mla_oracle.c into libmla_oracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _lib.oracle_max_threads.restype = ctypes.c_int
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _i(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _sel(sel):
    if sel is None:
        return None, 0, None
    s, p = _i(sel)
    return s, s.size, p


I64 = ctypes.c_int64
F64 = ctypes.c_double
VP = ctypes.c_void_p


def fold(q_nope, w_uk, nthreads: int = 0):
    """q_lat[..., h, :] = q_nope[..., h, :] @ W_UK[h]; q_nope [rows, H, n] -> [rows, H, r]."""
    lib = _load()
    q, qp = _d(q_nope)
    w, wp = _d(w_uk)
    H, n, r = w.shape
    rows = q.size // (H * n)
    out = np.empty((rows, H, r), dtype=np.float64)
    lib.oracle_fold(I64(rows), I64(H), I64(n), I64(r), qp, wp,
                    out.ctypes.data_as(VP), ctypes.c_int(nthreads))
    return out


def _offsets(offsets):
    o, op = _i(offsets)
    assert o.ndim == 1 and o.size >= 2
    return o, op, o.size - 1


def absorbed(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, offsets, L, scale, sel=None, nthreads: int = 0):
    """Whole absorbed path.  Returns [B*L*H, v] (or [len(sel), v])."""
    lib = _load()
    o, op, B = _offsets(offsets)
    w1, w1p = _d(w_uk)
    w2, w2p = _d(w_uv)
    H, n, r = w1.shape
    v = w2.shape[2]
    ckv, ckvp = _d(c_kv)
    kpe, kpep = _d(k_pe)
    rope = kpe.shape[1] if kpe.ndim == 2 else 0
    qn, qnp = _d(q_nope)
    qpe, qpep = _d(q_pe)
    s, ns, sp = _sel(sel)
    out = np.empty((ns if s is not None else B * L * H, v), dtype=np.float64)
    lib.oracle_absorbed(I64(r), I64(n), I64(v), I64(rope), I64(H), I64(B), I64(L), op,
                        qnp, qpep, ckvp, kpep, w1p, w2p, F64(scale), I64(ns), sp,
                        out.ctypes.data_as(VP), ctypes.c_int(nthreads))
    return out


def latent_attention(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale, sel=None, nthreads: int = 0):
    """Absorbed path after the fold, from a given q_lat [B, L, H, r]."""
    lib = _load()
    o, op, B = _offsets(offsets)
    w2, w2p = _d(w_uv)
    H, r, v = w2.shape
    ckv, ckvp = _d(c_kv)
    kpe, kpep = _d(k_pe)
    rope = kpe.shape[1] if kpe.ndim == 2 else 0
    ql, qlp = _d(q_lat)
    qpe, qpep = _d(q_pe)
    s, ns, sp = _sel(sel)
    out = np.empty((ns if s is not None else B * L * H, v), dtype=np.float64)
    lib.oracle_latent_attention(I64(r), I64(v), I64(rope), I64(H), I64(B), I64(L), op,
                                qlp, qpep, ckvp, kpep, w2p, F64(scale), I64(ns), sp,
                                out.ctypes.data_as(VP), ctypes.c_int(nthreads))
    return out


def expand(c_kv, k_pe, w_uk, w_uv, tsel=None, nthreads: int = 0):
    """Full per-head K [T', H, n+rope] and V [T', H, v] for all (or the listed) positions."""
    lib = _load()
    ckv, ckvp = _d(c_kv)
    kpe, kpep = _d(k_pe)
    w1, w1p = _d(w_uk)
    w2, w2p = _d(w_uv)
    H, n, r = w1.shape
    v = w2.shape[2]
    T = ckv.shape[0]
    rope = kpe.shape[1] if kpe.ndim == 2 else 0
    s, ns, sp = _sel(tsel)
    Tp = ns if s is not None else T
    K = np.empty((Tp, H, n + rope), dtype=np.float64)
    V = np.empty((Tp, H, v), dtype=np.float64)
    lib.oracle_expand(I64(T), I64(H), I64(r), I64(n), I64(v), I64(rope), ckvp, kpep, w1p, w2p,
                      I64(ns), sp, K.ctypes.data_as(VP), V.ctypes.data_as(VP), ctypes.c_int(nthreads))
    return K, V


def attention(q_nope, q_pe, K, V, offsets, L, scale, n, sel=None, nthreads: int = 0):
    """Ordinary causal attention over per-head K [T, H, n+rope], V [T, H, v]."""
    lib = _load()
    o, op, B = _offsets(offsets)
    Kd, Kp = _d(K)
    Vd, Vp = _d(V)
    T, H, dk = Kd.shape
    v = Vd.shape[2]
    rope = dk - n
    qn, qnp = _d(q_nope)
    qpe, qpep = _d(q_pe)
    s, ns, sp = _sel(sel)
    out = np.empty((ns if s is not None else B * L * H, v), dtype=np.float64)
    lib.oracle_attention(I64(n), I64(v), I64(rope), I64(H), I64(B), I64(L), op, qnp, qpep, Kp, Vp,
                         F64(scale), I64(ns), sp, out.ctypes.data_as(VP), ctypes.c_int(nthreads))
    return out


def materialized(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, offsets, L, scale, nthreads: int = 0):
    """Whole materialised path (expand per head, then attend).  Returns [B*L*H, v]."""
    lib = _load()
    o, op, B = _offsets(offsets)
    w1, w1p = _d(w_uk)
    w2, w2p = _d(w_uv)
    H, n, r = w1.shape
    v = w2.shape[2]
    ckv, ckvp = _d(c_kv)
    kpe, kpep = _d(k_pe)
    rope = kpe.shape[1] if kpe.ndim == 2 else 0
    qn, qnp = _d(q_nope)
    qpe, qpep = _d(q_pe)
    out = np.empty((B * L * H, v), dtype=np.float64)
    lib.oracle_materialized(I64(r), I64(n), I64(v), I64(rope), I64(H), I64(B), I64(L), op,
                            qnp, qpep, ckvp, kpep, w1p, w2p, F64(scale),
                            out.ctypes.data_as(VP), ctypes.c_int(nthreads))
    return out
