"""MI355X-native Multi-head Latent Attention for speculative-decoding verify.

A thin Python binding over libmla.so (include/mla.h).  Every function here
only marshals arguments -- tensor pointers, sizes and the current HIP stream
-- and calls the C ABI; all computation runs in the library's HIP kernels.
PyTorch supplies device memory and streams.

Entry points (same names as the C ABI, without the ``mla_`` prefix):
    select_path, fold_query, absorbed_workspace_size, absorbed_attention,
    materialize_kv, materialized_workspace_size, materialized_attention
and two conveniences that chain them: ``absorbed`` (fold + attention) and
``materialized`` (expand + attention).
"""

from __future__ import annotations

import ctypes
import math
from typing import Sequence

from . import _lib
from ._lib import Geom, MlaError, MLA_ABSORBED, MLA_MATERIALIZED, MLA_BF16, MLA_F32  # noqa: F401

__all__ = ["Geom", "MlaError", "MLA_ABSORBED", "MLA_MATERIALIZED", "Offsets", "select_path",
           "fold_query", "absorbed_workspace_size", "absorbed_attention", "absorbed_attention_noalloc",
           "absorbed_splits",
           "absorbed_merge", "materialize_kv",
           "materialized_workspace_size", "materialized_attention", "absorbed", "materialized",
           "library_path", "IndexerPool", "selection_offsets", "indexer_select", "update_list"]


def library_path() -> str:
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.MLA_BF16
    if t.dtype == torch.float32:
        return _lib.MLA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Offsets:
    """Per-sequence cache offsets [B+1] (int32), held on the host and on the device."""

    def __init__(self, offsets, device=None):
        torch = _torch()
        host = torch.as_tensor(offsets, dtype=torch.int32).contiguous().cpu()
        if host.dim() != 1 or host.numel() < 2:
            raise ValueError("offsets must be a 1-D sequence of B+1 integers")
        self.host = host
        self.dev = host.to(device if device is not None else "cuda")
        self.B = host.numel() - 1

    @classmethod
    def dense(cls, B: int, kv: int, device=None) -> "Offsets":
        return cls([b * kv for b in range(B + 1)], device)

    def host_ptr(self):
        return ctypes.c_void_p(self.host.data_ptr())

    def dev_ptr(self):
        return ctypes.c_void_p(self.dev.data_ptr())


def _as_offsets(kv_offsets, device) -> Offsets:
    return kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, device)


def select_path(geom: Geom, L: int, T: int = 0) -> tuple[int, int]:
    """(path, max_absorbed) for L query rows over T cached positions (T = 0: limit form)."""
    lib = _lib.load()
    path = ctypes.c_int32()
    m = ctypes.c_int64()
    _lib.check("mla_select_path", lib.mla_select_path(ctypes.byref(geom), int(L), int(T),
                                                      ctypes.byref(path), ctypes.byref(m)))
    return int(path.value), int(m.value)


def draft_cap(verify_cost, p: float, drafter: float) -> tuple[int, float, list[float]]:
    """Derived draft cap from a verify-cost curve (verify_cost[w - 1] = cost of a
    w-row pass, any unit): (cap, its speedup, speedup for caps 0..len - 1)."""
    lib = _lib.load()
    n = len(verify_cost)
    vc = (ctypes.c_double * max(n, 1))(*[float(x) for x in verify_cost])
    by_cap = (ctypes.c_double * max(n, 1))()
    cap = ctypes.c_int32()
    sp = ctypes.c_double()
    _lib.check("mla_draft_cap", lib.mla_draft_cap(vc, n, float(p), float(drafter), ctypes.byref(cap),
                                                  ctypes.byref(sp), by_cap))
    return int(cap.value), float(sp.value), [float(by_cap[i]) for i in range(n)]


def fold_query(q_nope, w_uk, out=None, stream=None):
    """q_lat[m, h, :] = q_nope[m, h, :] @ w_uk[h].  q_nope [..., H, n] -> [..., H, r]."""
    torch = _torch()
    lib = _lib.load()
    H, n, r = w_uk.shape
    rows = q_nope.numel() // (H * n)
    g = Geom(r, n, 1, 0, H)
    if out is None:
        out = torch.empty(q_nope.shape[:-1] + (r,), dtype=q_nope.dtype, device=q_nope.device)
    dt = _dtype_code(q_nope)
    if _dtype_code(w_uk) != dt or _dtype_code(out) != dt:
        raise TypeError("q_nope, w_uk and q_lat must share one dtype")
    _lib.check("mla_fold_query", lib.mla_fold_query(ctypes.byref(g), dt, rows, _ptr(_dev(q_nope, "q_nope")),
                                                    _ptr(_dev(w_uk, "w_uk")), _ptr(out), _stream(stream)))
    return out


def absorbed_workspace_size(geom: Geom, dtype_code: int, L: int, kv_offsets: Offsets) -> int:
    lib = _lib.load()
    sz = ctypes.c_size_t()
    _lib.check("mla_absorbed_workspace_size",
               lib.mla_absorbed_workspace_size(ctypes.byref(geom), dtype_code, kv_offsets.B, int(L),
                                               kv_offsets.host_ptr(), ctypes.byref(sz)))
    return int(sz.value)


def absorbed_attention(q_lat, q_pe, c_kv, k_pe, w_uv, kv_offsets, scale=None, out=None, workspace=None,
                       stream=None, n=None):
    """Absorbed attention after the fold.  q_lat [B, L, H, r], q_pe [B, L, H, rope],
    c_kv [sumKv, r], k_pe [sumKv, rope], w_uv [H, r, v] -> out [B, L, H, v] float32.
    ``scale`` defaults to 1/sqrt(n + rope) (n must then be given)."""
    torch = _torch()
    lib = _lib.load()
    B, L, H, r = q_lat.shape
    rope = q_pe.shape[-1] if q_pe is not None else 0
    v = w_uv.shape[-1]
    offs = _as_offsets(kv_offsets, q_lat.device)
    if offs.B != B:
        raise ValueError("offsets do not match the batch")
    if scale is None:
        if n is None:
            raise ValueError("give scale, or n to default it to 1/sqrt(n + rope)")
        scale = 1.0 / math.sqrt(n + rope)
    g = Geom(r, int(n) if n is not None else 0, v, rope, H)
    dt = _dtype_code(q_lat)
    need = absorbed_workspace_size(g, dt, L, offs)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q_lat.device)
    if out is None:
        out = torch.empty((B, L, H, v), dtype=torch.float32, device=q_lat.device)
    _lib.check("mla_absorbed_attention", lib.mla_absorbed_attention(
        ctypes.byref(g), dt, B, L, _ptr(_dev(q_lat, "q_lat")), _ptr(q_pe) if rope else None,
        _ptr(_dev(c_kv, "c_kv")), _ptr(k_pe) if rope else None, offs.host_ptr(), offs.dev_ptr(),
        _ptr(_dev(w_uv, "w_uv")), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def absorbed_attention_noalloc(q_lat, q_pe, c_kv, k_pe, w_uv, kv_offsets: Offsets, out, scale: float, n: int = 0,
                               stream=None):
    """absorbed_attention without a workspace (mla_absorbed_attention_noalloc): the
    split partials go to the library's static device array.  Every tensor,
    ``out`` and the offsets included, is the caller's; nothing is allocated here."""
    lib = _lib.load()
    B, L, H, r = q_lat.shape
    rope = q_pe.shape[-1] if q_pe is not None else 0
    v = w_uv.shape[-1]
    if not isinstance(kv_offsets, Offsets) or kv_offsets.B != B:
        raise ValueError("kv_offsets must be an Offsets of the batch")
    g = Geom(r, int(n), v, rope, H)
    _lib.check("mla_absorbed_attention_noalloc", lib.mla_absorbed_attention_noalloc(
        ctypes.byref(g), _dtype_code(q_lat), B, L, _ptr(_dev(q_lat, "q_lat")), _ptr(q_pe) if rope else None,
        _ptr(_dev(c_kv, "c_kv")), _ptr(k_pe) if rope else None, kv_offsets.host_ptr(), kv_offsets.dev_ptr(),
        _ptr(_dev(w_uv, "w_uv")), ctypes.c_float(scale), _ptr(_dev(out, "out")), _stream(stream)))
    return out


def absorbed_splits(q_lat, q_pe, c_kv, k_pe, kv_offsets: Offsets, geom: Geom, scale: float, workspace,
                    stream=None):
    """Split-KV pass of the absorbed attention (one kernel); partials go to ``workspace``."""
    lib = _lib.load()
    B, L = q_lat.shape[0], q_lat.shape[1]
    rope = geom.rope
    _lib.check("mla_absorbed_splits", lib.mla_absorbed_splits(
        ctypes.byref(geom), _dtype_code(q_lat), B, L, _ptr(_dev(q_lat, "q_lat")), _ptr(q_pe) if rope else None,
        _ptr(_dev(c_kv, "c_kv")), _ptr(k_pe) if rope else None, kv_offsets.host_ptr(), kv_offsets.dev_ptr(),
        ctypes.c_float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def absorbed_merge(w_uv, out, kv_offsets: Offsets, geom: Geom, L: int, workspace, stream=None):
    """Merge pass of the absorbed attention (one kernel): log-sum-exp combine and W_UV."""
    lib = _lib.load()
    _lib.check("mla_absorbed_merge", lib.mla_absorbed_merge(
        ctypes.byref(geom), _dtype_code(w_uv), kv_offsets.B, int(L), kv_offsets.host_ptr(), kv_offsets.dev_ptr(),
        _ptr(_dev(w_uv, "w_uv")), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def materialize_kv(c_kv, k_pe, w_uk, w_uv, k=None, v=None, stream=None):
    """K [T, H, n+rope], V [T, H, v] from the latent cache."""
    torch = _torch()
    lib = _lib.load()
    T, r = c_kv.shape
    rope = k_pe.shape[-1] if k_pe is not None else 0
    H, n, _ = w_uk.shape
    vd = w_uv.shape[-1]
    g = Geom(r, n, vd, rope, H)
    if k is None:
        k = torch.empty((T, H, n + rope), dtype=c_kv.dtype, device=c_kv.device)
    if v is None:
        v = torch.empty((T, H, vd), dtype=c_kv.dtype, device=c_kv.device)
    _lib.check("mla_materialize_kv", lib.mla_materialize_kv(
        ctypes.byref(g), _dtype_code(c_kv), T, _ptr(_dev(c_kv, "c_kv")), _ptr(k_pe) if rope else None,
        _ptr(w_uk), _ptr(w_uv), _ptr(k), _ptr(v), _stream(stream)))
    return k, v


def materialized_workspace_size(geom: Geom, dtype_code: int, L: int, kv_offsets: Offsets) -> int:
    lib = _lib.load()
    sz = ctypes.c_size_t()
    _lib.check("mla_materialized_workspace_size",
               lib.mla_materialized_workspace_size(ctypes.byref(geom), dtype_code, kv_offsets.B, int(L),
                                                   kv_offsets.host_ptr(), ctypes.byref(sz)))
    return int(sz.value)


def materialized_attention(q_nope, q_pe, k, v, kv_offsets, scale=None, out=None, workspace=None, stream=None):
    """Ordinary causal attention over expanded K [sumKv, H, n+rope] and V [sumKv, H, v]."""
    torch = _torch()
    lib = _lib.load()
    B, L, H, n = q_nope.shape
    rope = q_pe.shape[-1] if q_pe is not None else 0
    vd = v.shape[-1]
    offs = _as_offsets(kv_offsets, q_nope.device)
    if offs.B != B:
        raise ValueError("offsets do not match the batch")
    if scale is None:
        scale = 1.0 / math.sqrt(n + rope)
    g = Geom(1, n, vd, rope, H)
    dt = _dtype_code(q_nope)
    need = materialized_workspace_size(g, dt, L, offs)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q_nope.device)
    if out is None:
        out = torch.empty((B, L, H, vd), dtype=torch.float32, device=q_nope.device)
    _lib.check("mla_materialized_attention", lib.mla_materialized_attention(
        ctypes.byref(g), dt, B, L, _ptr(_dev(q_nope, "q_nope")), _ptr(q_pe) if rope else None,
        _ptr(_dev(k, "k")), _ptr(_dev(v, "v")), offs.host_ptr(), offs.dev_ptr(), ctypes.c_float(scale),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def quantize_latent_fp8(c_kv, k_pe, codes=None, scales=None, stream=None):
    """bf16 latent cache -> (codes uint8 [T, r + rope], scales float32 [T], powers of two)."""
    torch = _torch()
    lib = _lib.load()
    T, r = c_kv.shape
    rope = k_pe.shape[-1] if k_pe is not None else 0
    if codes is None:
        codes = torch.empty((T, r + rope), dtype=torch.uint8, device=c_kv.device)
    if scales is None:
        scales = torch.empty((T,), dtype=torch.float32, device=c_kv.device)
    if _dtype_code(c_kv) != MLA_BF16 or (rope and _dtype_code(k_pe) != MLA_BF16):
        raise TypeError("the fp8 cache is quantised from a bf16 cache")
    g = Geom(r, 0, 1, rope, 1)
    _lib.check("mla_quantize_latent_fp8", lib.mla_quantize_latent_fp8(
        ctypes.byref(g), T, _ptr(_dev(c_kv, "c_kv")), _ptr(k_pe) if rope else None, _ptr(_dev(codes, "codes")),
        _ptr(_dev(scales, "scales")), _stream(stream)))
    return codes, scales


def absorbed_attention_fp8(q_lat, q_pe, codes, scales, w_uv, kv_offsets, scale=None, out=None, workspace=None,
                           stream=None, n=None):
    """absorbed_attention over the fp8 cache (codes, scales) from quantize_latent_fp8."""
    torch = _torch()
    lib = _lib.load()
    B, L, H, r = q_lat.shape
    rope = q_pe.shape[-1] if q_pe is not None else 0
    v = w_uv.shape[-1]
    if codes.shape[-1] != r + rope:
        raise ValueError("codes rows must hold r + rope values")
    offs = _as_offsets(kv_offsets, q_lat.device)
    if offs.B != B:
        raise ValueError("offsets do not match the batch")
    if scale is None:
        if n is None:
            raise ValueError("give scale, or n to default it to 1/sqrt(n + rope)")
        scale = 1.0 / math.sqrt(n + rope)
    g = Geom(r, int(n) if n is not None else 0, v, rope, H)
    need = absorbed_workspace_size(g, MLA_BF16, L, offs)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q_lat.device)
    if out is None:
        out = torch.empty((B, L, H, v), dtype=torch.float32, device=q_lat.device)
    _lib.check("mla_absorbed_attention_fp8", lib.mla_absorbed_attention_fp8(
        ctypes.byref(g), B, L, _ptr(_dev(q_lat, "q_lat")), _ptr(q_pe) if rope else None,
        _ptr(_dev(codes, "codes")), _ptr(_dev(scales, "scales")), offs.host_ptr(), offs.dev_ptr(),
        _ptr(_dev(w_uv, "w_uv")), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def query_fp8_bytes(geom: Geom, B: int, L: int) -> int:
    """Bytes of the E4M3 query block of B sequences of L rows (fold_query_fp8)."""
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    _lib.check("mla_query_fp8_bytes", lib.mla_query_fp8_bytes(ctypes.byref(geom), B, L, ctypes.byref(n)))
    return n.value


def fold_query_fp8(q_nope, w_uk, q_pe, q_lat=False, q8=None, stream=None):
    """The fold for the fp8 route: q_nope [B, L, H, n], w_uk [H, n, r], q_pe
    [B, L, H, rope] (bf16) -> (q_lat [B, L, H, r] or None, q8 uint8: the block
    quantisation that absorbed_attention_fp8 applies to q_lat and q_pe, in the
    attention kernel's layout).  q_lat=True allocates q_lat, a tensor receives it."""
    torch = _torch()
    lib = _lib.load()
    B, L, H, n = q_nope.shape
    r = w_uk.shape[-1]
    rope = q_pe.shape[-1] if q_pe is not None else 0
    g = Geom(r, n, 1, rope, H)
    if q8 is None:
        q8 = torch.empty(query_fp8_bytes(g, B, L), dtype=torch.uint8, device=q_nope.device)
    if q_lat is True:
        q_lat = torch.empty((B, L, H, r), dtype=torch.bfloat16, device=q_nope.device)
    elif q_lat is False:
        q_lat = None
    _lib.check("mla_fold_query_fp8", lib.mla_fold_query_fp8(
        ctypes.byref(g), B, L, _ptr(_dev(q_nope, "q_nope")), _ptr(_dev(w_uk, "w_uk")), _ptr(q_pe) if rope else None,
        _ptr(q_lat) if q_lat is not None else None, _ptr(_dev(q8, "q8")), _stream(stream)))
    return q_lat, q8


def absorbed_attention_fp8q(q8, B, L, codes, scales, w_uv, kv_offsets, scale, rope=64, out=None, workspace=None,
                            stream=None):
    """absorbed_attention_fp8 with the queries given as fold_query_fp8's block q8."""
    torch = _torch()
    lib = _lib.load()
    H, r, v = w_uv.shape
    if codes.shape[-1] != r + rope:
        raise ValueError("codes rows must hold r + rope values")
    offs = _as_offsets(kv_offsets, q8.device)
    if offs.B != B:
        raise ValueError("offsets do not match the batch")
    g = Geom(r, 0, v, rope, H)
    need = absorbed_workspace_size(g, MLA_BF16, L, offs)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q8.device)
    if out is None:
        out = torch.empty((B, L, H, v), dtype=torch.float32, device=q8.device)
    _lib.check("mla_absorbed_attention_fp8q", lib.mla_absorbed_attention_fp8q(
        ctypes.byref(g), B, L, _ptr(_dev(q8, "q8")), _ptr(_dev(codes, "codes")), _ptr(_dev(scales, "scales")),
        offs.host_ptr(), offs.dev_ptr(), _ptr(_dev(w_uv, "w_uv")), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def absorbed_attention_sparse(q_lat, q_pe, c_kv, k_pe, w_uv, kv_offsets, sel, sel_offsets, scale=None, out=None,
                              workspace=None, stream=None, n=None):
    """Absorbed attention over selected positions: sequence b attends to
    sel[sel_offsets[b]:sel_offsets[b+1]] (positions from its start, increasing),
    row i to those below Kv_b - L + i + 1.  sel: int32 device tensor."""
    torch = _torch()
    lib = _lib.load()
    B, L, H, r = q_lat.shape
    rope = q_pe.shape[-1] if q_pe is not None else 0
    v = w_uv.shape[-1]
    offs = _as_offsets(kv_offsets, q_lat.device)
    soffs = _as_offsets(sel_offsets, q_lat.device)
    if offs.B != B or soffs.B != B:
        raise ValueError("offsets do not match the batch")
    if sel.dtype != torch.int32:
        raise TypeError("sel must be int32")
    if scale is None:
        if n is None:
            raise ValueError("give scale, or n to default it to 1/sqrt(n + rope)")
        scale = 1.0 / math.sqrt(n + rope)
    g = Geom(r, int(n) if n is not None else 0, v, rope, H)
    sz = ctypes.c_size_t()
    _lib.check("mla_absorbed_sparse_workspace_size", lib.mla_absorbed_sparse_workspace_size(
        ctypes.byref(g), B, L, offs.host_ptr(), soffs.host_ptr(), ctypes.byref(sz)))
    if workspace is None:
        workspace = torch.empty(max(int(sz.value), 256), dtype=torch.uint8, device=q_lat.device)
    if out is None:
        out = torch.empty((B, L, H, v), dtype=torch.float32, device=q_lat.device)
    _lib.check("mla_absorbed_attention_sparse", lib.mla_absorbed_attention_sparse(
        ctypes.byref(g), B, L, _ptr(_dev(q_lat, "q_lat")), _ptr(q_pe) if rope else None, _ptr(_dev(c_kv, "c_kv")),
        _ptr(k_pe) if rope else None, offs.host_ptr(), offs.dev_ptr(), _ptr(_dev(sel, "sel")), soffs.host_ptr(),
        soffs.dev_ptr(), _ptr(_dev(w_uv, "w_uv")), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


class IndexerPool:
    """Pooled keys of the top-k indexer (windows of four positions) for up to
    batch_max sequences of up to 4 * capacity cached positions, key width d.
    step() after every step that appended S positions per sequence: the tail
    only when the four guards hold, every window otherwise."""

    def __init__(self, capacity: int, batch_max: int, d: int, device=None):
        torch = _torch()
        self.pooled = torch.empty((batch_max, capacity, d), dtype=torch.float32,
                                  device=device if device is not None else "cuda")
        self.lengths = torch.zeros(batch_max, dtype=torch.int32)
        self.d = d
        self.state = _lib.Pool()
        _lib.check("mla_indexer_pool_init", _lib.load().mla_indexer_pool_init(
            ctypes.byref(self.state), ctypes.c_void_p(self.pooled.data_ptr()), capacity, batch_max,
            ctypes.c_void_p(self.lengths.data_ptr())))

    @property
    def capacity(self) -> int:
        return int(self.state.capacity)

    @property
    def valid(self) -> bool:
        return bool(self.state.valid)

    def plan(self, kv_offsets, S: int, padded: bool = False) -> bool:
        """Would a step of S new positions recompute only the tail?"""
        offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, self.pooled.device)
        inc = ctypes.c_int32()
        _lib.check("mla_indexer_pool_plan", _lib.load().mla_indexer_pool_plan(
            ctypes.byref(self.state), offs.B, self.d, offs.host_ptr(), S, int(padded), ctypes.byref(inc)))
        return bool(inc.value)

    def step(self, keys, kv_offsets, S: int, padded: bool = False, stream=None) -> bool:
        """Pool after a step; keys: bf16 device tensor whose rows are the cached
        positions (row stride keys.stride(0), first d columns).  Returns True if
        only the tail was recomputed."""
        torch = _torch()
        if keys.dtype != torch.bfloat16 or keys.dim() != 2 or keys.stride(1) != 1 or keys.shape[1] < self.d:
            raise ValueError("keys must be a bf16 [T, >= d] device tensor with unit column stride")
        offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, keys.device)
        inc = ctypes.c_int32()
        _lib.check("mla_indexer_pool_step", _lib.load().mla_indexer_pool_step(
            ctypes.byref(self.state), offs.B, self.d, ctypes.c_void_p(_dev(keys, "keys").data_ptr()),
            keys.stride(0), offs.host_ptr(), offs.dev_ptr(), S, int(padded), ctypes.byref(inc), _stream(stream)))
        return bool(inc.value)

    def step_fixed(self, keys, kv_offsets, S: int, target: int = 8, padded: bool = False, stream=None):
        """step() with a fixed-capacity update list (mla_indexer_pool_step_fixed):
        returns (incremental, capacity), capacity = target when the fixed launch
        shape ran and 0 when the ordinary step did."""
        torch = _torch()
        if keys.dtype != torch.bfloat16 or keys.dim() != 2 or keys.stride(1) != 1 or keys.shape[1] < self.d:
            raise ValueError("keys must be a bf16 [T, >= d] device tensor with unit column stride")
        offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, keys.device)
        inc, cap = ctypes.c_int32(), ctypes.c_int32()
        _lib.check("mla_indexer_pool_step_fixed", _lib.load().mla_indexer_pool_step_fixed(
            ctypes.byref(self.state), offs.B, self.d, ctypes.c_void_p(_dev(keys, "keys").data_ptr()),
            keys.stride(0), offs.host_ptr(), offs.dev_ptr(), S, int(padded), int(target), ctypes.byref(inc),
            ctypes.byref(cap), _stream(stream)))
        return bool(inc.value), int(cap.value)

    def step_scores(self, keys, kv_offsets, S: int, q, out=None, padded: bool = False, stream=None):
        """step() then scores() in one call (tail pooling fused into the scoring
        launch when the guards hold); returns (scores, incremental)."""
        torch = _torch()
        if keys.dtype != torch.bfloat16 or keys.dim() != 2 or keys.stride(1) != 1 or keys.shape[1] < self.d:
            raise ValueError("keys must be a bf16 [T, >= d] device tensor with unit column stride")
        offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, keys.device)
        if q.dtype != torch.float32 or tuple(q.shape) != (offs.B, self.d):
            raise ValueError("q must be float32 [B, d]")
        if out is None:
            out = torch.zeros((offs.B, self.capacity), dtype=torch.float32, device=q.device)
        inc = ctypes.c_int32()
        _lib.check("mla_indexer_pool_step_scores", _lib.load().mla_indexer_pool_step_scores(
            ctypes.byref(self.state), offs.B, self.d, ctypes.c_void_p(_dev(keys, "keys").data_ptr()),
            keys.stride(0), offs.host_ptr(), offs.dev_ptr(), S, int(padded), _ptr(_dev(q, "q")), _ptr(out),
            ctypes.byref(inc), _stream(stream)))
        return out, bool(inc.value)

    def trim(self, new_lengths) -> None:
        torch = _torch()
        nl = torch.as_tensor(new_lengths, dtype=torch.int32).contiguous()
        _lib.check("mla_indexer_pool_trim", _lib.load().mla_indexer_pool_trim(
            ctypes.byref(self.state), nl.numel(), ctypes.c_void_p(nl.data_ptr())))

    def scores(self, q, kv_offsets, out=None, stream=None):
        """Window scores [B, capacity] (float32; windows past a sequence's last untouched)."""
        torch = _torch()
        offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, q.device)
        if q.dtype != torch.float32 or tuple(q.shape) != (offs.B, self.d):
            raise ValueError("q must be float32 [B, d]")
        if out is None:
            out = torch.zeros((offs.B, self.capacity), dtype=torch.float32, device=q.device)
        _lib.check("mla_indexer_scores", _lib.load().mla_indexer_scores(
            ctypes.byref(self.state), offs.B, _ptr(_dev(q, "q")), offs.host_ptr(), offs.dev_ptr(), _ptr(out),
            _stream(stream)))
        return out


def update_list(first: int, windows: int, complete: int, S: int, target: int = 8) -> list[int]:
    """The fixed-capacity update list of one sequence (mla_indexer_update_list)."""
    lib = _lib.load()
    buf = (ctypes.c_int32 * max(1, windows - first, target))()
    cap = ctypes.c_int32()
    _lib.check("mla_indexer_update_list", lib.mla_indexer_update_list(int(first), int(windows), int(complete), int(S),
                                                                      int(target), buf, ctypes.byref(cap)))
    return [int(buf[i]) for i in range(cap.value)]


def selection_offsets(kv_offsets, budget: int, device=None) -> Offsets:
    """Offsets of the packed selection: sequence b gets min(budget, Kv_b) positions."""
    torch = _torch()
    offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, device)
    so = torch.empty(offs.B + 1, dtype=torch.int32)
    _lib.check("mla_indexer_selection_offsets", _lib.load().mla_indexer_selection_offsets(
        offs.B, offs.host_ptr(), budget, ctypes.c_void_p(so.data_ptr())))
    return Offsets(so, offs.dev.device if device is None else device)


def indexer_select(scores, kv_offsets, budget: int, sel_offsets: Offsets | None = None, out=None, stream=None):
    """Top-budget positions per sequence from window scores [B, capacity]:
    returns (sel int32 device tensor, sel_offsets)."""
    torch = _torch()
    offs = kv_offsets if isinstance(kv_offsets, Offsets) else Offsets(kv_offsets, scores.device)
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[0] != offs.B:
        raise ValueError("scores must be float32 [B, capacity]")
    if sel_offsets is None:
        sel_offsets = selection_offsets(offs, budget)
    if out is None:
        out = torch.empty(max(int(sel_offsets.host[-1]), 1), dtype=torch.int32, device=scores.device)
    _lib.check("mla_indexer_select", _lib.load().mla_indexer_select(
        offs.B, _ptr(_dev(scores, "scores")), scores.shape[1], offs.host_ptr(), offs.dev_ptr(), budget,
        sel_offsets.dev_ptr(), _ptr(out), _stream(stream)))
    return out, sel_offsets


def absorbed_attention_sparse_fp8(q_lat, q_pe, codes, scales, w_uv, kv_offsets, sel, sel_offsets, scale=None,
                                  out=None, workspace=None, stream=None, n=None):
    """absorbed_attention_sparse over the fp8 cache (codes, scales from quantize_latent_fp8)."""
    torch = _torch()
    lib = _lib.load()
    B, L, H, r = q_lat.shape
    rope = q_pe.shape[-1] if q_pe is not None else 0
    v = w_uv.shape[-1]
    offs = _as_offsets(kv_offsets, q_lat.device)
    soffs = _as_offsets(sel_offsets, q_lat.device)
    if offs.B != B or soffs.B != B:
        raise ValueError("offsets do not match the batch")
    if sel.dtype != torch.int32 or codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise TypeError("sel must be int32, codes uint8, scales float32")
    if scale is None:
        if n is None:
            raise ValueError("give scale, or n to default it to 1/sqrt(n + rope)")
        scale = 1.0 / math.sqrt(n + rope)
    g = Geom(r, int(n) if n is not None else 0, v, rope, H)
    sz = ctypes.c_size_t()
    _lib.check("mla_absorbed_sparse_workspace_size", lib.mla_absorbed_sparse_workspace_size(
        ctypes.byref(g), B, L, offs.host_ptr(), soffs.host_ptr(), ctypes.byref(sz)))
    if workspace is None:
        workspace = torch.empty(max(int(sz.value), 256), dtype=torch.uint8, device=q_lat.device)
    if out is None:
        out = torch.empty((B, L, H, v), dtype=torch.float32, device=q_lat.device)
    _lib.check("mla_absorbed_attention_sparse_fp8", lib.mla_absorbed_attention_sparse_fp8(
        ctypes.byref(g), B, L, _ptr(_dev(q_lat, "q_lat")), _ptr(q_pe) if rope else None, _ptr(_dev(codes, "codes")),
        _ptr(_dev(scales, "scales")), offs.host_ptr(), offs.dev_ptr(), _ptr(_dev(sel, "sel")), soffs.host_ptr(),
        soffs.dev_ptr(), _ptr(_dev(w_uv, "w_uv")), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def absorbed(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, kv_offsets, scale=None, stream=None, q_lat=None,
             out=None, workspace=None):
    """Whole absorbed path: fold_query then absorbed_attention."""
    q_lat = fold_query(q_nope, w_uk, out=q_lat, stream=stream)
    return absorbed_attention(q_lat, q_pe, c_kv, k_pe, w_uv, kv_offsets, scale=scale, out=out,
                              workspace=workspace, stream=stream, n=q_nope.shape[-1])


def materialized(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, kv_offsets, scale=None, stream=None, k=None, v=None,
                 out=None, workspace=None):
    """Whole materialised path: materialize_kv then materialized_attention."""
    k, v = materialize_kv(c_kv, k_pe, w_uk, w_uv, k=k, v=v, stream=stream)
    return materialized_attention(q_nope, q_pe, k, v, kv_offsets, scale=scale, out=out, workspace=workspace,
                                  stream=stream)


def chosen_path(geom: Geom, L: int, T: int) -> int:
    return select_path(geom, L, T)[0]


def forward(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, kv_offsets: Sequence[int] | Offsets, scale=None, stream=None):
    """Verify-step attention with the path picked by select_path (T = longest cache)."""
    offs = _as_offsets(kv_offsets, q_nope.device)
    H, n, r = w_uk.shape
    L = q_nope.shape[1]
    rope = q_pe.shape[-1] if q_pe is not None else 0
    T = int((offs.host[1:] - offs.host[:-1]).max())
    g = Geom(r, n, w_uv.shape[-1], rope, H)
    if select_path(g, L, T)[0] == MLA_ABSORBED:
        return absorbed(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, offs, scale=scale, stream=stream)
    return materialized(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, offs, scale=scale, stream=stream)
