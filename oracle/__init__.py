"""fp64 CPU oracle for exact attention forward and decode.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

``attention_fwd`` and ``decode`` wrap ``oracle.c`` (threaded C, IEEE double);
``brute`` is an independent pure-Python brute force for tiny shapes.  Inputs
are raw f16/bf16 bit patterns (``uint16`` arrays) as produced by
``fa_inputs``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_DT = {"f16": 0, "bf16": 1}
_lib = None


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB names another build to load instead (the sanitizer build)
        path = os.environ.get("ORACLE_LIB") or _build.build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        D = ctypes.c_double
        lib.oracle_fwd.argtypes = [P, P, P, I, I, I, I, I, I, I, D, I, P, P, L, P, P, I]
        lib.oracle_fwd.restype = I
        lib.oracle_decode.argtypes = [P, P, P, P, I, I, I, I, I, D, P, P, I]
        lib.oracle_decode.restype = I
        lib.oracle_bwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, I, P, P, L, P, P, P, P, I]
        lib.oracle_bwd.restype = I
        lib.oracle_widen.argtypes = [P, I, L, P]
        lib.oracle_widen.restype = None
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """The oracle's own f16/bf16 -> float64 decoding of raw bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_widen(_ptr(bits), _DT[dtype], bits.size, _ptr(out))
    return out


def attention_fwd(q, k, v, dtype: str, scale: float, causal: bool,
                  kv_lens: Optional[np.ndarray] = None,
                  rows: Optional[np.ndarray] = None, nthreads: int = 0):
    """O (float64) and LSE (float64) of exact attention.

    q: [B,H,Nq,d], k/v: [B,Hkv,Nk,d] uint16 bits, H a multiple of Hkv; query
    head h reads K/V head h // (H // Hkv).  ``rows``: optional flat row
    ids (b*H+h)*Nq+i; then O is [len(rows), d] and LSE [len(rows)] in the
    given order, else O is [B,H,Nq,d] and LSE [B,H,Nq].
    """
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    assert Hkv >= 1 and H % Hkv == 0
    assert k.shape == (B, Hkv, Nk, d) and v.shape == k.shape
    kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, np.int32)
    if kl is not None:
        assert kl.shape == (B,)
    if rows is None:
        o = np.empty((B, H, Nq, d), np.float64)
        lse = np.empty((B, H, Nq), np.float64)
        rc = _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dtype], B, H, Hkv, Nq, Nk,
                                d, float(scale), int(bool(causal)), _ptr(kl), None, 0,
                                _ptr(o), _ptr(lse), nthreads)
    else:
        rows = np.asarray(rows, np.int64).reshape(-1)
        order = np.argsort(rows, kind="stable")
        srt = np.ascontiguousarray(rows[order])
        assert srt.size == 0 or (srt[0] >= 0 and srt[-1] < B * H * Nq)
        o_s = np.empty((srt.size, d), np.float64)
        lse_s = np.empty((srt.size,), np.float64)
        rc = _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dtype], B, H, Hkv, Nq, Nk,
                                d, float(scale), int(bool(causal)), _ptr(kl), _ptr(srt),
                                srt.size, _ptr(o_s), _ptr(lse_s), nthreads)
        o = np.empty_like(o_s)
        lse = np.empty_like(lse_s)
        o[order] = o_s
        lse[order] = lse_s
    if rc != 0:
        raise RuntimeError(f"oracle_fwd self-check failed ({rc})")
    return o, lse


def decode(q, k, v, seq_off, dtype: str, scale: float, nthreads: int = 0):
    """Decode attention over logical per-sequence caches.

    q: [S,H,d]; k/v: [T,Hkv,d] with sequence s owning rows seq_off[s]:seq_off[s+1],
    H a multiple of Hkv; query head h reads K/V head h // (H // Hkv).
    Returns O [S,H,d] and LSE [S,H] (float64).
    """
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    off = np.ascontiguousarray(seq_off, np.int64)
    S, H, d = q.shape
    Hkv = k.shape[1]
    assert Hkv >= 1 and H % Hkv == 0
    assert off.shape == (S + 1,) and k.shape == (int(off[-1]), Hkv, d) and v.shape == k.shape
    o = np.empty((S, H, d), np.float64)
    lse = np.empty((S, H), np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(off), _DT[dtype], S, H, Hkv,
                               d, float(scale), _ptr(o), _ptr(lse), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_decode self-check failed ({rc})")
    return o, lse


def attention_bwd(q, k, v, dout, dtype: str, scale: float, causal: bool,
                  kv_lens: Optional[np.ndarray] = None, groups=None, nthreads: int = 0):
    """Gradients (float64) of exact attention for the output gradient ``dout``.

    q, dout: [B,H,Nq,d]; k, v: [B,Hkv,Nk,d] uint16 bits.  Returns
    (dq [B,H,Nq,d], dk [B,Hkv,Nk,d], dv [B,Hkv,Nk,d], delta [B,H,Nq]) where
    delta is the row term D_i = dO_i . O_i.  ``groups``: optional flat ids
    b*Hkv + kvh; then only those K/V heads (and the query heads reading them)
    are computed and every other entry is NaN.
    """
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    g = np.ascontiguousarray(dout, np.uint16)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    assert Hkv >= 1 and H % Hkv == 0
    assert k.shape == (B, Hkv, Nk, d) and v.shape == k.shape and g.shape == q.shape
    kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, np.int32)
    fill = np.nan if groups is not None else 0.0
    dq = np.full((B, H, Nq, d), fill)
    dk = np.full((B, Hkv, Nk, d), fill)
    dv = np.full((B, Hkv, Nk, d), fill)
    delta = np.full((B, H, Nq), fill)
    gr = None if groups is None else np.ascontiguousarray(np.sort(np.asarray(groups, np.int64)))
    if gr is not None:
        assert gr.size == 0 or (gr[0] >= 0 and gr[-1] < B * Hkv)
    rc = _load().oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _DT[dtype], B, H, Hkv, Nq, Nk,
                            d, float(scale), int(bool(causal)), _ptr(kl), _ptr(gr),
                            0 if gr is None else gr.size, _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(delta), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed ({rc})")
    return dq, dk, dv, delta


def threads_used(nthreads: int = 0) -> int:
    return nthreads if nthreads > 0 else (os.cpu_count() or 1)
