"""HGA CPU oracle (test infrastructure only).

A ctypes wrapper around ``liboracle_hga.so``, the plain fp64 C++ implementation
of Hierarchical Global Attention in ``hga_oracle.cpp``.  Only the tests, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP library.

All arrays are numpy float64 (int32 for routing indices), C-contiguous, in the
layouts documented at the top of ``hga_oracle.cpp``.  Chunk size ``C`` and group
size ``G`` default to the page's 64 and 8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hga_oracle.cpp")
# HGA_ORACLE_LIB selects another build of the same source (the tests' sanitizer
# build); it is used as it is, never rebuilt here
_LIB_ENV = os.environ.get("HGA_ORACLE_LIB")
_LIB = _LIB_ENV or os.path.join(_HERE, "liboracle_hga.so")
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lib = None


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compiles the oracle with g++ (no fast-math, no FP contraction); with
    `sanitize`, an address- and undefined-behaviour-sanitized build (to be
    loaded with those runtimes preloaded) into `out`."""
    lib = out or _LIB
    if _LIB_ENV and out is None:
        return lib
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp"
        opt = SANITIZE_FLAGS if sanitize else ["-O2"]
        cmd = ["g++", *opt, "-std=c++17", "-shared", "-fPIC", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB_ENV and (not os.path.exists(_LIB) or
                             os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i = ctypes.c_int
        lib.hgao_summaries.argtypes = [i, i, i, i, i, i, _dp, _dp, _dp]
        lib.hgao_route.argtypes = [i] * 10 + [_dp, _dp, _dp, _ip, _ip, _ip, _dp, _dp]
        lib.hgao_route_causal.argtypes = [i] * 10 + [_dp, _dp, _dp, _dp, _ip, _ip, _ip, _dp, _dp]
        lib.hgao_attend_fwd.argtypes = [i] * 9 + [ctypes.c_double, _dp, _dp, _dp, _ip, _dp, _dp]
        lib.hgao_attend_bwd.argtypes = ([i] * 9 + [ctypes.c_double, _dp, _dp, _dp, _ip, _dp,
                                                   _dp, _dp, _dp])
        lib.hgao_attended_pairs.argtypes = [i, i, i, i, i, i, _ip]
        lib.hgao_decode.argtypes = ([i] * 9 + [ctypes.c_double, _dp, _dp, _dp, _dp, _dp, _ip, _ip,
                                              _ip, _dp, _dp, _dp, _dp])
        lib.hgao_attended_pairs.restype = ctypes.c_longlong
        _lib = lib
    return _lib


def _d(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _i(a):
    return None if a is None else a.ctypes.data_as(_ip)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def summaries(K, C: int = 64, G: int = 8):
    """Chunk means [B,H,S/C,D] and group means [B,H,S/G,D] of K [B,H,S,D]."""
    K = _f64(K)
    B, H, S, D = K.shape
    cm = np.empty((B, H, S // C, D))
    gm = np.empty((B, H, S // G, D))
    _check(_load().hgao_summaries(B, H, S, D, C, G, _d(K), _d(cm), _d(gm)), "summaries")
    return cm, gm


def route(Q, chunk_mean, group_mean, Skv: int, top_k: int, top_g: int, C: int = 64,
          G: int = 8, forced_chunk_idx=None, want_scores: bool = False, causal: bool = False,
          Qprev=None):
    """Routing indices for every (b, hq, block).

    Returns ``(chunk_idx, group_idx)`` or, with ``want_scores``,
    ``(chunk_idx, group_idx, chunk_score, group_score)`` where the scores are
    fp64 with NaN at non-candidates.  With ``causal`` a block is routed with
    the mean of the C queries before it; ``Qprev`` [B,Hq,C,D] holds the C
    queries before the segment (needed when Skv > Sq).
    """
    Q = _f64(Q)
    chunk_mean = _f64(chunk_mean)
    group_mean = _f64(group_mean)
    B, Hq, Sq, D = Q.shape
    Hkv = chunk_mean.shape[1]
    nblk = Sq // C
    ci = np.empty((B, Hq, nblk, top_k), dtype=np.int32)
    gi = np.empty((B, Hq, nblk, top_g), dtype=np.int32)
    cs = np.empty((B, Hq, nblk, Skv // C)) if want_scores else None
    gs = np.empty((B, Hq, nblk, Skv // G)) if want_scores else None
    forced = None
    if forced_chunk_idx is not None:
        forced = np.ascontiguousarray(forced_chunk_idx, dtype=np.int32)
        assert forced.shape == ci.shape
    if causal:
        qp = None if Qprev is None else _f64(Qprev)
        if qp is not None:
            assert qp.shape == (B, Hq, C, D)
        rc = _load().hgao_route_causal(B, Hq, Hkv, Sq, Skv, D, C, G, top_k, top_g, _d(Q), _d(qp),
                                       _d(chunk_mean), _d(group_mean), _i(forced), _i(ci),
                                       _i(gi), _d(cs), _d(gs))
    else:
        rc = _load().hgao_route(B, Hq, Hkv, Sq, Skv, D, C, G, top_k, top_g, _d(Q),
                                _d(chunk_mean), _d(group_mean), _i(forced), _i(ci), _i(gi),
                                _d(cs), _d(gs))
    _check(rc, "route")
    if want_scores:
        return ci, gi, cs, gs
    return ci, gi


def decode(Q, K, V, chunk_mean, group_mean, top_k: int, top_g: int, scale: float = 0.0,
           C: int = 64, G: int = 8, forced_chunk_idx=None, want_scores: bool = False):
    """One query per (b, hq) at the last position of the L-token cache K, V.

    Q [B,Hq,D]; K, V [B,Hkv,L,D]; chunk_mean [B,Hkv,L//C,D]; group_mean
    [B,Hkv,(L//C)*(C//G),D].  Returns ``(chunk_idx, group_idx, O, lse)`` and,
    with ``want_scores``, also ``(chunk_score, group_score)`` (NaN where no
    candidate).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    chunk_mean, group_mean = _f64(chunk_mean), _f64(group_mean)
    B, Hq, D = Q.shape
    Hkv, L = K.shape[1], K.shape[2]
    nca = L // C
    ci = np.empty((B, Hq, top_k), dtype=np.int32)
    gi = np.empty((B, Hq, top_g), dtype=np.int32)
    O = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    cs = np.empty((B, Hq, nca)) if want_scores else None
    gs = np.empty((B, Hq, nca * (C // G))) if want_scores else None
    forced = None
    if forced_chunk_idx is not None:
        forced = np.ascontiguousarray(forced_chunk_idx, dtype=np.int32)
        assert forced.shape == ci.shape
    rc = _load().hgao_decode(B, Hq, Hkv, L, D, C, G, top_k, top_g, scale, _d(Q), _d(K), _d(V),
                             _d(chunk_mean), _d(group_mean), _i(forced), _i(ci), _i(gi), _d(O),
                             _d(lse), _d(cs), _d(gs))
    _check(rc, "decode")
    if want_scores:
        return ci, gi, O, lse, cs, gs
    return ci, gi, O, lse


def attend_fwd(Q, K, V, group_idx, scale: float = 0.0, C: int = 64, G: int = 8):
    """Exact-token attention output O [B,Hq,Sq,D] and lse [B,Hq,Sq]."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    gi = np.ascontiguousarray(group_idx, dtype=np.int32)
    B, Hq, Sq, D = Q.shape
    Hkv, Skv = K.shape[1], K.shape[2]
    top_g = gi.shape[-1]
    O = np.empty_like(Q)
    lse = np.empty((B, Hq, Sq))
    rc = _load().hgao_attend_fwd(B, Hq, Hkv, Sq, Skv, D, C, G, top_g, scale, _d(Q), _d(K),
                                 _d(V), _i(gi), _d(O), _d(lse))
    _check(rc, "attend_fwd")
    return O, lse


def attend_bwd(Q, K, V, group_idx, dO, scale: float = 0.0, C: int = 64, G: int = 8):
    """Gradients (dQ, dK, dV) of sum(O * dO) with the routing held fixed."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    gi = np.ascontiguousarray(group_idx, dtype=np.int32)
    B, Hq, Sq, D = Q.shape
    Hkv, Skv = K.shape[1], K.shape[2]
    top_g = gi.shape[-1]
    dQ = np.empty_like(Q)
    dK = np.empty_like(K)
    dV = np.empty_like(V)
    rc = _load().hgao_attend_bwd(B, Hq, Hkv, Sq, Skv, D, C, G, top_g, scale, _d(Q), _d(K),
                                 _d(V), _i(gi), _d(dO), _d(dQ), _d(dK), _d(dV))
    _check(rc, "attend_bwd")
    return dQ, dK, dV


def attended_pairs(group_idx, C: int = 64, G: int = 8) -> int:
    """Total attended (query, key) pairs for a routing result."""
    gi = np.ascontiguousarray(group_idx, dtype=np.int32)
    B, Hq, nblk, top_g = gi.shape
    return int(_load().hgao_attended_pairs(B, Hq, nblk * C, C, G, top_g, _i(gi)))
