"""CPU oracle for HiLS attention — TEST INFRASTRUCTURE ONLY.

Loads the single-threaded fp64 C++ oracle (hils_oracle.cpp) with ctypes and
wraps it for numpy arrays. Only tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hils_oracle.cpp")
_LIB = os.path.join(_HERE, "libhils_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)
_L = ctypes.POINTER(ctypes.c_long)
_U8 = ctypes.POINTER(ctypes.c_ubyte)


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (plain -O2, single thread)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def use_native_build(directory: str) -> str:
    """Compile the oracle with -O3 -march=native (vectorisation allowed, still one
    thread) into `directory` on the machine that will run it, and load that build
    in place of the portable one. Used by the benchmark's CPU baseline."""
    global _lib
    os.makedirs(directory, exist_ok=True)
    path = os.path.join(directory, "libhils_oracle_native.so")
    subprocess.check_call(["g++", "-O3", "-march=native", "-std=c++17", "-shared", "-fPIC", "-o",
                           path, _SRC])
    _lib = None
    lib(path)
    return path


def lib(path: Optional[str] = None):
    global _lib
    if _lib is None:
        if path is None:
            build(force=False)
        L = ctypes.CDLL(path or _LIB)
        ci, cl, cd = ctypes.c_int, ctypes.c_long, ctypes.c_double
        L.oracle_summarize.argtypes = [ci, ci, ci, ci, ci, ci, ci, cd, _D, _D, ci, ci, _D, _D, _D]
        L.oracle_score_topk.argtypes = [ci, ci, cl, ci, ci, ci, ci, ci, cd, cl, _D, _D, _D, cl,
                                        _L, _I, _D, _D]
        L.oracle_score_topk_group.argtypes = [ci, ci, cl, ci, ci, ci, ci, ci, ci, cd, cl, _D,
                                              _D, _D, cl, _L, _I, _D, _D]
        L.oracle_exact_chunk_lse.argtypes = [ci, ci, ci, cl, ci, ci, ci, ci, ci, cd, cl, _D, _D,
                                             cl, _L, _D]
        L.oracle_attend_fuse.argtypes = [ci, ci, ci, cl, ci, ci, ci, ci, ci, cd, cl, _D, _D, _D,
                                         _I, _D, cl, _L, _D, _D, _D]
        L.oracle_backward.argtypes = [ci, ci, ci, cl, ci, ci, ci, ci, ci, ci, cd, cl, _D, _D, _D,
                                      _D, _I, _D, _U8, _U8, _D, _D, _D, _D, _D, _D]
        for f in (L.oracle_summarize, L.oracle_score_topk, L.oracle_score_topk_group,
                  L.oracle_exact_chunk_lse, L.oracle_attend_fuse, L.oracle_backward):
            f.restype = None
        _lib = L
    return _lib


def _d(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x, t):
    return None if x is None else x.ctypes.data_as(t)


def _rows(rows):
    if rows is None:
        return 0, None
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r.size, r


def summarize(K, Ql, S, scale=0.0, c_begin=0, c_end=None):
    """Landmark summaries -> (ksum [B,NC,H,d], ent [B,NC,H], lse_l [B,NC,H])."""
    K, Ql = _d(K), _d(Ql)
    B, Tkv, Hkv, d = K.shape
    NC, H = Ql.shape[1], Ql.shape[2]
    c_end = NC if c_end is None else c_end
    ksum = np.zeros((B, NC, H, d))
    ent = np.zeros((B, NC, H))
    lse = np.zeros((B, NC, H))
    lib().oracle_summarize(B, Tkv, H, Hkv, d, S, NC, scale, _p(K, _D), _p(Ql, _D), c_begin,
                           c_end, _p(ksum, _D), _p(ent, _D), _p(lse, _D))
    return ksum, ent, lse


def score_topk(Q, ksum, ent, S, Ksel, q_pos0=0, scale=0.0, rows=None, group_hkv=None,
               window=0):
    """Top-K chunk selection -> (idx [B,Tq,H,K] int32, score [B,Tq,H,K], gap [B,Tq,H]).

    group_hkv=Hkv selects one chunk set per kv head by the maximum of the group's
    head scores (GQA group-max selection); None selects per query head. window is
    the local branch (0: own chunk; W > 0: the last W keys), which sets the
    candidates."""
    Q, ksum, ent = _d(Q), _d(ksum), _d(ent)
    B, Tq, H, d = Q.shape
    NC = ksum.shape[1]
    idx = np.full((B, Tq, H, Ksel), -1, dtype=np.int32)
    score = np.full((B, Tq, H, Ksel), -np.inf)
    gap = np.full((B, Tq, H), np.nan)
    n, r = _rows(rows)
    if group_hkv is None:
        lib().oracle_score_topk(B, Tq, q_pos0, H, d, S, NC, Ksel, scale, window, _p(Q, _D),
                                _p(ksum, _D), _p(ent, _D), n, _p(r, _L), _p(idx, _I),
                                _p(score, _D), _p(gap, _D))
    else:
        lib().oracle_score_topk_group(B, Tq, q_pos0, H, group_hkv, d, S, NC, Ksel, scale,
                                      window, _p(Q, _D), _p(ksum, _D), _p(ent, _D), n, _p(r, _L),
                                      _p(idx, _I), _p(score, _D), _p(gap, _D))
    return idx, score, gap


def exact_chunk_lse(Q, K, S, NC, q_pos0=0, scale=0.0, rows=None, window=0):
    """log Z_{i,c} of every candidate chunk -> [B,Tq,H,NC] (-inf where not a candidate)."""
    Q, K = _d(Q), _d(K)
    B, Tq, H, d = Q.shape
    Tkv, Hkv = K.shape[1], K.shape[2]
    out = np.full((B, Tq, H, NC), np.nan)
    n, r = _rows(rows)
    lib().oracle_exact_chunk_lse(B, Tq, Tkv, q_pos0, H, Hkv, d, S, NC, scale, window, _p(Q, _D),
                                 _p(K, _D), n, _p(r, _L), _p(out, _D))
    return out


def attend_fuse(Q, K, V, idx, score, S, q_pos0=0, scale=0.0, rows=None, window=0):
    """Hierarchical attention -> (O [B,Tq,H,d], lse_own [B,Tq,H], lse_tot [B,Tq,H]);
    lse_own is the local branch's log-mass (own chunk, or the last `window` keys)."""
    Q, K, V, score = _d(Q), _d(K), _d(V), _d(score)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, Tq, H, d = Q.shape
    Tkv, Hkv = K.shape[1], K.shape[2]
    Ksel = idx.shape[-1]
    O = np.full((B, Tq, H, d), np.nan)
    lo = np.full((B, Tq, H), np.nan)
    lt = np.full((B, Tq, H), np.nan)
    n, r = _rows(rows)
    lib().oracle_attend_fuse(B, Tq, Tkv, q_pos0, H, Hkv, d, S, Ksel, scale, window, _p(Q, _D),
                             _p(K, _D), _p(V, _D), _p(idx, _I), _p(score, _D), n, _p(r, _L),
                             _p(O, _D), _p(lo, _D), _p(lt, _D))
    return O, lo, lt


def forward(Q, K, V, Ql, S, Ksel, q_pos0=0, scale=0.0, rows=None, group=False, Qs=None,
            window=0):
    """Whole forward: summaries, scores/top-K, attend+fuse. Returns a dict.
    group=True selects one chunk set per kv head (GQA group-max selection);
    Qs is the Q-Cal scoring query (the chunk scores use it, the attention uses Q);
    window is the local branch (0: own chunk; W > 0: sliding window of W keys)."""
    ksum, ent, lse_l = summarize(K, Ql, S, scale)
    idx, score, gap = score_topk(Q if Qs is None else Qs, ksum, ent, S, Ksel, q_pos0, scale, rows,
                                 group_hkv=K.shape[2] if group else None, window=window)
    O, lo, lt = attend_fuse(Q, K, V, idx, score, S, q_pos0, scale, rows, window=window)
    return dict(ksum=ksum, ent=ent, lse_l=lse_l, idx=idx, score=score, gap=gap, O=O,
                lse_own=lo, lse_tot=lt)


def backward(Q, K, V, Ql, idx, dO, S, q_pos0=0, scale=0.0, row_mask=None, kv_mask=None,
             Qs=None, window=0):
    """Gradients (dQ, dK, dV, dQl) of sum(dO*O) with idx held fixed; NaN outside the masks.
    With a Q-Cal scoring query Qs the result is (dQ, dK, dV, dQl, dQs): dQs is the
    gradient through the chunk scores, dQ the one through the token attention."""
    Q, K, V, Ql, dO = _d(Q), _d(K), _d(V), _d(Ql), _d(dO)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, Tq, H, d = Q.shape
    Tkv, Hkv = K.shape[1], K.shape[2]
    NC = Ql.shape[1]
    Ksel = idx.shape[-1]
    dQ = np.full(Q.shape, np.nan)
    dK = np.full(K.shape, np.nan)
    dV = np.full(V.shape, np.nan)
    dQl = np.full(Ql.shape, np.nan)
    Qs = None if Qs is None else _d(Qs)
    dQs = None if Qs is None else np.full(Q.shape, np.nan)
    rm = None if row_mask is None else np.ascontiguousarray(row_mask, dtype=np.uint8)
    km = None if kv_mask is None else np.ascontiguousarray(kv_mask, dtype=np.uint8)
    lib().oracle_backward(B, Tq, Tkv, q_pos0, H, Hkv, d, S, NC, Ksel, scale, window, _p(Q, _D),
                          _p(K, _D),
                          _p(V, _D), _p(Ql, _D), _p(idx, _I), _p(dO, _D), _p(rm, _U8),
                          _p(km, _U8), _p(dQ, _D), _p(dK, _D), _p(dV, _D), _p(dQl, _D),
                          _p(Qs, _D), _p(dQs, _D))
    return (dQ, dK, dV, dQl) if Qs is None else (dQ, dK, dV, dQl, dQs)
