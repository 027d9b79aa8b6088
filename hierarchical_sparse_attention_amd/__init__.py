"""Python binding of libhils, the MI355X HiLS attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/hils.h. torch supplies device memory and the current HIP
stream. There is no CPU fallback: if libhils.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["HilsError", "lib", "make_dims", "summarize", "score_topk", "score_topk_noalloc",
           "attend_fuse", "decode", "decode_workspace", "backward",
           "forward", "workspace_size", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhils.so")

HILS_F32, HILS_BF16 = 0, 1
OP_SUMMARIZE, OP_SCORE_TOPK, OP_ATTEND_FUSE, OP_BACKWARD, OP_DECODE = 0, 1, 2, 3, 4
STATUS = {0: "HILS_OK", 1: "HILS_ERR_INVALID_ARG", 2: "HILS_ERR_UNSUPPORTED",
          3: "HILS_ERR_WORKSPACE", 4: "HILS_ERR_HIP", 5: "HILS_ERR_SCRATCH"}
EXPORTS = ("hils_workspace_size", "hils_summarize", "hils_score_topk", "hils_score_topk_noalloc",
           "hils_attend_fuse", "hils_decode", "hils_backward", "hils_status_string",
           "hils_version")


class hils_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("Tkv", ctypes.c_int32),
                ("Tkv_cap", ctypes.c_int32), ("NC_cap", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("S", ctypes.c_int32),
                ("K", ctypes.c_int32), ("dtype", ctypes.c_int32), ("select_mode", ctypes.c_int32),
                ("q_pos0", ctypes.c_int64), ("scale", ctypes.c_float),
                ("window", ctypes.c_int32)]


class HilsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None


def lib():
    """Load libhils.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m hierarchical_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, SZ = ctypes.POINTER(hils_dims), ctypes.c_void_p, ctypes.c_size_t
        i32 = ctypes.c_int32
        L.hils_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(SZ)]
        L.hils_summarize.argtypes = [P, VP, VP, i32, i32, VP, VP, VP, VP, SZ, VP]
        L.hils_score_topk.argtypes = [P, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.hils_score_topk_noalloc.argtypes = [P, VP, VP, VP, VP, VP, VP]
        L.hils_attend_fuse.argtypes = [P, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.hils_decode.argtypes = [P, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.hils_backward.argtypes = [P] + [VP] * 18 + [VP, SZ, VP]
        L.hils_status_string.argtypes = [ctypes.c_int]
        L.hils_status_string.restype = ctypes.c_char_p
        L.hils_version.restype = i32
        for f in ("hils_workspace_size", "hils_summarize", "hils_score_topk",
                  "hils_score_topk_noalloc", "hils_attend_fuse", "hils_decode",
                  "hils_backward"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HILS_F32
    if t.dtype == torch.bfloat16:
        return HILS_BF16
    raise ValueError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def make_dims(B, Tq, Tkv, H, Hkv, d, S, K, dtype, q_pos0=0, scale=0.0, Tkv_cap=0,
              NC_cap=0, select_mode=0, window=0) -> hils_dims:
    return hils_dims(B, Tq, Tkv, Tkv_cap, NC_cap, H, Hkv, d, S, K, dtype, select_mode, q_pos0,
                     scale, window)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise HilsError(fn, st)


def _need(t: torch.Tensor, name: str, shape=None, dtype=None, host_ok=False):
    """host_ok: the tensor may also live in pinned host memory (a decode cache's K/V)."""
    if not (t.is_cuda or (host_ok and t.is_pinned())):
        raise ValueError(f"{name} must be a GPU tensor" + (" or pinned host memory" if host_ok
                                                          else ""))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def workspace_size(dims: hils_dims, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("hils_workspace_size", lib().hils_workspace_size(ctypes.byref(dims), op, ctypes.byref(n)))
    return n.value


def _workspace(dims, op, device):
    n = workspace_size(dims, op)
    return (torch.empty(max(n, 256), dtype=torch.uint8, device=device), n)


def summarize(K: torch.Tensor, Ql: torch.Tensor, S: int = 64, c_begin: int = 0,
              c_end: Optional[int] = None, Tkv: Optional[int] = None, scale: float = 0.0,
              ksum=None, ent=None, lse_l=None):
    """Landmark summaries of chunks [c_begin, c_end). K [B,Tcap,Hkv,d], Ql [B,NCcap,H,d].
    K may be in pinned host memory (an offloaded cache).

    Returns (ksum [B,NCcap,H,d] f32, ent [B,NCcap,H] f32, lse_l [B,NCcap,H] f32).
    """
    B, Tcap, Hkv, d = K.shape
    NCcap, H = Ql.shape[1], Ql.shape[2]
    Tkv = Tcap if Tkv is None else Tkv
    c_end = Tkv // S if c_end is None else c_end
    _need(K, "K", host_ok=True), _need(Ql, "Ql", (B, NCcap, H, d), K.dtype)
    dev = Ql.device
    ksum = torch.empty(B, NCcap, H, d, dtype=torch.float32, device=dev) if ksum is None else ksum
    ent = torch.empty(B, NCcap, H, dtype=torch.float32, device=dev) if ent is None else ent
    lse_l = torch.empty(B, NCcap, H, dtype=torch.float32, device=dev) if lse_l is None else lse_l
    _need(ksum, "ksum", (B, NCcap, H, d), torch.float32)
    _need(ent, "ent", (B, NCcap, H), torch.float32)
    _need(lse_l, "lse_l", (B, NCcap, H), torch.float32)
    dims = make_dims(B, 0, Tkv, H, Hkv, d, S, 1, _dtype_code(K), 0, scale, Tcap, NCcap)
    _check("hils_summarize", lib().hils_summarize(
        ctypes.byref(dims), _ptr(K), _ptr(Ql), c_begin, c_end, _ptr(ksum), _ptr(ent), _ptr(lse_l),
        None, 0, _stream(dev)))
    return ksum, ent, lse_l


def score_topk(Q: torch.Tensor, ksum: torch.Tensor, ent: torch.Tensor, K_sel: int, S: int = 64,
               q_pos0: int = 0, Tkv: Optional[int] = None, scale: float = 0.0, Hkv: int = 1,
               idx=None, score=None, group: bool = False, window: int = 0):
    """Top-K chunk selection for query rows at positions q_pos0.. -> (idx int32, score f32).
    group=True selects one chunk set per kv head by the group maximum of the scores;
    window is the local branch (0: own chunk; W > 0: the last W keys)."""
    B, Tq, H, d = Q.shape
    NCcap = ksum.shape[1]
    Tkv = q_pos0 + Tq if Tkv is None else Tkv
    _need(Q, "Q"), _need(ksum, "ksum", (B, NCcap, H, d), torch.float32)
    _need(ent, "ent", (B, NCcap, H), torch.float32)
    dev = Q.device
    idx = torch.empty(B, Tq, H, K_sel, dtype=torch.int32, device=dev) if idx is None else idx
    score = torch.empty(B, Tq, H, K_sel, dtype=torch.float32, device=dev) if score is None else score
    _need(idx, "idx", (B, Tq, H, K_sel), torch.int32)
    _need(score, "score", (B, Tq, H, K_sel), torch.float32)
    dims = make_dims(B, Tq, Tkv, H, Hkv, d, S, K_sel, _dtype_code(Q), q_pos0, scale,
                     max(Tkv, NCcap * S), NCcap, 1 if group else 0, window)
    ws, n = _workspace(dims, OP_SCORE_TOPK, dev)
    _check("hils_score_topk", lib().hils_score_topk(
        ctypes.byref(dims), _ptr(Q), _ptr(ksum), _ptr(ent), _ptr(idx), _ptr(score), _ptr(ws), n,
        _stream(dev)))
    return idx, score


def score_topk_noalloc(Q: torch.Tensor, ksum: torch.Tensor, ent: torch.Tensor, K_sel: int,
                       S: int = 64, q_pos0: int = 0, Tkv: Optional[int] = None,
                       scale: float = 0.0, Hkv: int = 1, idx=None, score=None,
                       group: bool = False, window: int = 0):
    """score_topk through the entry point that takes no workspace (the library's static
    scratch); for callers that cannot allocate, pass idx and score."""
    B, Tq, H, d = Q.shape
    NCcap = ksum.shape[1]
    Tkv = q_pos0 + Tq if Tkv is None else Tkv
    _need(Q, "Q"), _need(ksum, "ksum", (B, NCcap, H, d), torch.float32)
    _need(ent, "ent", (B, NCcap, H), torch.float32)
    dev = Q.device
    idx = torch.empty(B, Tq, H, K_sel, dtype=torch.int32, device=dev) if idx is None else idx
    score = torch.empty(B, Tq, H, K_sel, dtype=torch.float32, device=dev) if score is None else score
    _need(idx, "idx", (B, Tq, H, K_sel), torch.int32)
    _need(score, "score", (B, Tq, H, K_sel), torch.float32)
    dims = make_dims(B, Tq, Tkv, H, Hkv, d, S, K_sel, _dtype_code(Q), q_pos0, scale,
                     max(Tkv, NCcap * S), NCcap, 1 if group else 0, window)
    _check("hils_score_topk_noalloc", lib().hils_score_topk_noalloc(
        ctypes.byref(dims), _ptr(Q), _ptr(ksum), _ptr(ent), _ptr(idx), _ptr(score), _stream(dev)))
    return idx, score


def attend_fuse(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                score: torch.Tensor, S: int = 64, q_pos0: int = 0, Tkv: Optional[int] = None,
                scale: float = 0.0, O=None, lse_own=None, lse_tot=None, window: int = 0):
    """Hierarchical attention -> (O [B,Tq,H,d], lse_own [B,Tq,H], lse_tot [B,Tq,H]);
    lse_own is the local branch's log-mass (own chunk, or the last `window` keys).
    K and V may be in pinned host memory (an offloaded decode cache): the kernels
    then read only the chunks the rows select and their local branch."""
    B, Tq, H, d = Q.shape
    Tcap, Hkv = K.shape[1], K.shape[2]
    K_sel = idx.shape[-1]
    Tkv = Tcap if Tkv is None else Tkv
    _need(Q, "Q"), _need(K, "K", (B, Tcap, Hkv, d), Q.dtype, host_ok=True)
    _need(V, "V", (B, Tcap, Hkv, d), Q.dtype, host_ok=True)
    _need(idx, "idx", (B, Tq, H, K_sel), torch.int32)
    _need(score, "score", (B, Tq, H, K_sel), torch.float32)
    dev = Q.device
    O = torch.empty_like(Q) if O is None else O
    lse_own = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if lse_own is None else lse_own
    lse_tot = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if lse_tot is None else lse_tot
    _need(O, "O", Q.shape, Q.dtype)
    _need(lse_own, "lse_own", (B, Tq, H), torch.float32)
    _need(lse_tot, "lse_tot", (B, Tq, H), torch.float32)
    dims = make_dims(B, Tq, Tkv, H, Hkv, d, S, K_sel, _dtype_code(Q), q_pos0, scale, Tcap, 0,
                     window=window)
    ws, n = _workspace(dims, OP_ATTEND_FUSE, dev)
    _check("hils_attend_fuse", lib().hils_attend_fuse(
        ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(score), _ptr(O),
        _ptr(lse_own), _ptr(lse_tot), _ptr(ws), n, _stream(dev)))
    return O, lse_own, lse_tot


def decode_workspace(Q: torch.Tensor, K: torch.Tensor, ksum: torch.Tensor, K_sel: int,
                     S: int = 64, q_pos0: int = 0, Tkv: Optional[int] = None,
                     window: int = 0) -> torch.Tensor:
    """A workspace for decode() calls of these shapes (allocate it once, outside any
    captured graph, and pass it to every call)."""
    B, Tq, H, d = Q.shape
    Tcap, Hkv = K.shape[1], K.shape[2]
    Tkv = q_pos0 + Tq if Tkv is None else Tkv
    dims = make_dims(B, Tq, Tkv, H, Hkv, d, S, K_sel, _dtype_code(Q), q_pos0, 0.0, Tcap,
                     ksum.shape[1], window=window)
    return torch.empty(max(workspace_size(dims, OP_DECODE), 256), dtype=torch.uint8,
                       device=Q.device)


def decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, ksum: torch.Tensor,
           ent: torch.Tensor, K_sel: int, S: int = 64, q_pos0: int = 0, Tkv: Optional[int] = None,
           scale: float = 0.0, idx=None, score=None, O=None, lse_own=None, lse_tot=None,
           ws: Optional[torch.Tensor] = None, window: int = 0):
    """One decode step of the query rows at q_pos0.. over the cache K, V (selection and
    attention in one call) -> (idx, score, O, lse_own, lse_tot). ws: a workspace from
    decode_workspace() (a zeroed one is made when it is None)."""
    B, Tq, H, d = Q.shape
    Tcap, Hkv = K.shape[1], K.shape[2]
    NCcap = ksum.shape[1]
    Tkv = q_pos0 + Tq if Tkv is None else Tkv
    _need(Q, "Q"), _need(K, "K", (B, Tcap, Hkv, d), Q.dtype, host_ok=True)
    _need(V, "V", (B, Tcap, Hkv, d), Q.dtype, host_ok=True)
    _need(ksum, "ksum", (B, NCcap, H, d), torch.float32)
    _need(ent, "ent", (B, NCcap, H), torch.float32)
    dev = Q.device
    idx = torch.empty(B, Tq, H, K_sel, dtype=torch.int32, device=dev) if idx is None else idx
    score = torch.empty(B, Tq, H, K_sel, dtype=torch.float32, device=dev) if score is None else score
    O = torch.empty_like(Q) if O is None else O
    lse_own = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if lse_own is None else lse_own
    lse_tot = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if lse_tot is None else lse_tot
    _need(idx, "idx", (B, Tq, H, K_sel), torch.int32)
    _need(score, "score", (B, Tq, H, K_sel), torch.float32)
    _need(O, "O", Q.shape, Q.dtype)
    _need(lse_own, "lse_own", (B, Tq, H), torch.float32)
    _need(lse_tot, "lse_tot", (B, Tq, H), torch.float32)
    dims = make_dims(B, Tq, Tkv, H, Hkv, d, S, K_sel, _dtype_code(Q), q_pos0, scale, Tcap, NCcap,
                     window=window)
    need = workspace_size(dims, OP_DECODE)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(ws, "ws", dtype=torch.uint8)
    _check("hils_decode", lib().hils_decode(
        ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(ksum), _ptr(ent), _ptr(idx),
        _ptr(score), _ptr(O), _ptr(lse_own), _ptr(lse_tot), _ptr(ws), ws.numel(), _stream(dev)))
    return idx, score, O, lse_own, lse_tot


def forward(Q, K, V, Ql, K_sel: int, S: int = 64, scale: float = 0.0, group: bool = False,
            Qs=None, window: int = 0):
    """Prefill forward: summaries, selection, attention. Returns a dict of tensors.
    Qs is an optional Q-Cal scoring query (the chunk scores use it, the attention Q);
    window is the local branch (0: own chunk; W > 0: sliding window of W keys)."""
    ksum, ent, lse_l = summarize(K, Ql, S, scale=scale)
    idx, score = score_topk(Q if Qs is None else Qs, ksum, ent, K_sel, S, 0, K.shape[1], scale,
                            Hkv=K.shape[2], group=group, window=window)
    O, lse_own, lse_tot = attend_fuse(Q, K, V, idx, score, S, 0, scale=scale, window=window)
    return dict(ksum=ksum, ent=ent, lse_l=lse_l, idx=idx, score=score, O=O, lse_own=lse_own,
                lse_tot=lse_tot)


def backward(Q, K, V, Ql, ksum, ent, lse_l, idx, score, lse_tot, O, dO, S: int = 64,
             scale: float = 0.0, Qs=None, window: int = 0):
    """Gradients (dQ, dK, dV, dQl) of sum(dO * O) with the selection held fixed; O is the
    forward's output. With a Q-Cal scoring query Qs (the query the chunk scores were
    computed from) the result is (dQ, dK, dV, dQl, dQs): dQs through the scores, dQ
    through the token attention."""
    B, T, H, d = Q.shape
    Hkv = K.shape[2]
    K_sel = idx.shape[-1]
    NC = Ql.shape[1]
    _dtype_code(Q)
    _need(Q, "Q")
    _need(K, "K", (B, T, Hkv, d), Q.dtype)
    _need(V, "V", (B, T, Hkv, d), Q.dtype)
    if NC < T // S:
        raise ValueError(f"Ql holds {NC} chunks, fewer than the {T // S} of the sequence")
    _need(Ql, "Ql", (B, NC, H, d), Q.dtype)
    _need(O, "O", tuple(Q.shape), Q.dtype)
    _need(dO, "dO", tuple(Q.shape), Q.dtype)
    if Qs is not None:
        _need(Qs, "Qs", tuple(Q.shape), Q.dtype)
    _need(ksum, "ksum", (B, NC, H, d), torch.float32)
    _need(ent, "ent", (B, NC, H), torch.float32)
    _need(lse_l, "lse_l", (B, NC, H), torch.float32)
    _need(idx, "idx", (B, T, H, K_sel), torch.int32)
    _need(score, "score", (B, T, H, K_sel), torch.float32)
    _need(lse_tot, "lse_tot", (B, T, H), torch.float32)
    dev = Q.device
    dQ, dK, dV, dQl = (torch.empty_like(x) for x in (Q, K, V, Ql))
    dQs = None if Qs is None else torch.empty_like(Q)
    dims = make_dims(B, T, T, H, Hkv, d, S, K_sel, _dtype_code(Q), 0, scale, T, NC,
                     window=window)
    ws, n = _workspace(dims, OP_BACKWARD, dev)
    _check("hils_backward", lib().hils_backward(
        ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(Ql), _ptr(ksum), _ptr(ent),
        _ptr(lse_l), _ptr(idx), _ptr(score), _ptr(lse_tot), _ptr(O), _ptr(dO), _ptr(dQ), _ptr(dK),
        _ptr(dV), _ptr(dQl), _ptr(Qs), _ptr(dQs), _ptr(ws), n, _stream(dev)))
    return (dQ, dK, dV, dQl) if Qs is None else (dQ, dK, dV, dQl, dQs)
