"""Seeded synthetic inputs for HiLS attention.

This module only draws and rounds random numbers; it holds none of the
attention arithmetic. Both the GPU path and the CPU oracle consume the arrays
it returns, so the two see bit-identical inputs.

Random source: a splitmix64 stream per (seed, stream id), read with random
access (value n of a stream is the splitmix64 finaliser applied to
key + (n + 1) * 0x9E3779B97F4A7C15, key derived from seed and stream id), then
Box-Muller in float64 for normals. Values are rounded to float32 with
round-to-nearest-even, and, for bf16 workloads, from float32 to bf16 with
round-to-nearest-even. Every tensor is returned as float32 (bf16 values are
exactly representable in float32).

Workload structure (the pages measure on pretraining text with trained
checkpoints, which are not available; these synthetic tensors stand in):
  * Q, K, V, landmark queries Ql and the upstream gradient dO ~ N(0, 1).
  * "planted peak" chunks: in a seeded choice of chunks, two keys per chunk
    (seeded positions) are set to 3 * u, where u is the unit vector along the
    mean of the queries of that batch element and kv-head group.
  * "near-uniform" chunks (7B-class workload): per chunk and kv head a shared
    vector a ~ N(0, I); every key of the chunk is a + 0.05 * noise.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

BASE_SEED = 0x48694C53  # ASCII "HiLS"

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream ids, one per drawn tensor
ST_Q, ST_K, ST_V, ST_QL, ST_DO = 1, 2, 3, 4, 5
ST_CHUNK_PICK, ST_KEY_PICK, ST_NU_SHARED, ST_NU_NOISE = 6, 7, 9, 10
ST_QS = 11


def _fmix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _stream_key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = np.array([(seed ^ (stream << 32)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
        return _fmix(k + _GAMMA)[0]


def uniform(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Values start..start+count-1 of a stream as float64 in the open interval (0, 1)."""
    key = _stream_key(seed, stream)
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = _fmix(key + n * _GAMMA)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, stream: int, count: int, start: int = 0,
           block: int = 1 << 24) -> np.ndarray:
    """count standard normals (float64) of a stream, beginning at (even) value index start.

    Box-Muller on consecutive uniform pairs (2m, 2m+1): r = sqrt(-2 ln u_2m),
    angle 2 pi u_2m+1, normals r cos, r sin.
    """
    if start % 2:
        raise ValueError("start must be even")
    out = np.empty(count, dtype=np.float64)
    pairs = (count + 1) // 2
    for p0 in range(0, pairs, block):
        p1 = min(pairs, p0 + block)
        u = uniform(seed, stream, start + 2 * p0, 2 * (p1 - p0))
        r = np.sqrt(-2.0 * np.log(u[0::2]))
        th = (2.0 * math.pi) * u[1::2]
        z = np.empty(2 * (p1 - p0), dtype=np.float64)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        lo, hi = 2 * p0, min(count, 2 * p1)
        out[lo:hi] = z[: hi - lo]
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (round to nearest even), returned as float32 with the low 16 bits zero."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32).reshape(x32.shape)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    f = round_f32(x)
    return round_bf16(f) if dtype == "bf16" else f


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int            # key rows (prefill: also query rows)
    H: int
    Hkv: int
    d: int
    S: int
    K: int
    dtype: str        # "f32" or "bf16"
    n_planted: int    # planted-peak chunks per batch element
    n_uniform: int = 0  # near-uniform chunks per batch element
    Tq: Optional[int] = None   # query rows (default T)
    q_pos0: int = 0            # absolute position of query row 0
    need_dO: bool = False
    seed: int = BASE_SEED
    decode_steps: int = 0      # decode workloads: number of timed steps

    @property
    def NC(self) -> int:
        return self.T // self.S

    @property
    def rows_q(self) -> int:
        return self.T if self.Tq is None else self.Tq


def frac_count(frac: float, nc: int) -> int:
    return max(1, int(round(frac * nc)))


def workloads() -> Dict[str, Workload]:
    """The five benchmark workloads: tiny fp32, 345M prefill, 128K decode, 7B GQA prefill, training."""
    s = BASE_SEED
    dec_T = 131072 + 256
    return {
        "tiny_f32": Workload("tiny_f32", 1, 2048, 4, 4, 64, 64, 8, "f32", 4, seed=s + 0),
        "prefill_345m": Workload("prefill_345m", 1, 8192, 16, 16, 64, 64, 16, "bf16",
                                 frac_count(0.01, 128), seed=s + 1),
        "decode_128k": Workload("decode_128k", 1, dec_T, 16, 16, 64, 64, 16, "bf16",
                                frac_count(0.01, 131072 // 64), Tq=256, q_pos0=131072,
                                seed=s + 2, decode_steps=256),
        "prefill_7b_gqa": Workload("prefill_7b_gqa", 1, 32768, 32, 8, 128, 64, 16, "bf16",
                                   frac_count(0.005, 512), frac_count(0.05, 512), seed=s + 3),
        "train_345m": Workload("train_345m", 2, 16384, 16, 16, 64, 64, 16, "bf16",
                               frac_count(0.01, 256), need_dO=True, seed=s + 4),
    }


def make_inputs(w: Workload) -> Dict[str, np.ndarray]:
    """Draw Q [B,Tq,H,d], K and V [B,T,Hkv,d], Ql [B,NC,H,d] (and dO [B,Tq,H,d]) as float32.

    Generation order is fixed: Q, K, V, Ql, dO, then planted / near-uniform
    edits of K (which read the rounded Q for the planted direction).
    """
    B, T, H, Hkv, d, S = w.B, w.T, w.H, w.Hkv, w.d, w.S
    Tq, NC, G = w.rows_q, w.NC, w.H // w.Hkv
    out = {}
    out["Q"] = to_dtype(normal(w.seed, ST_Q, B * Tq * H * d), w.dtype).reshape(B, Tq, H, d)
    K = to_dtype(normal(w.seed, ST_K, B * T * Hkv * d), w.dtype).reshape(B, T, Hkv, d)
    out["V"] = to_dtype(normal(w.seed, ST_V, B * T * Hkv * d), w.dtype).reshape(B, T, Hkv, d)
    out["Ql"] = to_dtype(normal(w.seed, ST_QL, B * NC * H * d), w.dtype).reshape(B, NC, H, d)
    if w.need_dO:
        out["dO"] = to_dtype(normal(w.seed, ST_DO, B * Tq * H * d), w.dtype).reshape(B, Tq, H, d)

    n_pick = w.n_planted + w.n_uniform
    if n_pick > NC:
        raise ValueError("more structured chunks than chunks")
    planted, uniform_chunks = [], []
    for b in range(B):
        perm = np.argsort(uniform(w.seed, ST_CHUNK_PICK, b * NC, NC), kind="stable")
        planted.append(perm[: w.n_planted])
        uniform_chunks.append(perm[w.n_planted:n_pick])
    if w.n_planted:
        q64 = out["Q"].astype(np.float64)
        for b in range(B):
            for g in range(Hkv):
                m = q64[b, :, g * G:(g + 1) * G, :].mean(axis=(0, 1))
                u = m / np.linalg.norm(m)
                peak = to_dtype(3.0 * u, w.dtype)
                for pi, c in enumerate(planted[b]):
                    key_u = uniform(w.seed, ST_KEY_PICK, ((b * w.n_planted + pi) * S), S)
                    pos = np.argsort(key_u, kind="stable")[:2]
                    for j in pos:
                        K[b, c * S + j, g, :] = peak
    if w.n_uniform:
        for b in range(B):
            for ui, c in enumerate(uniform_chunks[b]):
                base = (b * w.n_uniform + ui)
                a = normal(w.seed, ST_NU_SHARED, Hkv * d, start=base * Hkv * d).reshape(Hkv, d)
                eps = normal(w.seed, ST_NU_NOISE, S * Hkv * d,
                             start=base * S * Hkv * d).reshape(S, Hkv, d)
                K[b, c * S:(c + 1) * S, :, :] = to_dtype(a[None, :, :] + 0.05 * eps, w.dtype)
    out["K"] = K
    out["planted_chunks"] = np.array(planted, dtype=np.int64)
    out["uniform_chunks"] = np.array(uniform_chunks, dtype=np.int64)
    return out


def scoring_query(w: Workload, x: Dict[str, np.ndarray], spread: float = 0.5) -> np.ndarray:
    """A stand-in for a calibrated scoring query (Q-Cal): the workload's Q plus
    seeded N(0, spread^2) noise from a stream of its own, rounded to the dtype."""
    q = x["Q"]
    noise = normal(w.seed, ST_QS, q.size).reshape(q.shape)
    return to_dtype(q.astype(np.float64) + spread * noise, w.dtype)


def small(name: str, B=1, T=512, H=2, Hkv=1, d=64, S=64, K=4, dtype="f32", n_planted=1,
          n_uniform=0, Tq=None, q_pos0=0, need_dO=False, seed=BASE_SEED + 100) -> Workload:
    """A reduced workload with the same value distributions, for fast tests."""
    return Workload(name, B, T, H, Hkv, d, S, K, dtype, n_planted, n_uniform, Tq, q_pos0,
                    need_dO, seed)
