"""GPU selection contract and accumulation range, through the C ABI against the oracle.

* Exact ties: chunks are made in groups of three bit-identical copies (keys and
  landmark queries), so their summaries, and every query's scores of them, are
  bit-identical on the GPU and in the oracle. With K not a multiple of three the
  K-th and (K+1)-th places of most rows fall inside one group, and the rule that
  equal scores go to the lower chunk id decides the set. Every selection kernel
  is covered: prefill per head (bf16 matrix-core lists of 16/32/64 entries, float32
  rows), group-max (matrix-core G = 2, 4; float32 lane-shuffle), and decode
  (one workgroup per row; candidate splits with the rank, wavefront and
  workgroup merges).
* Selection lists whose entries do not all count (repeated, out-of-order, negative
  or beyond the candidates) give the oracle's result, forward and backward.
* A chunk of values 2^14 times larger than the rest leaves the rows that did not
  select it exact to the output tolerance (per-row fixed-point range).
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hsa
import oracle
import synth
from hils_testutil import (NEAR_TIE, TOL_BF16, TOL_F32, TOL_GRAD_BF16, all_scores, assert_close,
                           say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def tied_inputs(w, group=3):
    """Inputs whose chunks come in groups of `group` identical copies (keys of every
    kv head and landmark queries of every head copied from the group's first chunk)."""
    x = synth.make_inputs(w)
    S = w.S
    for c in range(w.NC):
        src = c - c % group
        if src != c:
            x["K"][:, c * S:(c + 1) * S] = x["K"][:, src * S:(src + 1) * S]
            x["Ql"][:, c] = x["Ql"][:, src]
    return x


def check_ties(gidx, Q, ksum, ent, S, K, q_pos0=0, group_hkv=None):
    """GPU index sets equal the oracle's on every row whose K-th score is at least
    NEAR_TIE away from every other score value (exact copies of it included, so ties
    at the K-th place are decided by the chunk id). Returns (clean rows, clean rows
    whose K-th and (K+1)-th scores are exactly equal)."""
    gi = gidx.reshape(-1, K)
    rows = np.arange(gi.shape[0])
    sc = all_scores(Q, ksum, ent, S, rows, q_pos0, group_hkv)
    if group_hkv is None:
        oi, _, _ = oracle.score_topk(Q, ksum, ent, S, K, q_pos0=q_pos0)
    else:
        oi, _, _ = oracle.score_topk(Q, ksum, ent, S, K, q_pos0=q_pos0, group_hkv=group_hkv)
    oi = oi.reshape(-1, K)
    n_clean = n_tie = 0
    for n in rows:
        s = sc[n]
        cand = np.isfinite(s)
        if cand.sum() <= K:
            assert np.array_equal(gi[n], oi[n]), (n, gi[n], oi[n])
            continue
        vals = np.sort(s[cand])[::-1]
        sk = vals[K - 1]
        others = vals[vals != sk]
        if others.size and np.min(np.abs(others - sk)) < NEAR_TIE:
            continue
        n_clean += 1
        n_tie += int(vals[K] == sk)
        assert np.array_equal(gi[n], oi[n]), (n, gi[n], oi[n], sk)
    return n_clean, n_tie


PREFILL = {
    "bf16_k8": synth.small("tie_bf16_k8", B=1, T=2048, H=2, Hkv=1, d=64, K=8, dtype="bf16"),
    "bf16_k16": synth.small("tie_bf16_k16", B=1, T=4096, H=2, Hkv=1, d=64, K=16, dtype="bf16"),
    "bf16_k32": synth.small("tie_bf16_k32", B=1, T=4096, H=2, Hkv=1, d=64, K=32, dtype="bf16"),
    "bf16_k40": synth.small("tie_bf16_k40", B=1, T=4096, H=1, Hkv=1, d=64, K=40, dtype="bf16"),
    "bf16_d128_k16": synth.small("tie_bf16_d128", B=1, T=2048, H=4, Hkv=2, d=128, K=16,
                                 dtype="bf16"),
    "f32_k8": synth.small("tie_f32_k8", B=1, T=2048, H=2, Hkv=1, d=64, K=8, dtype="f32"),
    "f32_k20": synth.small("tie_f32_k20", B=1, T=2048, H=2, Hkv=1, d=64, K=20, dtype="f32"),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_exact_ties_prefill(name):
    w = PREFILL[name]
    x = tied_inputs(w)
    say(f"[ties prefill] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "Ql")}
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    idx, _ = hsa.score_topk(t["Q"], ksum, ent, w.K, w.S, Hkv=w.Hkv)
    torch.cuda.synchronize()
    oks, oent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    n_clean, n_tie = check_ties(host(idx), x["Q"], oks, oent, w.S, w.K)
    say(f"  clean rows {n_clean}, ties at the K-th place {n_tie}")
    assert n_tie > 100


GROUP = {
    "bf16_g2_k8": synth.small("tie_grp_g2", B=1, T=2048, H=4, Hkv=2, d=64, K=8, dtype="bf16"),
    "bf16_d128_g4_k16": synth.small("tie_grp_g4", B=1, T=2048, H=8, Hkv=2, d=128, K=16,
                                    dtype="bf16"),
    "f32_g2_k8": synth.small("tie_grp_f32", B=1, T=2048, H=4, Hkv=2, d=64, K=8, dtype="f32"),
}


@pytest.mark.parametrize("name", list(GROUP))
def test_exact_ties_group_max(name):
    w = GROUP[name]
    x = tied_inputs(w)
    say(f"[ties group-max] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "Ql")}
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    idx, _ = hsa.score_topk(t["Q"], ksum, ent, w.K, w.S, Hkv=w.Hkv, group=True)
    torch.cuda.synchronize()
    oks, oent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    n_clean, n_tie = check_ties(host(idx), x["Q"], oks, oent, w.S, w.K, group_hkv=w.Hkv)
    say(f"  clean rows {n_clean}, ties at the K-th place {n_tie}")
    assert n_tie > 100


# decode: the query rows sit at the end of the cache (q_pos0 = T - Tq); candidate
# splits of 128 and a merge whose kind follows the list count
DECODE = {
    # 128 splits x 16 entries: rank merge
    "bf16_rank_k16": (synth.small("tie_dec_rank", B=1, T=16384, H=2, Hkv=1, d=64, K=16,
                                  dtype="bf16", Tq=8, q_pos0=16384 - 8), 8),
    # 17 lists of 64 entries: wavefront merge
    "bf16_wave_k64": (synth.small("tie_dec_wave", B=1, T=2112 * 64, H=1, Hkv=1, d=64, K=64,
                                  dtype="bf16", Tq=4, q_pos0=2112 * 64 - 4), 4),
    # 65 lists: the workgroup merge
    "bf16_wg_k16": (synth.small("tie_dec_wg", B=1, T=8256 * 64, H=1, Hkv=1, d=64, K=16,
                                dtype="bf16", Tq=4, q_pos0=8256 * 64 - 4), 4),
    "f32_rank_k16": (synth.small("tie_dec_f32", B=1, T=16384, H=2, Hkv=1, d=64, K=16,
                                 dtype="f32", Tq=8, q_pos0=16384 - 8), 8),
    # 128 positions x 2 heads = 256 rows
    "bf16_rowwg_k16": (synth.small("tie_dec_row", B=1, T=8192, H=2, Hkv=1, d=64, K=16,
                                   dtype="bf16", Tq=128, q_pos0=8192 - 128), 128),
}


@pytest.mark.parametrize("name", list(DECODE))
def test_exact_ties_decode(name):
    w, nq = DECODE[name]
    x = tied_inputs(w)
    say(f"[ties decode] {name}: cache {w.T}, {nq} query positions")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    idx, sc = hsa.score_topk(t["Q"], ksum, ent, w.K, w.S, q_pos0=w.q_pos0, Tkv=w.T, Hkv=w.Hkv)
    # hils_decode (with fewer than 256 rows its slot kernel merges the split lists
    # itself) selects the same chunks
    ws = hsa.decode_workspace(t["Q"], t["K"], ksum, w.K, w.S, w.q_pos0, w.T)
    got = hsa.decode(t["Q"], t["K"], t["V"], ksum, ent, w.K, w.S, q_pos0=w.q_pos0, Tkv=w.T, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(got[0], idx) and torch.equal(got[1], sc)
    oks, oent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    n_clean, n_tie = check_ties(host(idx), x["Q"], oks, oent, w.S, w.K, q_pos0=w.q_pos0)
    say(f"  clean rows {n_clean}, ties at the K-th place {n_tie}")
    assert n_tie >= max(1, n_clean // 2)


# ------------------------------------------------------------------ selection lists
def messy(idx, score, ncand_of_row, seed):
    """Selection lists with entries that do not count: per row one of a repeated id,
    two entries swapped (the later, smaller one no longer counts), an id beyond the
    candidates, a negative id other than -1, or the list unchanged."""
    rng = np.random.default_rng(seed)
    idx, score = idx.copy(), score.copy()
    fi, fs = idx.reshape(-1, idx.shape[-1]), score.reshape(-1, idx.shape[-1])
    K = fi.shape[1]
    for r in range(fi.shape[0]):
        nv = int((fi[r] >= 0).sum())
        kind = rng.integers(0, 5)
        if nv < 2 or kind == 0:
            continue
        k = int(rng.integers(0, nv - 1))
        if kind == 1:
            fi[r, k + 1], fs[r, k + 1] = fi[r, k], fs[r, k]
        elif kind == 2:
            fi[r, [k, k + 1]] = fi[r, [k + 1, k]]
            fs[r, [k, k + 1]] = fs[r, [k + 1, k]]
        elif kind == 3:
            fi[r, k] = ncand_of_row(r) + int(rng.integers(0, 3)) if rng.integers(0, 2) else 1 << 20
        else:
            fi[r, k] = -5
    return idx, score


LISTS = {
    "bf16_d64_g2": (synth.small("list_bf16", B=1, T=1024, H=4, Hkv=2, d=64, K=5, dtype="bf16",
                                need_dO=True), 0),
    "bf16_d128": (synth.small("list_d128", B=1, T=768, H=4, Hkv=1, d=128, K=4, dtype="bf16",
                              need_dO=True), 0),
    "f32": (synth.small("list_f32", B=1, T=640, H=2, Hkv=1, d=64, K=4, dtype="f32",
                        need_dO=True), 0),
    "bf16_window": (synth.small("list_win", B=1, T=1024, H=2, Hkv=1, d=64, K=6, dtype="bf16",
                                need_dO=True), 128),
}


@pytest.mark.parametrize("name", list(LISTS))
def test_selection_lists_with_entries_that_do_not_count(name):
    w, W = LISTS[name]
    x = synth.make_inputs(w)
    say(f"[selection lists] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql", "dO")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, window=W)
    torch.cuda.synchronize()

    def ncand(r):
        pos = (r // w.H) % w.T
        lstart = max(0, pos - W + 1) if W else pos - pos % w.S
        return lstart // w.S

    idx_m, sc_m = messy(host(f["idx"]), host(f["score"]), ncand, 5)
    ti, ts = torch.from_numpy(idx_m).to(DEV), torch.from_numpy(sc_m).to(DEV)
    O, lo, lt = hsa.attend_fuse(t["Q"], t["K"], t["V"], ti, ts, w.S, window=W)
    g = hsa.backward(t["Q"], t["K"], t["V"], t["Ql"], f["ksum"], f["ent"], f["lse_l"], ti, ts, lt,
                     O, t["dO"], w.S, window=W)
    torch.cuda.synchronize()
    oO, olo, olt = oracle.attend_fuse(x["Q"], x["K"], x["V"], idx_m, sc_m.astype(np.float64),
                                      w.S, window=W)
    tol = TOL_BF16 if w.dtype == "bf16" else TOL_F32
    assert_close(host(O), oO, tol, "O")
    assert_close(host(lo), olo, TOL_F32, "lse_own")
    assert_close(host(lt), olt, TOL_F32, "lse_tot")
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], idx_m, x["dO"], w.S, window=W)
    gtol = TOL_GRAD_BF16 if w.dtype == "bf16" else TOL_F32
    for nm, a, b in zip(("dQ", "dK", "dV", "dQl"), g, og):
        assert_close(host(a), b, gtol, nm)
    # decode rows take the same lists
    for p in (w.T - 1, w.T // 2 + 3):
        q = t["Q"][:, p:p + 1].contiguous()
        Od, _, ltd = hsa.attend_fuse(q, t["K"], t["V"], ti[:, p:p + 1].contiguous(),
                                     ts[:, p:p + 1].contiguous(), w.S, q_pos0=p, Tkv=p + 1,
                                     window=W)
        torch.cuda.synchronize()
        assert_close(host(Od)[:, 0], oO[:, p], tol, f"decode O {p}")
        assert_close(host(ltd)[:, 0], olt[:, p], TOL_F32, f"decode lse_tot {p}")


# ------------------------------------------------------------------ value range
@pytest.mark.parametrize("name,d", [("range_d64", 64), ("range_d128", 128)])
def test_large_values_in_one_chunk(name, d):
    """V of one chunk scaled by 2^14 (exact in bf16): rows that read it match the
    oracle, and so, at the output tolerance of their own magnitude, do the rows
    that share its workgroups but never read it."""
    w = synth.small(name, B=1, T=2048, H=4, Hkv=2, d=d, K=6, dtype="bf16")
    x = synth.make_inputs(w)
    say(f"[value range] {name}")
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    cstar, g = 5, 0
    V = x["V"].copy()
    V[:, cstar * w.S:(cstar + 1) * w.S, g] *= 16384.0
    O_ref, lo_ref, lt_ref = oracle.attend_fuse(x["Q"], x["K"], V, o["idx"], o["score"], w.S)
    t = {k: dev(v, w.dtype) for k, v in (("Q", x["Q"]), ("K", x["K"]), ("V", V))}
    idx = torch.from_numpy(o["idx"]).to(DEV)
    score = torch.from_numpy(o["score"].astype(np.float32)).to(DEV)
    O, lo, lt = hsa.attend_fuse(t["Q"], t["K"], t["V"], idx, score, w.S)
    torch.cuda.synchronize()
    G = w.H // w.Hkv
    heads = np.arange(w.H) // G == g
    pos = np.arange(w.T)
    reads = np.any(o["idx"] == cstar, axis=-1) | (pos // w.S == cstar)[None, :, None]
    reads &= heads[None, None, :]
    quiet = ~reads
    say(f"  rows reading the chunk {int(reads.sum())}, others {int(quiet.sum())}")
    assert reads.sum() > 0
    Og = host(O)
    assert_close(Og[reads], O_ref[reads], TOL_BF16, "O (rows reading the chunk)")
    assert_close(Og[quiet], O_ref[quiet], TOL_BF16, "O (other rows)")
    assert_close(host(lt), lt_ref, TOL_F32, "lse_tot")
