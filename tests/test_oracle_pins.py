"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test ties the oracle to something other than itself: closed forms stated
on the pages (entropy limits, mean pooling), identities that follow from the
first-order expansion (exact at the expansion point, tangent-plane lower
bound), torch's dense causal attention (the hierarchical factorisation with
exact chunk masses and every chunk selected is full attention), a brute-force
sort for the top-K rule, and autograd / finite differences for the backward.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "entropy_limits.json")))


def normals(shape, seed, stream=1):
    return synth.normal(seed, stream, int(np.prod(shape))).reshape(shape)


def all_scores(Q, ksum, ent, S, q_pos0=0):
    """Every candidate score, by asking the oracle for K >= NC (all candidates kept)."""
    NC = ksum.shape[1]
    idx, score, _ = oracle.score_topk(Q, ksum, ent, S, NC, q_pos0)
    return idx, score


def dense_causal(Q, K, V, q_pos0=0, keep=None):
    """torch fp64 scaled-dot-product attention, causal over absolute positions;
    keep [Tq, Tkv] (bool), when given, further restricts the keys each row sees."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    B, Tq, H, d = Q.shape
    Tkv, Hkv = K.shape[1], K.shape[2]
    G = H // Hkv
    q = torch.from_numpy(np.ascontiguousarray(Q.transpose(0, 2, 1, 3)))
    k = torch.from_numpy(np.ascontiguousarray(np.repeat(K, G, axis=2).transpose(0, 2, 1, 3)))
    v = torch.from_numpy(np.ascontiguousarray(np.repeat(V, G, axis=2).transpose(0, 2, 1, 3)))
    pos = q_pos0 + np.arange(Tq)[:, None]
    m = np.arange(Tkv)[None, :] <= pos
    mask = torch.from_numpy(m if keep is None else m & keep)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    logits = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


# ---------------------------------------------------------------- summaries
@pytest.mark.parametrize("S", [16, 64])
def test_entropy_uniform_and_one_hot(S):
    """Page 2 §5.1: b' -> log S for uniform landmark logits, -> 0 for one dominant token."""
    d, H, Hkv = 16, 2, 1
    K = normals((1, 3 * S, Hkv, d), 11)
    Ql = normals((1, 3, H, d), 12)
    a = normals((d,), 13)
    K[0, 0:S, 0, :] = a                       # chunk 0: identical keys
    Ql[0, 1] = 0.0                            # chunk 1: zero landmark query
    jstar = 5                                 # chunk 2: one key dominates by a logit of 40
    K[0, 2 * S:3 * S, 0, :] *= 1e-3
    ql = Ql[0, 2, 0]
    K[0, 2 * S + jstar, 0, :] = 40.0 * math.sqrt(d) * ql / (ql @ ql)
    Ql[0, 2, 1] = Ql[0, 2, 0]
    ksum, ent, lse = oracle.summarize(K, Ql, S)
    logS = GOLD["uniform"][str(S)]
    for h in range(H):
        assert ent[0, 0, h] == pytest.approx(logS, abs=1e-12)
        np.testing.assert_allclose(ksum[0, 0, h], a, rtol=0, atol=1e-12)
        assert lse[0, 0, h] == pytest.approx((Ql[0, 0, h] @ a) / math.sqrt(d) + logS, abs=1e-12)
        assert ent[0, 1, h] == pytest.approx(logS, abs=1e-12)
        np.testing.assert_allclose(ksum[0, 1, h], K[0, S:2 * S, 0].mean(0), rtol=0, atol=1e-12)
        assert 0.0 <= ent[0, 2, h] < GOLD["one_hot_max"]
        np.testing.assert_allclose(ksum[0, 2, h], K[0, 2 * S + jstar, 0], rtol=1e-12, atol=1e-12)


def test_entropy_between_limits():
    """Entropy of a distribution over S outcomes lies in [0, log S] (page 2 §5.1 limits)."""
    w = synth.workloads()["tiny_f32"]
    x = synth.make_inputs(w)
    _, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    assert np.all(ent >= 0) and np.all(ent <= math.log(w.S) + 1e-12)


# ---------------------------------------------------------------- scores
def _small(seed, T=256, S=16, H=2, Hkv=1, d=16):
    return normals((1, T, H, d), seed), normals((1, T, Hkv, d), seed + 1), \
        normals((1, T, Hkv, d), seed + 2), normals((1, T // S, H, d), seed + 3)


def test_score_exact_at_expansion_point():
    """First-order expansion at q'_c (page 2 §5.1): at q = q'_c the score equals log Z exactly."""
    S = 16
    Q, K, V, Ql = _small(21, S=S)
    pairs = [(100, 3, 0), (200, 0, 1), (255, 14, 0), (40, 1, 1)]   # (row i, chunk c, head h)
    for i, c, h in pairs:
        Q[0, i, h] = Ql[0, c, h]
    ksum, ent, _ = oracle.summarize(K, Ql, S)
    idx, sc = all_scores(Q, ksum, ent, S)
    lz = oracle.exact_chunk_lse(Q, K, S, K.shape[1] // S)
    for i, c, h in pairs:
        assert idx[0, i, h, c] == c
        assert sc[0, i, h, c] == pytest.approx(lz[0, i, h, c], rel=1e-13, abs=1e-13)


def test_score_tangent_plane_lower_bound():
    """log Z is convex in q and the score is its tangent plane at q'_c, so score <= log Z."""
    w = synth.workloads()["tiny_f32"]
    x = synth.make_inputs(w)
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    idx, sc = all_scores(x["Q"], ksum, ent, w.S)
    lz = oracle.exact_chunk_lse(x["Q"], x["K"], w.S, w.NC)
    valid = idx >= 0
    c = np.where(valid, idx, 0)
    lz_sel = np.take_along_axis(lz, c, axis=-1)
    assert valid.sum() == sum(min(i // w.S, w.NC) for i in range(w.T)) * w.H
    assert np.all(sc[valid] <= lz_sel[valid] + 1e-10)


def test_score_identical_key_chunk_is_exact():
    """All keys of a chunk equal: log Z = q.a/sqrt d + log S = score for every q."""
    S = 16
    Q, K, V, Ql = _small(31, S=S)
    a = normals((16,), 35)
    K[0, 3 * S:4 * S, 0, :] = a
    ksum, ent, _ = oracle.summarize(K, Ql, S)
    idx, sc = all_scores(Q, ksum, ent, S)
    lz = oracle.exact_chunk_lse(Q, K, S, K.shape[1] // S)
    rows = np.arange(4 * S, K.shape[1])
    np.testing.assert_allclose(sc[0, rows, :, 3], lz[0, rows, :, 3], rtol=1e-13, atol=1e-13)


def test_score_zero_landmark_is_mean_pooling():
    """q' = 0: uniform landmark weights, score = q.mean(k)/sqrt d + log S (page 2 §3)."""
    S, d = 16, 16
    Q, K, V, Ql = _small(41, S=S)
    Ql[:] = 0.0
    ksum, ent, _ = oracle.summarize(K, Ql, S)
    idx, sc = all_scores(Q, ksum, ent, S)
    NC = K.shape[1] // S
    kmean = K[0, :, 0, :].reshape(NC, S, d).mean(1)
    for i in (17, 100, 255):
        for h in range(2):
            want = Q[0, i, h] @ kmean[: i // S].T / math.sqrt(d) + math.log(S)
            np.testing.assert_allclose(sc[0, i, h, : i // S], want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- top-K
def test_topk_brute_force_sort():
    """I_i = chunks of rank < K by score, ties to the lower id (page 2 §5.2), by full sort."""
    w = synth.workloads()["tiny_f32"]
    x = synth.make_inputs(w)
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    idx_all, sc_all = all_scores(x["Q"], ksum, ent, w.S)
    idx, score, gap = oracle.score_topk(x["Q"], ksum, ent, w.S, w.K)
    for i in range(w.T):
        n = i // w.S
        for h in range(w.H):
            cand = sorted(range(n), key=lambda c: (-sc_all[0, i, h, c], c))
            take = sorted(cand[: w.K])
            want = take + [-1] * (w.K - len(take))
            assert list(idx[0, i, h]) == want
            np.testing.assert_array_equal(score[0, i, h, : len(take)], sc_all[0, i, h, take])
            assert np.all(np.isneginf(score[0, i, h, len(take):]))
            if n > w.K:
                assert gap[0, i, h] == sc_all[0, i, h, cand[w.K - 1]] - sc_all[0, i, h, cand[w.K]]
            else:
                assert np.isinf(gap[0, i, h])


def test_topk_exact_tie_goes_to_lower_chunk():
    S, d = 16, 16
    Q, K, V, Ql = _small(51, T=96, S=S, H=1)
    a = normals((d,), 55)
    base = K[0, S:2 * S, 0, :] + 3.0 * a
    for c in (1, 3):                       # chunks 1 and 3 identical, strongly aligned with q
        K[0, c * S:(c + 1) * S, 0, :] = base
        Ql[0, c, 0] = Ql[0, 1, 0]
    Q[0, 5 * S:, 0, :] = 3.0 * a
    ksum, ent, _ = oracle.summarize(K, Ql, S)
    idx_all, sc_all = all_scores(Q, ksum, ent, S)
    row = 5 * S + 7
    assert sc_all[0, row, 0, 1] == sc_all[0, row, 0, 3]
    assert sc_all[0, row, 0, 1] == sc_all[0, row, 0, :5].max()
    idx, score, gap = oracle.score_topk(Q, ksum, ent, S, 1)
    assert idx[0, row, 0, 0] == 1 and gap[0, row, 0] == 0.0


# ---------------------------------------------------------------- GQA group-max top-K
def _gqa_case(seed, T=512, S=16, H=8, Hkv=2, d=16):
    Q, K, V, Ql = _small(seed, T=T, S=S, H=H, Hkv=Hkv, d=d)
    ksum, ent, _ = oracle.summarize(K, Ql, S)
    return Q, ksum, ent, S


def test_group_topk_brute_force():
    """Group-max selection (page 2 §5.4): per kv head, the top-K of the maximum over the
    group's query-head scores (ties to the lower id) is every head's index set, and
    each head keeps its own score; checked by a full sort of the aggregated scores."""
    Q, ksum, ent, S = _gqa_case(61)
    B, T, H, d = Q.shape
    Hkv, G, Ksel = 2, 4, 5
    idx_all, sc_all = all_scores(Q, ksum, ent, S)
    idx, score, gap = oracle.score_topk(Q, ksum, ent, S, Ksel, group_hkv=Hkv)
    for i in range(0, T, 7):
        n = i // S
        for g in range(Hkv):
            heads = range(g * G, g * G + G)
            agg = [max(sc_all[0, i, h, c] for h in heads) for c in range(n)]
            cand = sorted(range(n), key=lambda c: (-agg[c], c))
            take = sorted(cand[:Ksel])
            want = take + [-1] * (Ksel - len(take))
            for h in heads:
                assert list(idx[0, i, h]) == want
                np.testing.assert_array_equal(score[0, i, h, : len(take)], sc_all[0, i, h, take])
                assert np.all(np.isneginf(score[0, i, h, len(take):]))
                if n > Ksel:
                    assert gap[0, i, h] == agg[cand[Ksel - 1]] - agg[cand[Ksel]]


def test_group_topk_one_head_per_group_is_per_head_selection():
    """G = 1: the group maximum is the head's own score, so both modes agree exactly."""
    Q, ksum, ent, S = _gqa_case(71, H=2, Hkv=2)
    a = oracle.score_topk(Q, ksum, ent, S, 4)
    b = oracle.score_topk(Q, ksum, ent, S, 4, group_hkv=2)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_group_topk_identical_heads():
    """Heads of a group with the same query and landmark queries have equal scores, so
    the group selection is each head's own selection."""
    S, d, H, Hkv = 16, 16, 4, 2
    Q, K, V, Ql = _small(81, T=384, S=S, H=H, Hkv=Hkv, d=d)
    for g in range(Hkv):
        for h in range(g * 2 + 1, g * 2 + 2):
            Q[:, :, h] = Q[:, :, g * 2]
            Ql[:, :, h] = Ql[:, :, g * 2]
    ksum, ent, _ = oracle.summarize(K, Ql, S)
    a = oracle.score_topk(Q, ksum, ent, S, 3)
    b = oracle.score_topk(Q, ksum, ent, S, 3, group_hkv=Hkv)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------- attend + fuse
@pytest.mark.parametrize("H,Hkv", [(2, 1), (4, 2)])
def test_full_attention_equivalence(H, Hkv):
    """Exact chunk masses as scores and every candidate selected: the hierarchical
    weights reduce to full causal attention (page 4 Fig. 3, 'equivalent when Z'_c = Z_c')."""
    S, d, T = 32, 32, 512
    Q = normals((1, T, H, d), 61)
    K = normals((1, T, Hkv, d), 62)
    V = normals((1, T, Hkv, d), 63)
    NC = T // S
    lz = oracle.exact_chunk_lse(Q, K, S, NC)
    idx = np.full((1, T, H, NC), -1, dtype=np.int32)
    score = np.full((1, T, H, NC), -np.inf)
    for i in range(T):
        n = i // S
        idx[0, i, :, :n] = np.arange(n)
        score[0, i, :, :n] = lz[0, i, :, :n]
    O, lo, lt = oracle.attend_fuse(Q, K, V, idx, score, S)
    Od, lse = dense_causal(Q, K, V)
    np.testing.assert_allclose(O, Od, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(lt, lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [64, 96, 128])
def test_window_full_attention_equivalence(W):
    """Sliding-window local branch (page 2 §5.2: SWA with chunk selection): with exact
    chunk masses as scores and every candidate selected, each row attends exactly to
    the chunks wholly before its window plus the window's keys, as one softmax."""
    S, d, T, H, Hkv = 32, 32, 512, 2, 1
    Q = normals((1, T, H, d), 81)
    K = normals((1, T, Hkv, d), 82)
    V = normals((1, T, Hkv, d), 83)
    NC = T // S
    lz = oracle.exact_chunk_lse(Q, K, S, NC, window=W)
    idx = np.full((1, T, H, NC), -1, dtype=np.int32)
    score = np.full((1, T, H, NC), -np.inf)
    keep = np.zeros((T, T), dtype=bool)
    for i in range(T):
        first = max(0, i - W + 1)              # the window: the last W keys
        n = first // S                          # chunks ending before the window
        assert np.all(np.isinf(lz[0, i, :, n:])) and np.all(np.isfinite(lz[0, i, :, :n]))
        idx[0, i, :, :n] = np.arange(n)
        score[0, i, :, :n] = lz[0, i, :, :n]
        keep[i, :n * S] = True
        keep[i, first:i + 1] = True
    O, lo, lt = oracle.attend_fuse(Q, K, V, idx, score, S, window=W)
    Od, lse = dense_causal(Q, K, V, keep=keep)
    np.testing.assert_allclose(O, Od, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(lt, lse, rtol=1e-12, atol=1e-12)
    # the window's own log-mass is the dense LSE over the window alone
    wonly = np.zeros((T, T), dtype=bool)
    for i in range(T):
        wonly[i, max(0, i - W + 1):i + 1] = True
    np.testing.assert_allclose(lo, dense_causal(Q, K, V, keep=wonly)[1], rtol=1e-12, atol=1e-12)


def test_window_covering_the_prefix_is_causal_attention():
    """A window at least as long as the sequence leaves no candidate chunk: every row
    is plain causal attention, whatever K."""
    w = synth.small("wfull", T=384, H=2, Hkv=1, d=32, S=64, K=3)
    x = synth.make_inputs(w)
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, window=512)
    Od, lse = dense_causal(x["Q"], x["K"], x["V"])
    np.testing.assert_allclose(f["O"], Od, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f["lse_tot"], lse, rtol=1e-12, atol=1e-12)
    assert np.all(f["idx"] == -1)


def test_window_candidates_lie_wholly_before_the_window():
    """With W = 2S the candidate chunks are exactly those whose last key precedes the
    window's first key: a chunk the window cuts is never scored."""
    w = synth.small("wcand", T=640, H=2, Hkv=1, d=32, S=64, K=20)
    x = synth.make_inputs(w)
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    idx, score, _ = oracle.score_topk(x["Q"], ksum, ent, w.S, w.NC, window=128)
    for i in (0, 126, 127, 128, 190, 191, 192, 255, 256, 639):
        first = max(0, i - 127)
        got = set(int(c) for c in idx[0, i, 0] if c >= 0)
        want = {c for c in range(w.NC) if (c + 1) * w.S - 1 < first}
        assert got == want, (i, sorted(got))


def test_first_chunk_rows_are_causal_attention():
    """Rows in chunk 0 have no candidates: plain causal attention over positions <= i."""
    w = synth.small("c0", T=256, H=2, Hkv=1, d=32, S=64, K=2)
    x = synth.make_inputs(w)
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    Od, lse = dense_causal(x["Q"][:, :64], x["K"][:, :64], x["V"][:, :64])
    np.testing.assert_allclose(f["O"][:, :64], Od, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f["lse_own"][:, :64], lse, rtol=1e-12, atol=1e-12)
    assert np.all(f["idx"][:, :64] == -1)


def test_partition_of_unity():
    """The fused weights sum to one: V constant => O equals that constant (page 2 §5.3)."""
    w = synth.small("pu", T=512, H=4, Hkv=2, d=32, S=32, K=3)
    x = synth.make_inputs(w)
    c = normals((32,), 71)
    V = np.broadcast_to(c, x["V"].shape).copy()
    f = oracle.forward(x["Q"], x["K"], V, x["Ql"], w.S, w.K)
    np.testing.assert_allclose(f["O"], np.broadcast_to(c, f["O"].shape), rtol=1e-12, atol=1e-12)


def test_decode_equals_prefill_row():
    """A decode query at position p over a cache of p+1 tokens equals prefill row p."""
    w = synth.small("dec", T=1024, H=2, Hkv=1, d=32, S=64, K=4)
    x = synth.make_inputs(w)
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    for p in (63, 64, 700, 767, 1000, 1023):
        nc = (p + 1) // w.S
        Kc, Vc = x["K"][:, : p + 1], x["V"][:, : p + 1]
        ksum, ent, _ = oracle.summarize(Kc, x["Ql"][:, :nc], w.S)
        q = x["Q"][:, p:p + 1]
        idx, score, _ = oracle.score_topk(q, ksum, ent, w.S, w.K, q_pos0=p)
        O, lo, lt = oracle.attend_fuse(q, Kc, Vc, idx, score, w.S, q_pos0=p)
        np.testing.assert_array_equal(idx[:, 0], f["idx"][:, p])
        np.testing.assert_allclose(O[:, 0], f["O"][:, p], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lt[:, 0], f["lse_tot"][:, p], rtol=1e-13)


# ---------------------------------------------------------------- backward
def torch_hils(Q, K, V, Ql, idx, S, Qs=None, window=0):
    """Dense, differentiable restatement of the forward with fixed idx (torch fp64);
    Qs, when given, is the scoring query of the chunk scores (Q-Cal); window > 0
    makes the local branch the last `window` keys instead of the own chunk."""
    B, T, H, d = Q.shape
    Hkv = K.shape[2]
    G, NC, tau = H // Hkv, Ql.shape[1], 1.0 / math.sqrt(d)
    Kh = K.repeat_interleave(G, dim=2)
    Vh = V.repeat_interleave(G, dim=2)
    Kc = Kh[:, : NC * S].reshape(B, NC, S, H, d)
    lp = torch.log_softmax(tau * torch.einsum("bchd,bcshd->bchs", Ql, Kc), dim=-1)
    p = lp.exp()
    ksum = torch.einsum("bchs,bcshd->bchd", p, Kc)
    ent = -(p * lp).sum(-1)
    out = []
    for b in range(B):
        for i in range(T):
            for h in range(H):
                q = Q[b, i, h]
                qs = q if Qs is None else Qs[b, i, h]
                logits, outs = [], []
                for c in [int(c) for c in idx[b, i, h] if c >= 0]:
                    logits.append(tau * (ksum[b, c, h] @ qs) + ent[b, c, h])
                    s = tau * (Kh[b, c * S:(c + 1) * S, h] @ q)
                    outs.append(torch.softmax(s, 0) @ Vh[b, c * S:(c + 1) * S, h])
                own = (i // S) * S if window == 0 else max(0, i - window + 1)
                s = tau * (Kh[b, own:i + 1, h] @ q)
                logits.append(torch.logsumexp(s, 0))
                outs.append(torch.softmax(s, 0) @ Vh[b, own:i + 1, h])
                a = torch.softmax(torch.stack(logits), 0)
                out.append((a[:, None] * torch.stack(outs)).sum(0))
    return torch.stack(out).reshape(B, T, H, d)


def _bwd_case():
    w = synth.small("bwd", B=1, T=256, H=4, Hkv=2, d=16, S=16, K=3, n_planted=1, need_dO=True)
    x = synth.make_inputs(w)
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    return w, x, f


def test_backward_matches_autograd():
    w, x, f = _bwd_case()
    dQ, dK, dV, dQl = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S)
    t = {k: torch.from_numpy(x[k].astype(np.float64)).requires_grad_(True)
         for k in ("Q", "K", "V", "Ql")}
    O = torch_hils(t["Q"], t["K"], t["V"], t["Ql"], f["idx"], w.S)
    np.testing.assert_allclose(O.detach().numpy(), f["O"], rtol=1e-11, atol=1e-12)
    (O * torch.from_numpy(x["dO"].astype(np.float64))).sum().backward()
    for name, g in (("Q", dQ), ("K", dK), ("V", dV), ("Ql", dQl)):
        np.testing.assert_allclose(g, t[name].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def test_backward_finite_differences():
    """Central differences of the oracle's own forward (selection unchanged) match its backward."""
    w, x, f = _bwd_case()
    assert np.nanmin(f["gap"]) > 1e-4
    dQ, dK, dV, dQl = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S)
    grads = {"Q": dQ, "K": dK, "V": dV, "Ql": dQl}
    base = {k: x[k].astype(np.float64) for k in ("Q", "K", "V", "Ql")}
    dO = x["dO"].astype(np.float64)
    rng = np.random.default_rng(5)
    h = 1e-6
    for name in ("Q", "K", "V", "Ql"):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in base[name].shape)
            vals = []
            for sgn in (1, -1):
                arrs = {k: v.copy() for k, v in base.items()}
                arrs[name][pos] += sgn * h
                g = oracle.forward(arrs["Q"], arrs["K"], arrs["V"], arrs["Ql"], w.S, w.K)
                assert np.array_equal(g["idx"], f["idx"])
                vals.append(np.sum(g["O"] * dO))
            fd = (vals[0] - vals[1]) / (2 * h)
            assert fd == pytest.approx(grads[name][pos], rel=1e-5, abs=1e-7), (name, pos)


def _qcal_case():
    """Backward case with a Q-Cal scoring query: Qs = Q + a low-rank update of
    seeded hidden states (the caller's W_up W_down h of page 2 §5.4)."""
    w, x, _ = _bwd_case()
    rng = np.random.default_rng(11)
    hdim, rank = 24, 4
    hid = rng.standard_normal((w.B, w.T, hdim))
    Wd = rng.standard_normal((rank, hdim)) / np.sqrt(hdim)
    Wu = rng.standard_normal((w.H, w.d, rank)) / np.sqrt(rank)
    Qs = x["Q"].astype(np.float64) + np.einsum("hdr,rk,btk->bthd", Wu, Wd, hid)
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, Qs=Qs)
    return w, x, Qs, f


def test_qcal_backward_matches_autograd():
    w, x, Qs, f = _qcal_case()
    dQ, dK, dV, dQl, dQs = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"],
                                           w.S, Qs=Qs)
    t = {k: torch.from_numpy(x[k].astype(np.float64)).requires_grad_(True)
         for k in ("Q", "K", "V", "Ql")}
    t["Qs"] = torch.from_numpy(Qs).requires_grad_(True)
    O = torch_hils(t["Q"], t["K"], t["V"], t["Ql"], f["idx"], w.S, Qs=t["Qs"])
    np.testing.assert_allclose(O.detach().numpy(), f["O"], rtol=1e-11, atol=1e-12)
    (O * torch.from_numpy(x["dO"].astype(np.float64))).sum().backward()
    for name, g in (("Q", dQ), ("Qs", dQs), ("K", dK), ("V", dV), ("Ql", dQl)):
        np.testing.assert_allclose(g, t[name].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def test_qcal_backward_finite_differences():
    """Central differences in the scoring query and the token query (selection unchanged)."""
    w, x, Qs, f = _qcal_case()
    assert np.nanmin(f["gap"]) > 1e-5   # a step of 1e-6 moves a score by far less
    dQ, _, _, _, dQs = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S,
                                       Qs=Qs)
    dO = x["dO"].astype(np.float64)
    Q0 = x["Q"].astype(np.float64)
    rng = np.random.default_rng(6)
    h = 1e-6
    for which, grad in (("Qs", dQs), ("Q", dQ)):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in Q0.shape)
            vals = []
            for sgn in (1, -1):
                q, qs = Q0.copy(), Qs.copy()
                (qs if which == "Qs" else q)[pos] += sgn * h
                g = oracle.forward(q, x["K"], x["V"], x["Ql"], w.S, w.K, Qs=qs)
                assert np.array_equal(g["idx"], f["idx"])
                vals.append(np.sum(g["O"] * dO))
            fd = (vals[0] - vals[1]) / (2 * h)
            assert fd == pytest.approx(grad[pos], rel=1e-5, abs=1e-7), (which, pos)


def test_qcal_with_token_query_splits_the_plain_gradient():
    """Qs = Q: the scoring and token parts add up to the plain query gradient and
    every other gradient is unchanged."""
    w, x, f = _bwd_case()
    plain = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S)
    split = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S, Qs=x["Q"])
    np.testing.assert_allclose(split[0] + split[4], plain[0], rtol=1e-12, atol=1e-13)
    assert np.abs(split[4]).max() > 1e-3 * np.abs(plain[0]).max()
    for a, b in zip(split[1:4], plain[1:4]):
        np.testing.assert_array_equal(a, b)


def test_window_backward_matches_autograd_and_differences():
    """Sliding-window local branch (W = 40 keys, S = 16): the backward equals autograd
    of the dense restatement and central differences of the oracle's own forward."""
    w = synth.small("bwdw", B=1, T=256, H=4, Hkv=2, d=16, S=16, K=3, n_planted=1,
                    need_dO=True)
    x = synth.make_inputs(w)
    W = 40
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, window=W)
    grads = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S, window=W)
    t = {k: torch.from_numpy(x[k].astype(np.float64)).requires_grad_(True)
         for k in ("Q", "K", "V", "Ql")}
    O = torch_hils(t["Q"], t["K"], t["V"], t["Ql"], f["idx"], w.S, window=W)
    np.testing.assert_allclose(O.detach().numpy(), f["O"], rtol=1e-11, atol=1e-12)
    (O * torch.from_numpy(x["dO"].astype(np.float64))).sum().backward()
    for name, g in zip(("Q", "K", "V", "Ql"), grads):
        np.testing.assert_allclose(g, t[name].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
    base = {k: x[k].astype(np.float64) for k in ("Q", "K", "V", "Ql")}
    dO = x["dO"].astype(np.float64)
    rng = np.random.default_rng(7)
    h = 1e-6
    for gi, name in enumerate(("Q", "K", "V", "Ql")):
        for _ in range(3):
            pos = tuple(rng.integers(0, sz) for sz in base[name].shape)
            vals = []
            for sgn in (1, -1):
                arrs = {k: v.copy() for k, v in base.items()}
                arrs[name][pos] += sgn * h
                g = oracle.forward(arrs["Q"], arrs["K"], arrs["V"], arrs["Ql"], w.S, w.K, window=W)
                assert np.array_equal(g["idx"], f["idx"])
                vals.append(np.sum(g["O"] * dO))
            fd = (vals[0] - vals[1]) / (2 * h)
            assert fd == pytest.approx(grads[gi][pos], rel=1e-5, abs=1e-7), (name, pos)


def test_window_decode_equals_prefill_row():
    """Decode with a sliding window: position p over a cache of p+1 keys = prefill row p."""
    w = synth.small("decw", T=1024, H=2, Hkv=1, d=32, S=64, K=4)
    x = synth.make_inputs(w)
    W = 256
    f = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, window=W)
    for p in (63, 255, 256, 319, 320, 700, 1023):
        nc = (p + 1) // w.S
        Kc, Vc = x["K"][:, : p + 1], x["V"][:, : p + 1]
        ksum, ent, _ = oracle.summarize(Kc, x["Ql"][:, :nc], w.S)
        q = x["Q"][:, p:p + 1]
        idx, score, _ = oracle.score_topk(q, ksum, ent, w.S, w.K, q_pos0=p, window=W)
        O, lo, lt = oracle.attend_fuse(q, Kc, Vc, idx, score, w.S, q_pos0=p, window=W)
        np.testing.assert_array_equal(idx[:, 0], f["idx"][:, p])
        np.testing.assert_allclose(O[:, 0], f["O"][:, p], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lt[:, 0], f["lse_tot"][:, p], rtol=1e-13)


def test_backward_masks_restrict_work():
    """Masked backward reproduces the full backward on the requested entries."""
    w, x, f = _bwd_case()
    full = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S)
    row_mask = np.zeros((1, w.T, w.H), np.uint8)
    row_mask[0, [3, 77, 255], :] = 1
    kv_mask = np.zeros((1, w.NC, w.Hkv), np.uint8)
    kv_mask[0, [2, 15], 1] = 1
    kv_mask[0, 9, 0] = 1
    part = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], f["idx"], x["dO"], w.S,
                           row_mask=row_mask, kv_mask=kv_mask)
    rm = row_mask.astype(bool)
    np.testing.assert_array_equal(part[0][rm], full[0][rm])
    for c, g in ((2, 1), (15, 1), (9, 0)):
        sl = slice(c * w.S, (c + 1) * w.S)
        np.testing.assert_allclose(part[1][0, sl, g], full[1][0, sl, g], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(part[2][0, sl, g], full[2][0, sl, g], rtol=1e-12, atol=1e-14)
        G = w.H // w.Hkv
        np.testing.assert_allclose(part[3][0, c, g * G:(g + 1) * G],
                                   full[3][0, c, g * G:(g + 1) * G], rtol=1e-12, atol=1e-14)


def test_selection_lists_count_only_ascending_candidates():
    """A selection list handed to the attention or the backward counts entry k only
    when its id is a candidate of the row and above every earlier entry; the others
    (a repeated id, an out-of-order id, an id past the candidates, a negative id)
    contribute nothing. Pinned against the same lists with those entries replaced by
    padding: the oracle's forward, and the dense autograd restatement for the
    gradients."""
    w, x, f = _bwd_case()
    rng = np.random.default_rng(3)
    idx = f["idx"].copy()
    score = f["score"].copy()
    fi, fs = idx.reshape(-1, w.K), score.reshape(-1, w.K)
    H = w.H
    ncand = ((np.arange(fi.shape[0]) // H) % w.T) // w.S
    for r in range(fi.shape[0]):
        nv = int((fi[r] >= 0).sum())
        if nv < 2:
            continue
        kind = r % 5
        k = int(rng.integers(0, nv - 1))
        if kind == 1:
            fi[r, k + 1], fs[r, k + 1] = fi[r, k], fs[r, k]
        elif kind == 2:
            fi[r, [k, k + 1]] = fi[r, [k + 1, k]]
            fs[r, [k, k + 1]] = fs[r, [k + 1, k]]
        elif kind == 3:
            fi[r, k] = ncand[r]
        elif kind == 4:
            fi[r, k] = -3
    clean = idx.copy()
    fc = clean.reshape(-1, w.K)
    for r in range(fc.shape[0]):
        seen = -1
        for k in range(w.K):
            c = int(fi[r, k])
            if not (0 <= c < ncand[r] and c > seen):
                fc[r, k] = -1
            seen = max(seen, c)
    assert (clean != idx).any()
    O1, lo1, lt1 = oracle.attend_fuse(x["Q"], x["K"], x["V"], idx, score, w.S)
    sc_clean = np.where(clean >= 0, score, -np.inf)
    O2, lo2, lt2 = oracle.attend_fuse(x["Q"], x["K"], x["V"], clean, sc_clean, w.S)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(lt1, lt2)
    g = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], idx, x["dO"], w.S)
    t = {k: torch.from_numpy(x[k].astype(np.float64)).requires_grad_(True)
         for k in ("Q", "K", "V", "Ql")}
    O = torch_hils(t["Q"], t["K"], t["V"], t["Ql"], clean, w.S)
    (O * torch.from_numpy(x["dO"].astype(np.float64))).sum().backward()
    for name, gg in zip(("Q", "K", "V", "Ql"), g):
        np.testing.assert_allclose(gg, t[name].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
