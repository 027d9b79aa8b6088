"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Oracle inputs never come from the GPU: stage tests feed oracle outputs (e.g.
the oracle's selection) into the GPU kernels, never the reverse. Selection is
compared bit-exactly on rows whose oracle K-th/(K+1)-th score gap is at least
1e-4; excluded rows are counted. Outputs use |x-y| <= tol|y| + tol*rms(y).
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hsa
import oracle
import synth
from hils_testutil import (NEAR_TIE, TOL_BF16, TOL_F32, TOL_GRAD_BF16, all_scores, assert_close,
                           check_band, compare_selection, say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def out_tol(w):
    return TOL_BF16 if w.dtype == "bf16" else TOL_F32


SMALL = {
    "f32_d64_B2": synth.small("f32_d64_B2", B=2, T=640, H=2, Hkv=1, d=64, K=4, dtype="f32"),
    "bf16_gqa_ragged": synth.small("bf16_gqa_ragged", B=1, T=704, H=4, Hkv=2, d=64, K=5,
                                   dtype="bf16", n_planted=2),
    "bf16_d128_gqa4": synth.small("bf16_d128_gqa4", B=1, T=1024, H=8, Hkv=2, d=128, K=6,
                                  dtype="bf16", n_planted=1, n_uniform=2),
    "f32_d128": synth.small("f32_d128", B=1, T=512, H=2, Hkv=2, d=128, K=3, dtype="f32"),
    "f32_kmax": synth.small("f32_kmax", B=1, T=4224, H=1, Hkv=1, d=64, K=64, dtype="f32"),
    "bf16_kmax": synth.small("bf16_kmax", B=1, T=4224, H=2, Hkv=1, d=64, K=64, dtype="bf16"),
    "single_chunk": synth.small("single_chunk", B=1, T=64, H=2, Hkv=1, d=64, K=2, dtype="bf16"),
}
_cache = {}


def case(name):
    if name not in _cache:
        w = SMALL[name] if name in SMALL else synth.workloads()[name]
        x = synth.make_inputs(w)
        _cache[name] = (w, x)
    return _cache[name]


def gpu_forward(w, x):
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S)
    torch.cuda.synchronize()
    return t, f


@pytest.mark.parametrize("name", list(SMALL) + ["tiny_f32"])
def test_summarize(name):
    w, x = case(name)
    say(f"[summarize] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("K", "Ql")}
    ksum, ent, lse = hsa.summarize(t["K"], t["Ql"], w.S)
    torch.cuda.synchronize()
    oks, oent, olse = oracle.summarize(x["K"], x["Ql"], w.S)
    assert_close(host(ksum), oks, TOL_F32, "ksum")
    assert_close(host(ent), oent, TOL_F32, "ent")
    assert_close(host(lse), olse, TOL_F32, "lse_l")


# groups of query heads per kv head: bf16 takes up to 16 heads per matrix-core
# round (3 and 8 in one round, 20 in rounds of 16 and 4); float32 runs a round
# with an idle wavefront (3 heads on 2)
GROUPS = {
    "bf16_g3": synth.small("sum_g3", B=1, T=640, H=3, Hkv=1, d=64, K=4, dtype="bf16"),
    "bf16_d128_g8": synth.small("sum_g8", B=2, T=512, H=16, Hkv=2, d=128, K=4, dtype="bf16"),
    "bf16_g20": synth.small("sum_g20", B=1, T=320, H=40, Hkv=2, d=64, K=4, dtype="bf16"),
    "bf16_d128_g20": synth.small("sum_g20d", B=1, T=256, H=20, Hkv=1, d=128, K=4, dtype="bf16"),
    "f32_g3": synth.small("sum_g3f", B=1, T=384, H=6, Hkv=2, d=64, K=4, dtype="f32"),
}


@pytest.mark.parametrize("name", list(GROUPS) + ["peaked_bf16", "peaked_bf16_d128"])
def test_summarize_head_groups(name):
    """Summaries per head group against the oracle. The peaked cases scale the
    landmark queries by 16 (exact in bf16), so each chunk's landmark softmax
    puts almost all of its mass on one or two keys (entropy near 0)."""
    if name.startswith("peaked"):
        w = GROUPS["bf16_d128_g8" if name.endswith("d128") else "bf16_g3"]
        x = synth.make_inputs(w)
        x["Ql"] = x["Ql"] * 16.0
    else:
        w = GROUPS[name]
        x = synth.make_inputs(w)
    say(f"[summarize groups] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("K", "Ql")}
    ksum, ent, lse = hsa.summarize(t["K"], t["Ql"], w.S)
    torch.cuda.synchronize()
    oks, oent, olse = oracle.summarize(x["K"], x["Ql"], w.S)
    assert_close(host(ksum), oks, TOL_F32, "ksum")
    assert_close(host(ent), oent, TOL_F32, "ent")
    assert_close(host(lse), olse, TOL_F32, "lse_l")


@pytest.mark.parametrize("name", list(SMALL) + ["tiny_f32"])
def test_forward_end_to_end(name):
    w, x = case(name)
    say(f"[forward] {name}")
    t, f = gpu_forward(w, x)
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    excl, eq = compare_selection(host(f["idx"]), o["idx"], o["gap"], w.K,
                                 lambda d: all_scores(x["Q"], o["ksum"], o["ent"], w.S, d))
    say(f"  near-tie rows excluded: {int(excl.sum())}/{excl.size}; differing among them: "
        f"{int((~eq).sum())}")
    sel = eq[..., None].repeat(w.K, -1) & (o["idx"] >= 0)
    assert_close(host(f["score"])[sel], o["score"][sel], TOL_F32, "score")
    assert np.all(host(f["score"])[eq[..., None].repeat(w.K, -1) & (o["idx"] < 0)] == -np.inf)
    assert_close(host(f["O"])[eq], o["O"][eq], out_tol(w), "O")
    assert_close(host(f["lse_own"])[eq], o["lse_own"][eq], TOL_F32, "lse_own")
    assert_close(host(f["lse_tot"])[eq], o["lse_tot"][eq], TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", ["f32_d64_B2", "bf16_d128_gqa4", "tiny_f32"])
def test_attend_stage_with_oracle_selection(name):
    """attend_fuse fed the oracle's selection and scores covers every row, near-ties included."""
    w, x = case(name)
    say(f"[attend stage] {name}")
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V")}
    idx = torch.from_numpy(o["idx"]).to(DEV)
    score = torch.from_numpy(o["score"].astype(np.float32)).to(DEV)
    O, lo, lt = hsa.attend_fuse(t["Q"], t["K"], t["V"], idx, score, w.S)
    torch.cuda.synchronize()
    assert_close(host(O), o["O"], out_tol(w), "O")
    assert_close(host(lo), o["lse_own"], TOL_F32, "lse_own")
    assert_close(host(lt), o["lse_tot"], TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", ["bf16_gqa_ragged", "bf16_d128_gqa4"])
def test_attend_stage_scores_far_from_chunk_mass(name):
    """Scores that are not HiLS chunk scores (offsets of up to +-100 from the oracle's,
    so exp(s - score) over a chunk can overflow or vanish) still give the oracle's output:
    the intra-chunk softmax must not depend on the score being close to the chunk's mass."""
    w, x = case(name)
    say(f"[attend stage, shifted scores] {name}")
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    rng = np.random.default_rng(7)
    sc = (o["score"] + rng.uniform(-100.0, 100.0, o["score"].shape)).astype(np.float32)
    sc[o["idx"] < 0] = -np.inf
    O_ref, lo_ref, lt_ref = oracle.attend_fuse(x["Q"], x["K"], x["V"], o["idx"], sc, w.S)
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V")}
    idx = torch.from_numpy(o["idx"]).to(DEV)
    score = torch.from_numpy(sc).to(DEV)
    O, lo, lt = hsa.attend_fuse(t["Q"], t["K"], t["V"], idx, score, w.S)
    torch.cuda.synchronize()
    assert_close(host(O), O_ref, out_tol(w), "O")
    assert_close(host(lo), lo_ref, TOL_F32, "lse_own")
    assert_close(host(lt), lt_ref, TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", ["bf16_gqa_ragged", "bf16_d128_gqa4"])
def test_attend_stage_large_logits(name):
    """Queries scaled by 32 (exact in bf16) make logits of several hundred, so weights
    taken without a running maximum would overflow: the kernels must still match."""
    w, x = case(name)
    say(f"[attend stage, large logits] {name}")
    Q = x["Q"] * 32.0
    o = oracle.forward(Q, x["K"], x["V"], x["Ql"], w.S, w.K)
    t = {k: dev(v, w.dtype) for k, v in (("Q", Q), ("K", x["K"]), ("V", x["V"]))}
    idx = torch.from_numpy(o["idx"]).to(DEV)
    score = torch.from_numpy(o["score"].astype(np.float32)).to(DEV)
    O, lo, lt = hsa.attend_fuse(t["Q"], t["K"], t["V"], idx, score, w.S)
    torch.cuda.synchronize()
    assert_close(host(O), o["O"], out_tol(w), "O")
    assert_close(host(lo), o["lse_own"], TOL_F32, "lse_own")
    assert_close(host(lt), o["lse_tot"], TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", ["bf16_gqa_ragged", "bf16_d128_gqa4"])
def test_attend_rows_independent_of_tile_mates(name):
    """A row's output does not depend on the rows that share its MFMA tiles. With
    every other query position scaled by 32 (logits of several hundred: those rows'
    weight sums leave the no-maximum fast path), the unscaled rows equal a run
    without scaling bit for bit (selection and scores held fixed), and the scaled
    rows match the oracle."""
    w, x = case(name)
    say(f"[attend stage, tile mates] {name}")
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    Q2 = x["Q"].copy()
    Q2[:, 1::2] *= 32.0                      # exact in bf16
    idx = torch.from_numpy(o["idx"]).to(DEV)
    score = torch.from_numpy(o["score"].astype(np.float32)).to(DEV)
    K, V = dev(x["K"], w.dtype), dev(x["V"], w.dtype)
    Oa, loa, _ = hsa.attend_fuse(dev(x["Q"], w.dtype), K, V, idx, score, w.S)
    Ob, lob, ltb = hsa.attend_fuse(dev(Q2, w.dtype), K, V, idx, score, w.S)
    torch.cuda.synchronize()
    assert torch.equal(Oa[:, 0::2], Ob[:, 0::2])
    assert torch.equal(loa[:, 0::2], lob[:, 0::2])
    O_ref, lo_ref, lt_ref = oracle.attend_fuse(Q2, x["K"], x["V"], o["idx"], o["score"], w.S)
    assert_close(host(Ob), O_ref, out_tol(w), "O")
    assert_close(host(lob), lo_ref, TOL_F32, "lse_own")
    assert_close(host(ltb), lt_ref, TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", ["bf16_gqa_ragged", "bf16_d128_gqa4", "f32_kmax"])
def test_decode_rows_equal_prefill_rows(name):
    """A query scored alone (split path) selects what the prefill pass selected, bit for bit,
    and attends to the same output (decode = prefill row)."""
    w, x = case(name)
    say(f"[decode=prefill] {name}")
    t, f = gpu_forward(w, x)
    idx_p, sc_p, O_p = host(f["idx"]), host(f["score"]), host(f["O"])
    for p in (63, 64, 300, w.T - 65, w.T - 1):
        q = t["Q"][:, p:p + 1].contiguous()
        idx, sc = hsa.score_topk(q, f["ksum"], f["ent"], w.K, w.S, q_pos0=p, Tkv=p + 1,
                                 Hkv=w.Hkv)
        O, lo, lt = hsa.attend_fuse(q, t["K"], t["V"], idx, sc, w.S, q_pos0=p, Tkv=p + 1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(idx)[:, 0], idx_p[:, p])
        np.testing.assert_array_equal(host(sc)[:, 0], sc_p[:, p])
        # single rows and prefill tiles may run different attention kernels
        assert_close(host(O)[:, 0], O_p[:, p], out_tol(w), f"O row {p}")


def test_empty_query_range_is_noop():
    w, x = case("bf16_gqa_ragged")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    q = t["Q"][:, :0].contiguous()
    idx, sc = hsa.score_topk(q, ksum, ent, w.K, w.S, Tkv=w.T, Hkv=w.Hkv)
    O, lo, lt = hsa.attend_fuse(q, t["K"], t["V"], idx, sc, w.S)
    torch.cuda.synchronize()
    assert O.numel() == 0


def test_incremental_summaries_match_full():
    """Summarising chunk ranges one at a time (decode) equals one pass over all chunks."""
    w, x = case("bf16_d128_gqa4")
    say("[summarize incremental]")
    t = {k: dev(x[k], w.dtype) for k in ("K", "Ql")}
    full = hsa.summarize(t["K"], t["Ql"], w.S)
    parts = [torch.full_like(a, float("nan")) for a in full]
    for c in range(w.NC):
        hsa.summarize(t["K"], t["Ql"], w.S, c, c + 1, ksum=parts[0], ent=parts[1],
                      lse_l=parts[2])
    torch.cuda.synchronize()
    for a, b in zip(full, parts):
        assert torch.equal(a, b)


def test_forward_deterministic():
    w, x = case("bf16_d128_gqa4")
    _, f1 = gpu_forward(w, x)
    _, f2 = gpu_forward(w, x)
    for k in f1:
        assert torch.equal(f1[k], f2[k]), k


# ------------------------------------------------------------------ full-size workloads
def sampled_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    B, Tq, H = w.B, w.rows_q, w.H
    rows = rng.choice(B * Tq * H, size=n, replace=False)
    # always include the last row of each batch element and a chunk-0 row
    extra = [((b * Tq + Tq - 1) * H + H - 1) for b in range(B)] + [3 * H]
    return np.unique(np.concatenate([rows, extra]))


@pytest.mark.parametrize("name,nrows", [("prefill_345m", None), ("prefill_7b_gqa", 1024)])
def test_full_size_prefill(name, nrows):
    """The full workload on the GPU; every row compared for the 345M prefill; for the
    7B GQA prefill every row of kv head 5 (all 32768 positions of its 4 query heads)
    and sampled rows of the other heads (plus the last row and a chunk-0 row)."""
    w, x = case(name)
    say(f"[full prefill] {name}: B{w.B} T{w.T} H{w.H}/{w.Hkv} d{w.d} K{w.K}")
    t, f = gpu_forward(w, x)
    ksum, ent, lse = oracle.summarize(x["K"], x["Ql"], w.S)
    assert_close(host(f["ksum"]), ksum, TOL_F32, "ksum")
    assert_close(host(f["ent"]), ent, TOL_F32, "ent")
    if nrows is None:
        rows = np.arange(w.B * w.T * w.H)
    else:
        G, g0 = w.H // w.Hkv, 5
        group = np.array([(b * w.T + i) * w.H + g0 * G + hh for b in range(w.B)
                          for i in range(w.T) for hh in range(G)])
        rows = np.unique(np.concatenate([group, sampled_rows(w, nrows, 7)]))
    idx, score, gap = oracle.score_topk(x["Q"], ksum, ent, w.S, w.K, rows=rows)
    O, lo, lt = oracle.attend_fuse(x["Q"], x["K"], x["V"], idx, score, w.S, rows=rows)
    flat = lambda a: a.reshape(-1, *a.shape[3:])  # noqa: E731
    gi, gs = flat(host(f["idx"]))[rows], flat(host(f["score"]))[rows]
    excl, eq = compare_selection(gi, flat(idx)[rows], flat(gap)[rows], w.K,
                                 lambda d: all_scores(x["Q"], ksum, ent, w.S, rows[d]))
    say(f"  rows compared {len(rows)}, near-tie excluded {int(excl.sum())}")
    m = eq[:, None].repeat(w.K, 1) & (flat(idx)[rows] >= 0)
    assert_close(gs[m], flat(score)[rows][m], TOL_F32, "score")
    assert_close(flat(host(f["O"]))[rows][eq], flat(O)[rows][eq], out_tol(w), "O")
    assert_close(flat(host(f["lse_tot"]))[rows][eq], flat(lt)[rows][eq], TOL_F32, "lse_tot")
    # every row: selection is valid (ascending, distinct, causal, padded only when n < K)
    gi_all = host(f["idx"])
    n = (np.arange(w.T) // w.S)[None, :, None]
    cnt = (gi_all >= 0).sum(-1)
    assert np.all(cnt == np.minimum(n, w.K))
    valid = gi_all >= 0
    assert np.all(valid[..., :-1] | ~valid[..., 1:])          # pads only at the end
    both = valid[..., :-1] & valid[..., 1:]
    assert np.all((np.diff(gi_all, axis=-1) > 0) | ~both)     # ascending, distinct
    assert np.all(gi_all < n[..., None])


def test_full_size_decode_sampled_steps():
    w, x = case("decode_128k")
    say(f"[full decode] cache {w.T} H{w.H} d{w.d} K{w.K}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    ksum, ent, lse = hsa.summarize(t["K"], t["Ql"], w.S)
    oks, oent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    assert_close(host(ksum), oks, TOL_F32, "ksum")
    for step in (0, 63, 64, 200, 255):
        p = w.q_pos0 + step
        q = t["Q"][:, step:step + 1].contiguous()
        idx, sc = hsa.score_topk(q, ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, Hkv=w.Hkv)
        O, lo, lt = hsa.attend_fuse(q, t["K"], t["V"], idx, sc, w.S, q_pos0=p, Tkv=p + 1)
        torch.cuda.synchronize()
        qn = x["Q"][:, step:step + 1]
        oidx, osc, ogap = oracle.score_topk(qn, oks, oent, w.S, w.K, q_pos0=p)
        oO, olo, olt = oracle.attend_fuse(qn, x["K"][:, :p + 1], x["V"][:, :p + 1], oidx, osc,
                                          w.S, q_pos0=p)
        excl, eq = compare_selection(host(idx), oidx, ogap, w.K,
                                     lambda d: all_scores(qn, oks, oent, w.S, d, q_pos0=p))
        assert_close(host(O)[eq], oO[eq], TOL_BF16, f"O step {step}")
        assert_close(host(lt)[eq], olt[eq], TOL_F32, f"lse_tot step {step}")


# ------------------------------------------------------------------ GQA group-max selection
GROUP = {
    "grp_bf16_g2": synth.small("grp_bf16_g2", B=1, T=704, H=4, Hkv=2, d=64, K=5, dtype="bf16",
                               n_planted=2),
    "grp_bf16_d128_g4": synth.small("grp_bf16_d128_g4", B=1, T=1024, H=8, Hkv=2, d=128, K=6,
                                    dtype="bf16", n_planted=1, n_uniform=2),
    "grp_f32_g8_k20": synth.small("grp_f32_g8_k20", B=2, T=640, H=8, Hkv=1, d=64, K=20,
                                  dtype="f32"),
    "grp_f32_g1": synth.small("grp_f32_g1", B=1, T=512, H=2, Hkv=2, d=64, K=4, dtype="f32"),
}


def check_group_forward(w, x, f, rows=None):
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, group=True)
    gi = host(f["idx"])
    G = w.H // w.Hkv
    # one chunk set per kv group, on every row
    grp = gi.reshape(w.B, w.T, w.Hkv, G, w.K)
    assert np.all(grp == grp[:, :, :, :1])
    excl, eq = compare_selection(gi, o["idx"], o["gap"], w.K,
                                 lambda d: all_scores(x["Q"], o["ksum"], o["ent"], w.S, d,
                                                      group_hkv=w.Hkv))
    say(f"  near-tie rows excluded: {int(excl.sum())}/{excl.size}")
    sel = eq[..., None].repeat(w.K, -1) & (o["idx"] >= 0)
    assert_close(host(f["score"])[sel], o["score"][sel], TOL_F32, "score")
    assert np.all(host(f["score"])[eq[..., None].repeat(w.K, -1) & (o["idx"] < 0)] == -np.inf)
    assert_close(host(f["O"])[eq], o["O"][eq], out_tol(w), "O")
    assert_close(host(f["lse_tot"])[eq], o["lse_tot"][eq], TOL_F32, "lse_tot")
    return o


@pytest.mark.parametrize("name", list(GROUP))
def test_forward_group_max(name):
    w = GROUP[name]
    x = synth.make_inputs(w)
    say(f"[forward group-max] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, group=True)
    torch.cuda.synchronize()
    check_group_forward(w, x, f)


# Long contexts: the matrix-core group scorer's second pass keeps a per-(position,
# bitmask word) prefix table that grows with the candidate count; past 65 G 32
# candidates (4160 at G = 2, 8320 at G = 4) it is larger than the first pass's
# score blocks. Summaries are drawn directly (float32 normals; the query rows are
# bf16 values) and the 64 query positions sit at the end of the context.
LONG_GROUP = {"g2_4800": (2, 4800), "g4_8500": (4, 8500)}


@pytest.mark.parametrize("name", list(LONG_GROUP))
def test_group_max_long_context(name):
    G, NC = LONG_GROUP[name]
    B, Hkv, d, S, K, Tq = 1, 1, 128, 64, 16, 64
    H = G * Hkv
    Tkv = NC * S + S // 2          # the last position's candidates: chunks 0 .. NC - 1
    q_pos0 = Tkv - Tq
    say(f"[group-max long context] G{G} candidates {NC}")
    rng = np.random.default_rng(1000 + G)
    Qg = torch.from_numpy(rng.standard_normal((B, Tq, H, d)).astype(np.float32)).to(torch.bfloat16)
    Qo = Qg.double().numpy()
    ksum = (0.5 * rng.standard_normal((B, NC + 1, H, d))).astype(np.float32)
    ent = (0.3 * rng.standard_normal((B, NC + 1, H))).astype(np.float32)
    idx, sc = hsa.score_topk(Qg.to(DEV), torch.from_numpy(ksum).to(DEV),
                             torch.from_numpy(ent).to(DEV), K, S, q_pos0=q_pos0, Tkv=Tkv,
                             Hkv=Hkv, group=True)
    torch.cuda.synchronize()
    ko, eo = ksum.astype(np.float64), ent.astype(np.float64)
    oi, os_, gap = oracle.score_topk(Qo, ko, eo, S, K, q_pos0=q_pos0, group_hkv=Hkv)
    gi, gs = host(idx), host(sc)
    excl, eq = compare_selection(gi, oi, gap, K,
                                 lambda r: all_scores(Qo, ko, eo, S, r, q_pos0, group_hkv=Hkv))
    say(f"  near-tie rows excluded: {int(excl.sum())}/{excl.size}")
    assert eq.sum() >= excl.size // 2
    m = eq[..., None].repeat(K, -1) & (oi >= 0)
    assert_close(gs[m], os_[m], TOL_F32, "score")


def test_backward_with_group_selection():
    """The backward takes any fixed selection: here a group-max one (bf16, G = 4)."""
    w = synth.small("bwd_grp", B=1, T=768, H=8, Hkv=2, d=64, K=5, dtype="bf16", need_dO=True)
    x = synth.make_inputs(w)
    say("[backward group-max] bwd_grp")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql", "dO")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, group=True)
    g = hsa.backward(t["Q"], t["K"], t["V"], t["Ql"], f["ksum"], f["ent"], f["lse_l"], f["idx"],
                     f["score"], f["lse_tot"], f["O"], t["dO"], w.S)
    torch.cuda.synchronize()
    o = check_group_forward(w, x, f)
    eq = np.all(host(f["idx"]) == o["idx"], axis=-1)
    assert eq.all(), "this case needs identical selections"
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], o["idx"], x["dO"], w.S)
    for nm, a, b in zip(("dQ", "dK", "dV", "dQl"), g, og):
        assert_close(host(a), b, TOL_GRAD_BF16, nm)


def test_full_size_group_max_7b_sampled():
    w, x = case("prefill_7b_gqa")
    say(f"[full group-max] B{w.B} T{w.T} H{w.H}/{w.Hkv} d{w.d} K{w.K}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, group=True)
    torch.cuda.synchronize()
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    rows = sampled_rows(w, 256, 13)
    idx, score, gap = oracle.score_topk(x["Q"], ksum, ent, w.S, w.K, rows=rows,
                                        group_hkv=w.Hkv)
    O, lo, lt = oracle.attend_fuse(x["Q"], x["K"], x["V"], idx, score, w.S, rows=rows)
    flat = lambda a: a.reshape(-1, *a.shape[3:])  # noqa: E731
    gi, gs = flat(host(f["idx"]))[rows], flat(host(f["score"]))[rows]
    excl, eq = compare_selection(gi, flat(idx)[rows], flat(gap)[rows], w.K,
                                 lambda d: all_scores(x["Q"], ksum, ent, w.S, rows[d],
                                                      group_hkv=w.Hkv))
    say(f"  rows compared {len(rows)}, near-tie excluded {int(excl.sum())}")
    m = eq[:, None].repeat(w.K, 1) & (flat(idx)[rows] >= 0)
    assert_close(gs[m], flat(score)[rows][m], TOL_F32, "score")
    assert_close(flat(host(f["O"]))[rows][eq], flat(O)[rows][eq], out_tol(w), "O")
    G = w.H // w.Hkv
    grp = host(f["idx"]).reshape(w.B, w.T, w.Hkv, G, w.K)
    assert np.all(grp == grp[:, :, :, :1])


# ------------------------------------------------------------------ backward
BWD = {
    "bwd_bf16_gqa": synth.small("bwd_bf16_gqa", B=2, T=512, H=4, Hkv=2, d=64, K=3, dtype="bf16",
                                need_dO=True),
    "bwd_bf16_g1": synth.small("bwd_bf16_g1", B=1, T=1024, H=2, Hkv=2, d=64, K=4, dtype="bf16",
                               n_planted=2, need_dO=True),
    "bwd_bf16_gqa4": synth.small("bwd_bf16_gqa4", B=1, T=768, H=8, Hkv=2, d=64, K=5,
                                 dtype="bf16", n_planted=1, need_dO=True),
    # K above the candidate count of every row (padded selections) and above 16
    "bwd_bf16_k20": synth.small("bwd_bf16_k20", B=1, T=1024, H=2, Hkv=1, d=64, K=20,
                                dtype="bf16", need_dO=True),
    "bwd_f32": synth.small("bwd_f32", B=1, T=640, H=2, Hkv=1, d=64, K=4, dtype="f32",
                           need_dO=True),
    "bwd_f32_d128": synth.small("bwd_f32_d128", B=1, T=256, H=2, Hkv=1, d=128, K=2,
                                dtype="f32", need_dO=True),
    "bwd_bf16_d128": synth.small("bwd_bf16_d128", B=1, T=512, H=4, Hkv=1, d=128, K=3,
                                 dtype="bf16", need_dO=True),
    # the largest top-K with real selections (up to 65 candidates per row)
    "bwd_bf16_kmax": synth.small("bwd_bf16_kmax", B=1, T=4224, H=2, Hkv=1, d=64, K=64,
                                 dtype="bf16", need_dO=True),
}


def gpu_train(w, x):
    t, f = gpu_forward(w, x)
    dO = dev(x["dO"], w.dtype)
    g = hsa.backward(t["Q"], t["K"], t["V"], t["Ql"], f["ksum"], f["ent"], f["lse_l"], f["idx"],
                     f["score"], f["lse_tot"], f["O"], dO, w.S)
    torch.cuda.synchronize()
    return f, g


def test_full_size_training_backward_one_head():
    """Every dQ row of one (batch element, head) of the training workload, and dK, dV
    and dQl of every chunk of its kv head (one query head per kv head), against the
    oracle. Rows whose near-tie selection differs from the oracle's, and the chunks
    they touch, are left out (their gradients follow a different, equally valid
    selection)."""
    w, x = case("train_345m")
    G = w.H // w.Hkv
    assert G == 1
    b0, h0 = 1, 9
    say(f"[full backward, one head] b{b0} h{h0}: {w.T} rows, {w.NC} chunks")
    f, g = gpu_train(w, x)
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    rows = np.array([(b0 * w.T + i) * w.H + h0 for i in range(w.T)])
    idx, score, gap = oracle.score_topk(x["Q"], ksum, ent, w.S, w.K, rows=rows)
    gi = host(f["idx"]).reshape(-1, w.K)
    oi = idx.reshape(-1, w.K)
    differ = rows[np.any(gi[rows] != oi[rows], axis=1)]
    assert np.all(gap.reshape(-1)[differ] < NEAR_TIE)
    if differ.size:  # a valid top-K within the near-tie band
        check_band(gi[differ], all_scores(x["Q"], ksum, ent, w.S, differ), w.K)
    row_mask = np.zeros(w.B * w.T * w.H, np.uint8)
    row_mask[np.setdiff1d(rows, differ)] = 1
    kv_mask = np.zeros((w.B, w.NC, w.Hkv), np.uint8)
    kv_mask[b0, :, h0] = 1
    for r in differ:
        for c in set(gi[r].tolist()) | set(oi[r].tolist()):
            if c >= 0:
                kv_mask[b0, c, h0] = 0
    say(f"  rows with differing near-tie selections: {len(differ)}; "
        f"chunks compared {int(kv_mask.sum())} of {w.NC}")
    oidx_full = np.full((w.B, w.T, w.H, w.K), -1, np.int32)
    oidx_full.reshape(-1, w.K)[rows] = oi[rows]
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], oidx_full, x["dO"], w.S,
                         row_mask=row_mask.reshape(w.B, w.T, w.H), kv_mask=kv_mask)
    dQ, dK, dV, dQl = (host(a) for a in g)
    rm = row_mask.astype(bool)
    assert_close(dQ.reshape(-1, w.d)[rm], og[0].reshape(-1, w.d)[rm], TOL_GRAD_BF16, "dQ")
    cs = np.flatnonzero(kv_mask[b0, :, h0])
    keys = (cs[:, None] * w.S + np.arange(w.S)[None, :]).reshape(-1)
    assert_close(dK[b0, keys, h0], og[1][b0, keys, h0], TOL_GRAD_BF16, "dK")
    assert_close(dV[b0, keys, h0], og[2][b0, keys, h0], TOL_GRAD_BF16, "dV")
    assert_close(dQl[b0, cs, h0], og[3][b0, cs, h0], TOL_GRAD_BF16, "dQl")


@pytest.mark.parametrize("name", list(BWD))
def test_backward_small(name):
    w = BWD[name]
    x = synth.make_inputs(w)
    say(f"[backward] {name}")
    f, g = gpu_train(w, x)
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K)
    eq = np.all(host(f["idx"]) == o["idx"], axis=-1)
    assert eq.all(), "small backward cases need identical selections"
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], o["idx"], x["dO"], w.S)
    tol = TOL_GRAD_BF16 if w.dtype == "bf16" else TOL_F32
    for nm, a, b in zip(("dQ", "dK", "dV", "dQl"), g, og):
        assert_close(host(a), b, tol, nm)


@pytest.mark.parametrize("name", ["bwd_bf16_gqa", "bwd_bf16_k20", "bwd_f32", "bwd_bf16_d128"])
def test_backward_qcal(name):
    """Q-Cal: the chunk scores use a separate scoring query Qs; the backward
    returns its gradient dQs apart from dQ (matrix-core and vector paths)."""
    w = BWD[name]
    x = synth.make_inputs(w)
    qs = synth.scoring_query(w, x)
    say(f"[backward q-cal] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql", "dO")}
    tqs = dev(qs, w.dtype)
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, Qs=tqs)
    g = hsa.backward(t["Q"], t["K"], t["V"], t["Ql"], f["ksum"], f["ent"], f["lse_l"], f["idx"],
                     f["score"], f["lse_tot"], f["O"], t["dO"], w.S, Qs=tqs)
    torch.cuda.synchronize()
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, Qs=qs)
    eq = np.all(host(f["idx"]) == o["idx"], axis=-1)
    assert eq.all(), "small backward cases need identical selections"
    tol = TOL_GRAD_BF16 if w.dtype == "bf16" else TOL_F32
    assert_close(host(f["O"]), o["O"], out_tol(w), "O")
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], o["idx"], x["dO"], w.S, Qs=qs)
    for nm, a, b in zip(("dQ", "dK", "dV", "dQl", "dQs"), g, og):
        assert_close(host(a), b, tol, nm)


def test_backward_deterministic():
    w = BWD["bwd_bf16_gqa"]
    x = synth.make_inputs(w)
    _, g1 = gpu_train(w, x)
    _, g2 = gpu_train(w, x)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_full_size_training_backward_sampled():
    w, x = case("train_345m")
    say(f"[full backward] B{w.B} T{w.T} H{w.H} d{w.d} K{w.K}")
    f, g = gpu_train(w, x)
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    c_min = w.NC - 5
    # rows that can select chunks >= c_min, plus sampled rows for dQ
    late = np.array([(b * w.T + i) * w.H + h for b in range(w.B)
                     for i in range(c_min * w.S, w.T) for h in range(w.H)])
    dq_rows = sampled_rows(w, 96, 11)
    rows = np.unique(np.concatenate([late, dq_rows]))
    idx, score, gap = oracle.score_topk(x["Q"], ksum, ent, w.S, w.K, rows=rows)
    gi = host(f["idx"]).reshape(-1, w.K)
    oi = idx.reshape(-1, w.K)
    differ = rows[np.any(gi[rows] != oi[rows], axis=1)]
    assert np.all(gap.reshape(-1)[differ] < NEAR_TIE)
    if differ.size:  # a valid top-K within the near-tie band
        check_band(gi[differ], all_scores(x["Q"], ksum, ent, w.S, differ), w.K)
    row_mask = np.zeros(w.B * w.T * w.H, np.uint8)
    row_mask[np.setdiff1d(dq_rows, differ)] = 1
    kv_mask = np.zeros((w.B, w.NC, w.Hkv), np.uint8)
    chosen = [(0, w.NC - 1, 0), (0, w.NC - 3, 5), (1, w.NC - 2, 15), (1, c_min, 7)]
    # drop a chunk if a row whose selection differs touches it
    keep = []
    for b, c, gh in chosen:
        touched = False
        for r in differ:
            h = r % w.H
            if r // (w.T * w.H) == b and h // (w.H // w.Hkv) == gh and (
                    c in gi[r] or c in oi[r]):
                touched = True
        if not touched:
            keep.append((b, c, gh))
            kv_mask[b, c, gh] = 1
    say(f"  rows with differing near-tie selections: {len(differ)}; chunks checked {keep}")
    oidx_full = np.full((w.B, w.T, w.H, w.K), -1, np.int32)
    oidx_full.reshape(-1, w.K)[rows] = oi[rows]
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], oidx_full, x["dO"], w.S,
                         row_mask=row_mask.reshape(w.B, w.T, w.H), kv_mask=kv_mask)
    dQ, dK, dV, dQl = (host(a) for a in g)
    rm = row_mask.astype(bool)
    assert_close(dQ.reshape(-1, w.d)[rm], og[0].reshape(-1, w.d)[rm], TOL_GRAD_BF16, "dQ")
    for b, c, gh in keep:
        sl = slice(c * w.S, (c + 1) * w.S)
        assert_close(dK[b, sl, gh], og[1][b, sl, gh], TOL_GRAD_BF16, f"dK {b,c,gh}")
        assert_close(dV[b, sl, gh], og[2][b, sl, gh], TOL_GRAD_BF16, f"dV {b,c,gh}")
        G = w.H // w.Hkv
        assert_close(dQl[b, c, gh * G:(gh + 1) * G], og[3][b, c, gh * G:(gh + 1) * G],
                     TOL_GRAD_BF16, f"dQl {b,c,gh}")
