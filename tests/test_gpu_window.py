"""GPU parity of the sliding-window local branch (note §5.2 main setting: the last
512 keys attended exactly, the top-K chosen among the chunks wholly before the
window) against the CPU oracle, through the C ABI: prefill forward on the
matrix-core and vector paths, group-max selection, decode rows, the backward,
and the pages' main configuration (S = 64, K = 32, W = 512) at full size.
Same comparison rules as the other parity tests."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hsa
import oracle
import synth
from hils_testutil import (TOL_BF16, TOL_F32, TOL_GRAD_BF16, all_scores, assert_close,
                           compare_selection,
                           say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def out_tol(w):
    return TOL_BF16 if w.dtype == "bf16" else TOL_F32


# (workload, window in keys)
WIN = {
    "w_bf16_g1": (synth.small("w_bf16_g1", B=1, T=1024, H=2, Hkv=2, d=64, K=4, dtype="bf16",
                              n_planted=2), 256),
    "w_bf16_gqa_k32": (synth.small("w_bf16_gqa_k32", B=1, T=1536, H=4, Hkv=2, d=64, K=32,
                                   dtype="bf16"), 512),
    "w_bf16_d128_g4": (synth.small("w_bf16_d128_g4", B=1, T=1024, H=8, Hkv=2, d=128, K=5,
                                   dtype="bf16"), 192),
    "w_bf16_ragged": (synth.small("w_bf16_ragged", B=2, T=704, H=4, Hkv=2, d=64, K=3,
                                  dtype="bf16"), 320),
    "w_f32": (synth.small("w_f32", B=1, T=640, H=2, Hkv=1, d=64, K=3, dtype="f32"), 128),
    "w_f32_d128": (synth.small("w_f32_d128", B=1, T=512, H=2, Hkv=1, d=128, K=2,
                               dtype="f32"), 64),
    # the window covers every row's prefix: no candidates anywhere
    "w_cover": (synth.small("w_cover", B=1, T=384, H=2, Hkv=1, d=64, K=3, dtype="bf16"), 512),
    # the largest top-K and the largest window
    "w_bf16_kmax_wmax": (synth.small("w_bf16_kmax_wmax", B=1, T=3072, H=2, Hkv=1, d=64, K=64,
                                     dtype="bf16"), 2048),
}
_cache = {}


def case(name):
    if name not in _cache:
        w, W = WIN[name]
        _cache[name] = (w, W, synth.make_inputs(w))
    return _cache[name]


def check_forward(w, x, f, o, W, group=False):
    excl, eq = compare_selection(host(f["idx"]), o["idx"], o["gap"], w.K,
                                 lambda d: all_scores(x["Q"], o["ksum"], o["ent"], w.S, d,
                                                      group_hkv=w.Hkv if group else None,
                                                      window=W))
    say(f"  near-tie rows excluded: {int(excl.sum())}/{excl.size}")
    sel = eq[..., None].repeat(w.K, -1) & (o["idx"] >= 0)
    assert_close(host(f["score"])[sel], o["score"][sel], TOL_F32, "score")
    assert np.all(host(f["score"])[eq[..., None].repeat(w.K, -1) & (o["idx"] < 0)] == -np.inf)
    assert_close(host(f["O"])[eq], o["O"][eq], out_tol(w), "O")
    assert_close(host(f["lse_own"])[eq], o["lse_own"][eq], TOL_F32, "lse_own")
    assert_close(host(f["lse_tot"])[eq], o["lse_tot"][eq], TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", list(WIN))
def test_forward_window(name):
    w, W, x = case(name)
    say(f"[forward window {W}] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, window=W)
    torch.cuda.synchronize()
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, window=W)
    check_forward(w, x, f, o, W)
    if name == "w_cover":
        assert np.all(host(f["idx"]) == -1)


@pytest.mark.parametrize("name", ["w_bf16_gqa_k32", "w_bf16_d128_g4", "w_f32"])
def test_attend_window_with_oracle_selection(name):
    """attend_fuse fed the oracle's selection covers every row, near-ties included."""
    w, W, x = case(name)
    say(f"[attend stage, window {W}] {name}")
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, window=W)
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V")}
    idx = torch.from_numpy(o["idx"]).to(DEV)
    score = torch.from_numpy(o["score"].astype(np.float32)).to(DEV)
    O, lo, lt = hsa.attend_fuse(t["Q"], t["K"], t["V"], idx, score, w.S, window=W)
    torch.cuda.synchronize()
    assert_close(host(O), o["O"], out_tol(w), "O")
    assert_close(host(lo), o["lse_own"], TOL_F32, "lse_own")
    assert_close(host(lt), o["lse_tot"], TOL_F32, "lse_tot")


@pytest.mark.parametrize("name", ["w_bf16_gqa_k32", "w_bf16_d128_g4"])
def test_forward_window_group_max(name):
    w, W, x = case(name)
    say(f"[forward window {W}, group-max] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, group=True, window=W)
    torch.cuda.synchronize()
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, group=True, window=W)
    check_forward(w, x, f, o, W, group=True)


@pytest.mark.parametrize("name", ["w_bf16_gqa_k32", "w_bf16_d128_g4", "w_f32", "w_bf16_kmax_wmax"])
def test_decode_window_rows_equal_prefill_rows(name):
    """Single rows (split scoring, slot-parallel decode attention with one slot per
    local chunk) select and attend as the prefill pass does."""
    w, W, x = case(name)
    say(f"[decode=prefill, window {W}] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, window=W)
    torch.cuda.synchronize()
    idx_p, sc_p, O_p, lt_p = host(f["idx"]), host(f["score"]), host(f["O"]), host(f["lse_tot"])
    for p in (0, 63, W - 1, W, W + 64, w.T - 65, w.T - 1):
        q = t["Q"][:, p:p + 1].contiguous()
        idx, sc = hsa.score_topk(q, f["ksum"], f["ent"], w.K, w.S, q_pos0=p, Tkv=p + 1,
                                 Hkv=w.Hkv, window=W)
        O, lo, lt = hsa.attend_fuse(q, t["K"], t["V"], idx, sc, w.S, q_pos0=p, Tkv=p + 1,
                                    window=W)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(idx)[:, 0], idx_p[:, p])
        np.testing.assert_array_equal(host(sc)[:, 0], sc_p[:, p])
        assert_close(host(O)[:, 0], O_p[:, p], out_tol(w), f"O row {p}")
        assert_close(host(lt)[:, 0], lt_p[:, p], TOL_F32, f"lse_tot row {p}")


BWD = {
    "bw_bf16_g1": (synth.small("bw_bf16_g1", B=1, T=1024, H=2, Hkv=2, d=64, K=4, dtype="bf16",
                               need_dO=True), 256),
    "bw_bf16_gqa_k32": (synth.small("bw_bf16_gqa_k32", B=1, T=1536, H=4, Hkv=2, d=64, K=32,
                                    dtype="bf16", need_dO=True), 512),
    "bw_bf16_ragged_b2": (synth.small("bw_bf16_ragged_b2", B=2, T=704, H=4, Hkv=2, d=64, K=3,
                                      dtype="bf16", need_dO=True), 320),
    "bw_f32": (synth.small("bw_f32", B=1, T=640, H=2, Hkv=1, d=64, K=3, dtype="f32",
                           need_dO=True), 128),
    "bw_bf16_d128": (synth.small("bw_bf16_d128", B=1, T=512, H=4, Hkv=1, d=128, K=3,
                                 dtype="bf16", need_dO=True), 192),
    # the largest window of the matrix-core backward (1024 keys) and, past it, the
    # vector path with the largest window and top-K
    "bw_bf16_w1024": (synth.small("bw_bf16_w1024", B=1, T=2048, H=2, Hkv=1, d=64, K=8,
                                  dtype="bf16", need_dO=True), 1024),
    "bw_bf16_kmax_wmax": (synth.small("bw_bf16_kmax_wmax", B=1, T=3072, H=2, Hkv=1, d=64,
                                      K=64, dtype="bf16", need_dO=True), 2048),
}


@pytest.mark.parametrize("name", list(BWD))
def test_backward_window(name):
    w, W = BWD[name]
    x = synth.make_inputs(w)
    say(f"[backward window {W}] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql", "dO")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, window=W)
    g = hsa.backward(t["Q"], t["K"], t["V"], t["Ql"], f["ksum"], f["ent"], f["lse_l"], f["idx"],
                     f["score"], f["lse_tot"], f["O"], t["dO"], w.S, window=W)
    torch.cuda.synchronize()
    o = oracle.forward(x["Q"], x["K"], x["V"], x["Ql"], w.S, w.K, window=W)
    eq = np.all(host(f["idx"]) == o["idx"], axis=-1)
    assert eq.all(), "small backward cases need identical selections"
    og = oracle.backward(x["Q"], x["K"], x["V"], x["Ql"], o["idx"], x["dO"], w.S, window=W)
    tol = TOL_GRAD_BF16 if w.dtype == "bf16" else TOL_F32
    for nm, a, b in zip(("dQ", "dK", "dV", "dQl"), g, og):
        assert_close(host(a), b, tol, nm)


def sampled_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    B, Tq, H = w.B, w.rows_q, w.H
    rows = rng.choice(B * Tq * H, size=n, replace=False)
    extra = [((b * Tq + Tq - 1) * H + H - 1) for b in range(B)] + [3 * H, 600 * H]
    return np.unique(np.concatenate([rows, extra]))


def test_full_size_main_config_sampled():
    """The pages' main setting on the 345M-class prefill: S = 64, top-K = 32, a
    sliding window of 512 keys (B=1, T=8192, H=16, d=64, bf16); sampled rows."""
    base = synth.workloads()["prefill_345m"]
    w = synth.Workload("prefill_345m_k32", base.B, base.T, base.H, base.Hkv, base.d, base.S, 32,
                       base.dtype, base.n_planted, seed=base.seed)
    W = 512
    x = synth.make_inputs(w)
    say(f"[full main config] B{w.B} T{w.T} H{w.H} d{w.d} K{w.K} window {W}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    f = hsa.forward(t["Q"], t["K"], t["V"], t["Ql"], w.K, w.S, window=W)
    torch.cuda.synchronize()
    ksum, ent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    rows = sampled_rows(w, 384, 17)
    idx, score, gap = oracle.score_topk(x["Q"], ksum, ent, w.S, w.K, rows=rows, window=W)
    O, lo, lt = oracle.attend_fuse(x["Q"], x["K"], x["V"], idx, score, w.S, rows=rows, window=W)
    flat = lambda a: a.reshape(-1, *a.shape[3:])  # noqa: E731
    gi, gs = flat(host(f["idx"]))[rows], flat(host(f["score"]))[rows]
    excl, eq = compare_selection(gi, flat(idx)[rows], flat(gap)[rows], w.K,
                                 lambda d: all_scores(x["Q"], ksum, ent, w.S, rows[d], window=W))
    say(f"  sampled rows {len(rows)}, near-tie excluded {int(excl.sum())}")
    m = eq[:, None].repeat(w.K, 1) & (flat(idx)[rows] >= 0)
    assert_close(gs[m], flat(score)[rows][m], TOL_F32, "score")
    assert_close(flat(host(f["O"]))[rows][eq], flat(O)[rows][eq], TOL_BF16, "O")
    assert_close(flat(host(f["lse_own"]))[rows][eq], flat(lo)[rows][eq], TOL_F32, "lse_own")
    assert_close(flat(host(f["lse_tot"]))[rows][eq], flat(lt)[rows][eq], TOL_F32, "lse_tot")
