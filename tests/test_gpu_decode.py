"""hils_decode (one decode step in one call) through the C ABI.

Its results are those of hils_score_topk followed by hils_attend_fuse, bit for
bit (selection, scores, outputs, log-masses), also where its slot kernel merges
the candidate splits' lists itself (few rows, at most 32 splits) and where one
workgroup per row merges, attends and fuses (128 rows and more). Also checked
against the oracle, over many steps in a row on one workspace (whose contents do
not matter), with windows, K = 64, several rows per call, rows with no
candidates, d = 128, float32 and a host-resident cache.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hsa
import oracle
import synth
from hils_testutil import TOL_BF16, TOL_F32, all_scores, assert_close, compare_selection, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


CASES = {
    # name: workload, window, query rows per call
    "bf16_d64": (synth.small("dec_d64", B=1, T=8192, H=4, Hkv=2, d=64, K=16, dtype="bf16",
                             n_planted=2), 0, 1),
    "bf16_d64_rows4_b2": (synth.small("dec_rows", B=2, T=4096, H=2, Hkv=1, d=64, K=8,
                                      dtype="bf16"), 0, 4),
    "bf16_d128_g4": (synth.small("dec_d128", B=1, T=8192, H=8, Hkv=2, d=128, K=16, dtype="bf16",
                                 n_uniform=3), 0, 1),
    "bf16_window_k32": (synth.small("dec_win", B=1, T=8192, H=4, Hkv=4, d=64, K=32,
                                    dtype="bf16"), 512, 1),
    "bf16_k64_window2048": (synth.small("dec_k64", B=1, T=12288, H=2, Hkv=1, d=64, K=64,
                                        dtype="bf16"), 2048, 2),
    "f32_d64": (synth.small("dec_f32", B=1, T=4096, H=2, Hkv=1, d=64, K=8, dtype="f32"), 0, 1),
    # 8 candidate splits of 64-entry lists merged inside the slot kernel
    "bf16_k64_splits8": (synth.small("dec_k64s", B=1, T=65536, H=2, Hkv=1, d=64, K=64,
                                     dtype="bf16"), 0, 1),
    # 64 query positions per call: over the long cache the slot kernels serve
    # them (at the first positions the matrix-core kernel does)
    "bf16_64pos": (synth.small("dec_64pos", B=1, T=65536, H=2, Hkv=1, d=64, K=8,
                               dtype="bf16"), 0, 64),
    # 17 splits of 32-entry lists at the last positions (the 24-list merge)
    "bf16_k32_splits17": (synth.small("dec_k32s", B=1, T=17 * 128 * 64 + 128, H=4, Hkv=2,
                                      d=64, K=32, dtype="bf16"), 0, 1),
    # 128 rows per call (4 sequences x 8 positions x 4 heads): one workgroup per
    # row merges, attends every slot and fuses in LDS
    "bf16_rows128": (synth.small("dec_r128", B=4, T=10240, H=4, Hkv=2, d=64, K=16,
                                 dtype="bf16"), 0, 8),
    "bf16_d128_rows128": (synth.small("dec_r128d", B=2, T=10240, H=8, Hkv=2, d=128, K=16,
                                      dtype="bf16"), 0, 8),
    "bf16_window_k32_rows128": (synth.small("dec_r128w", B=4, T=10240, H=4, Hkv=4, d=64, K=32,
                                            dtype="bf16"), 512, 8),
    "f32_rows128": (synth.small("dec_r128f", B=4, T=10240, H=4, Hkv=2, d=64, K=8,
                                dtype="f32"), 0, 8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_steps_match_two_calls_and_oracle(name):
    w, W, nq = CASES[name]
    x = synth.make_inputs(w)
    say(f"[decode] {name}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    oks, oent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    # positions: the first chunk (no candidates), chunk edges, late rows
    starts = [0, 63, 64, 1000, w.T // 2 + 5, w.T - 64, w.T - nq]
    ws = None
    for p in starts:
        q = t["Q"][:, p:p + nq].contiguous()
        if ws is None:
            ws = hsa.decode_workspace(t["Q"][:, :nq], t["K"], ksum, w.K, w.S, w.T - nq, w.T,
                                      window=W)
        got = hsa.decode(q, t["K"], t["V"], ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + nq, ws=ws,
                         window=W)
        idx, sc = hsa.score_topk(q, ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + nq, Hkv=w.Hkv,
                                 window=W)
        O, lo, lt = hsa.attend_fuse(q, t["K"], t["V"], idx, sc, w.S, q_pos0=p, Tkv=p + nq,
                                    window=W)
        torch.cuda.synchronize()
        assert torch.equal(got[0], idx), p
        assert torch.equal(got[1], sc), p
        assert torch.equal(got[2], O), p
        assert torch.equal(got[4], lt), p
        assert torch.equal(got[3], lo), p
        qn = x["Q"][:, p:p + nq]
        oidx, osc, ogap = oracle.score_topk(qn, oks, oent, w.S, w.K, q_pos0=p, window=W)
        oO, olo, olt = oracle.attend_fuse(qn, x["K"][:, :p + nq], x["V"][:, :p + nq], oidx, osc,
                                          w.S, q_pos0=p, window=W)
        excl, eq = compare_selection(host(got[0]), oidx, ogap, w.K,
                                     lambda d: all_scores(qn, oks, oent, w.S, d, q_pos0=p,
                                                          window=W))
        tol = TOL_BF16 if w.dtype == "bf16" else TOL_F32
        assert_close(host(got[2])[eq], oO[eq], tol, f"O {p}")
        assert_close(host(got[4])[eq], olt[eq], TOL_F32, f"lse_tot {p}")
        assert_close(host(got[3])[eq], olo[eq], TOL_F32, f"lse_own {p}")


def test_decode_workspace_contents_do_not_matter():
    """A workspace full of arbitrary bytes gives the same results as a fresh one."""
    w, W, nq = CASES["bf16_d64"]
    x = synth.make_inputs(w)
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    ws = hsa.decode_workspace(t["Q"][:, :1], t["K"], ksum, w.K, w.S, w.T - 1, w.T)
    for p in range(w.T - 40, w.T, 7):
        q = t["Q"][:, p:p + 1].contiguous()
        ws.fill_(0xA5)
        a = hsa.decode(q, t["K"], t["V"], ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, ws=ws)
        ws.fill_(0xFF)
        b = hsa.decode(q, t["K"], t["V"], ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, ws=ws)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v), p


def test_decode_full_size_cache_steps():
    """The 128K-token cache, 256 steps with incremental summaries; every step against
    the oracle and against the two-call path (bit for bit)."""
    w = synth.workloads()["decode_128k"]
    x = synth.make_inputs(w)
    say(f"[decode full] cache {w.T} H{w.H} d{w.d} K{w.K}")
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    p0 = w.q_pos0
    NC = w.T // w.S
    ksum = torch.empty(1, NC, w.H, w.d, device=DEV)
    ent = torch.empty(1, NC, w.H, device=DEV)
    hsa.summarize(t["K"], t["Ql"], w.S, 0, p0 // w.S, Tkv=p0, ksum=ksum, ent=ent)
    oks, oent, _ = oracle.summarize(x["K"], x["Ql"], w.S)
    ws = hsa.decode_workspace(t["Q"][:, :1], t["K"], ksum, w.K, w.S, w.T - 1, w.T)
    # the oracle takes the whole cache (keys past a row's position are never read),
    # converted to float64 once
    Kd = np.ascontiguousarray(x["K"], dtype=np.float64)
    Vd = np.ascontiguousarray(x["V"], dtype=np.float64)
    n_excl = 0
    for s in range(w.rows_q):
        p = p0 + s
        if p % w.S == 0 and p > p0:
            c = p // w.S - 1
            hsa.summarize(t["K"], t["Ql"], w.S, c, c + 1, Tkv=p, ksum=ksum, ent=ent)
        q = t["Q"][:, s:s + 1].contiguous()
        got = hsa.decode(q, t["K"], t["V"], ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, ws=ws)
        idx, sc = hsa.score_topk(q, ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, Hkv=w.Hkv)
        O, lo, lt = hsa.attend_fuse(q, t["K"], t["V"], idx, sc, w.S, q_pos0=p, Tkv=p + 1)
        torch.cuda.synchronize()
        for a, b, nm in zip(got, (idx, sc, O, lo, lt), ("idx", "score", "O", "lse_own", "lse_tot")):
            assert torch.equal(a, b), (s, nm)
        qn = x["Q"][:, s:s + 1]
        oidx, osc, ogap = oracle.score_topk(qn, oks, oent, w.S, w.K, q_pos0=p)
        oO, _, olt = oracle.attend_fuse(qn, Kd, Vd, oidx, osc, w.S, q_pos0=p)
        excl, eq = compare_selection(host(got[0]), oidx, ogap, w.K,
                                     lambda d: all_scores(qn, oks, oent, w.S, d, q_pos0=p))
        n_excl += int(excl.sum())
        assert_close(host(got[2])[eq], oO[eq], TOL_BF16, f"O step {s}")
        assert_close(host(got[4])[eq], olt[eq], TOL_F32, f"lse_tot step {s}")
    say(f"  {w.rows_q} steps x {w.H} heads; near-tie rows excluded: {n_excl}")


def test_decode_host_resident_cache():
    """K and V in pinned host memory: the step reads the selected chunks and the local
    branch through the device mapping; results equal the device-resident cache."""
    w, W, nq = CASES["bf16_d64"]
    x = synth.make_inputs(w)
    t = {k: dev(x[k], w.dtype) for k in ("Q", "K", "V", "Ql")}
    Kh = torch.empty(t["K"].shape, dtype=torch.bfloat16, pin_memory=True)
    Vh = torch.empty(t["V"].shape, dtype=torch.bfloat16, pin_memory=True)
    Kh.copy_(t["K"])
    Vh.copy_(t["V"])
    ksum, ent, _ = hsa.summarize(t["K"], t["Ql"], w.S)
    ws = hsa.decode_workspace(t["Q"][:, :1], t["K"], ksum, w.K, w.S, w.T - 1, w.T)
    for p in (w.T - 1, w.T // 2):
        q = t["Q"][:, p:p + 1].contiguous()
        a = hsa.decode(q, t["K"], t["V"], ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, ws=ws)
        b = hsa.decode(q, Kh, Vh, ksum, ent, w.K, w.S, q_pos0=p, Tkv=p + 1, ws=ws)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v), p
