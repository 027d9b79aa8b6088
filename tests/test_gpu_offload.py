"""Decode over a host-resident KV cache (the news article's inference story: the
KV of unselected chunks sits in CPU memory). K and V live in pinned host memory;
the summaries, the selection and the outputs stay on the GPU. The kernels read
the cache through its device mapping, so every result must equal, bit for bit,
the one computed from the same cache in device memory."""
import ctypes

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hsa
import oracle
import synth
from hils_testutil import TOL_BF16, TOL_F32, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_decode(td, K, V, w, steps, K_sel, window):
    """Summaries of the cached prefix, then decode steps that summarise each chunk as
    it completes; returns the per-step (idx, score, O, lse_tot) on the host."""
    NC = w.T // w.S
    p0 = w.q_pos0
    ksum, ent, lse_l = hsa.summarize(K, td["Ql"], w.S, 0, p0 // w.S, Tkv=p0)
    out = []
    for s in steps:
        p = p0 + s
        if p % w.S == 0 and p > p0:
            c = p // w.S - 1
            hsa.summarize(K, td["Ql"], w.S, c, c + 1, Tkv=p, ksum=ksum, ent=ent, lse_l=lse_l)
        q = td["Q"][:, s:s + 1].contiguous()
        idx, sc = hsa.score_topk(q, ksum, ent, K_sel, w.S, p, p + 1, Hkv=w.Hkv, window=window)
        O, lo, lt = hsa.attend_fuse(q, K, V, idx, sc, w.S, p, p + 1, window=window)
        torch.cuda.synchronize()
        out.append(tuple(a.cpu() for a in (idx, sc, O, lt)))
    assert NC >= (p0 + max(steps)) // w.S
    return out


@pytest.mark.parametrize("K_sel,window", [(8, 0), (16, 512)])
def test_decode_with_host_resident_cache(K_sel, window):
    w = synth.small("offload", B=1, T=4096 + 128, H=4, Hkv=2, d=64, K=K_sel, dtype="bf16",
                    Tq=128, q_pos0=4096, n_planted=3)
    x = synth.make_inputs(w)
    say(f"[decode, host-resident cache] K {K_sel} window {window}")
    td = {k: torch.from_numpy(x[k]).to(DEV, torch.bfloat16) for k in ("Q", "K", "V", "Ql")}
    Kh = torch.empty(td["K"].shape, dtype=torch.bfloat16, pin_memory=True)
    Vh = torch.empty(td["V"].shape, dtype=torch.bfloat16, pin_memory=True)
    Kh.copy_(td["K"])
    Vh.copy_(td["V"])
    torch.cuda.synchronize()
    steps = [0, 1, 63, 64, 65, 127]
    dev_run = run_decode(td, td["K"], td["V"], w, steps, K_sel, window)
    host_run = run_decode(td, Kh, Vh, w, steps, K_sel, window)
    for s, a, b in zip(steps, dev_run, host_run):
        for name, u, v in zip(("idx", "score", "O", "lse_tot"), a, b):
            assert torch.equal(u, v), (s, name)
    # and the device-resident result is the oracle's (last step)
    s = steps[-1]
    p = w.q_pos0 + s
    Kc, Vc = x["K"][:, :p + 1], x["V"][:, :p + 1]
    oks, oent, _ = oracle.summarize(Kc, x["Ql"][:, :(p + 1) // w.S], w.S)
    q = x["Q"][:, s:s + 1]
    oidx, osc, ogap = oracle.score_topk(q, oks, oent, w.S, K_sel, q_pos0=p, window=window)
    oO, _, olt = oracle.attend_fuse(q, Kc, Vc, oidx, osc, w.S, q_pos0=p, window=window)
    eq = np.all(host_run[-1][0].numpy() == oidx, axis=-1)
    assert eq.all()
    assert_close(host_run[-1][2].float().numpy(), oO, TOL_BF16, "O")
    assert_close(host_run[-1][3].numpy(), olt, TOL_F32, "lse_tot")


def test_pageable_host_cache_is_rejected():
    """Memory no kernel can read (pageable host memory) is refused before any launch."""
    w = synth.small("offload_bad", B=1, T=256, H=2, Hkv=1, d=64, K=2, dtype="bf16")
    L = hsa.lib()
    K = np.zeros((1, 256, 1, 64), dtype=np.uint16)   # pageable host buffer
    Ql = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    ksum = torch.empty(1, 4, 2, 64, device=DEV)
    ent = torch.empty(1, 4, 2, device=DEV)
    dims = hsa.make_dims(1, 0, 256, 2, 1, 64, 64, 1, hsa.HILS_BF16)
    st = L.hils_summarize(ctypes.byref(dims), ctypes.c_void_p(K.ctypes.data),
                          ctypes.c_void_p(Ql.data_ptr()), 0, 4, ctypes.c_void_p(ksum.data_ptr()),
                          ctypes.c_void_p(ent.data_ptr()), None, None, 0, None)
    assert st == 1
    assert w.T == 256
    with pytest.raises(ValueError):   # the binding refuses it first
        hsa.summarize(torch.from_numpy(K.view(np.int16)).view(torch.bfloat16), Ql, 64)
