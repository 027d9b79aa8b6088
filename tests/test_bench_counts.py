"""The bench's algorithmic work counts, checked on the CPU against direct
enumeration: for every query row, the chunks it may select are the complete
chunks that end before its local branch starts (its own chunk, or its sliding
window), and it reads every key of its local branch and S keys per selected
chunk. Roofline blocks divide that work by the launch duration."""
import os
import sys
from types import SimpleNamespace

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def enumerate_counts(B, T, H, S, window, idx):
    cand = own = 0
    for i in range(T):
        first_local = max(0, i - window + 1) if window else (i // S) * S
        chunks = [c for c in range(T // S) if (c + 1) * S - 1 < first_local]
        cand += len(chunks)
        own += len(range(first_local, i + 1))
    cand *= B * H
    own *= B * H
    sel = int(np.count_nonzero(idx >= 0))
    return cand, sel * S + own


@pytest.mark.parametrize("window", [0, 128, 64])
def test_prefill_counts_match_enumeration(window):
    B, T, H, Hkv, d, S, K = 2, 512, 4, 2, 64, 64, 3
    rng = np.random.default_rng(7)
    idx = rng.integers(-1, T // S, size=(B, T, H, K)).astype(np.int32)
    w = SimpleNamespace(B=B, T=T, H=H, Hkv=Hkv, d=d, S=S, K=K)
    c = bench.prefill_counts(w, idx, window)
    cand, visits = enumerate_counts(B, T, H, S, window, idx)
    assert c["candidates"] == cand
    assert c["key_visits"] == visits
    assert c["attend_flops"] == 4 * d * visits       # q.k and p.v per key visit
    assert c["backward_flops"] == 10 * d * visits
    assert c["score_flops"] == 2 * d * cand


def test_summary_bytes_of_the_7b_gqa_prefill():
    # K read once per kv head, every landmark query read, a (d + 2)-float record
    # written per (chunk, head): 67,108,864 + 4,194,304 + 8,519,680 bytes
    w = SimpleNamespace(B=1, T=32768, H=32, Hkv=8, d=128, S=64, K=16)
    c = bench.prefill_counts(w, np.full((1, 1, 1, 1), -1, np.int32))
    assert c["summarize_bytes"] == 79_822_848


@pytest.mark.parametrize("p", [0, 63, 64, 1000, 131071])
@pytest.mark.parametrize("window", [0, 512])
def test_decode_step_bytes_match_enumeration(p, window):
    wd = SimpleNamespace(H=16, Hkv=16, d=64, S=64)
    K = 16
    first_local = max(0, p - window + 1) if window else (p // 64) * 64
    n = sum(1 for c in range(p // 64 + 1) if (c + 1) * 64 - 1 < first_local)
    nloc = p + 1 - first_local
    want = (n * 16 * 65 * 4                 # summary keys and entropies of the candidates
            + 16 * min(K, n) * 64 * 64 * 4  # K and V of the selected chunks
            + 16 * nloc * 64 * 4            # K and V of the local branch
            + 2 * 16 * 64 * 2               # query and output
            + 16 * K * 8)                   # selected ids and scores
    assert bench.decode_step_bytes(wd, K, window, p) == want


def test_roofline_block():
    b = bench.roofline("k", "mfma", 2.5e12, 2.0, traffic=1e9)
    assert b["bound"] == "mfma" and b["unit"] == "TFLOP/s" and b["peak"] == 2500.0
    assert b["achieved"] == pytest.approx(1250.0) and b["frac"] == pytest.approx(0.5)
    b = bench.roofline("k", "hbm", 8e9, 1.0)
    assert b["unit"] == "GB/s" and b["frac"] == pytest.approx(1.0) and b["traffic"] is None
