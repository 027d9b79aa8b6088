"""Seeded input generator: determinism, rounding and workload structure."""
import numpy as np

import synth


def test_deterministic_and_streams_differ():
    a = synth.normal(7, 1, 1001)
    b = synth.normal(7, 1, 1001)
    c = synth.normal(7, 2, 1001)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # random access: a window equals the slice of the full stream
    assert np.array_equal(synth.normal(7, 1, 10, start=500), a[500:510])
    assert abs(a.mean()) < 0.15 and abs(a.std() - 1) < 0.1


def test_bf16_round_to_nearest_even():
    one = 1.0
    vals = np.array([one + 2.0**-8, one + 3 * 2.0**-8, -(one + 2.0**-8), 3.0, 1e-3], np.float32)
    r = synth.round_bf16(vals)
    assert r[0] == 1.0 and r[1] == 1.0 + 2.0**-6 and r[2] == -1.0 and r[3] == 3.0
    assert np.all(r.view(np.uint32) & 0xFFFF == 0)


def test_workload_structure():
    w = synth.small("s", T=1024, H=4, Hkv=2, d=32, S=64, K=4, dtype="bf16", n_planted=2,
                    n_uniform=3)
    x = synth.make_inputs(w)
    assert x["Q"].shape == (1, 1024, 4, 32) and x["K"].shape == (1, 1024, 2, 32)
    assert x["Ql"].shape == (1, 16, 4, 32)
    pc, uc = x["planted_chunks"][0], x["uniform_chunks"][0]
    assert len(set(pc) | set(uc)) == 5
    for c in pc:   # two keys per planted chunk share the planted vector of norm ~3
        for g in range(2):
            rows = x["K"][0, c * 64:(c + 1) * 64, g]
            norms = np.linalg.norm(rows, axis=1)
            hits = np.where(np.abs(norms - 3.0) < 0.05)[0]
            assert len(hits) >= 2
    for c in uc:   # near-uniform: keys within 0.05-noise of a shared vector
        rows = x["K"][0, c * 64:(c + 1) * 64, 0].astype(np.float64)
        assert np.std(rows - rows.mean(0)) < 0.07
    for k in ("Q", "K", "V", "Ql"):
        assert np.all(x[k].view(np.uint32) & 0xFFFF == 0)


def test_named_workload_counts():
    ws = synth.workloads()
    assert ws["prefill_345m"].n_planted == 1
    assert ws["decode_128k"].n_planted == 20
    assert (ws["prefill_7b_gqa"].n_planted, ws["prefill_7b_gqa"].n_uniform) == (3, 26)
    assert ws["train_345m"].n_planted == 3
