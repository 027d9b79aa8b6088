"""C-ABI checks that need no GPU: exports, status strings, workspace sizing and
argument validation (every error path returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import hierarchical_sparse_attention_amd as hsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "hils.h")).read()
    return sorted(set(re.findall(r"^\s*(?:hils_status|const char\*|int32_t)\s+(hils_\w+)\s*\(",
                                 text, re.M)))


def test_library_exports_every_declared_function():
    L = hsa.lib()
    names = header_functions()
    assert set(names) == set(hsa.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = hsa.lib()
    for code, name in hsa.STATUS.items():
        assert L.hils_status_string(code).decode().startswith(name)
    assert L.hils_status_string(99) == b"unknown hils_status"
    assert L.hils_version() == 100


def base(**kw):
    a = dict(B=1, Tq=128, Tkv=128, H=2, Hkv=1, d=64, S=64, K=4, dtype=hsa.HILS_BF16)
    a.update(kw)
    return hsa.make_dims(**a)


def ws_size(dims, op):
    n = ctypes.c_size_t(12345)
    st = hsa.lib().hils_workspace_size(ctypes.byref(dims), op, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(S=32), 2), (dict(d=96), 2), (dict(K=65), 2),
    (dict(S=0), 1), (dict(d=0), 1), (dict(K=0), 1),
    (dict(H=3, Hkv=2), 1), (dict(B=0), 1), (dict(Tkv=0), 1), (dict(Tq=-1), 1),
    (dict(dtype=7), 1), (dict(q_pos0=1), 1), (dict(Tkv_cap=64), 1), (dict(NC_cap=1), 1),
    (dict(scale=-1.0), 1), (dict(scale=float("nan")), 1),
])
def test_dims_validation(kw, status):
    st, _ = ws_size(base(**kw), hsa.OP_ATTEND_FUSE)
    assert st == status


def test_window_field_and_select_mode():
    for wnd, status in ((-64, 1), (32, 2), (96, 2), (64 * 33, 2), (64, 0), (512, 0), (2048, 0)):
        assert ws_size(base(window=wnd), hsa.OP_ATTEND_FUSE)[0] == status, wnd
    d = base()
    d.select_mode = 2                                    # no such selection
    assert ws_size(d, hsa.OP_SCORE_TOPK)[0] == 1
    d = base(H=8, Hkv=2)
    d.select_mode = 1                                    # group max, G = 4
    assert ws_size(d, hsa.OP_SCORE_TOPK)[0] == 0
    d = base(H=6, Hkv=2)
    d.select_mode = 1                                    # G = 3: not a power of two
    assert ws_size(d, hsa.OP_SCORE_TOPK)[0] == 2


def test_workspace_sizes():
    assert ws_size(base(), hsa.OP_SUMMARIZE) == (0, 0)
    assert ws_size(base(), 9)[0] == 1
    # decode-like: few rows, many candidates -> split scoring needs workspace
    st, n = ws_size(base(Tq=1, Tkv=131073, q_pos0=131072, H=16, Hkv=16, K=16),
                    hsa.OP_SCORE_TOPK)
    assert st == 0 and n >= 16 * 8 * 16 * 8
    st, n = ws_size(base(Tq=4096, Tkv=4096), hsa.OP_BACKWARD)
    assert st == 0 and n >= 4096 * 2 * 4 * 4
    # backward needs a prefill layout
    assert ws_size(base(Tq=64, Tkv=128, q_pos0=64), hsa.OP_BACKWARD)[0] == 2


def test_entry_points_reject_bad_pointers_without_launching():
    L = hsa.lib()
    d = base()
    p = ctypes.c_void_p(4096)       # aligned but never dereferenced: validation fails first
    mis = ctypes.c_void_p(4100)     # misaligned
    nul = None
    assert L.hils_summarize(ctypes.byref(d), nul, p, 0, 2, p, p, p, nul, 0, nul) == 1
    assert L.hils_summarize(ctypes.byref(d), p, p, 0, 3, p, p, p, nul, 0, nul) == 1  # c_end > NC
    assert L.hils_summarize(ctypes.byref(d), p, p, 2, 1, p, p, p, nul, 0, nul) == 1
    assert L.hils_summarize(ctypes.byref(d), p, p, 1, 1, p, p, p, nul, 0, nul) == 0  # empty range
    assert L.hils_score_topk(ctypes.byref(d), mis, p, p, p, p, nul, 0, nul) == 1
    assert L.hils_attend_fuse(ctypes.byref(d), p, p, p, p, p, nul, p, p, nul, 0, nul) == 1
    assert L.hils_backward(ctypes.byref(d), *([p] * 15), nul, nul, nul, nul, 0, nul) == 1
    d2 = base(Tq=4096, Tkv=4096)
    n = ws_size(d2, hsa.OP_BACKWARD)[1]
    big = ctypes.c_void_p(1 << 40)
    # the Q-Cal pair is both NULL or both set, 16-byte aligned
    assert L.hils_backward(ctypes.byref(d2), *([p] * 16), p, nul, big, n, nul) == 1
    assert L.hils_backward(ctypes.byref(d2), *([p] * 16), nul, p, big, n, nul) == 1
    assert L.hils_backward(ctypes.byref(d2), *([p] * 16), mis, p, big, n, nul) == 1
    assert L.hils_backward(ctypes.byref(d2), *([p] * 16), p, p, big, n - 1, nul) == 3
    dd = base(Tq=1, Tkv=131073, q_pos0=131072, H=16, Hkv=16, K=16)
    assert L.hils_score_topk(ctypes.byref(dd), p, p, p, p, p, p, 8, nul) == 3   # workspace short
    assert L.hils_score_topk(None, p, p, p, p, p, nul, 0, nul) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    K = torch.zeros(1, 128, 1, 64, dtype=torch.bfloat16)
    Ql = torch.zeros(1, 2, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hsa.summarize(K, Ql)


@pytest.mark.parametrize("B,H", [(1, 16), (8, 16), (16, 16), (4, 32)])
def test_decode_workspace_covers_both_calls(B, H):
    """hils_decode takes the two calls (score_topk, then attend_fuse) where its
    merged or per-row plans do not apply: in the first chunk, with no
    candidates, and for a batch of 128 rows and more at shapes the per-row
    kernel does not take. Wherever it may take them, its workspace is at least
    what either call needs; and it never shrinks as the cache grows, so a
    workspace sized for the last position of a decode serves every earlier one."""
    prev = 0
    for p in (0, 1, 63, 64, 65, 1000, 4096, 65536, 131071):
        d = base(B=B, Tq=1, Tkv=p + 1, q_pos0=p, H=H, Hkv=H, K=16)
        st_dec, dec = ws_size(d, hsa.OP_DECODE)
        st_sc, sc = ws_size(d, hsa.OP_SCORE_TOPK)
        st_at, at = ws_size(d, hsa.OP_ATTEND_FUSE)
        assert st_dec == st_sc == st_at == 0, (p, st_dec, st_sc, st_at)
        if B * H >= 128 or p < 64:
            assert dec >= max(sc, at), (B, H, p, dec, sc, at)
        assert dec >= prev, (B, H, p, dec, prev)
        prev = dec
