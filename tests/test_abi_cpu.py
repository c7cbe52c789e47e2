"""The C-ABI library loads, exports what its header declares, and rejects bad
host arguments before touching the GPU (CPU only: no kernel is launched)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
LIB = os.path.join(ROOT, "draft_token_verification_row_amd", "libspecverify.so")


@pytest.fixture(scope="module")
def sv():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._build_module().build(verbose=False)
    import draft_token_verification_row_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for need in ("spec_verify_greedy", "spec_verify_sample", "spec_verify_workspace_bytes",
                 "spec_verify_status_string"):
        assert need in names


def test_library_exports_every_declared_symbol(sv):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (spec_verify_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(sv.EXPORTED) == set(declared_functions())


def test_status_strings(sv):
    assert sv.spec_verify_status_string(0) == "ok"
    for s in range(1, 5):
        assert sv.spec_verify_status_string(s) not in ("ok", "unknown status")
    assert sv.spec_verify_status_string(99) == "unknown status"


def test_workspace_sizes(sv):
    assert sv.spec_verify_workspace_bytes(0, 0, 10) == 0
    assert sv.spec_verify_workspace_bytes(1, -1, 10) == 0
    assert sv.spec_verify_workspace_bytes(1, 0, 0) == 0
    assert sv.spec_verify_workspace_bytes(1, 0, (1 << 30) + 1) == 0
    a = sv.spec_verify_workspace_bytes(64, 192, 32000)
    b = sv.spec_verify_workspace_bytes(64, 192, 64000)
    c = sv.spec_verify_workspace_bytes(128, 192, 32000)
    assert 0 < a < b and a < c
    # the largest workload needs a few MB, not a copy of the logits
    assert sv.spec_verify_workspace_bytes(512, 3584, 262144) < 16 << 20
    # row units and residual units of one early-exit round together must fit
    # a 32-bit count, even when each alone does (V = 2^28: 32768 / 131072 units)
    assert sv.spec_verify_workspace_bytes(10000, 10000, 1 << 28) == 0
    assert sv.spec_verify_workspace_bytes(5000, 10000, 1 << 28) > 0


FAKE = 1 << 20   # never dereferenced: every call below fails a host check first


def _batch(sv, **kw):
    d = dict(B=4, K=8, V=1000, dtype=0, target_ld=1000, draft_ld=1000, num_draft=FAKE,
             target=FAKE, draft=FAKE, draft_tokens=FAKE)
    d.update(kw)
    return sv.SvBatch(**d)


def _sample(sv, bt, T=1.0, ws_bytes=None, ws=FAKE, ua=FAKE, uf=FAKE, acc=FAKE, out=FAKE):
    need = sv.spec_verify_workspace_bytes(max(bt.B, 1), max(bt.K, 0), max(bt.V, 1))
    wsb = need if ws_bytes is None else ws_bytes
    return sv.lib().spec_verify_sample(ctypes.byref(bt), ctypes.c_float(T), None, ua, uf, acc, out,
                                      None, None, None, ws, wsb, None)


def _greedy(sv, bt, ws_bytes=None, ws=FAKE, acc=FAKE, out=FAKE):
    need = sv.spec_verify_workspace_bytes(max(bt.B, 1), max(bt.K, 0), max(bt.V, 1))
    wsb = need if ws_bytes is None else ws_bytes
    return sv.lib().spec_verify_greedy(ctypes.byref(bt), acc, out, ws, wsb, None)


def test_host_validation_rejects_bad_arguments(sv):
    INV, UNS, WS = sv.SV_ERR_INVALID_ARG, sv.SV_ERR_UNSUPPORTED, sv.SV_ERR_WORKSPACE
    assert sv.lib().spec_verify_sample(None, ctypes.c_float(1.0), None, FAKE, FAKE, FAKE, FAKE,
                                      None, None, None, FAKE, 1 << 20, None) == INV
    assert _sample(sv, _batch(sv, B=0)) == INV
    assert _sample(sv, _batch(sv, K=-1)) == INV
    assert _sample(sv, _batch(sv, V=0)) == INV
    assert _sample(sv, _batch(sv, dtype=7)) == UNS
    assert _sample(sv, _batch(sv, target_ld=999)) == INV
    assert _sample(sv, _batch(sv, draft_ld=10)) == INV
    assert _sample(sv, _batch(sv, num_draft=None)) == INV
    assert _sample(sv, _batch(sv, target=None)) == INV
    assert _sample(sv, _batch(sv, draft=None)) == INV
    assert _sample(sv, _batch(sv, draft_tokens=None)) == INV
    assert _sample(sv, _batch(sv, target=FAKE + 2)) == INV          # fp32 rows must be 4-byte aligned
    assert _sample(sv, _batch(sv, dtype=1, target=FAKE + 1)) == INV  # bf16 rows 2-byte aligned
    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-39, 1e-45):
        assert _sample(sv, _batch(sv), T=T) == INV, T
    assert _sample(sv, _batch(sv), ua=None) == INV
    assert _sample(sv, _batch(sv), uf=None) == INV
    assert _sample(sv, _batch(sv), acc=None) == INV
    assert _sample(sv, _batch(sv), out=None) == INV
    assert _sample(sv, _batch(sv), ws=None) == WS
    need = sv.spec_verify_workspace_bytes(4, 8, 1000)
    assert _sample(sv, _batch(sv), ws_bytes=need - 1) == WS
    # greedy: no draft, temperature or uniforms needed, but the same size checks
    assert _greedy(sv, _batch(sv, B=0)) == INV
    assert _greedy(sv, _batch(sv, target_ld=3)) == INV
    assert _greedy(sv, _batch(sv), ws_bytes=need - 1) == WS
    assert _greedy(sv, _batch(sv), out=None) == INV
    # K = 0 needs no token pointer; still no launch because the workspace is short
    assert _greedy(sv, _batch(sv, K=0, draft_tokens=None), ws_bytes=0) == WS


def test_binding_argument_checks(sv):
    import torch
    t = torch.zeros(5, 10, dtype=torch.float16)
    with pytest.raises(ValueError):
        sv.make_batch_struct(t, None, torch.zeros(1, dtype=torch.int32),
                             torch.zeros(4, dtype=torch.int32))
    t = torch.zeros(10, 5).t()       # non-unit stride along the vocabulary
    with pytest.raises(ValueError):
        sv.make_batch_struct(t, None, torch.zeros(1, dtype=torch.int32),
                             torch.zeros(4, dtype=torch.int32))


def test_synthetic_layouts():
    import synth
    for cfg in (1, 2, 3, 4, 5):
        b = synth.make_batch(cfg, B=6, V=257)
        assert b.target.shape == (b.K + b.B, 257)
        assert b.tokens.shape == (b.K,)
        toks = b.tokens.numpy()
        assert toks.min(initial=0) >= 0 and toks.max(initial=0) < 257
        ua = b.u_accept.numpy().astype(np.float64)
        assert np.all((ua >= 0) & (ua < 1)) and np.all(ua * 2 ** 24 == np.round(ua * 2 ** 24))
        if cfg == 5:
            assert set(np.unique(b.greedy)) <= {0, 1} and b.greedy[1] == 1 and b.greedy[0] == 0
        if cfg == 2:
            assert b.draft is None and b.temperature is None
        else:
            assert b.draft.shape == (b.K, 257)
    # the same seed reproduces the batch
    x, y = synth.make_batch(3, B=3, V=100), synth.make_batch(3, B=3, V=100)
    assert torch_equal(x.target, y.target) and torch_equal(x.tokens, y.tokens)


def torch_equal(a, b):
    import torch
    return bool(torch.equal(a, b))


def test_accept_stats_host_validation(sv):
    INV = sv.SV_ERR_INVALID_ARG
    f = sv.lib().spec_verify_accept_stats
    assert f(None, FAKE, 4, 3, FAKE, None) == INV
    assert f(FAKE, None, 4, 3, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 3, None, None) == INV
    assert f(FAKE, FAKE, 0, 3, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 0, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 4097, FAKE, None) == INV


def test_early_exit_host_validation(sv):
    INV, WS = sv.SV_ERR_INVALID_ARG, sv.SV_ERR_WORKSPACE
    need = sv.spec_verify_workspace_bytes(4, 8, 1000)
    g = sv.lib().spec_verify_greedy_early_exit
    s = sv.lib().spec_verify_sample_early_exit

    def smp(bt, max_k, T=1.0, wsb=need, ua=FAKE):
        return s(ctypes.byref(bt), max_k, ctypes.c_float(T), None, ua, FAKE, FAKE, FAKE, None,
                 None, None, FAKE, wsb, None)

    for mk in (-1, 4097, -(1 << 30)):
        assert g(ctypes.byref(_batch(sv)), mk, FAKE, FAKE, FAKE, need, None) == INV, mk
        assert smp(_batch(sv), mk) == INV, mk
    assert g(None, 4, FAKE, FAKE, FAKE, need, None) == INV
    assert g(ctypes.byref(_batch(sv, B=0)), 4, FAKE, FAKE, FAKE, need, None) == INV
    assert g(ctypes.byref(_batch(sv)), 4, FAKE, None, FAKE, need, None) == INV
    assert g(ctypes.byref(_batch(sv)), 4, FAKE, FAKE, FAKE, need - 1, None) == WS
    assert smp(_batch(sv), 4, T=0.0) == INV
    assert smp(_batch(sv), 4, ua=None) == INV
    assert smp(_batch(sv), 4, wsb=need - 1) == WS
    assert smp(_batch(sv, draft=None), 4) == INV


def _tree(sv, **kw):
    d = dict(B=2, N=9, V=1000, dtype=0, target_ld=1000, num_nodes=FAKE, parent=FAKE, tokens=FAKE,
             target=FAKE)
    d.update(kw)
    return sv.SvTree(**d)


def test_tree_host_validation(sv):
    INV, UNS, WS = sv.SV_ERR_INVALID_ARG, sv.SV_ERR_UNSUPPORTED, sv.SV_ERR_WORKSPACE
    need = sv.spec_verify_tree_workspace_bytes(2, 9, 1000)
    assert need > 0
    assert sv.spec_verify_tree_workspace_bytes(2, 1, 1000) == 0      # N < B
    assert sv.spec_verify_tree_workspace_bytes(0, 1, 1000) == 0
    assert sv.spec_verify_tree_workspace_bytes(1, 1, 0) == 0
    g = sv.lib().spec_verify_tree_greedy
    e = sv.lib().spec_verify_tree_greedy_early_exit

    def call(tr, wsb=need, acc=FAKE, path=FAKE, out=FAKE, ws=FAKE):
        return g(ctypes.byref(tr) if tr is not None else None, acc, path, out, ws, wsb, None)

    assert call(None) == INV
    assert call(_tree(sv, B=0)) == INV
    assert call(_tree(sv, N=1)) == INV
    assert call(_tree(sv, V=0)) == INV
    assert call(_tree(sv, dtype=3)) == UNS
    assert call(_tree(sv, target_ld=10)) == INV
    for f in ("num_nodes", "parent", "tokens", "target"):
        assert call(_tree(sv, **{f: None})) == INV, f
    assert call(_tree(sv, target=FAKE + 2)) == INV
    assert call(_tree(sv), acc=None) == INV
    assert call(_tree(sv), path=None) == INV
    assert call(_tree(sv), out=None) == INV
    assert call(_tree(sv), ws=None) == WS
    assert call(_tree(sv), wsb=need - 1) == WS
    for md in (-1, 4097):
        assert e(ctypes.byref(_tree(sv)), md, FAKE, FAKE, FAKE, FAKE, need, None) == INV
    assert e(ctypes.byref(_tree(sv)), 3, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WS


def test_tree_binding_checks(sv):
    import torch
    t = torch.zeros(4, 10)
    i32 = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        sv.make_tree_struct(t, i32.long(), i32, torch.ones(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.make_tree_struct(t, i32, torch.zeros(3, dtype=torch.int32), torch.ones(1, dtype=torch.int32))


def test_tree_synthetic_shapes():
    import synth
    tb = synth.make_tree_batch(1)
    off = tb.offsets
    par = tb.parent.numpy()
    tok = tb.tokens.numpy()
    for b in range(tb.B):
        s, n = int(off[b]), int(tb.num_nodes[b])
        assert par[s] == -1
        for i in range(1, n):
            assert 0 <= par[s + i] < i
        for i in range(n):      # sibling tokens are distinct
            kids = [tok[s + c] for c in range(1, n) if par[s + c] == i]
            assert len(kids) == len(set(kids))


def test_adaptive_and_gather_host_validation(sv):
    INV, UNS = sv.SV_ERR_INVALID_ARG, sv.SV_ERR_UNSUPPORTED
    f = sv.lib().spec_verify_adaptive_length
    assert f(0, 7, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == INV
    assert f(4, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == INV
    assert f(4, 4097, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == INV
    assert f(4, 7, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == INV
    assert f(4, 7, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, None) == INV
    assert f(4, 7, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None) == INV
    assert f(4, 7, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, None) == INV
    assert f(4, 7, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None) == INV
    assert f(4, 7, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None) == INV
    g = sv.lib().spec_verify_gather_rows
    assert g(5, 100, FAKE, 100, 4, FAKE, FAKE, 4, FAKE, 100, None) == UNS
    assert g(1, 0, FAKE, 100, 4, FAKE, FAKE, 4, FAKE, 100, None) == INV
    assert g(1, 100, FAKE, 99, 4, FAKE, FAKE, 4, FAKE, 100, None) == INV
    assert g(1, 100, FAKE, 100, 4, FAKE, FAKE, 4, FAKE, 50, None) == INV
    assert g(1, 100, None, 100, 4, FAKE, FAKE, 4, FAKE, 100, None) == INV
    assert g(1, 100, FAKE, 100, 4, None, FAKE, 4, FAKE, 100, None) == INV
    assert g(1, 100, FAKE, 100, 4, FAKE, None, 4, FAKE, 100, None) == INV
    assert g(1, 100, FAKE, 100, 4, FAKE, FAKE, -1, FAKE, 100, None) == INV
    assert g(1, 100, FAKE + 1, 100, 4, FAKE, FAKE, 4, FAKE, 100, None) == INV
    assert g(1, 100, FAKE, 100, 4, FAKE, FAKE, 0, FAKE, 100, None) == sv.SV_OK   # nothing to copy


def test_launch_plan_values(sv):
    for bad in (-1, 3, 99):
        assert sv.lib().spec_verify_set_launch_plan(bad) == sv.SV_ERR_INVALID_ARG
    for ok in (1, 2, 0):
        assert sv.lib().spec_verify_set_launch_plan(ok) == sv.SV_OK


def test_read_probe_rejects_bad_arguments(sv):
    f = sv.lib().spec_verify_read_probe
    assert f(None, 16, 8, None) == sv.SV_ERR_INVALID_ARG          # no source
    assert f(16, 16, None, None) == sv.SV_ERR_INVALID_ARG          # no sink
    assert f(16, 24, 8, None) == sv.SV_ERR_INVALID_ARG             # not whole 16-byte chunks
    assert f(8, 16, 8, None) == sv.SV_ERR_INVALID_ARG              # misaligned source


def _noalloc(sv, bt, T=1.0, ua=FAKE, uf=FAKE, acc=FAKE, out=FAKE):
    return sv.lib().spec_verify_sample_noalloc(ctypes.byref(bt), ctypes.c_float(T), None, ua, uf,
                                              acc, out, None, None, None, None)


def test_noalloc_host_validation(sv):
    """The entry point that uses the library's static workspace runs the same
    host checks as spec_verify_sample, and refuses a call whose workspace
    would exceed its array, before any HIP call (so also without a GPU)."""
    INV, UNS, WS = sv.SV_ERR_INVALID_ARG, sv.SV_ERR_UNSUPPORTED, sv.SV_ERR_WORKSPACE
    assert sv.lib().spec_verify_sample_noalloc(None, ctypes.c_float(1.0), None, FAKE, FAKE, FAKE,
                                              FAKE, None, None, None, None) == INV
    assert _noalloc(sv, _batch(sv, B=0)) == INV
    assert _noalloc(sv, _batch(sv, dtype=7)) == UNS
    assert _noalloc(sv, _batch(sv, draft=None)) == INV
    assert _noalloc(sv, _batch(sv), T=0.0) == INV
    assert _noalloc(sv, _batch(sv), uf=None) == INV
    assert _noalloc(sv, _batch(sv), out=None) == INV
    big = dict(B=4096, K=65536, V=262144, target_ld=262144, draft_ld=262144)
    assert sv.spec_verify_workspace_bytes(4096, 65536, 262144) > sv.NOALLOC_MAX_BYTES
    assert _noalloc(sv, _batch(sv, **big)) == WS
