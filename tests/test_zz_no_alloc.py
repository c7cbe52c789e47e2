"""spec_verify_sample_noalloc (static device workspace) against
spec_verify_sample (caller workspace), through the C ABI (needs the GPU).

Two calls in a row on the same device, the second with a smaller batch: the
outputs must equal those of the workspace entry point bit for bit, so nothing
the first call left in the static array leaks into the second.  A batch whose
workspace exceeds SPEC_VERIFY_NOALLOC_MAX_BYTES is refused before any launch.
"""
import ctypes
import os
import re
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _header_max_bytes():
    text = open(os.path.join(ROOT, "include", "spec_verify.h")).read()
    m = re.search(r"#define\s+SPEC_VERIFY_NOALLOC_MAX_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    return int(m.group(1)) << int(m.group(2))


def _outputs(batch, fill):
    dev = batch.target.device
    return dict(acc=torch.full((batch.B,), fill, dtype=torch.int32, device=dev),
                out=torch.full((batch.K + batch.B,), fill, dtype=torch.int32, device=dev),
                p=torch.full((max(batch.K, 1),), float(fill), dtype=torch.float32, device=dev),
                q=torch.full((max(batch.K, 1),), float(fill), dtype=torch.float32, device=dev),
                rm=torch.full((batch.B,), float(fill), dtype=torch.float32, device=dev))


def _call(sv, batch, noalloc, fill):
    lib = sv.lib()
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
    bt = sv.make_batch_struct(batch.target, batch.draft, batch.tokens, nd)
    o = _outputs(batch, fill)
    T = ctypes.c_float(batch.temperature)
    ptrs = (gm.data_ptr(), batch.u_accept.data_ptr(), batch.u_final.data_ptr(),
            o["acc"].data_ptr(), o["out"].data_ptr(), o["p"].data_ptr(), o["q"].data_ptr(),
            o["rm"].data_ptr())
    sh = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = lib.spec_verify_sample_noalloc(ctypes.byref(bt), T, *ptrs, sh)
    else:
        wsb = sv.spec_verify_workspace_bytes(batch.B, batch.K, batch.V)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        st = lib.spec_verify_sample(ctypes.byref(bt), T, *ptrs, ws.data_ptr(), wsb, sh)
    torch.cuda.synchronize()
    return st, {k: v.cpu().numpy() for k, v in o.items()}


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    import draft_token_verification_row_amd as sv
    assert sv.NOALLOC_MAX_BYTES == _header_max_bytes()
    big = synth.make_batch(5, DEV, B=48, V=70001)
    small = synth.make_batch(3, DEV, B=5, V=3001, seed=9)
    for label, batch in (("first, B=48 V=70001", big), ("second, smaller: B=5 V=3001", small)):
        _log(f"[noalloc] {label}")
        st_n, got = _call(sv, batch, True, -7)
        st_w, want = _call(sv, batch, False, -9)
        assert st_n == 0 and st_w == 0, (st_n, st_w)
        for k in want:
            assert np.array_equal(got[k].view(np.int32), want[k].view(np.int32)), (label, k)
        assert np.all(got["acc"] >= 0)


def test_noalloc_refuses_a_workspace_beyond_the_static_array():
    import draft_token_verification_row_amd as sv
    # a batch whose workspace exceeds the array; only its sizes are checked,
    # so small tensors stand in for the logits (nothing is launched)
    B, K, V = 1 << 16, 1 << 20, 1 << 14
    assert sv.spec_verify_workspace_bytes(B, K, V) > sv.NOALLOC_MAX_BYTES
    t = torch.zeros((4, 16), dtype=torch.float32, device=DEV)
    nd = torch.zeros(4, dtype=torch.int32, device=DEV)
    toks = torch.zeros(1, dtype=torch.int32, device=DEV)
    bt = sv.make_batch_struct(t, t, toks, nd)
    bt.B, bt.K, bt.V, bt.target_ld, bt.draft_ld = B, K, V, V, V
    out = torch.full((8,), 5, dtype=torch.int32, device=DEV)
    st = sv.lib().spec_verify_sample_noalloc(ctypes.byref(bt), ctypes.c_float(1.0), None,
                                             t.data_ptr(), t.data_ptr(), out.data_ptr(),
                                             out.data_ptr(), None, None, None,
                                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == sv.SV_ERR_WORKSPACE
    assert torch.all(out == 5)
