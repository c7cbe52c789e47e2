"""Confidence-driven verification length and row gather on the GPU (needs the GPU).

The lengths, offsets, compacted tokens and source indices are integers and must
equal the oracle's exactly; the progress values are formed in fp64 in the same
order on both sides and must be identical too.  The gather is a copy and must
reproduce the selected rows bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.adaptive as oa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(ab_conf, cost, tokens, got, label):
    ref = oa.adaptive_batch(ab_conf, cost, tokens)
    nd = got["num_draft"].cpu().numpy().astype(np.int64)
    off = got["offsets"].cpu().numpy().astype(np.int64)
    assert np.array_equal(nd, ref["num_draft"]), label
    assert np.array_equal(off, ref["offsets"]), label
    K = int(ref["offsets"][-1])
    assert np.array_equal(got["tokens"].cpu().numpy()[:K].astype(np.int64), ref["tokens"]), label
    if got["src_index"] is not None:
        assert np.array_equal(got["src_index"].cpu().numpy()[:K].astype(np.int64), ref["src_index"]), label
    if got["progress"] is not None:
        assert np.array_equal(got["progress"].cpu().numpy(), ref["progress"]), label
    return ref


CASES = [("block7_B512", dict(B=512, N=7)), ("block15_B64", dict(B=64, N=15)),
         ("block1_B3000", dict(B=3000, N=1)), ("block0", dict(B=10, N=0)),
         ("steep_cost", dict(B=300, N=7, slope=0.6)), ("flat_cost", dict(B=300, N=7, slope=0.0)),
         ("block64_B33", dict(B=33, N=64))]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_adaptive_parity(label, kw):
    import draft_token_verification_row_amd as sv
    ab = synth.make_adaptive_batch(device=DEV, V=100, with_rows=False, **kw)
    got = sv.spec_verify_adaptive_length(ab.conf, ab.cost, ab.tokens)
    torch.cuda.synchronize()
    ref = _check(ab.conf.cpu().numpy(), ab.cost.cpu().numpy(), ab.tokens.cpu().numpy(), got, label)
    _log(f"[adaptive] {label}: K'={int(ref['offsets'][-1])} of {ab.B * ab.N}, "
         f"k histogram {np.bincount(ref['num_draft'], minlength=ab.N + 1).tolist()}")


def test_adaptive_ties_and_errors():
    import draft_token_verification_row_amd as sv
    conf = torch.tensor([[0.9, 0.9, 0.0, 0.5], [0.0, 0.9, 0.9, 0.9], [0.9, 0.9, 0.9, 0.9],
                         [1.0, 1.0, 1.0, 1.0]], dtype=torch.float32, device=DEV)
    toks = torch.arange(16, dtype=torch.int32, device=DEV).reshape(4, 4) + 100
    for cost in ([1.0] * 5, [1.0, 2.0, 3.0, 4.0, 5.0], [1.0, 1.5, 2.0, 2.5, 3.0]):
        c = torch.tensor(cost, dtype=torch.float64, device=DEV)
        got = sv.spec_verify_adaptive_length(conf, c, toks)
        torch.cuda.synchronize()
        _check(conf.cpu().numpy(), np.array(cost), toks.cpu().numpy(), got, str(cost))
    for bad in ([1.0, 1.0, 0.0, 1.0, 1.0], [1.0, -2.0, 1.0, 1.0, 1.0],
                [1.0, float("nan"), 1.0, 1.0, 1.0], [1.0, 1.0, float("inf"), 1.0, 1.0]):
        c = torch.tensor(bad, dtype=torch.float64, device=DEV)
        got = sv.spec_verify_adaptive_length(conf, c, toks)
        torch.cuda.synchronize()
        assert torch.all(got["num_draft"] == -1) and torch.all(got["offsets"] == 0), bad
        assert torch.all(got["progress"] == -1.0), bad


@pytest.mark.parametrize("V,dtype,pad", [(262144, "bf16", 0), (4097, "f32", 0), (1003, "bf16", 5),
                                         (33, "f32", 3)])
def test_gather_rows(V, dtype, pad):
    import draft_token_verification_row_amd as sv
    B, N = (512, 7) if V == 262144 else (40, 5)
    ab = synth.make_adaptive_batch(B=B, N=N, V=V, dtype=dtype, device=DEV)
    src = ab.draft
    if pad:
        big = torch.zeros(B * N, V + pad, dtype=src.dtype, device=DEV)
        big[:, :V] = src
        src = big[:, :V]
    sel = sv.spec_verify_adaptive_length(ab.conf, ab.cost, ab.tokens)
    K = int(sel["offsets"][-1].item())
    out = torch.full((B * N, V + pad), 7.0, dtype=src.dtype, device=DEV)[:, :V]
    sv.spec_verify_gather_rows(src, sel["src_index"], sel["offsets"][B:], B * N, out=out)
    torch.cuda.synchronize()
    idx = sel["src_index"][:K].long()
    assert torch.equal(out[:K], src.index_select(0, idx)), (V, dtype, pad)
    assert torch.all(out[K:] == 7.0)                     # rows past the count untouched
    _log(f"[gather] V={V} {dtype} pad={pad}: {K} rows")


def test_gather_skips_bad_indices_and_caps_rows():
    import draft_token_verification_row_amd as sv
    src = torch.randn(10, 300, device=DEV).to(torch.bfloat16)
    index = torch.tensor([3, -1, 9, 10, 0, 2], dtype=torch.int32, device=DEV)
    count = torch.tensor([6], dtype=torch.int32, device=DEV)
    out = torch.zeros(6, 300, dtype=torch.bfloat16, device=DEV)
    sv.spec_verify_gather_rows(src, index, count, 5, out=out)   # cap at 5 rows
    torch.cuda.synchronize()
    assert torch.equal(out[0], src[3]) and torch.equal(out[2], src[9]) and torch.equal(out[4], src[0])
    assert torch.all(out[1] == 0) and torch.all(out[3] == 0)    # index -1 and 10: skipped
    assert torch.all(out[5] == 0)                                # beyond max_rows
