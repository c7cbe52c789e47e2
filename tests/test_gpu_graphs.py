"""The entry points can be captured into a HIP graph by the caller (no memsets,
no synchronising calls inside).  Each graph is replayed several times with eager
work and synchronisations between replays and new inputs copied in place; every
replay must equal an eager call on the same inputs (needs the GPU)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _eager_then_graph(make_call, refresh, outputs, n_replays=4, written=None):
    """make_call() launches on the current stream into fixed output tensors;
    written(outputs) -> the views the call defines (default: all of them)."""
    written = written or (lambda outs: outs)
    make_call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        make_call()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        make_call()
    for r in range(n_replays):
        refresh(r)                       # new inputs, in place
        torch.cuda.synchronize()
        make_call()                      # eager reference on the same inputs
        torch.cuda.synchronize()
        want = [o.clone() for o in written(outputs)]
        for o in outputs:
            o.fill_(-7)
        _ = torch.ones(1 << 20, device=DEV).sum()    # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(written(outputs), want):
            assert torch.equal(o, w), f"replay {r}"


@pytest.mark.parametrize("plan,max_k", [(1, None), (2, None), (0, "ee")])
def test_sample_in_graph(plan, max_k):
    import draft_token_verification_row_amd as sv
    batch = synth.make_batch(5, DEV, B=24, V=50000)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
    acc = torch.empty(batch.B, dtype=torch.int32, device=DEV)
    out = torch.empty(batch.K + batch.B, dtype=torch.int32, device=DEV)
    pq = torch.empty(2, batch.K, dtype=torch.float32, device=DEV)
    rm = torch.empty(batch.B, dtype=torch.float32, device=DEV)
    ws = torch.empty(sv.spec_verify_workspace_bytes(batch.B, batch.K, batch.V), dtype=torch.uint8,
                     device=DEV)
    mk = int(batch.num_draft.max()) if max_k == "ee" else None
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)

    def call():
        sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm, accepted_len=acc,
                              out_tokens=out, p_draft=pq[0], q_draft=pq[1], resid_mass=rm,
                              workspace=ws, max_k=mk)

    def refresh(r):
        batch.u_accept.copy_(torch.rand(batch.K, generator=gen, device=DEV))
        batch.u_final.copy_(torch.rand(batch.B, generator=gen, device=DEV))

    sv.spec_verify_set_launch_plan(plan)
    try:
        _eager_then_graph(call, refresh, [acc, out, pq, rm])
    finally:
        sv.spec_verify_set_launch_plan(0)


def test_tree_and_adaptive_in_graph():
    import draft_token_verification_row_amd as sv
    tb = synth.make_tree_batch(2, DEV, B=6, V=20000)
    nn = torch.as_tensor(tb.num_nodes, dtype=torch.int32, device=DEV)
    acc = torch.empty(tb.B, dtype=torch.int32, device=DEV)
    path = torch.empty(tb.N, dtype=torch.int32, device=DEV)
    out = torch.empty(tb.N, dtype=torch.int32, device=DEV)
    ws = torch.empty(sv.spec_verify_tree_workspace_bytes(tb.B, tb.N, tb.V), dtype=torch.uint8,
                     device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(6)
    for md in (None, 12):
        def call():
            sv.spec_verify_tree_greedy(tb.target, tb.parent, tb.tokens, nn, max_depth=md,
                                       accepted_len=acc, path_nodes=path, out_tokens=out,
                                       workspace=ws)

        def refresh(r):
            tb.target.copy_(torch.randn(tb.target.shape, generator=gen, device=DEV).to(tb.target.dtype))
        _eager_then_graph(call, refresh, [acc, path, out])

    ab = synth.make_adaptive_batch(B=64, N=7, V=3000, device=DEV)
    dst = torch.empty(64 * 7, 3000, dtype=ab.draft.dtype, device=DEV)
    res = sv.spec_verify_adaptive_length(ab.conf, ab.cost, ab.tokens)

    def call_a():
        st = sv.lib().spec_verify_adaptive_length(
            64, 7, ab.conf.data_ptr(), ab.cost.data_ptr(), ab.tokens.data_ptr(),
            res["num_draft"].data_ptr(), res["offsets"].data_ptr(), res["tokens"].data_ptr(),
            res["src_index"].data_ptr(), res["progress"].data_ptr(),
            torch.cuda.current_stream().cuda_stream)
        assert st == 0
        sv.spec_verify_gather_rows(ab.draft, res["src_index"], res["offsets"][64:], 64 * 7, out=dst)

    def refresh_a(r):
        ab.conf.copy_(torch.rand(ab.conf.shape, generator=gen, device=DEV))
    def kept(outs):
        nd, off, toks, rows = outs
        k = int(off[64].item())
        return [nd, off, toks[:k], rows[:k]]
    _eager_then_graph(call_a, refresh_a, [res["num_draft"], res["offsets"], res["tokens"], dst],
                      written=kept)
