"""Seeded synthetic inputs for one round of draft-token verification.

This module only draws numbers.  It holds none of the verification arithmetic
(no tempered softmax, no ratio test, no residual, no inverse CDF), so the CPU
oracle and the HIP path can both consume its batches without sharing any of
the method's code.

Workload shapes follow the serving workloads the pages describe:

* sequential drafters propose 1..7 tokens per round and block drafters use
  blocks of 16 = one anchor + 15 drafts (vLLM blog "speculative-decoding-amd-gpus",
  section "Match the sweep to the workload" and the DFlash tuning paragraph);
* a ragged batch packs per-request verification windows of different lengths
  back to back (chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash,
  DDTree, and DSpark", section 5 DSpark: compact, variable-length verification).

Packed layout (the same one the C ABI takes).  Request b owns k_b draft tokens
and k_b + 1 target rows (k_b verified positions plus the row the bonus token is
drawn from).  With off[b] = sum of k over earlier requests:

* target row of (b, i), i = 0..k_b        -> off[b] + b + i
* draft row and draft token of (b, i), i < k_b -> off[b] + i

Draft tokens "sampled from q" are drawn with the Gumbel-max trick on the
draft logits divided by the temperature, which the verification step itself
never uses.  Uniforms are fp32 values on the 2**-24 grid.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

BASE_SEED = 20261202

# The five verification workloads.  sigma / noise are standard deviations.
CONFIGS = {
    1: dict(name="tiny_stochastic", B=1, k=4, V=1000, dtype="f32", sigma=2.0,
            noise=1.0, T=1.0, mode="stochastic"),
    2: dict(name="greedy_v32000", B=64, k=3, V=32000, dtype="bf16", sigma=3.0,
            noise=None, T=None, mode="greedy", p_match=0.7),
    3: dict(name="stochastic_f32_v128256", B=256, k=5, V=128256, dtype="f32",
            sigma=2.5, noise=1.0, T=0.7, mode="stochastic"),
    4: dict(name="dflash_block16_v151936", B=32, k=15, V=151936, dtype="bf16",
            sigma=2.0, noise=1.5, T=1.0, mode="stochastic"),
    5: dict(name="ragged_mixed_v262144", B=512, k=(0, 7), V=262144, dtype="bf16",
            sigma=2.0, noise=1.2, T=0.8, mode="mixed"),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Batch:
    """One packed verification batch.  Tensors live on `device`."""
    name: str
    B: int
    K: int
    V: int
    dtype: str
    num_draft: np.ndarray          # int32 [B]   (host copy)
    greedy: np.ndarray             # uint8 [B]   (host copy, 1 = greedy request)
    temperature: Optional[float]   # fp32 value, None for all-greedy batches
    target: torch.Tensor           # [K+B, V]
    draft: Optional[torch.Tensor]  # [K, V] or None
    tokens: torch.Tensor           # int32 [K]
    u_accept: torch.Tensor         # fp32 [K]
    u_final: torch.Tensor          # fp32 [B]

    @property
    def offsets(self) -> np.ndarray:
        off = np.zeros(self.B + 1, dtype=np.int64)
        np.cumsum(self.num_draft, out=off[1:])
        return off

    def target_row(self, b: int, i: int) -> int:
        return int(self.offsets[b]) + b + i

    def draft_row(self, b: int, i: int) -> int:
        return int(self.offsets[b]) + i

    @property
    def positions(self) -> int:
        return int(self.K)

    def bytes_read_once(self) -> int:
        """Every target row, plus the draft rows of stochastic requests, read once."""
        es = 4 if self.dtype == "f32" else 2
        stoch_drafts = int(self.num_draft[self.greedy == 0].sum())
        return (self.K + self.B + stoch_drafts) * self.V * es

    def to(self, device) -> "Batch":
        def mv(t):
            return None if t is None else t.to(device)
        return dataclasses.replace(
            self, target=mv(self.target), draft=mv(self.draft), tokens=mv(self.tokens),
            u_accept=mv(self.u_accept), u_final=mv(self.u_final))


def _streams(cfg_id: int, seed: Optional[int]):
    ss = np.random.SeedSequence(BASE_SEED + cfg_id if seed is None else seed)
    return ss.spawn(5)   # target, noise, draw, uniforms, layout


def _torch_gen(ss: np.random.SeedSequence, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1)))
    return g


def uniforms_f32(rng: np.random.Generator, n: int) -> np.ndarray:
    """fp32 uniforms on [0, 1): (32-bit draw >> 8) * 2**-24."""
    bits = rng.integers(0, 1 << 32, size=n, dtype=np.uint64)
    return ((bits >> np.uint64(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _layout(cfg: dict, B: int, k, rng: np.random.Generator):
    if isinstance(k, tuple):
        num_draft = rng.integers(k[0], k[1] + 1, size=B).astype(np.int32)
    else:
        num_draft = np.full(B, int(k), dtype=np.int32)
    if cfg["mode"] == "greedy":
        greedy = np.ones(B, dtype=np.uint8)
    elif cfg["mode"] == "stochastic":
        greedy = np.zeros(B, dtype=np.uint8)
    else:  # mixed: odd requests greedy, even requests stochastic
        greedy = (np.arange(B) % 2).astype(np.uint8)
    return num_draft, greedy


def _gumbel_argmax(logits_f32: torch.Tensor, T: float, g: torch.Generator,
                   chunk_rows: int = 256) -> torch.Tensor:
    """One draw per row from softmax(logits / T) by the Gumbel-max trick."""
    out = torch.empty(logits_f32.shape[0], dtype=torch.int64, device=logits_f32.device)
    for r0 in range(0, logits_f32.shape[0], chunk_rows):
        x = logits_f32[r0:r0 + chunk_rows]
        u = torch.rand(x.shape, generator=g, device=x.device, dtype=torch.float32)
        u.clamp_(min=1e-38)
        gumbel = -torch.log(-torch.log(u))
        out[r0:r0 + chunk_rows] = torch.argmax(x / T + gumbel, dim=1)
    return out


def make_batch(cfg_id: int, device="cpu", *, B: Optional[int] = None,
               V: Optional[int] = None, k=None, seed: Optional[int] = None,
               dtype: Optional[str] = None, target_ld: Optional[int] = None) -> Batch:
    """Build configuration `cfg_id` (1..5), optionally with smaller B / V / k.

    `target_ld` > V pads every logit row (a strided layout); pad columns hold NaN
    so a kernel that reads past V is caught by the parity tests.
    """
    cfg = CONFIGS[cfg_id]
    B = cfg["B"] if B is None else B
    V = cfg["V"] if V is None else V
    k = cfg["k"] if k is None else k
    dt = cfg["dtype"] if dtype is None else dtype
    s_target, s_noise, s_draw, s_unif, s_layout = _streams(cfg_id, seed)
    num_draft, greedy = _layout(cfg, B, k, np.random.default_rng(s_layout))
    K = int(num_draft.sum())
    off = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(num_draft, out=off[1:])
    req_of_draft = np.repeat(np.arange(B), num_draft)
    pos_of_draft = np.arange(K) - off[req_of_draft]
    trow_of_draft = torch.as_tensor(off[req_of_draft] + req_of_draft + pos_of_draft,
                                    dtype=torch.int64, device=device)

    g_t = _torch_gen(s_target, device)
    ld = V if target_ld is None else int(target_ld)
    tdt = TORCH_DTYPE[dt]
    target32 = torch.randn((K + B, V), generator=g_t, device=device,
                           dtype=torch.float32) * cfg["sigma"]
    target = target32.to(tdt)
    target32 = target.to(torch.float32)          # exact widening of what is stored
    T = cfg["T"]

    draft = None
    draft32 = None
    if cfg["noise"] is not None and K > 0:
        g_n = _torch_gen(s_noise, device)
        noise = torch.randn((K, V), generator=g_n, device=device,
                            dtype=torch.float32) * cfg["noise"]
        draft = (target32.index_select(0, trow_of_draft) + noise).to(tdt)
        draft32 = draft.to(torch.float32)
        del noise
    elif cfg["noise"] is not None:
        draft = torch.empty((0, V), dtype=tdt, device=device)

    g_d = _torch_gen(s_draw, device)
    tokens = torch.empty(K, dtype=torch.int64, device=device)
    if K > 0:
        if cfg["mode"] == "greedy":
            # draft equals the target argmax with prob p_match, else uniform id
            tgt_rows = target32.index_select(0, trow_of_draft)
            amax = torch.argmax(tgt_rows, dim=1)
            coin = torch.rand(K, generator=g_d, device=device) < cfg["p_match"]
            rand_ids = torch.randint(0, V, (K,), generator=g_d, device=device)
            tokens = torch.where(coin, amax, rand_ids)
            del tgt_rows
        else:
            sampled = _gumbel_argmax(draft32, float(np.float32(T)), g_d)
            greedy_d = torch.as_tensor(greedy[req_of_draft].astype(bool), device=device)
            if bool(greedy_d.any()):
                amax = torch.argmax(draft32, dim=1)
                tokens = torch.where(greedy_d, amax, sampled)
            else:
                tokens = sampled
    del draft32

    if ld != V:
        pad_t = torch.full((K + B, ld), float("nan"), dtype=tdt, device=device)
        pad_t[:, :V] = target
        target = pad_t[:, :V]
        if draft is not None:
            pad_d = torch.full((K, ld), float("nan"), dtype=tdt, device=device)
            pad_d[:, :V] = draft
            draft = pad_d[:, :V]

    rng_u = np.random.default_rng(s_unif)
    u_accept = uniforms_f32(rng_u, K)
    u_final = uniforms_f32(rng_u, B)
    return Batch(
        name=cfg["name"], B=B, K=K, V=V, dtype=dt, num_draft=num_draft, greedy=greedy,
        temperature=None if T is None else float(np.float32(T)),
        target=target, draft=draft, tokens=tokens.to(torch.int32),
        u_accept=torch.as_tensor(u_accept, device=device),
        u_final=torch.as_tensor(u_final, device=device))


RANDOM_VOCABS = (1, 2, 7, 63, 64, 65, 1000, 4099, 16385, 30011, 50000)


def make_random_batch(seed: int, device="cpu", max_elems: int = 8 << 20) -> Batch:
    """A batch of random shape for broad parity sweeps: dtype, vocabulary (odd,
    tiny and multiple-of-chunk sizes), request count, ragged k_b, greedy share,
    temperature (log-uniform in [0.05, 20]), logit scale, draft noise, strided
    rows and masked (-inf) columns all drawn from `seed`.  Drafts are the draft
    row's argmax with probability 1/2, else a uniform id, so that cuts fall
    both early and late.  Rows x V stays under max_elems."""
    rng = np.random.default_rng(np.random.SeedSequence([BASE_SEED, 7, int(seed)]))
    dt = "f32" if rng.random() < 0.5 else "bf16"
    V = int(rng.choice(RANDOM_VOCABS)) if rng.random() < 0.6 else int(rng.integers(1, 50001))
    kmax = int(rng.choice([0, 1, 3, 7, 15]))
    B = int(rng.integers(1, 33))
    while True:
        num_draft = rng.integers(0, kmax + 1, size=B).astype(np.int32)
        K = int(num_draft.sum())
        if (2 * K + B) * V <= max_elems or B == 1:
            break
        B = max(1, B // 2)
    share = float(rng.choice([0.0, 0.5, 1.0]))
    greedy = (rng.random(B) < share).astype(np.uint8)
    T = float(np.float32(np.exp(rng.uniform(np.log(0.05), np.log(20.0)))))
    sigma = float(rng.uniform(0.5, 4.0))
    noise = float(rng.uniform(0.1, 2.0))
    tdt = TORCH_DTYPE[dt]
    target = torch.as_tensor(rng.normal(0.0, sigma, size=(K + B, V)).astype(np.float32))
    off = np.concatenate([[0], np.cumsum(num_draft)]).astype(np.int64)
    trow = np.concatenate([np.arange(off[b] + b, off[b] + b + num_draft[b]) for b in range(B)]
                          + [np.zeros(0, np.int64)]).astype(np.int64)
    draft = target[torch.as_tensor(trow)] + torch.as_tensor(
        rng.normal(0.0, noise, size=(K, V)).astype(np.float32))
    if V > 8 and rng.random() < 0.2:          # masked columns (never all of a row)
        cols = rng.choice(V, size=V // 8, replace=False)
        target[:, cols] = float("-inf")
        draft[:, cols] = float("-inf")
    target = target.to(tdt)
    draft = draft.to(tdt)
    d32 = draft.to(torch.float32)
    amax = torch.argmax(d32, dim=1).numpy() if K else np.zeros(0, np.int64)
    tokens = np.where(rng.random(K) < 0.5, amax, rng.integers(0, V, size=K)).astype(np.int64)
    if K and V > 8 and bool(torch.isinf(d32[0]).any()):
        finite = ~torch.isinf(d32).numpy()
        for i in range(K):                     # keep tokens on unmasked ids
            if not finite[i, tokens[i]]:
                tokens[i] = int(amax[i])
    ld = V + int(rng.integers(1, 18)) if rng.random() < 0.3 else V
    b = Batch(name=f"random_{seed}", B=B, K=K, V=V, dtype=dt, num_draft=num_draft, greedy=greedy,
              temperature=T, target=target, draft=draft,
              tokens=torch.as_tensor(tokens).to(torch.int32),
              u_accept=torch.as_tensor(uniforms_f32(rng, K)),
              u_final=torch.as_tensor(uniforms_f32(rng, B))).to(device)
    if ld != V:                               # strided rows, NaN in the pads (built on the device)
        pt = torch.full((K + B, ld), float("nan"), dtype=tdt, device=device)
        pt[:, :V] = b.target
        pd = torch.full((K, ld), float("nan"), dtype=tdt, device=device)
        pd[:, :V] = b.draft
        b = dataclasses.replace(b, target=pt[:, :V], draft=pd[:, :V])
    return b


def from_arrays(target, draft, tokens, num_draft, greedy=None, temperature=None,
                u_accept=None, u_final=None, dtype="f32", name="custom",
                device="cpu") -> Batch:
    """Wrap hand-built arrays (fixtures) into a Batch."""
    num_draft = np.asarray(num_draft, dtype=np.int32)
    B = int(num_draft.shape[0])
    K = int(num_draft.sum())
    greedy = np.zeros(B, np.uint8) if greedy is None else np.asarray(greedy, np.uint8)
    tdt = TORCH_DTYPE[dtype]
    tgt = torch.as_tensor(np.asarray(target, dtype=np.float32)).to(tdt)
    V = int(tgt.shape[1])
    dr = None if draft is None else torch.as_tensor(
        np.asarray(draft, dtype=np.float32).reshape(K, V)).to(tdt)
    ua = np.zeros(K, np.float32) if u_accept is None else np.asarray(u_accept, np.float32)
    uf = np.zeros(B, np.float32) if u_final is None else np.asarray(u_final, np.float32)
    b = Batch(name=name, B=B, K=K, V=V, dtype=dtype, num_draft=num_draft, greedy=greedy,
              temperature=None if temperature is None else float(np.float32(temperature)),
              target=tgt, draft=dr,
              tokens=torch.as_tensor(np.asarray(tokens, np.int64).reshape(K)).to(torch.int32),
              u_accept=torch.as_tensor(ua), u_final=torch.as_tensor(uf))
    return b.to(device)


def select_requests(batch: Batch, reqs: Sequence[int], device="cpu") -> Batch:
    """Copy the rows of the listed requests into a smaller packed batch.

    Requests are independent in one verification round, so the result of request
    reqs[j] in the sub-batch equals its result in the full batch.
    """
    off = batch.offsets
    t_rows, d_rows, f_idx = [], [], []
    for b in reqs:
        k = int(batch.num_draft[b])
        t_rows.extend(range(int(off[b]) + b, int(off[b]) + b + k + 1))
        d_rows.extend(range(int(off[b]), int(off[b]) + k))
        f_idx.append(b)
    dev = batch.target.device
    ti = torch.as_tensor(t_rows, dtype=torch.int64, device=dev)
    di = torch.as_tensor(d_rows, dtype=torch.int64, device=dev)
    fi = torch.as_tensor(f_idx, dtype=torch.int64, device=dev)
    nd = batch.num_draft[list(reqs)].copy()
    return Batch(
        name=batch.name + "_subset", B=len(reqs), K=int(nd.sum()), V=batch.V,
        dtype=batch.dtype, num_draft=nd, greedy=batch.greedy[list(reqs)].copy(),
        temperature=batch.temperature,
        target=batch.target.index_select(0, ti).to(device),
        draft=None if batch.draft is None else batch.draft.index_select(0, di).to(device),
        tokens=batch.tokens.index_select(0, di).to(device),
        u_accept=batch.u_accept.index_select(0, di).to(device),
        u_final=batch.u_final.index_select(0, fi).to(device))


def as_numpy(batch: Batch) -> dict:
    """Host fp32/int views of a batch (bf16 widens to fp32 exactly)."""
    def f32(t):
        return None if t is None else t.detach().to("cpu", torch.float32).numpy()
    return dict(
        target=f32(batch.target), draft=f32(batch.draft),
        tokens=batch.tokens.cpu().numpy().astype(np.int64),
        num_draft=batch.num_draft.astype(np.int64), greedy=batch.greedy.astype(bool),
        temperature=batch.temperature,
        u_accept=batch.u_accept.cpu().numpy(), u_final=batch.u_final.cpu().numpy())


# ---------------------------------------------------------------------------
# Token trees (greedy tree verification).  Shapes only: the verification walk
# is not computed here.
#
# Request b owns n_b nodes (node 0 = root, the last committed token) in
# creation order, so every parent index is below its child's.  Shapes grow by
# best-first expansion of random factorized scores: a candidate child of node
# i at sibling rank r scores score(i) * w_i[r], with w_i a random Dirichlet
# draw sorted descending (the shape of the candidate sets that chzhyang,
# "Speculative Decoding: ...", section 5 DDTree describes; the scores here are
# random numbers, not a drafter's marginals).  Target logits are N(0, sigma^2)
# per node row.  Sibling tokens are distinct; with probability p_match one
# child of a node carries the argmax of the node's target row (so walks go
# deep), the other children random other ids.

TREE_CONFIGS = {
    1: dict(name="tree_tiny_v1000", B=3, nodes=(1, 12), V=1000, dtype="f32", sigma=2.0,
            p_match=0.7, branch=3),
    2: dict(name="ddtree_budget32_v151936", B=32, nodes=33, V=151936, dtype="bf16",
            sigma=2.0, p_match=0.75, branch=4),
}


@dataclasses.dataclass
class TreeBatch:
    """One packed batch of token trees.  Tensors live on `device`."""
    name: str
    B: int
    N: int
    V: int
    dtype: str
    num_nodes: np.ndarray          # int32 [B] (host copy)
    parent: torch.Tensor           # int32 [N], local parent index (root's entry -1)
    tokens: torch.Tensor           # int32 [N]
    target: torch.Tensor           # [N, V]

    @property
    def offsets(self) -> np.ndarray:
        off = np.zeros(self.B + 1, dtype=np.int64)
        np.cumsum(self.num_nodes, out=off[1:])
        return off

    def to(self, device) -> "TreeBatch":
        return dataclasses.replace(self, parent=self.parent.to(device),
                                   tokens=self.tokens.to(device),
                                   target=self.target.to(device))


def _tree_shape(n: int, branch: int, rng: np.random.Generator) -> np.ndarray:
    import heapq
    parent = np.full(n, -1, dtype=np.int64)
    score = np.zeros(n)
    score[0] = 1.0
    heap = []

    def push_children(i):
        w = np.sort(rng.dirichlet(np.ones(branch)))[::-1]
        for r in range(branch):
            heapq.heappush(heap, (-score[i] * w[r], int(rng.integers(1 << 30)), i))

    push_children(0)
    for i in range(1, n):
        s, _, p = heapq.heappop(heap)
        parent[i] = p
        score[i] = -s
        push_children(i)
    return parent


def make_tree_batch(cfg_id: int, device="cpu", *, B: Optional[int] = None,
                    V: Optional[int] = None, nodes=None, seed: Optional[int] = None,
                    dtype: Optional[str] = None, p_match: Optional[float] = None,
                    branch: Optional[int] = None) -> TreeBatch:
    cfg = TREE_CONFIGS[cfg_id]
    branch = cfg["branch"] if branch is None else int(branch)
    B = cfg["B"] if B is None else B
    V = cfg["V"] if V is None else V
    nodes = cfg["nodes"] if nodes is None else nodes
    dt = cfg["dtype"] if dtype is None else dtype
    pm = cfg["p_match"] if p_match is None else p_match
    ss = np.random.SeedSequence(BASE_SEED + 100 + cfg_id if seed is None else seed)
    s_shape, s_target, s_tok = ss.spawn(3)
    rng = np.random.default_rng(s_shape)
    if isinstance(nodes, tuple):
        num_nodes = rng.integers(nodes[0], nodes[1] + 1, size=B).astype(np.int32)
    else:
        num_nodes = np.full(B, int(nodes), dtype=np.int32)
    N = int(num_nodes.sum())
    parent = np.concatenate([_tree_shape(int(n), branch, rng) for n in num_nodes]) \
        if N else np.zeros(0, np.int64)
    g_t = _torch_gen(s_target, device)
    target = (torch.randn((N, V), generator=g_t, device=device, dtype=torch.float32)
              * cfg["sigma"]).to(TORCH_DTYPE[dt])
    amax = torch.argmax(target.to(torch.float32), dim=1).cpu().numpy() if N else np.zeros(0)
    rt = np.random.default_rng(s_tok)
    tokens = np.zeros(N, dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(num_nodes)]).astype(np.int64)
    for b in range(B):
        s, n = int(off[b]), int(num_nodes[b])
        tokens[s] = rt.integers(0, V)                       # root: not verified
        for i in range(n):
            kids = [c for c in range(i + 1, n) if parent[s + c] == i]
            if not kids:
                continue
            used = set()
            if rt.random() < pm and V > len(kids):
                tokens[s + kids[0]] = amax[s + i]
                used.add(int(amax[s + i]))
                kids = kids[1:]
            banned = {int(amax[s + i])}
            for c in kids:
                while True:
                    t = int(rt.integers(0, V))
                    if t not in used and (t not in banned or V <= len(used) + 1):
                        break
                tokens[s + c] = t
                used.add(t)
    return TreeBatch(name=cfg["name"], B=B, N=N, V=V, dtype=dt, num_nodes=num_nodes,
                     parent=torch.as_tensor(parent.astype(np.int32), device=device),
                     tokens=torch.as_tensor(tokens.astype(np.int32), device=device),
                     target=target)


def tree_from_arrays(target, parent, tokens, num_nodes, dtype="f32", name="custom_tree",
                     device="cpu") -> TreeBatch:
    num_nodes = np.asarray(num_nodes, dtype=np.int32)
    tgt = torch.as_tensor(np.asarray(target, dtype=np.float32)).to(TORCH_DTYPE[dtype])
    return TreeBatch(name=name, B=int(num_nodes.shape[0]), N=int(num_nodes.sum()),
                     V=int(tgt.shape[1]), dtype=dtype, num_nodes=num_nodes,
                     parent=torch.as_tensor(np.asarray(parent, np.int64).astype(np.int32)),
                     tokens=torch.as_tensor(np.asarray(tokens, np.int64).astype(np.int32)),
                     target=tgt).to(device)


def select_trees(batch: TreeBatch, reqs: Sequence[int], device="cpu") -> TreeBatch:
    off = batch.offsets
    rows = []
    for b in reqs:
        rows.extend(range(int(off[b]), int(off[b]) + int(batch.num_nodes[b])))
    ri = torch.as_tensor(rows, dtype=torch.int64, device=batch.target.device)
    nn = batch.num_nodes[list(reqs)].copy()
    return TreeBatch(name=batch.name + "_subset", B=len(reqs), N=int(nn.sum()), V=batch.V,
                     dtype=batch.dtype, num_nodes=nn,
                     parent=batch.parent.index_select(0, ri).to(device),
                     tokens=batch.tokens.index_select(0, ri).to(device),
                     target=batch.target.index_select(0, ri).to(device))


def tree_as_numpy(batch: TreeBatch) -> dict:
    return dict(target=batch.target.detach().to("cpu", torch.float32).numpy(),
                parent=batch.parent.cpu().numpy().astype(np.int64),
                tokens=batch.tokens.cpu().numpy().astype(np.int64),
                num_nodes=batch.num_nodes.astype(np.int64))


# ---------------------------------------------------------------------------
# Confidence-driven verification length.  A drafter proposes a block of N
# tokens per request with per-position confidences (chzhyang, "Speculative
# Decoding: ...", section 5 DSpark; blocks of 7 as in the DSpark checkpoints the
# vLLM blog's tuning section names).  Confidences fall with the position:
# c_i = clip(c_0 * decay^i + noise, 0, 1), c_0 ~ U(0.6, 1).  The cost table is
# a synthetic linear one, cost(k) = 1 + slope * k (time units of one round with
# k verification positions), standing in for the per-deployment profiled table
# the pages call for.

@dataclasses.dataclass
class AdaptiveBatch:
    name: str
    B: int
    N: int
    V: int
    dtype: str
    conf: torch.Tensor             # fp32 [B, N]
    tokens: torch.Tensor           # int32 [B, N]
    cost: torch.Tensor             # fp64 [N + 1]
    draft: Optional[torch.Tensor]  # [B * N, V] draft logits (row b * N + i), or None


def make_adaptive_batch(B: int = 512, N: int = 7, V: int = 262144, dtype: str = "bf16",
                        device="cpu", *, slope: float = 0.12, with_rows: bool = True,
                        seed: Optional[int] = None) -> AdaptiveBatch:
    ss = np.random.SeedSequence(BASE_SEED + 200 if seed is None else seed)
    s_conf, s_tok, s_rows = ss.spawn(3)
    rng = np.random.default_rng(s_conf)
    c0 = rng.uniform(0.6, 1.0, size=(B, 1))
    decay = rng.uniform(0.75, 0.97, size=(B, 1))
    conf = np.clip(c0 * decay ** np.arange(N)[None, :] + rng.normal(0, 0.05, size=(B, N)), 0, 1)
    tokens = np.random.default_rng(s_tok).integers(0, V, size=(B, N))
    cost = 1.0 + slope * np.arange(N + 1, dtype=np.float64)
    draft = None
    if with_rows:
        g = _torch_gen(s_rows, device)
        draft = (torch.randn((B * N, V), generator=g, device=device, dtype=torch.float32)
                 * 2.0).to(TORCH_DTYPE[dtype])
    return AdaptiveBatch(name=f"adaptive_block{N}_v{V}", B=B, N=N, V=V, dtype=dtype,
                         conf=torch.as_tensor(conf.astype(np.float32), device=device),
                         tokens=torch.as_tensor(tokens.astype(np.int32), device=device),
                         cost=torch.as_tensor(cost, device=device), draft=draft)
