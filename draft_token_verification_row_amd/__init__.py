"""Python binding of libspecverify.so (one-round draft-token verification, gfx950).

Argument marshalling only: every step of the verification runs in the HIP
kernels behind the C ABI of include/spec_verify.h.  PyTorch supplies device
memory and the current stream.  The functions carry the C names.

The library is loaded on first use (lib()), so the package and its build
module import on a tree where libspecverify.so has not been built yet.  Any
call made without the built library raises LibraryMissingError: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP = range(5)
SV_F32, SV_BF16 = 0, 1
_DTYPES = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}

# Every function the C header declares (checked by the CPU test suite).
EXPORTED = ("spec_verify_workspace_bytes", "spec_verify_status_string",
            "spec_verify_greedy", "spec_verify_sample", "spec_verify_greedy_early_exit",
            "spec_verify_sample_early_exit", "spec_verify_accept_stats",
            "spec_verify_set_profile_events", "spec_verify_tree_workspace_bytes",
            "spec_verify_tree_greedy", "spec_verify_tree_greedy_early_exit",
            "spec_verify_adaptive_length", "spec_verify_gather_rows",
            "spec_verify_set_launch_plan", "spec_verify_sample_noalloc",
            "spec_verify_read_probe")

# SPEC_VERIFY_NOALLOC_MAX_BYTES of the C header: the largest workspace that
# spec_verify_sample_noalloc serves from its static device array.
NOALLOC_MAX_BYTES = 32 << 20


class SvBatch(ctypes.Structure):
    """Mirror of sv_batch_t."""
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("target_ld", ctypes.c_int64), ("draft_ld", ctypes.c_int64),
        ("num_draft", ctypes.c_void_p), ("target", ctypes.c_void_p),
        ("draft", ctypes.c_void_p), ("draft_tokens", ctypes.c_void_p),
    ]


class SvTree(ctypes.Structure):
    """Mirror of sv_tree_t."""
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("V", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("target_ld", ctypes.c_int64),
        ("num_nodes", ctypes.c_void_p), ("parent", ctypes.c_void_p),
        ("tokens", ctypes.c_void_p), ("target", ctypes.c_void_p),
    ]


class LibraryMissingError(ImportError):
    """libspecverify.so has not been built (no fallback path exists)."""


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise LibraryMissingError(
            f"{LIB_PATH} is missing: build it with `python draft_token_verification_row_amd/build.py` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_status_string.argtypes = [i32]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_greedy.argtypes = [ctypes.POINTER(SvBatch), vp, vp, vp, sz, vp]
    lib.spec_verify_greedy.restype = i32
    lib.spec_verify_sample.argtypes = [ctypes.POINTER(SvBatch), ctypes.c_float, vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_sample.restype = i32
    lib.spec_verify_greedy_early_exit.argtypes = [ctypes.POINTER(SvBatch), i32, vp, vp, vp, sz,
                                                  vp]
    lib.spec_verify_greedy_early_exit.restype = i32
    lib.spec_verify_sample_early_exit.argtypes = [ctypes.POINTER(SvBatch), i32, ctypes.c_float,
                                                  vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_sample_early_exit.restype = i32
    lib.spec_verify_sample_noalloc.argtypes = [ctypes.POINTER(SvBatch), ctypes.c_float, vp, vp, vp,
                                               vp, vp, vp, vp, vp, vp]
    lib.spec_verify_sample_noalloc.restype = i32
    lib.spec_verify_read_probe.argtypes = [vp, sz, vp, vp]
    lib.spec_verify_read_probe.restype = i32
    lib.spec_verify_accept_stats.argtypes = [vp, vp, i32, i32, vp, vp]
    lib.spec_verify_accept_stats.restype = i32
    lib.spec_verify_tree_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_verify_tree_workspace_bytes.restype = sz
    lib.spec_verify_tree_greedy.argtypes = [ctypes.POINTER(SvTree), vp, vp, vp, vp, sz, vp]
    lib.spec_verify_tree_greedy.restype = i32
    lib.spec_verify_tree_greedy_early_exit.argtypes = [ctypes.POINTER(SvTree), i32, vp, vp, vp, vp,
                                                       sz, vp]
    lib.spec_verify_tree_greedy_early_exit.restype = i32
    lib.spec_verify_adaptive_length.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.spec_verify_adaptive_length.restype = i32
    lib.spec_verify_gather_rows.argtypes = [i32, i32, vp, ctypes.c_int64, i32, vp, vp, i32, vp,
                                            ctypes.c_int64, vp]
    lib.spec_verify_gather_rows.restype = i32
    lib.spec_verify_set_launch_plan.argtypes = [i32]
    lib.spec_verify_set_launch_plan.restype = i32
    lib.spec_verify_set_profile_events.argtypes = [vp, vp]
    lib.spec_verify_set_profile_events.restype = i32
    return lib


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on the first call; raises LibraryMissingError
    when it has not been built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    # `_lib` stays available as an attribute for callers of the raw C functions
    if name == "_lib":
        return lib()
    raise AttributeError(name)


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"spec_verify status {status}: {spec_verify_status_string(status)}")
        self.status = status


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or (t.stride(1) != 1 and t.numel() > 0):
        raise ValueError(f"{name} must be 2-D with unit stride along the vocabulary")
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} dtype {t.dtype} unsupported (float32 or bfloat16)")
    return max(t.stride(0), t.shape[1]) if t.numel() == 0 else t.stride(0)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def spec_verify_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(lib().spec_verify_workspace_bytes(B, K, V))


def spec_verify_status_string(status: int) -> str:
    return lib().spec_verify_status_string(status).decode()


def spec_verify_set_launch_plan(plan: int) -> None:
    """0 automatic, 1 multi-kernel pipeline, 2 single launch (calling thread only)."""
    st = lib().spec_verify_set_launch_plan(int(plan))
    if st != SV_OK:
        raise SpecVerifyError(st)


def spec_verify_set_profile_events(ev_begin: Optional[int], ev_end: Optional[int]) -> int:
    return int(lib().spec_verify_set_profile_events(ev_begin, ev_end))


def spec_verify_read_probe(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Plain streaming read of src (diagnostic: the read-bandwidth ceiling)."""
    st = lib().spec_verify_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                      _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st)


def make_batch_struct(target: torch.Tensor, draft: Optional[torch.Tensor],
                      draft_tokens: torch.Tensor, num_draft: torch.Tensor) -> SvBatch:
    tld = _rows(target, "target")
    dld = 0
    if draft is not None:
        dld = _rows(draft, "draft")
        if draft.dtype != target.dtype:
            raise ValueError("target and draft logits must share a dtype")
    B = int(num_draft.numel())
    K = int(draft_tokens.numel())
    return SvBatch(B=B, K=K, V=int(target.shape[1]), dtype=_DTYPES[target.dtype],
                   target_ld=tld, draft_ld=dld, num_draft=_ptr(num_draft), target=_ptr(target),
                   draft=_ptr(draft), draft_tokens=_ptr(draft_tokens) if K > 0 else None)


def _workspace(B, K, V, workspace, device):
    need = spec_verify_workspace_bytes(B, K, V)
    if need == 0:
        raise SpecVerifyError(SV_ERR_INVALID_ARG)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def spec_verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor, num_draft: torch.Tensor,
                       *, accepted_len=None, out_tokens=None, workspace=None, stream=None,
                       max_k: Optional[int] = None):
    """Greedy verification; returns (accepted_len [B], out_tokens [K+B]) int32 tensors.

    With max_k given, calls spec_verify_greedy_early_exit (reads rows only up to
    each request's cut; every num_draft[b] must be <= max_k)."""
    bt = make_batch_struct(target, None, draft_tokens, num_draft)
    dev = target.device
    if accepted_len is None:
        accepted_len = torch.empty(bt.B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(bt.K + bt.B, dtype=torch.int32, device=dev)
    workspace, wsb = _workspace(bt.B, bt.K, bt.V, workspace, dev)
    if max_k is None:
        st = lib().spec_verify_greedy(ctypes.byref(bt), _ptr(accepted_len), _ptr(out_tokens),
                                     _ptr(workspace), wsb, _stream_handle(stream))
    else:
        st = lib().spec_verify_greedy_early_exit(ctypes.byref(bt), int(max_k), _ptr(accepted_len),
                                                _ptr(out_tokens), _ptr(workspace), wsb,
                                                _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accepted_len, out_tokens


def spec_verify_sample(target: torch.Tensor, draft: Optional[torch.Tensor],
                       draft_tokens: torch.Tensor, num_draft: torch.Tensor, temperature: float,
                       u_accept: torch.Tensor, u_final: torch.Tensor, *, greedy_mask=None,
                       accepted_len=None, out_tokens=None, p_draft=None, q_draft=None,
                       resid_mass=None, want_probs: bool = True, workspace=None, stream=None,
                       max_k: Optional[int] = None):
    """Stochastic (optionally mixed greedy) verification.

    Returns a dict of device tensors: accepted_len, out_tokens, p_draft, q_draft,
    resid_mass (the last three None when want_probs is False and none was given).
    With max_k given, calls spec_verify_sample_early_exit.
    """
    bt = make_batch_struct(target, draft, draft_tokens, num_draft)
    dev = target.device
    if accepted_len is None:
        accepted_len = torch.empty(bt.B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(bt.K + bt.B, dtype=torch.int32, device=dev)
    if want_probs:
        if p_draft is None:
            p_draft = torch.empty(bt.K, dtype=torch.float32, device=dev)
        if q_draft is None:
            q_draft = torch.empty(bt.K, dtype=torch.float32, device=dev)
        if resid_mass is None:
            resid_mass = torch.empty(bt.B, dtype=torch.float32, device=dev)
    workspace, wsb = _workspace(bt.B, bt.K, bt.V, workspace, dev)
    rest = (ctypes.c_float(temperature), _ptr(greedy_mask), _ptr(u_accept), _ptr(u_final),
            _ptr(accepted_len), _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft), _ptr(resid_mass),
            _ptr(workspace), wsb, _stream_handle(stream))
    if max_k is None:
        st = lib().spec_verify_sample(ctypes.byref(bt), *rest)
    else:
        st = lib().spec_verify_sample_early_exit(ctypes.byref(bt), int(max_k), *rest)
    if st != SV_OK:
        raise SpecVerifyError(st)
    return dict(accepted_len=accepted_len, out_tokens=out_tokens, p_draft=p_draft,
                q_draft=q_draft, resid_mass=resid_mass)


def spec_verify_sample_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor],
                               draft_tokens: torch.Tensor, num_draft: torch.Tensor,
                               temperature: float, u_accept: torch.Tensor, u_final: torch.Tensor,
                               *, greedy_mask=None, accepted_len=None, out_tokens=None,
                               p_draft=None, q_draft=None, resid_mass=None, stream=None):
    """spec_verify_sample with the library's static device workspace (the C
    call allocates nothing; pass preallocated outputs to allocate nothing at
    all).  Returns the same dict of device tensors."""
    bt = make_batch_struct(target, draft, draft_tokens, num_draft)
    dev = target.device
    if accepted_len is None:
        accepted_len = torch.empty(bt.B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(bt.K + bt.B, dtype=torch.int32, device=dev)
    st = lib().spec_verify_sample_noalloc(
        ctypes.byref(bt), ctypes.c_float(temperature), _ptr(greedy_mask), _ptr(u_accept),
        _ptr(u_final), _ptr(accepted_len), _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft),
        _ptr(resid_mass), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return dict(accepted_len=accepted_len, out_tokens=out_tokens, p_draft=p_draft,
                q_draft=q_draft, resid_mass=resid_mass)


def spec_verify_accept_stats(accepted_len: torch.Tensor, num_draft: torch.Tensor, max_pos: int,
                             *, out=None, stream=None) -> torch.Tensor:
    """Acceptance statistics of one call's outcome; returns a float64 device tensor
    [4 + max_pos]: rounds, mean kept drafts, MAL (counts the final token), AR,
    per-position acceptance p_1..p_max_pos (-1 where undefined)."""
    B = int(accepted_len.numel())
    if int(num_draft.numel()) != B:
        raise ValueError("accepted_len and num_draft must have the same length")
    if out is None:
        out = torch.empty(4 + max_pos, dtype=torch.float64, device=accepted_len.device)
    st = lib().spec_verify_accept_stats(_ptr(accepted_len), _ptr(num_draft), B, max_pos, _ptr(out),
                                       _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return out


def spec_verify_tree_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(lib().spec_verify_tree_workspace_bytes(B, N, V))


def make_tree_struct(target: torch.Tensor, parent: torch.Tensor, tokens: torch.Tensor,
                     num_nodes: torch.Tensor) -> SvTree:
    tld = _rows(target, "target")
    for name, t in (("parent", parent), ("tokens", tokens), ("num_nodes", num_nodes)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    N = int(parent.numel())
    if int(tokens.numel()) != N or int(target.shape[0]) < N:
        raise ValueError("parent, tokens and target rows must cover the same N nodes")
    return SvTree(B=int(num_nodes.numel()), N=N, V=int(target.shape[1]),
                  dtype=_DTYPES[target.dtype], target_ld=tld, num_nodes=_ptr(num_nodes),
                  parent=_ptr(parent), tokens=_ptr(tokens), target=_ptr(target))


def spec_verify_tree_greedy(target: torch.Tensor, parent: torch.Tensor, tokens: torch.Tensor,
                            num_nodes: torch.Tensor, *, max_depth: Optional[int] = None,
                            accepted_len=None, path_nodes=None, out_tokens=None, workspace=None,
                            stream=None):
    """Greedy token-tree verification; returns (accepted_len [B], path_nodes [N],
    out_tokens [N]) int32 tensors.  With max_depth given, calls the early-exit
    entry point (reads only the rows the walks visit)."""
    tr = make_tree_struct(target, parent, tokens, num_nodes)
    dev = target.device
    if accepted_len is None:
        accepted_len = torch.empty(tr.B, dtype=torch.int32, device=dev)
    if path_nodes is None:
        path_nodes = torch.empty(tr.N, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(tr.N, dtype=torch.int32, device=dev)
    need = spec_verify_tree_workspace_bytes(tr.B, tr.N, tr.V)
    if need == 0:
        raise SpecVerifyError(SV_ERR_INVALID_ARG)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    ptrs = (_ptr(accepted_len), _ptr(path_nodes), _ptr(out_tokens), _ptr(workspace), wsb,
            _stream_handle(stream))
    if max_depth is None:
        st = lib().spec_verify_tree_greedy(ctypes.byref(tr), *ptrs)
    else:
        st = lib().spec_verify_tree_greedy_early_exit(ctypes.byref(tr), int(max_depth), *ptrs)
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accepted_len, path_nodes, out_tokens


def verify_tree_batch(tb, *, max_depth=None, workspace=None, stream=None):
    """Run a synthetic tree batch (fields as produced by the input generator)."""
    nn = torch.as_tensor(tb.num_nodes, dtype=torch.int32, device=tb.target.device)
    acc, path, out = spec_verify_tree_greedy(tb.target, tb.parent, tb.tokens, nn,
                                             max_depth=max_depth, workspace=workspace,
                                             stream=stream)
    return dict(accepted_len=acc, path_nodes=path, out_tokens=out)


def spec_verify_adaptive_length(conf: torch.Tensor, cost: torch.Tensor, draft_tokens: torch.Tensor,
                                *, want_src_index: bool = True, want_progress: bool = True,
                                stream=None) -> dict:
    """Per-request verification length from confidences [B, N] (fp32) and a cost
    table [N + 1] (fp64); returns device tensors num_draft [B], offsets [B + 1],
    tokens [B * N] (first offsets[B] entries used), src_index [B * N], progress [B]."""
    if conf.dim() != 2 or conf.dtype != torch.float32 or not conf.is_contiguous():
        raise ValueError("conf must be a contiguous float32 [B, N] tensor")
    B, N = conf.shape
    if cost.dtype != torch.float64 or cost.numel() != N + 1:
        raise ValueError("cost must be a float64 tensor of N + 1 entries")
    if draft_tokens.dtype != torch.int32 or draft_tokens.numel() != B * N \
            or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [B, N] tensor")
    dev = conf.device
    nd = torch.empty(B, dtype=torch.int32, device=dev)
    off = torch.empty(B + 1, dtype=torch.int32, device=dev)
    toks = torch.empty(max(B * N, 1), dtype=torch.int32, device=dev)
    src = torch.empty(max(B * N, 1), dtype=torch.int32, device=dev) if want_src_index else None
    prog = torch.empty(B, dtype=torch.float64, device=dev) if want_progress else None
    st = lib().spec_verify_adaptive_length(B, N, _ptr(conf), _ptr(cost), _ptr(draft_tokens),
                                          _ptr(nd), _ptr(off), _ptr(toks), _ptr(src), _ptr(prog),
                                          _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return dict(num_draft=nd, offsets=off, tokens=toks, src_index=src, progress=prog)


def spec_verify_gather_rows(src: torch.Tensor, index: torch.Tensor, count: torch.Tensor,
                            max_rows: int, *, out=None, stream=None) -> torch.Tensor:
    """dst[r] = src[index[r]] for r < min(count[0], max_rows) (count on the device)."""
    ld = _rows(src, "src")
    if out is None:
        out = torch.empty(max(max_rows, 1), src.shape[1], dtype=src.dtype, device=src.device)
    st = lib().spec_verify_gather_rows(_DTYPES[src.dtype], int(src.shape[1]), _ptr(src), ld,
                                      int(src.shape[0]), _ptr(index), _ptr(count), int(max_rows),
                                      _ptr(out), _rows(out, "out"), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return out


def verify_batch(batch, *, workspace=None, want_probs=True, stream=None, max_k=None):
    """Run a synthetic batch object (fields as produced by the input generator).
    max_k selects the early-exit entry points."""
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=batch.target.device)
    if batch.temperature is None:
        acc, out = spec_verify_greedy(batch.target, batch.tokens, nd, workspace=workspace,
                                      stream=stream, max_k=max_k)
        return dict(accepted_len=acc, out_tokens=out, p_draft=None, q_draft=None,
                    resid_mass=None)
    gm = None
    if batch.greedy.any():
        gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=batch.target.device)
    return spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm,
                              want_probs=want_probs, workspace=workspace, stream=stream,
                              max_k=max_k)
