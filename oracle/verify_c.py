"""ctypes binding of the fp64 C oracle (oracle/verify_ref.c).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import it.  It shares no code with the HIP path, and none
with oracle/verify.py either: the functions below have that module's names,
arguments and results, so the same pins run on both oracles, but every step
is computed in C (see the header of verify_ref.c for the passages and
readings it follows).

The library is built in place by `build_library()` (gcc, OpenMP, no
fast-math, no FMA contraction); `default()` builds it when it is missing or
older than its source.  `COracle(path)` binds another build of the same
source (the mutant tests build copies with one mistake planted).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import tempfile
from typing import Optional

import numpy as np

ORACLE_IS_TEST_INFRASTRUCTURE = True

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "verify_ref.c")
LIB_PATH = os.path.join(HERE, "liboracle_verify.so")
GCC_FLAGS = ["-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math"]


def build_library(verbose: bool = False, source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile verify_ref.c (or a copy of it) into a shared library."""
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out))
    os.close(fd)
    cmd = ["gcc", *GCC_FLAGS, source, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    d, i64, i32, vp = ctypes.c_double, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_widen_temperature.restype = d
    lib.oracle_widen_temperature.argtypes = [d]
    lib.oracle_tempered_softmax.restype = None
    lib.oracle_tempered_softmax.argtypes = [vp, i64, d, vp]
    lib.oracle_lowest_argmax.restype = i64
    lib.oracle_lowest_argmax.argtypes = [vp, i64]
    lib.oracle_keeps_draft.restype = i32
    lib.oracle_keeps_draft.argtypes = [d, d, d]
    lib.oracle_accept_margin.restype = d
    lib.oracle_accept_margin.argtypes = [d, d, d]
    lib.oracle_positive_residual.restype = None
    lib.oracle_positive_residual.argtypes = [vp, vp, i64, vp]
    lib.oracle_inverse_cdf.restype = i32
    lib.oracle_inverse_cdf.argtypes = [vp, i64, d, ctypes.POINTER(i64),
                                       ctypes.POINTER(d), ctypes.POINTER(d)]
    lib.oracle_verify_batch.restype = i32
    lib.oracle_verify_batch.argtypes = [vp, vp, i32, i64, i64, vp, vp, vp, i64, i64, d,
                                        vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(x) -> np.ndarray:
    """fp32 logits stay fp32 (the C side widens each one exactly); anything
    else becomes fp64."""
    a = np.asarray(x)
    if a.dtype == np.float32:
        return np.ascontiguousarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


class COracle:
    """The functions of oracle/verify.py, computed by one build of the C oracle."""

    def __init__(self, lib_path: str):
        self.lib = _bind(lib_path)

    # ------------------------------------------------------------ single steps
    def widen_temperature(self, T) -> float:
        return float(self.lib.oracle_widen_temperature(float(T)))

    def tempered_softmax(self, logits, T: float) -> np.ndarray:
        z = _f64(logits)
        p = np.empty_like(z)
        self.lib.oracle_tempered_softmax(_ptr(z), z.size, float(T), _ptr(p))
        return p

    def lowest_argmax(self, logits) -> int:
        z = _f64(logits)
        return int(self.lib.oracle_lowest_argmax(_ptr(z), z.size))

    def keeps_draft(self, u: float, p_y: float, q_y: float) -> bool:
        return bool(self.lib.oracle_keeps_draft(float(u), float(p_y), float(q_y)))

    def accept_margin(self, u: float, p_y: float, q_y: float) -> float:
        return float(self.lib.oracle_accept_margin(float(u), float(p_y), float(q_y)))

    def positive_residual(self, p, q) -> np.ndarray:
        p, q = _f64(p), _f64(q)
        r = np.empty_like(p)
        self.lib.oracle_positive_residual(_ptr(p), _ptr(q), p.size, _ptr(r))
        return r

    def inverse_cdf(self, weights, w: float):
        wt = _f64(weights)
        t, tot, m = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
        if self.lib.oracle_inverse_cdf(_ptr(wt), wt.size, float(w), ctypes.byref(t),
                                       ctypes.byref(tot), ctypes.byref(m)) != 0:
            raise ValueError("no positive weight to draw from")
        return int(t.value), float(tot.value), float(m.value)

    # ------------------------------------------------------------ batches
    def verify_batch(self, target, draft, tokens, num_draft, greedy, temperature,
                     u_accept, u_final, early_exit: bool = False, threads: int = 1) -> dict:
        """A packed batch (layout of the C ABI) -> per-request results, as
        oracle.verify.verify_batch; `threads` OpenMP threads over the requests."""
        nd = np.ascontiguousarray(np.asarray(num_draft, dtype=np.int64))
        B = int(nd.shape[0])
        K = int(nd.sum())
        tgt = _logits(target)
        V = int(tgt.shape[1]) if tgt.ndim == 2 else 0
        g = np.ones(B, np.uint8) if greedy is None else np.ascontiguousarray(
            np.asarray(greedy).astype(bool).astype(np.uint8))
        drf = None
        if draft is not None and not g.all():
            drf = _logits(draft)
            if drf.dtype != tgt.dtype:
                drf = np.ascontiguousarray(drf, dtype=np.float64)
                tgt = np.ascontiguousarray(tgt, dtype=np.float64)
            if K > 0:
                assert drf.ndim == 2 and drf.shape[1] == V and drf.shape[0] >= K
        assert tgt.ndim == 2 and tgt.shape[0] >= K + B
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(-1))
        ua = _f64(np.asarray(u_accept, dtype=np.float64).reshape(-1)) if K > 0 else np.zeros(1)
        uf = _f64(np.asarray(u_final, dtype=np.float64).reshape(-1))
        T = 1.0 if temperature is None else float(temperature)
        acc = np.zeros(B, np.int64)
        out = np.full(K + B, -1, np.int64)
        p_y = np.full(max(K, 1), -1.0)
        q_y = np.full(max(K, 1), -1.0)
        resid = np.full(B, -1.0)
        margin = np.full(B, math.inf)
        eb = 4 if tgt.dtype == np.float32 else 8
        rc = self.lib.oracle_verify_batch(
            _ptr(tgt), _ptr(drf), eb, V, V, _ptr(toks if K > 0 else np.zeros(1, np.int64)),
            _ptr(nd), _ptr(g), B, V, T, _ptr(ua), _ptr(uf), int(bool(early_exit)),
            int(threads), _ptr(acc), _ptr(out), _ptr(p_y), _ptr(q_y), _ptr(resid),
            _ptr(margin))
        if rc == -1:
            raise ValueError("a stochastic draft token lies outside [0, V)")
        if rc != 0:
            raise RuntimeError(f"oracle_verify_batch returned {rc}")
        return dict(accepted_len=acc, out_tokens=out, p_draft=p_y[:K], q_draft=q_y[:K],
                    resid_mass=resid, margin=margin)

    def verify_request(self, target_rows, draft_rows, tokens, greedy: bool,
                       T: Optional[float], u_accept, w: float, early_exit: bool = False) -> dict:
        """One request, with the results of oracle.verify.verify_request."""
        tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
        k = int(tokens.size)
        tgt = np.asarray(target_rows)
        assert tgt.shape[0] == k + 1
        res = self.verify_batch(tgt, None if greedy else draft_rows, tokens, [k],
                                [bool(greedy)], T,
                                np.asarray(u_accept, dtype=np.float64).reshape(-1),
                                [float(w)], early_exit=early_exit)
        a = int(res["accepted_len"][0])
        return dict(a=a, committed=[int(x) for x in res["out_tokens"][:a + 1]],
                    p_y=res["p_draft"], q_y=res["q_draft"],
                    resid_mass=float(res["resid_mass"][0]), margin=float(res["margin"][0]))


_DEFAULT: Optional[COracle] = None


def default() -> COracle:
    """The build next to the source, rebuilt when missing or older than it."""
    global _DEFAULT
    if _DEFAULT is None:
        if (not os.path.exists(LIB_PATH)
                or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE)):
            build_library()
        _DEFAULT = COracle(LIB_PATH)
    return _DEFAULT


def widen_temperature(T):
    return default().widen_temperature(T)


def tempered_softmax(logits, T):
    return default().tempered_softmax(logits, T)


def lowest_argmax(logits):
    return default().lowest_argmax(logits)


def keeps_draft(u, p_y, q_y):
    return default().keeps_draft(u, p_y, q_y)


def accept_margin(u, p_y, q_y):
    return default().accept_margin(u, p_y, q_y)


def positive_residual(p, q):
    return default().positive_residual(p, q)


def inverse_cdf(weights, w):
    return default().inverse_cdf(weights, w)


def verify_batch(*args, **kw):
    return default().verify_batch(*args, **kw)


def verify_request(*args, **kw):
    return default().verify_request(*args, **kw)
