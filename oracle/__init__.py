"""ctypes wrapper of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline import this module; the product path never does. The oracle shares no
code with the HIP path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
ACCEPT, SAMPLE, DRAFT = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, IEEE fp64, OpenMP over sequences)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


class _Diag(ctypes.Structure):
    _fields_ = [("row_max", ctypes.c_void_p), ("row_sumexp", ctypes.c_void_p),
                ("p_tok", ctypes.c_void_p), ("q_tok", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("Z", ctypes.c_void_p),
                ("cdf_lo", ctypes.c_void_p), ("cdf_hi", ctypes.c_void_p),
                ("degenerate", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # an alternate build of the oracle (the planted-mistake tests use this)
        path = os.environ.get("SPECVERIFY_ORACLE_LIB") or build(force=False)
        L = ctypes.CDLL(path)
        vp, i32, i64, u32, u64, f64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double)
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_philox4x32_10.restype = None
        L.orc_uniform.argtypes = [u64, u32, u32, u32]
        L.orc_uniform.restype = f64
        L.orc_uniform_batch.argtypes = [u64, vp, vp, vp, i64, vp]
        L.orc_uniform_batch.restype = None
        L.orc_row_softmax.argtypes = [vp, ctypes.c_int, i64, f64, vp, vp, vp]
        L.orc_row_softmax.restype = ctypes.c_int
        L.orc_residual_cdf.argtypes = [vp, vp, ctypes.c_int, i64, f64, vp]
        L.orc_residual_cdf.restype = f64
        L.orc_verify_u.argtypes = [vp, vp, vp, i32, i32, i64, ctypes.c_int, f64, vp, vp,
                                   vp, vp, ctypes.POINTER(_Diag)]
        L.orc_verify_u.restype = ctypes.c_int
        L.orc_verify.argtypes = [vp, vp, vp, i32, i32, i64, ctypes.c_int, f64, u64, i64,
                                 vp, vp, ctypes.POINTER(_Diag)]
        L.orc_verify.restype = ctypes.c_int
        L.orc_draft_sample.argtypes = [vp, i32, i32, i64, ctypes.c_int, f64, u64, i64, i64, vp, vp,
                                       vp, vp]
        L.orc_draft_sample.restype = ctypes.c_int
        L.orc_row_entropy.argtypes = [vp, ctypes.c_int, i64, f64]
        L.orc_row_entropy.restype = f64
        L.orc_expected_accept.argtypes = [vp, vp, i32, i32, i64, ctypes.c_int, f64, vp]
        L.orc_expected_accept.restype = ctypes.c_int
        L.orc_tree_verify.argtypes = [vp, vp, vp, vp, i32, i32, i64, ctypes.c_int, f64, f64, vp, vp, vp]
        L.orc_tree_verify.restype = ctypes.c_int
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(a, dtype):
    if a is None:
        return None
    want = np.float32 if dtype == F32 else np.uint16
    a = np.ascontiguousarray(a)
    assert a.dtype == want, (a.dtype, want)
    return a


def philox(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, b, i, purpose):
    return lib().orc_uniform(seed, b, i, purpose)


def uniforms(seed, b, i, purpose):
    b = np.ascontiguousarray(b, dtype=np.uint32)
    i = np.ascontiguousarray(np.broadcast_to(i, b.shape), dtype=np.uint32)
    pu = np.ascontiguousarray(np.broadcast_to(purpose, b.shape), dtype=np.uint32)
    out = np.empty(b.shape, np.float64)
    lib().orc_uniform_batch(seed, _ptr(b), _ptr(i), _ptr(pu), b.size, _ptr(out))
    return out


def row_softmax(row, dtype, T):
    row = _storage(row, dtype)
    V = row.shape[-1]
    p = np.empty(V, np.float64)
    m = ctypes.c_double()
    S = ctypes.c_double()
    ok = lib().orc_row_softmax(_ptr(row), dtype, V, T, _ptr(p), ctypes.byref(m), ctypes.byref(S))
    return bool(ok), p, m.value, S.value


def residual_cdf(p_row, q_row, dtype, T):
    p_row = _storage(p_row, dtype)
    q_row = _storage(q_row, dtype)
    V = p_row.shape[-1]
    cdf = np.empty(V, np.float64)
    Z = lib().orc_residual_cdf(_ptr(p_row), _ptr(q_row), dtype, V, T, _ptr(cdf))
    return Z, cdf


class Result:
    """Outputs and diagnostics of one oracle call."""

    def __init__(self, B, gamma):
        R = 2 * gamma + 1
        self.tokens = np.full((B, gamma + 1), -7, np.int32)
        self.n = np.full(B, -7, np.int32)
        self.row_max = np.full((B, R), np.nan)
        self.row_sumexp = np.full((B, R), np.nan)
        self.p_tok = np.full((B, gamma), np.nan)
        self.q_tok = np.full((B, gamma), np.nan)
        self.alpha = np.full((B, gamma), np.nan)
        self.Z = np.full(B, np.nan)
        self.cdf_lo = np.full(B, np.nan)
        self.cdf_hi = np.full(B, np.nan)
        self.degenerate = np.zeros(B, np.int32)

    def diag(self):
        return _Diag(*[_ptr(a) for a in (self.row_max, self.row_sumexp, self.p_tok,
                                         self.q_tok, self.alpha, self.Z, self.cdf_lo,
                                         self.cdf_hi, self.degenerate)])


def verify(target, draft, tokens, dtype, T, seed=0, b_offset=0, diag=True):
    """Run the oracle on storage arrays (float32, or uint16 bf16 bits).
    target [B, g+1, V], draft [B, g, V] (may be None at T == 0), tokens [B, g]."""
    target = _storage(target, dtype)
    draft = _storage(draft, dtype)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, g1, V = target.shape
    g = g1 - 1
    res = Result(B, g)
    d = res.diag() if diag else None
    rc = lib().orc_verify(_ptr(target), _ptr(draft), _ptr(tokens), B, g, V, dtype, float(T),
                          int(seed) & 0xFFFFFFFFFFFFFFFF, int(b_offset), _ptr(res.tokens),
                          _ptr(res.n), ctypes.byref(d) if d is not None else None)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return res


def verify_u(target, draft, tokens, dtype, T, u_accept, u_sample, diag=True):
    """Oracle with explicit uniforms: u_accept [B, g], u_sample [B, g+1]."""
    target = _storage(target, dtype)
    draft = _storage(draft, dtype)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, g1, V = target.shape
    g = g1 - 1
    ua = None if u_accept is None else np.ascontiguousarray(u_accept, dtype=np.float64)
    us = None if u_sample is None else np.ascontiguousarray(u_sample, dtype=np.float64)
    if ua is not None:
        assert ua.shape == (B, g)
    if us is not None:
        assert us.shape == (B, g + 1)
    res = Result(B, g)
    d = res.diag() if diag else None
    rc = lib().orc_verify_u(_ptr(target), _ptr(draft), _ptr(tokens), B, g, V, dtype, float(T),
                            _ptr(ua), _ptr(us), _ptr(res.tokens), _ptr(res.n),
                            ctypes.byref(d) if d is not None else None)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return res


class DraftResult:
    """Draft-side sampling outputs of one oracle call, each [B, n]."""

    def __init__(self, B, n):
        self.tokens = np.full((B, n), -7, np.int32)
        self.q = np.full((B, n), np.nan)
        self.cdf_lo = np.full((B, n), np.nan)
        self.cdf_hi = np.full((B, n), np.nan)


def draft_sample(logits, dtype, T, seed=0, pos0=0, b_offset=0):
    """Draft tokens drawn from softmax(logits / T) (argmax at T == 0) for
    logits [B, n, V] in storage form; row (b, t) draws with the DRAFT uniform
    of counter (b + b_offset, pos0 + t)."""
    logits = _storage(logits, dtype)
    B, n, V = logits.shape
    res = DraftResult(B, n)
    rc = lib().orc_draft_sample(_ptr(logits), B, n, V, dtype, float(T), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                int(pos0), int(b_offset), _ptr(res.tokens), _ptr(res.q),
                                _ptr(res.cdf_lo), _ptr(res.cdf_hi))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return res


def row_entropy(row, dtype, T):
    """H = -sum p ln p of softmax(row / T) (0 at T == 0; NaN if unusable)."""
    row = _storage(row, dtype)
    return lib().orc_row_entropy(_ptr(row), dtype, row.shape[-1], float(T))


def entropies(logits, dtype, T):
    """row_entropy of every row of logits [..., V]."""
    a = _storage(logits, dtype)
    flat = a.reshape(-1, a.shape[-1])
    return np.array([row_entropy(r, dtype, T) for r in flat]).reshape(a.shape[:-1])


def expected_accept(target, draft, dtype, T):
    """beta [B, g] = sum_x min(p_i(x), q_i(x)) for target [B, g+1, V], draft [B, g, V]."""
    target = _storage(target, dtype)
    draft = _storage(draft, dtype)
    B, g1, V = target.shape
    out = np.full((B, g1 - 1), np.nan)
    rc = lib().orc_expected_accept(_ptr(target), _ptr(draft), B, g1 - 1, V, dtype, float(T), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def tree_verify(target, draft, parent, token, dtype, T, threshold):
    """Token-tree verification (the pages' heuristic): target/draft [B, N, V]
    storage arrays (draft may be None at T == 0), parent/token [B, N] int32.
    Returns (tokens [B, N-1], nodes [B, N-1], n [B])."""
    target = _storage(target, dtype)
    draft = _storage(draft, dtype)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    token = np.ascontiguousarray(token, dtype=np.int32)
    B, N, V = target.shape
    tok = np.full((B, N - 1), -7, np.int32)
    nodes = np.full((B, N - 1), -7, np.int32)
    n = np.full(B, -7, np.int32)
    rc = lib().orc_tree_verify(_ptr(target), _ptr(draft), _ptr(parent), _ptr(token), B, N, V, dtype, float(T),
                               float(threshold), _ptr(tok), _ptr(nodes), _ptr(n))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return tok, nodes, n


def max_threads():
    return lib().orc_max_threads()


def set_threads(n):
    lib().orc_set_threads(int(n))
