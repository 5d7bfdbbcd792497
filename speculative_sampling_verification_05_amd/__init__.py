"""Python binding of libspecverify (batched speculative-sampling verification on gfx950).

Argument marshalling only: every step of the verification runs in the HIP
kernels behind the C ABI declared in include/specverify.h. PyTorch provides
device memory and the current stream. There is no fallback: if the shared
library is missing, importing the entry points raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB names another build of the same library (e.g. one whose host
# code carries address and undefined-behaviour checks)
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(HERE, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EHIP, SPEC_ENOMEM = 0, -1, -2, -3, -4
SPEC_F32, SPEC_BF16 = 0, 1
SCHEDULE_AUTO, SCHEDULE_GROUP, SCHEDULE_EARLY_STOP, SCHEDULE_POSITION, SCHEDULE_GROUP_TWO_PHASE = 0, 1, 2, 3, 4
MAX_GAMMA = 63

# every symbol include/specverify.h declares
EXPORTS = (
    "spec_verify",
    "spec_verify_ex",
    "spec_verify_noalloc",
    "spec_row_stats",
    "spec_draft_sample",
    "spec_draft_sample_ex",
    "spec_expected_accept",
    "spec_tree_verify",
    "spec_verify_schedule",
    "spec_verify_status",
    "spec_verify_set_wait_limit",
    "spec_verify_workspace_bytes",
    "spec_verify_release_workspace",
    "spec_verify_last_error",
    "spec_verify_abi_version",
)


class SpecVerifyError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"spec_verify failed ({code}): {msg}")
        self.code = code


class Extras(ctypes.Structure):
    """Mirror of spec_extras_t."""
    _fields_ = [
        ("row_max", ctypes.c_void_p),
        ("row_sumexp", ctypes.c_void_p),
        ("p_draft", ctypes.c_void_p),
        ("q_draft", ctypes.c_void_p),
        ("Z", ctypes.c_void_p),
        ("argmax", ctypes.c_void_p),
        ("b_offset", ctypes.c_int64),
        ("events", ctypes.c_void_p * 3),
        ("schedule", ctypes.c_int32),
    ]


class DraftExtras(ctypes.Structure):
    """Mirror of spec_draft_extras_t."""
    _fields_ = [
        ("entropy", ctypes.c_void_p),
        ("events", ctypes.c_void_p * 2),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspecverify.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    vp, i32, i64, u64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
    L.spec_verify.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, u64, vp, vp, vp]
    L.spec_verify.restype = ctypes.c_int
    L.spec_verify_ex.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, u64, vp, vp, vp,
                                 ctypes.POINTER(Extras)]
    L.spec_verify_ex.restype = ctypes.c_int
    L.spec_verify_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, u64, vp, vp, vp]
    L.spec_verify_noalloc.restype = ctypes.c_int
    L.spec_row_stats.argtypes = [vp, i64, i32, i32, f32, vp, vp, vp]
    L.spec_row_stats.restype = ctypes.c_int
    L.spec_draft_sample.argtypes = [vp, i32, i32, i32, i32, f32, u64, i64, i64, vp, vp, vp]
    L.spec_draft_sample.restype = ctypes.c_int
    L.spec_draft_sample_ex.argtypes = [vp, i32, i32, i32, i32, f32, u64, i64, i64, vp, vp, vp,
                                       ctypes.POINTER(DraftExtras)]
    L.spec_draft_sample_ex.restype = ctypes.c_int
    L.spec_expected_accept.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp]
    L.spec_expected_accept.restype = ctypes.c_int
    L.spec_tree_verify.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, vp, vp]
    L.spec_tree_verify.restype = ctypes.c_int
    L.spec_verify_schedule.argtypes = [i32, i32, i32, i32, f32]
    L.spec_verify_schedule.restype = i32
    L.spec_verify_status.argtypes = [vp, ctypes.POINTER(i32)]
    L.spec_verify_status.restype = ctypes.c_int
    L.spec_verify_set_wait_limit.argtypes = [i64]
    L.spec_verify_set_wait_limit.restype = i64
    L.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, i32, f32]
    L.spec_verify_workspace_bytes.restype = ctypes.c_size_t
    L.spec_verify_release_workspace.argtypes = []
    L.spec_verify_release_workspace.restype = None
    L.spec_verify_last_error.argtypes = []
    L.spec_verify_last_error.restype = ctypes.c_char_p
    L.spec_verify_abi_version.argtypes = []
    L.spec_verify_abi_version.restype = i32
    _lib = L
    return L


def last_error() -> str:
    return load_library().spec_verify_last_error().decode()


def _check(rc):
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, last_error())


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def verify(target_logits, draft_logits, draft_tokens, temperature: float, seed: int,
           out_tokens=None, out_n_accepted=None, stream=None, extras: Extras | None = None):
    """One verification step.

    target_logits [B, gamma+1, V] and draft_logits [B, gamma, V] (float32 or
    bfloat16, contiguous, on the GPU; draft_logits may be None at temperature 0),
    draft_tokens [B, gamma] int32. Returns (out_tokens [B, gamma+1] int32,
    out_n_accepted [B] int32), enqueued on `stream` (default: torch's current
    stream)."""
    import torch
    L = load_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    dt = _dtype_code(target_logits)
    for name, t in (("target_logits", target_logits), ("draft_logits", draft_logits),
                    ("draft_tokens", draft_tokens)):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if draft_logits is not None:
        if draft_logits.dtype != target_logits.dtype or tuple(draft_logits.shape) != (B, gamma, V):
            raise ValueError("draft_logits must be [B, gamma, V] with the target's dtype")
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, gamma):
        raise ValueError("draft_tokens must be int32 [B, gamma]")
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    if out_n_accepted is None:
        out_n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    args = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, gamma, V, dt,
            float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out_tokens),
            _ptr(out_n_accepted), _stream_handle(stream))
    if extras is None:
        _check(L.spec_verify(*args))
    else:
        _check(L.spec_verify_ex(*args, ctypes.byref(extras)))
    return out_tokens, out_n_accepted


def verify_noalloc(target_logits, draft_logits, draft_tokens, temperature: float, seed: int,
                   out_tokens, out_n_accepted, stream=None):
    """spec_verify_noalloc: the verification step with no device allocation,
    in the library or here. The caller passes every tensor, outputs included
    (out_tokens [B, gamma+1], out_n_accepted [B], int32, contiguous, on the
    GPU); shapes as verify()."""
    import torch
    L = load_library()
    B, g1, V = target_logits.shape
    for t in (target_logits, draft_logits, draft_tokens, out_tokens, out_n_accepted):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous GPU tensors")
    if tuple(out_tokens.shape) != (B, g1) or tuple(out_n_accepted.shape) != (B,) or \
            out_tokens.dtype != torch.int32 or out_n_accepted.dtype != torch.int32:
        raise ValueError("out_tokens must be int32 [B, gamma+1] and out_n_accepted int32 [B]")
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, g1 - 1):
        raise ValueError("draft_tokens must be int32 [B, gamma]")
    _check(L.spec_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, g1 - 1, V,
                                 _dtype_code(target_logits), float(temperature),
                                 int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out_tokens), _ptr(out_n_accepted),
                                 _stream_handle(stream)))
    return out_tokens, out_n_accepted


def verify_raw(target_ptr, draft_ptr, tokens_ptr, B, gamma, V, dtype, temperature, seed,
               out_tokens_ptr, out_n_ptr, stream_handle, extras: Extras | None = None) -> int:
    """Direct C-ABI call on raw device pointers; returns the status code."""
    L = load_library()
    args = (ctypes.c_void_p(target_ptr), ctypes.c_void_p(draft_ptr) if draft_ptr else None,
            ctypes.c_void_p(tokens_ptr), B, gamma, V, dtype, float(temperature),
            int(seed) & 0xFFFFFFFFFFFFFFFF, ctypes.c_void_p(out_tokens_ptr),
            ctypes.c_void_p(out_n_ptr), ctypes.c_void_p(stream_handle))
    if extras is None:
        return L.spec_verify(*args)
    return L.spec_verify_ex(*args, ctypes.byref(extras))


def row_stats(logits, temperature: float, stream=None):
    """Softmax statistics of every row of a [rows, V] tensor: (row_max float32,
    row_sumexp float64)."""
    import torch
    L = load_library()
    if logits.dim() != 2 or not logits.is_cuda or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, V] GPU tensor")
    rows, V = logits.shape
    m = torch.empty(rows, dtype=torch.float32, device=logits.device)
    s = torch.empty(rows, dtype=torch.float64, device=logits.device)
    _check(L.spec_row_stats(_ptr(logits), rows, V, _dtype_code(logits), float(temperature),
                            _ptr(m), _ptr(s), _stream_handle(stream)))
    return m, s


def draft_sample(logits, temperature: float, seed: int, pos0: int = 0, b_offset: int = 0,
                 want_q: bool = True, out_tokens=None, out_q=None, stream=None, events=None,
                 want_entropy: bool = False):
    """Draft tokens drawn from softmax(logits / T) (the first argmax at T == 0)
    for logits [B, n, V] (or [B, V], one position), float32 or bfloat16,
    contiguous, on the GPU; row (b, t) draws with the DRAFT uniform of counter
    (b + b_offset, pos0 + t). Returns (tokens int32, q float64 or None), each
    [B, n] (or [B]); -1 and NaN mark unusable rows. With want_entropy, a third
    tensor holds each row's entropy (float64, natural log)."""
    import torch
    L = load_library()
    if logits.dim() not in (2, 3) or not logits.is_cuda or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [B, n, V] or [B, V] GPU tensor")
    shape = tuple(logits.shape[:-1])
    B = shape[0]
    n = shape[1] if logits.dim() == 3 else 1
    V = logits.shape[-1]
    dev = logits.device
    if out_tokens is None:
        out_tokens = torch.empty(shape, dtype=torch.int32, device=dev)
    if want_q and out_q is None:
        out_q = torch.empty(shape, dtype=torch.float64, device=dev)
    args = (_ptr(logits), B, n, V, _dtype_code(logits), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
            int(pos0), int(b_offset), _ptr(out_tokens), _ptr(out_q if want_q else None), _stream_handle(stream))
    ent = torch.empty(shape, dtype=torch.float64, device=dev) if want_entropy else None
    if events is None and ent is None:
        _check(L.spec_draft_sample(*args))
    else:
        ex = DraftExtras()
        ex.entropy = ent.data_ptr() if ent is not None else None
        if events is not None:
            ex.events[0], ex.events[1] = events
        _check(L.spec_draft_sample_ex(*args, ctypes.byref(ex)))
    if want_entropy:
        return out_tokens, (out_q if want_q else None), ent
    return out_tokens, (out_q if want_q else None)


def expected_accept(target_logits, draft_logits, temperature: float, out=None, stream=None):
    """beta [B, gamma] float64: sum_x min(p_i(x), q_i(x)) for every position,
    the probability that a reached position accepts its draft token; target
    [B, gamma+1, V] and draft [B, gamma, V] on the GPU, same dtype, T > 0."""
    import torch
    L = load_library()
    if target_logits.dim() != 3 or draft_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V] and draft_logits [B, gamma, V]")
    B, g1, V = target_logits.shape
    for t in (target_logits, draft_logits):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("logits must be contiguous GPU tensors")
    if draft_logits.dtype != target_logits.dtype or tuple(draft_logits.shape) != (B, g1 - 1, V):
        raise ValueError("draft_logits must be [B, gamma, V] with the target's dtype")
    if out is None:
        out = torch.empty((B, g1 - 1), dtype=torch.float64, device=target_logits.device)
    _check(L.spec_expected_accept(_ptr(target_logits), _ptr(draft_logits), B, g1 - 1, V, _dtype_code(target_logits),
                                  float(temperature), _ptr(out), _stream_handle(stream)))
    return out


def tree_verify(target_logits, draft_logits, parent, token, temperature: float, threshold: float, stream=None):
    """Token-tree verification, the pages' heuristic mode (not distribution-
    preserving): target/draft [B, N, V] (draft may be None at T == 0), parent
    and token [B, N] int32, all on the GPU. Returns (tokens [B, N-1], nodes
    [B, N-1], n [B]) int32: the accepted path, -1 after it; n = -1 marks
    invalid input."""
    import torch
    L = load_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, N, V]")
    B, N, V = target_logits.shape
    for t in (target_logits, draft_logits, parent, token):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("inputs must be contiguous GPU tensors")
    if draft_logits is not None and (draft_logits.dtype != target_logits.dtype or
                                     tuple(draft_logits.shape) != (B, N, V)):
        raise ValueError("draft_logits must be [B, N, V] with the target's dtype")
    for name, t in (("parent", parent), ("token", token)):
        if t.dtype != torch.int32 or tuple(t.shape) != (B, N):
            raise ValueError(f"{name} must be int32 [B, N]")
    dev = target_logits.device
    tok = torch.empty((B, N - 1), dtype=torch.int32, device=dev)
    nodes = torch.empty((B, N - 1), dtype=torch.int32, device=dev)
    n = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(L.spec_tree_verify(_ptr(target_logits), _ptr(draft_logits), _ptr(parent), _ptr(token), B, N, V,
                              _dtype_code(target_logits), float(temperature), float(threshold), _ptr(tok),
                              _ptr(nodes), _ptr(n), _stream_handle(stream)))
    return tok, nodes, n


def auto_schedule(B, gamma, V, dtype, temperature) -> int:
    """The schedule SCHEDULE_AUTO takes for this shape (a rule of the shape
    alone, evaluated on the host)."""
    rc = load_library().spec_verify_schedule(B, gamma, V, dtype, float(temperature))
    if rc < 0:
        raise SpecVerifyError(rc, last_error())
    return rc


def status(stream=None) -> bool:
    """Whether a bounded in-kernel wait on `stream` (default: torch's current
    stream) ran out since the last status call; synchronises the stream and
    clears the flag."""
    flag = ctypes.c_int32(0)
    _check(load_library().spec_verify_status(_stream_handle(stream), ctypes.byref(flag)))
    return bool(flag.value)


def set_wait_limit(ticks: int) -> int:
    """Bound on every in-kernel wait of later calls, in device wall-clock ticks
    (100 MHz); negative restores the default. Returns the previous setting.
    For tests of the failure path only."""
    return int(load_library().spec_verify_set_wait_limit(int(ticks)))


def workspace_bytes(B, gamma, V, dtype, temperature) -> int:
    return int(load_library().spec_verify_workspace_bytes(B, gamma, V, dtype, float(temperature)))


def release_workspace():
    load_library().spec_verify_release_workspace()
