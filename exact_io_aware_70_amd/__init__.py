"""Python binding of libfa.so (exact IO-aware attention on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels behind
the C ABI declared in ``include/fa.h``.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing or cannot be loaded, every call raises.

    o, lse = fa_fwd(q, k, v, causal=True)               # q, k, v: [B, H, N, d] on the GPU
    dq, dk, dv = fa_bwd(q, k, v, o, lse, do, causal=True)

Tensors must be contiguous, on one GPU, all float32 or all bfloat16, d in {64, 128}.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FAError", "library_path", "load_library", "fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_workspace_size",
           "fa_status_string", "fa_version", "FA_OK", "FA_F32", "FA_BF16", "FA_BWD_LAUNCHES",
           "FA_NOALLOC_SCRATCH_BYTES", "fa_std_ld", "fa_std_fwd", "fa_std_bwd"]

FA_OK = 0
FA_F32 = 0
FA_BF16 = 1
FA_BWD_LAUNCHES = 2  # kernel launches per fa_bwd call: dQ (which also forms D), then dK/dV
FA_NOALLOC_SCRATCH_BYTES = 16 << 20  # static backward scratch of fa_bwd_noalloc, per GPU

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FAError(RuntimeError):
    """A libfa call returned a non-zero fa_status."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {fa_status_string(code)} (status {code})")


def library_path() -> str:
    return os.environ.get("FA_LIBRARY", os.path.join(_HERE, "libfa.so"))


def load_library() -> ctypes.CDLL:
    """Load libfa.so once and declare the C signatures; raises if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libfa.so not found at {path}; build it with "
                           "`python -m exact_io_aware_70_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp,
                                 ctypes.POINTER(vp)]
    lib.fa_bwd_timed.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, f, u64, u32, vp]
    lib.fa_fwd_dropout.restype = i
    lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, f, u64, u32, vp, sz, vp,
                                   ctypes.POINTER(vp)]
    lib.fa_bwd_dropout.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_softmax_rows.argtypes = [vp, vp, vp, ctypes.c_longlong, i, i, vp]
    lib.fa_softmax_rows.restype = i
    lib.fa_std_ld.argtypes = [i]
    lib.fa_std_ld.restype = i
    lib.fa_std_matrix_bytes.argtypes = [i, i, i]
    lib.fa_std_matrix_bytes.restype = sz
    lib.fa_std_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_std_fwd.restype = i
    lib.fa_std_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_std_bwd.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    _LIB = lib
    return lib


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def fa_version() -> int:
    return int(load_library().fa_version())


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int, dtype: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d, dtype))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check(name: str, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _workspace(workspace, need: int, device):
    """The caller's backward workspace, checked (on `device`, contiguous, >= need bytes), or a
    new one.  The C side sees only a raw pointer and a byte count."""
    import torch
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.device != device:
        raise ValueError(f"workspace: on {workspace.device}, expected {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError(f"workspace: {have} bytes, fa_bwd_workspace_size gives {need}")
    return workspace


def _event_handles(events, stream, device):
    """ctypes array of the FA_BWD_LAUNCHES + 1 torch events' HIP handles (None passes through)."""
    import torch
    if events is None:
        return None
    if len(events) != FA_BWD_LAUNCHES + 1:
        raise ValueError(f"events: need {FA_BWD_LAUNCHES + 1} events")
    s = stream if stream is not None else torch.cuda.current_stream(device)
    handles = (ctypes.c_void_p * len(events))()
    for n, ev in enumerate(events):
        if ev.cuda_event == 0:  # torch creates the underlying event on its first record
            ev.record(s)
        handles[n] = ev.cuda_event
    return handles


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def fa_fwd(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None):
    """Forward pass: returns (o [B,H,N,d] in q's dtype, lse [B,H,N] float32).

    ``o`` and ``lse`` may be passed preallocated; ``scale`` defaults to 1/sqrt(d).
    Work is enqueued on ``stream`` (default: the current torch stream) without waiting.
    """
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check("o", o, (B, H, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, N, d, sc, 1 if causal else 0, _dtype_code(q), _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return o, lse


def fa_bwd(q, k, v, o, lse, do, dq=None, dk=None, dv=None, scale=None, causal=False,
           workspace=None, stream=None, events=None):
    """Backward pass: returns (dq, dk, dv) for the loss sum(o * do).

    ``o`` and ``lse`` are what fa_fwd returned for (q, k, v).  ``workspace`` (a uint8 device
    tensor of at least fa_bwd_workspace_size bytes) may be passed to avoid an allocation.
    ``events``: optional list of FA_BWD_LAUNCHES + 1 torch.cuda.Event(enable_timing=True);
    the library records events[i] before its launch i and the last one after (fa_bwd_timed),
    so events[i].elapsed_time(events[i + 1]) is the duration of launch i.
    """
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    code = _dtype_code(q)
    workspace = _workspace(workspace, fa_bwd_workspace_size(B, H, N, d, code), dev)
    if events is not None and len(events) != FA_BWD_LAUNCHES + 1:
        raise ValueError(f"events: need {FA_BWD_LAUNCHES + 1} events")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, sc, 1 if causal else 0, code,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    if events is None:
        st = lib.fa_bwd(*args)
        where = "fa_bwd"
    else:
        st = lib.fa_bwd_timed(*args, _event_handles(events, stream, dev))
        where = "fa_bwd_timed"
    if st != FA_OK:
        raise FAError(st, where)
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale=None, causal=False, stream=None):
    """fa_bwd without a workspace argument, for callers that cannot allocate device memory:
    the library keeps the workspace in a static per-GPU array (FA_NOALLOC_SCRATCH_BYTES),
    and calls that overlap on one GPU race.  dq, dk, dv must be passed preallocated; nothing
    is allocated here or in the library.  Returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, sc, 1 if causal else 0,
                            _dtype_code(q), _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_std_ld(N: int) -> int:
    """Row stride of the standard path's N x N matrices (N rounded up to 128; 0 if N is out of range)."""
    return int(load_library().fa_std_ld(N))


def fa_std_fwd(q, k, v, o=None, lse=None, p=None, scale=None, causal=False, stream=None):
    """Standard (materialising) attention forward, bf16: S = scale q k^T is written to HBM,
    softmaxed in place into P, then o = P v.  Returns (o, lse, p) with p the probability
    matrix [B, H, N, fa_std_ld(N)] bf16 (padding columns 0), which fa_std_bwd reads."""
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    ld = fa_std_ld(N)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    p = torch.empty((B, H, N, max(ld, 1)), dtype=q.dtype, device=dev) if p is None else p
    _check("o", o, (B, H, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    _check("p", p, (B, H, N, ld), q.dtype, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_std_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), p.data_ptr(),
                        B, H, N, d, sc, 1 if causal else 0, _dtype_code(q), _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_std_fwd")
    return o, lse, p


def fa_std_bwd(q, k, v, do, p, dq=None, dk=None, dv=None, dp=None, scale=None, causal=False, stream=None):
    """Standard attention backward from the stored P of fa_std_fwd: dP = do v^T is written to
    ``dp`` (workspace, the shape of p; allocated if None), turned into dS in place, then
    dq = scale dS k, dk = scale dS^T q, dv = P^T do.  Returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    ld = fa_std_ld(N)
    _check("p", p, (B, H, N, ld), q.dtype, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    dp = torch.empty_like(p) if dp is None else dp
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    _check("dp", dp, (B, H, N, ld), q.dtype, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_std_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), p.data_ptr(), dq.data_ptr(),
                        dk.data_ptr(), dv.data_ptr(), dp.data_ptr(), B, H, N, d, sc, 1 if causal else 0,
                        _dtype_code(q), _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_std_bwd")
    return dq, dk, dv


def fa_softmax_rows(x, y=None, lse=None, with_lse=True, stream=None):
    """Row-wise softmax of a 2-D [rows, cols] tensor: returns (y, lse or None).

    ``y`` (x's shape and dtype; may be ``x`` itself for in place) and ``lse`` ([rows]
    float32) may be passed preallocated; ``with_lse=False`` skips the logsumexp.  Work is
    enqueued on ``stream`` (default: the current torch stream) without waiting.
    """
    import torch
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = x.shape
    dev = x.device
    _check("x", x, (rows, cols), x.dtype, dev)
    y = torch.empty_like(x) if y is None else y
    _check("y", y, (rows, cols), x.dtype, dev)
    if with_lse and lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    if lse is not None:
        _check("lse", lse, (rows,), torch.float32, dev)
    st = lib.fa_softmax_rows(x.data_ptr(), y.data_ptr(), None if lse is None else lse.data_ptr(), rows, cols,
                             _dtype_code(x), _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_softmax_rows")
    return y, lse


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o=None, lse=None, scale=None, causal=False,
               stream=None):
    """FP8 forward: q8, k8, v8 are uint8 E4M3 codes [B,H,N,d] (or torch.float8_e4m3fn);
    the descales are float32 [B,H].  Returns (o [B,H,N,d] bfloat16, lse [B,H,N] float32)."""
    import torch
    lib = load_library()
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    dev = q8.device
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name}: dtype {t.dtype}, expected uint8 codes or float8_e4m3fn")
        _check(name, t, (B, H, N, d), t.dtype, dev)
    for name, t in (("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)):
        _check(name, t, (B, H), torch.float32, dev)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check("o", o, (B, H, N, d), torch.bfloat16, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(),
                        v_descale.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, sc, 1 if causal else 0,
                        _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return o, lse


def fa_fwd_dropout(q, k, v, dropout_p, seed, offset=0, o=None, lse=None, scale=None, causal=False, stream=None):
    """Forward pass with dropout on the probabilities (bf16): returns (o, lse)."""
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check("o", o, (B, H, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, sc,
                            1 if causal else 0, _dtype_code(q), float(dropout_p), int(seed), int(offset),
                            _stream_handle(stream, dev))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_dropout")
    return o, lse


def fa_bwd_dropout(q, k, v, o, lse, do, dropout_p, seed, offset=0, dq=None, dk=None, dv=None, scale=None,
                   causal=False, workspace=None, stream=None, events=None):
    """Backward pass of fa_fwd_dropout (same seed and offset): returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    code = _dtype_code(q)
    workspace = _workspace(workspace, fa_bwd_workspace_size(B, H, N, d, code), dev)
    if events is not None and len(events) != FA_BWD_LAUNCHES + 1:
        raise ValueError(f"events: need {FA_BWD_LAUNCHES + 1} events")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    handles = _event_handles(events, stream, dev)
    st = lib.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, sc, 1 if causal else 0, code,
                            float(dropout_p), int(seed), int(offset), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream_handle(stream, dev), handles)
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dropout")
    return dq, dk, dv
