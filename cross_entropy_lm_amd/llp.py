"""ctypes binding of ``libllp.so`` with the C ABI's names (include/llp.h).

Argument marshalling only: every step of the computation runs in the HIP
library. torch provides device memory and the current stream; outputs and
workspaces that the caller does not pass are allocated here with
``torch.empty`` (the library itself allocates nothing). There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllp.so")

LLP_F32, LLP_BF16, LLP_F16 = 0, 1, 2
LLP_SCRATCH_BYTES = 64 << 20  # the device-global scratch of linear_logp_fwd_noalloc
LLP_OK, LLP_EINVAL, LLP_EWORKSPACE, LLP_EOVERFLOW, LLP_EHIP = 0, 1, 2, 3, 4

_lib = None

_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/llp.h
SIGNATURES = {
    "llp_version": (_int, []),
    "llp_strerror": (ctypes.c_char_p, [_int]),
    "linear_logp_chunk_rows": (_i64, [_i64, _i64, _i64]),
    "linear_logp_num_chunks": (_i64, [_i64, _i64, _i64]),
    "linear_logp_fwd_workspace_size": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_sz)]),
    "linear_logp_fwd": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "linear_logp_fwd_noalloc": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "linear_logp_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int, _i64, _int, _int, _int, _int,
                                              ctypes.POINTER(_sz)]),
    "linear_logp_bwd": (_int, [_i64, _i64, _i64, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _int, _vp, _int, _vp, _sz, _vp]),
    "linear_logp_fwd_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int, _i64, _int, _int, _int, _int,
                                                  ctypes.POINTER(_sz)]),
    "linear_logp_fwd_bwd": (_int, [_i64, _i64, _i64, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _int, _vp, _int, _vp, _sz, _vp]),
    "linear_logp_shard_fwd": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _sz, _vp]),
    "linear_logp_shard_combine": (_int, [_i64, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "linear_logp_shard_bwd": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _int, _vp, _int, _vp, _int, _vp, _sz, _vp]),
    "logp_fwd": (_int, [_i64, _i64, _int, _vp, _vp, _vp, _vp, _vp]),
    "logp_bwd": (_int, [_i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "llp_trace_enable": (_int, [_int]),
    "llp_trace_read": (_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64), _int]),
}

# kernel kinds of the launch trace (llp_kernel_kind)
TRACE_KINDS = ["fwd_lse", "combine", "dlogits", "dh_dw", "transpose", "small", "rows_fwd", "rows_bwd", "dh_dw_fwd",
               "dh_reduce", "dh_dw_dlogits"]


class LlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {llp_strerror(status)} (status {status})")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m cross_entropy_lm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(st: int, where: str):
    if st != LLP_OK:
        raise LlpError(st, where)


def _torch():
    import torch

    return torch


def dtype_code(dt) -> int:
    torch = _torch()
    codes = {torch.float32: LLP_F32, torch.bfloat16: LLP_BF16, torch.float16: LLP_F16}
    if dt not in codes:
        raise TypeError(f"unsupported dtype {dt}")
    return codes[dt]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ----------------------------------------------------------------------------- argument checks
# Everything the C ABI cannot see (a tensor's dtype, its shape beyond the sizes
# passed, its device) is checked here before the library is called, so that a
# mismatch raises instead of letting a kernel read or write past a buffer.
# dtype and shape checks come first; the device check last.

def _expect(t, name, shape, dtypes):
    """t is None, or a contiguous tensor of one of `dtypes` and exactly `shape`."""
    if t is None:
        return
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        want = " or ".join(str(d) for d in dtypes)
        raise TypeError(f"{name} must have dtype {want}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _contig(t, name)


def _operands(h, W):
    """(N, D, V, torch dtype) of h [N, D] and W [V, D] of one operand dtype."""
    torch = _torch()
    if not isinstance(h, torch.Tensor) or h.dim() != 2:
        raise ValueError("h must be a 2-D tensor [N, D]")
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor [V, D]")
    dtype_code(h.dtype)
    N, D = h.shape
    V = W.shape[0]
    _expect(h, "h", (N, D), (h.dtype,))
    _expect(W, "W", (V, D), (h.dtype,))
    return N, D, V, h.dtype


def _table_dtypes(op_dtype):
    torch = _torch()
    return (torch.float32,) if op_dtype == torch.float32 else (torch.float32, op_dtype)


def _same_device(named):
    """Every given tensor lives on one GPU; returns that device."""
    devs = [(n, t.device) for n, t in named if t is not None]
    for n, d in devs:
        if d.type != "cuda":
            raise ValueError(f"{n} must be a GPU tensor, got device {d}")
    if len({d for _, d in devs}) > 1:
        raise ValueError("tensors on different devices: " + ", ".join(f"{n}={d}" for n, d in devs))
    return devs[0][1] if devs else None


def _workspace_arg(workspace):
    if workspace is not None:
        torch = _torch()
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        _contig(workspace, "workspace")
    return workspace


class _OnStream:
    """Allocations made inside run on the caller's stream (the caching
    allocator then reuses a freed workspace only for later work on that
    stream); with no stream given, torch's current stream is used."""

    def __init__(self, stream, device):
        torch = _torch()
        self.ctx = None
        if stream is None:
            self.ptr = torch.cuda.current_stream(device).cuda_stream if device is not None else 0
        elif isinstance(stream, torch.cuda.Stream):
            self.ptr = stream.cuda_stream
            self.ctx = torch.cuda.stream(stream)
        else:
            self.ptr = int(stream)
            self.ctx = torch.cuda.stream(torch.cuda.ExternalStream(self.ptr, device=device))

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            return self.ctx.__exit__(*exc)
        return False


def llp_version() -> int:
    return lib().llp_version()


def llp_strerror(status: int) -> str:
    return lib().llp_strerror(status).decode()


def linear_logp_chunk_rows(N: int, V: int, chunk: int = 0) -> int:
    return lib().linear_logp_chunk_rows(N, V, chunk)


def linear_logp_num_chunks(N: int, V: int, chunk: int = 0) -> int:
    return lib().linear_logp_num_chunks(N, V, chunk)


def linear_logp_fwd_workspace_size(N: int, D: int, V: int, dtype: int) -> int:
    out = _sz(0)
    _check(lib().linear_logp_fwd_workspace_size(N, D, V, dtype, ctypes.byref(out)),
           "linear_logp_fwd_workspace_size")
    return out.value


def linear_logp_bwd_workspace_size(N, D, V, dtype, chunk=0, want_dH=True, want_dW=True,
                                   want_db=False, have_lse=True) -> int:
    out = _sz(0)
    _check(lib().linear_logp_bwd_workspace_size(N, D, V, dtype, chunk, int(want_dH), int(want_dW),
                                                int(want_db), int(have_lse), ctypes.byref(out)),
           "linear_logp_bwd_workspace_size")
    return out.value


def _workspace(nbytes, workspace, device):
    if workspace is not None:
        return workspace
    return _torch().empty(max(nbytes, 1), dtype=_torch().uint8, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


def _check_tables(V, D, op_dtype, dW_dtype, dW, db):
    """dW [V, D] and db [V] (each optional) share one dtype, float32 or the
    operand dtype; returns that dtype."""
    torch = _torch()
    ok = _table_dtypes(op_dtype)
    tdt = torch.float32 if dW_dtype is None else dW_dtype
    if tdt not in ok:
        raise TypeError(f"dW_dtype must be float32 or the operand dtype {op_dtype}, got {tdt}")
    _expect(dW, "dW", (V, D), ok)
    _expect(db, "db", (V,), ok)
    if dW is not None and db is not None and dW.dtype != db.dtype:
        raise TypeError(f"dW and db must share one dtype, got {dW.dtype} and {db.dtype}")
    if dW is not None:
        tdt = dW.dtype
    elif db is not None:
        tdt = db.dtype
    return tdt


def _grad_tables(V, D, op_dtype, dW_dtype, dW, db, accumulate, want_dW, want_db, device):
    """The dW / db tables to pass (allocated when requested and not given) and
    their common dtype (checked by _check_tables first)."""
    torch = _torch()
    tdt = _check_tables(V, D, op_dtype, dW_dtype, dW, db)
    if want_dW and dW is None:
        dW = (torch.zeros if accumulate else torch.empty)((V, D), dtype=tdt, device=device)
    if want_db and db is None:
        db = (torch.zeros if accumulate else torch.empty)((V,), dtype=tdt, device=device)
    return dW, db, tdt


def linear_logp_fwd(h, W, b, targets, logp=None, lse=None, workspace=None, stream=None,
                    want_lse=True):
    """logp [N] (and lse [N]) for h [N, D], W [V, D], b [V] or None, targets [N] int64."""
    torch = _torch()
    N, D, V, odt = _operands(h, W)
    _expect(b, "b", (V,), (odt,))
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(logp, "logp", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    _workspace_arg(workspace)
    dev = _same_device([("h", h), ("W", W), ("b", b), ("targets", targets), ("logp", logp), ("lse", lse),
                        ("workspace", workspace)])
    dt = dtype_code(odt)
    with _OnStream(stream, dev) as st_:
        if logp is None:
            logp = torch.empty(N, dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty(N, dtype=torch.float32, device=dev)
        ws = _workspace(linear_logp_fwd_workspace_size(N, D, V, dt), workspace, dev)
        st = lib().linear_logp_fwd(N, D, V, dt, _ptr(h), _ptr(W), _ptr(b), _ptr(targets), _ptr(logp),
                                   _ptr(lse), _ptr(ws), _nbytes(ws), st_.ptr)
    _check(st, "linear_logp_fwd")
    return logp, lse


def linear_logp_fwd_noalloc(h, W, b, targets, logp, lse=None, stream=None):
    """linear_logp_fwd into the caller's logp [N] (and lse [N] or None) with the
    library's device-global scratch instead of a workspace: nothing is
    allocated, here or in the library. Calls that overlap on one device race
    on that scratch."""
    torch = _torch()
    N, D, V, odt = _operands(h, W)
    _expect(b, "b", (V,), (odt,))
    _expect(targets, "targets", (N,), (torch.int64,))
    if logp is None:
        raise ValueError("logp is required (this call allocates nothing)")
    _expect(logp, "logp", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    dev = _same_device([("h", h), ("W", W), ("b", b), ("targets", targets), ("logp", logp), ("lse", lse)])
    ptr = _OnStream(stream, dev).ptr
    st = lib().linear_logp_fwd_noalloc(N, D, V, dtype_code(odt), _ptr(h), _ptr(W), _ptr(b), _ptr(targets),
                                       _ptr(logp), _ptr(lse), ptr)
    _check(st, "linear_logp_fwd_noalloc")
    return logp, lse


def linear_logp_bwd(h, W, b, targets, g, lse=None, want_dH=True, want_dW=True, want_db=False,
                    dW_dtype=None, chunk=0, accumulate=False, dH=None, dW=None, db=None,
                    workspace=None, stream=None):
    """(dH, dW, db) for the requested outputs (None for the others).

    ``dW_dtype`` is the dW/db table dtype (torch.float32 by default, or the
    operand dtype). With ``accumulate`` the caller's dW/db are added into.
    """
    torch = _torch()
    N, D, V, odt = _operands(h, W)
    _expect(b, "b", (V,), (odt,))
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(g, "g", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    _expect(dH, "dH", (N, D), (odt,))
    _workspace_arg(workspace)
    if (want_db or db is not None) and b is None:
        raise ValueError("db needs a bias b")
    _check_tables(V, D, odt, dW_dtype, dW, db)
    dev = _same_device([("h", h), ("W", W), ("b", b), ("targets", targets), ("g", g), ("lse", lse),
                        ("dH", dH), ("dW", dW), ("db", db), ("workspace", workspace)])
    dt = dtype_code(odt)
    with _OnStream(stream, dev) as st_:
        dW, db, tdt = _grad_tables(V, D, odt, dW_dtype, dW, db, accumulate, want_dW, want_db, dev)
        if want_dH and dH is None:
            dH = torch.empty((N, D), dtype=odt, device=dev)
        nbytes = linear_logp_bwd_workspace_size(N, D, V, dt, chunk, dH is not None, dW is not None,
                                                db is not None, lse is not None)
        ws = _workspace(nbytes, workspace, dev)
        st = lib().linear_logp_bwd(N, D, V, dt, chunk, _ptr(h), _ptr(W), _ptr(b), _ptr(targets), _ptr(g),
                                   _ptr(lse), _ptr(dH), _ptr(dW), dtype_code(tdt), _ptr(db),
                                   int(bool(accumulate)), _ptr(ws), _nbytes(ws), st_.ptr)
    _check(st, "linear_logp_bwd")
    return dH, dW, db


def linear_logp_fwd_bwd_workspace_size(N, D, V, dtype, chunk=0, want_dH=True, want_dW=True,
                                       want_db=False, have_lse=True) -> int:
    out = _sz(0)
    _check(lib().linear_logp_fwd_bwd_workspace_size(N, D, V, dtype, chunk, int(want_dH), int(want_dW),
                                                    int(want_db), int(have_lse), ctypes.byref(out)),
           "linear_logp_fwd_bwd_workspace_size")
    return out.value


def linear_logp_fwd_bwd(h, W, b, targets, g, want_dH=True, want_dW=True, want_db=False, dW_dtype=None,
                        chunk=0, accumulate=False, logp=None, lse=None, want_lse=True, dH=None, dW=None,
                        db=None, workspace=None, stream=None):
    """(logp, lse, dH, dW, db) in one call, for an upstream g known before the forward."""
    torch = _torch()
    N, D, V, odt = _operands(h, W)
    _expect(b, "b", (V,), (odt,))
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(g, "g", (N,), (torch.float32,))
    _expect(logp, "logp", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    _expect(dH, "dH", (N, D), (odt,))
    _workspace_arg(workspace)
    if (want_db or db is not None) and b is None:
        raise ValueError("db needs a bias b")
    _check_tables(V, D, odt, dW_dtype, dW, db)
    dev = _same_device([("h", h), ("W", W), ("b", b), ("targets", targets), ("g", g), ("logp", logp),
                        ("lse", lse), ("dH", dH), ("dW", dW), ("db", db), ("workspace", workspace)])
    dt = dtype_code(odt)
    with _OnStream(stream, dev) as st_:
        dW, db, tdt = _grad_tables(V, D, odt, dW_dtype, dW, db, accumulate, want_dW, want_db, dev)
        if logp is None:
            logp = torch.empty(N, dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty(N, dtype=torch.float32, device=dev)
        if want_dH and dH is None:
            dH = torch.empty((N, D), dtype=odt, device=dev)
        nbytes = linear_logp_fwd_bwd_workspace_size(N, D, V, dt, chunk, dH is not None, dW is not None,
                                                    db is not None, lse is not None)
        ws = _workspace(nbytes, workspace, dev)
        st = lib().linear_logp_fwd_bwd(N, D, V, dt, chunk, _ptr(h), _ptr(W), _ptr(b), _ptr(targets), _ptr(g),
                                       _ptr(logp), _ptr(lse), _ptr(dH), _ptr(dW), dtype_code(tdt), _ptr(db),
                                       int(bool(accumulate)), _ptr(ws), _nbytes(ws), st_.ptr)
    _check(st, "linear_logp_fwd_bwd")
    return logp, lse, dH, dW, db


def linear_logp_shard_fwd(h, W_shard, b_shard, targets, v0, Vt, lse_shard=None, zt_shard=None,
                          workspace=None, stream=None):
    """(lse_shard [N], zt_shard [N]) of the vocabulary share W_shard = rows [v0, v0 + Vs) of a
    Vt-row vocabulary; zt_shard is -inf where the share does not hold the target."""
    torch = _torch()
    N, D, Vs, odt = _operands(h, W_shard)
    _expect(b_shard, "b_shard", (Vs,), (odt,))
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(lse_shard, "lse_shard", (N,), (torch.float32,))
    _expect(zt_shard, "zt_shard", (N,), (torch.float32,))
    _workspace_arg(workspace)
    dev = _same_device([("h", h), ("W_shard", W_shard), ("b_shard", b_shard), ("targets", targets),
                        ("lse_shard", lse_shard), ("zt_shard", zt_shard), ("workspace", workspace)])
    dt = dtype_code(odt)
    with _OnStream(stream, dev) as st_:
        if lse_shard is None:
            lse_shard = torch.empty(N, dtype=torch.float32, device=dev)
        if zt_shard is None:
            zt_shard = torch.empty(N, dtype=torch.float32, device=dev)
        ws = _workspace(linear_logp_fwd_workspace_size(N, D, Vs, dt), workspace, dev)
        st = lib().linear_logp_shard_fwd(N, D, Vs, v0, Vt, dt, _ptr(h), _ptr(W_shard), _ptr(b_shard),
                                         _ptr(targets), _ptr(lse_shard), _ptr(zt_shard), _ptr(ws), _nbytes(ws),
                                         st_.ptr)
    _check(st, "linear_logp_shard_fwd")
    return lse_shard, zt_shard


def linear_logp_shard_combine(lse_shards, zt_shards, targets, Vt, logp=None, lse=None, want_lse=True,
                              stream=None):
    """(logp [N], lse [N]) from the shares' [P, N] lse and target-logit rows."""
    torch = _torch()
    if not isinstance(lse_shards, torch.Tensor) or lse_shards.dim() != 2:
        raise ValueError("lse_shards must be a 2-D tensor [P, N]")
    P, N = lse_shards.shape
    _expect(lse_shards, "lse_shards", (P, N), (torch.float32,))
    _expect(zt_shards, "zt_shards", (P, N), (torch.float32,))
    if zt_shards is None:
        raise ValueError("zt_shards is required")
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(logp, "logp", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    dev = _same_device([("lse_shards", lse_shards), ("zt_shards", zt_shards), ("targets", targets),
                        ("logp", logp), ("lse", lse)])
    with _OnStream(stream, dev) as st_:
        if logp is None:
            logp = torch.empty(N, dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty(N, dtype=torch.float32, device=dev)
        st = lib().linear_logp_shard_combine(N, P, _ptr(lse_shards), _ptr(zt_shards), _ptr(targets), Vt,
                                             _ptr(logp), _ptr(lse), st_.ptr)
    _check(st, "linear_logp_shard_combine")
    return logp, lse


def linear_logp_shard_bwd(h, W_shard, b_shard, targets, g, lse, v0, Vt, want_dH=True, want_dW=True,
                          want_db=False, dH_dtype=None, dW_dtype=None, chunk=0, accumulate=False, dH=None,
                          dW=None, db=None, workspace=None, stream=None):
    """(dH partial [N, D], dW_shard [Vs, D], db_shard [Vs]) of one vocabulary share, given the
    global lse. ``dH_dtype`` is float32 by default (the partials are summed by the caller)."""
    torch = _torch()
    N, D, Vs, odt = _operands(h, W_shard)
    _expect(b_shard, "b_shard", (Vs,), (odt,))
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(g, "g", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    if lse is None:
        raise ValueError("lse (the merged lse of every share) is required")
    hdt = torch.float32 if dH_dtype is None else dH_dtype
    if hdt not in _table_dtypes(odt):
        raise TypeError(f"dH_dtype must be float32 or the operand dtype {odt}, got {hdt}")
    _expect(dH, "dH", (N, D), _table_dtypes(odt))
    if dH is not None:
        hdt = dH.dtype
    _workspace_arg(workspace)
    if (want_db or db is not None) and b_shard is None:
        raise ValueError("db needs a bias b_shard")
    _check_tables(Vs, D, odt, dW_dtype, dW, db)
    dev = _same_device([("h", h), ("W_shard", W_shard), ("b_shard", b_shard), ("targets", targets), ("g", g),
                        ("lse", lse), ("dH", dH), ("dW", dW), ("db", db), ("workspace", workspace)])
    dt = dtype_code(odt)
    with _OnStream(stream, dev) as st_:
        dW, db, tdt = _grad_tables(Vs, D, odt, dW_dtype, dW, db, accumulate, want_dW, want_db, dev)
        if want_dH and dH is None:
            dH = torch.empty((N, D), dtype=hdt, device=dev)
        nbytes = linear_logp_bwd_workspace_size(N, D, Vs, dt, chunk, dH is not None, dW is not None,
                                                db is not None, True)
        ws = _workspace(nbytes, workspace, dev)
        st = lib().linear_logp_shard_bwd(N, D, Vs, v0, Vt, dt, chunk, _ptr(h), _ptr(W_shard), _ptr(b_shard),
                                         _ptr(targets), _ptr(g), _ptr(lse), _ptr(dH), dtype_code(hdt), _ptr(dW),
                                         dtype_code(tdt), _ptr(db), int(bool(accumulate)), _ptr(ws), _nbytes(ws),
                                         st_.ptr)
    _check(st, "linear_logp_shard_bwd")
    return dH, dW, db


def _logits_arg(logits):
    torch = _torch()
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits must be a 2-D tensor [N, V]")
    dtype_code(logits.dtype)
    _contig(logits, "logits")
    return logits.shape


def logp_fwd(logits, targets, logp=None, lse=None, want_lse=True, stream=None):
    """Logits-only forward: logp [N] (and lse [N]) from logits [N, V]."""
    torch = _torch()
    N, V = _logits_arg(logits)
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(logp, "logp", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    dev = _same_device([("logits", logits), ("targets", targets), ("logp", logp), ("lse", lse)])
    with _OnStream(stream, dev) as st_:
        if logp is None:
            logp = torch.empty(N, dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty(N, dtype=torch.float32, device=dev)
        st = lib().logp_fwd(N, V, dtype_code(logits.dtype), _ptr(logits), _ptr(targets), _ptr(logp),
                            _ptr(lse), st_.ptr)
    _check(st, "logp_fwd")
    return logp, lse


def logp_bwd(logits, targets, g, lse=None, dlogits=None, stream=None):
    """Logits-only backward: dlogits [N, V] (the logits' dtype; may be the logits tensor itself)."""
    torch = _torch()
    N, V = _logits_arg(logits)
    _expect(targets, "targets", (N,), (torch.int64,))
    _expect(g, "g", (N,), (torch.float32,))
    _expect(lse, "lse", (N,), (torch.float32,))
    _expect(dlogits, "dlogits", (N, V), (logits.dtype,))
    dev = _same_device([("logits", logits), ("targets", targets), ("g", g), ("lse", lse), ("dlogits", dlogits)])
    with _OnStream(stream, dev) as st_:
        if dlogits is None:
            dlogits = torch.empty_like(logits)
        st = lib().logp_bwd(N, V, dtype_code(logits.dtype), _ptr(logits), _ptr(targets), _ptr(g),
                            _ptr(lse), _ptr(dlogits), st_.ptr)
    _check(st, "logp_bwd")
    return dlogits


def llp_trace_enable(on: bool = True) -> None:
    _check(lib().llp_trace_enable(int(bool(on))), "llp_trace_enable")


def llp_trace_read() -> dict:
    """{kind: (total ms, launches)} of the current thread's trace (waits for its events)."""
    n = len(TRACE_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (_i64 * n)()
    st = lib().llp_trace_read(ms, cnt, n)
    if st not in (LLP_OK, LLP_EOVERFLOW):
        _check(st, "llp_trace_read")
    return {k: (ms[i], cnt[i]) for i, k in enumerate(TRACE_KINDS)}
