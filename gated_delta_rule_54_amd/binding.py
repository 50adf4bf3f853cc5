"""Thin ctypes binding of libgdr (include/gdr.h): argument marshalling only.

Every function here has the name of the C entry point it wraps.  Torch is
used for device memory (outputs and workspace are allocated as torch
tensors) and for the current HIP stream; all arithmetic runs in libgdr's
kernels.  If libgdr.so has not been built, loading fails loudly.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK = 0
GDR_F32, GDR_BF16 = 0, 1
GDR_ALGO_AUTO, GDR_ALGO_SEQUENTIAL, GDR_ALGO_CHUNKED = 0, 1, 2
GDR_USE_QK_L2NORM, GDR_CHANNELWISE, GDR_FUSED_GATES, GDR_SAVE_CHUNKS = 1, 2, 4, 8
ALGOS = {"auto": GDR_ALGO_AUTO, "sequential": GDR_ALGO_SEQUENTIAL,
         "chunked": GDR_ALGO_CHUNKED}

# Every symbol include/gdr.h declares.
SYMBOLS = ("gdr_keeps_chunks", "gdr_forward_workspace", "gdr_backward_workspace", "gdr_forward",
           "gdr_backward", "gdr_forward_noalloc", "gdr_forward_varlen", "gdr_backward_varlen",
           "gdr_profile_enable", "gdr_profile_read",
           "gdr_status_str", "gdr_last_hip_error", "gdr_abi_version")
# Every symbol include/gdr_calib.h declares (device ceilings for the benchmark).
CALIB_SYMBOLS = ("gdr_calib_copy", "gdr_calib_mfma")


class GdrProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64),
                ("Hk", ctypes.c_int32), ("Hv", ctypes.c_int32),
                ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("algo", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32)]


class GdrKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("total_ms", ctypes.c_double),
                ("launches", ctypes.c_int64)]


class GdrError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().gdr_status_str(status).decode()
        if status == 6:
            msg += ": " + lib().gdr_last_hip_error().decode()
        super().__init__(f"{where}: status {status} ({msg})")


_lib = None


def lib():
    """The loaded libgdr.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GdrProblem)
        vp, fp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
        L.gdr_keeps_chunks.argtypes = [P, ctypes.POINTER(ctypes.c_int)]
        L.gdr_forward_workspace.argtypes = [P, ctypes.POINTER(sz)]
        L.gdr_backward_workspace.argtypes = [P, ctypes.POINTER(sz)]
        L.gdr_forward.argtypes = [P, vp, vp, vp, fp, fp, fp, vp, fp, vp, sz, vp]
        L.gdr_backward.argtypes = [P, vp, vp, vp, fp, fp, fp, vp, fp,
                                   vp, vp, vp, fp, fp, fp, vp, sz, vp]
        L.gdr_forward_noalloc.argtypes = [P, vp, vp, vp, fp, fp, fp, vp, fp, vp]
        L.gdr_forward_varlen.argtypes = [P, vp, vp, vp, vp, fp, fp, fp, vp, fp, vp, sz, vp]
        L.gdr_backward_varlen.argtypes = [P, vp, vp, vp, vp, fp, fp, fp, vp, fp,
                                          vp, vp, vp, fp, fp, fp, vp, sz, vp]
        L.gdr_calib_copy.argtypes = [vp, vp, sz, vp]
        L.gdr_calib_mfma.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_double), vp]
        for name in ("gdr_keeps_chunks", "gdr_calib_copy", "gdr_calib_mfma",
                     "gdr_forward_workspace", "gdr_backward_workspace",
                     "gdr_forward", "gdr_backward", "gdr_forward_noalloc", "gdr_forward_varlen",
                     "gdr_backward_varlen"):
            getattr(L, name).restype = ctypes.c_int
        L.gdr_profile_enable.argtypes = [ctypes.c_int]
        L.gdr_profile_enable.restype = ctypes.c_int
        L.gdr_profile_read.argtypes = [ctypes.POINTER(GdrKernelTime), ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int)]
        L.gdr_profile_read.restype = ctypes.c_int
        L.gdr_status_str.argtypes = [ctypes.c_int]
        L.gdr_status_str.restype = ctypes.c_char_p
        L.gdr_last_hip_error.restype = ctypes.c_char_p
        L.gdr_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _dt(t):
    if t == torch.float32:
        return GDR_F32
    if t == torch.bfloat16:
        return GDR_BF16
    raise TypeError(f"unsupported dtype {t}")


def make_problem(B, T, Hk, Hv, Dk, Dv, io_dtype, out_dtype, use_qk_l2norm=True,
                 channelwise=False, algo="auto", chunk_size=0, fused_gates=False, save_chunks=False):
    flags = ((GDR_USE_QK_L2NORM if use_qk_l2norm else 0) | (GDR_CHANNELWISE if channelwise else 0)
             | (GDR_FUSED_GATES if fused_gates else 0) | (GDR_SAVE_CHUNKS if save_chunks else 0))
    return GdrProblem(B, T, Hk, Hv, Dk, Dv, _dt(io_dtype), _dt(out_dtype), flags,
                      ALGOS[algo], chunk_size)


def gdr_keeps_chunks(prob):
    """Whether GDR_SAVE_CHUNKS takes effect for this problem."""
    n = ctypes.c_int(0)
    st = lib().gdr_keeps_chunks(ctypes.byref(prob), ctypes.byref(n))
    if st != GDR_OK:
        raise GdrError(st, "gdr_keeps_chunks")
    return bool(n.value)


def gdr_calib_copy(src, dst, stream=None):
    """dst <- src with the library's streaming copy kernel (same byte size)."""
    _check(src, "src")
    _check(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    st = lib().gdr_calib_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream))
    if st != GDR_OK:
        raise GdrError(st, "gdr_calib_copy")


def gdr_calib_mfma(out, workgroups, iters, stream=None):
    """The matrix-core loop of gdr_calib_mfma into out (float32, at least
    workgroups * 256 elements); returns the FLOPs the launch executes."""
    _check(out, "out", torch.float32)
    if out.numel() < workgroups * 256:
        raise ValueError("out holds fewer than workgroups * 256 floats")
    fl = ctypes.c_double(0.0)
    st = lib().gdr_calib_mfma(_ptr(out), workgroups, iters, ctypes.byref(fl), _stream(stream))
    if st != GDR_OK:
        raise GdrError(st, "gdr_calib_mfma")
    return fl.value


def gdr_forward_workspace(prob):
    n = ctypes.c_size_t(0)
    st = lib().gdr_forward_workspace(ctypes.byref(prob), ctypes.byref(n))
    if st != GDR_OK:
        raise GdrError(st, "gdr_forward_workspace")
    return n.value


def gdr_backward_workspace(prob):
    n = ctypes.c_size_t(0)
    st = lib().gdr_backward_workspace(ctypes.byref(prob), ctypes.byref(n))
    if st != GDR_OK:
        raise GdrError(st, "gdr_backward_workspace")
    return n.value


def gdr_profile_enable(on=True):
    st = lib().gdr_profile_enable(1 if on else 0)
    if st != GDR_OK:
        raise GdrError(st, "gdr_profile_enable")


def gdr_profile_read():
    """{kernel name: (total ms, launches)} of the events recorded since the
    last read; waits for them to complete."""
    cap = 32
    buf = (GdrKernelTime * cap)()
    n = ctypes.c_int(0)
    st = lib().gdr_profile_read(buf, cap, ctypes.byref(n))
    if st != GDR_OK:
        raise GdrError(st, "gdr_profile_read")
    return {buf[i].name.decode(): (buf[i].total_ms, buf[i].launches) for i in range(min(n.value, cap))}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


class SavedChunks:
    """What a ``gdr_forward(..., save_for_backward=True)`` call leaves for the
    ``gdr_backward`` of the same problem and inputs: the workspace holding its
    chunk images and chunk entry states (GDR_SAVE_CHUNKS), or, where the
    library does not keep chunks for the problem (``kept`` False: the
    sequential algorithm, fp32 io, Dk = 16, the channelwise gate), nothing,
    and the backward then recomputes."""

    def __init__(self, ws, key, kept=True):
        self.ws, self.key, self.kept = ws, key, kept


def _save_key(prob):
    return (prob.B, prob.T, prob.Hk, prob.Hv, prob.Dk, prob.Dv, prob.io_dtype,
            prob.flags & ~GDR_SAVE_CHUNKS, prob.algo, prob.chunk_size)


def _ragged_dims(q, cu_seqlens, max_seqlen):
    """(number of sequences, length bound) of a ragged batch.  Without
    ``max_seqlen`` the offsets are read back once and checked (start at or
    after row 0, non-decreasing, end at or before the last row); with it the
    caller vouches for them and nothing waits on the device."""
    if q.shape[0] != 1:
        raise ValueError("a ragged batch holds its sequences in one row: q must be [1, rows, Hk, Dk]")
    if cu_seqlens.dtype != torch.int64 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-d int64 device tensor")
    if cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be on the device of q")
    n = cu_seqlens.numel() - 1
    if n < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        lens = cu[1:] - cu[:-1]
        if int(cu[0]) < 0 or int(cu[-1]) > q.shape[1] or (n > 0 and int(lens.min()) < 0):
            raise ValueError(f"cu_seqlens must rise from >= 0 to <= {q.shape[1]} rows")
        max_seqlen = int(lens.max()) if n > 0 else 0
    elif max_seqlen < 0:
        raise ValueError("max_seqlen must be >= 0")
    return n, max_seqlen


def _check_shapes(B, T, Hk, Hv, Dk, Dv, N, channelwise, tensors):
    """Every operand's shape against the problem the call describes (the
    library takes pointers and sizes only, so this is the last place a
    mismatch can be caught), and every operand on one device.  B, T are the
    tensor dims (1, rows for a ragged batch); N is the number of states."""
    want = {"q": (B, T, Hk, Dk), "k": (B, T, Hk, Dk), "v": (B, T, Hv, Dv), "dout": (B, T, Hv, Dv),
            "g": (B, T, Hv, Dk) if channelwise else (B, T, Hv), "beta": (B, T, Hv),
            "h0": (N, Hv, Dk, Dv), "ht": (N, Hv, Dk, Dv), "dht": (N, Hv, Dk, Dv)}
    dev = tensors["q"].device
    for name, t in tensors.items():
        if t is None:
            continue
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want[name]}")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")


def gdr_forward(q, k, v, g, beta, h0=None, *, use_qk_l2norm=True, channelwise=False,
                algo="auto", chunk_size=0, out_dtype=torch.float32, ht=True,
                stream=None, fused_gates=False, save_for_backward=False,
                cu_seqlens=None, max_seqlen=None):
    """Returns (o, ht), or (o, ht, saved) with ``save_for_backward`` (pass
    ``saved`` to ``gdr_backward``).  ``ht`` may be True (allocate), None (not
    wanted) or a tensor to write the final state into (it may be ``h0``
    itself).  With ``fused_gates`` g and beta are pre-activations
    (GDR_FUSED_GATES).  ``cu_seqlens`` (int64 device tensor [N + 1]) makes
    the batch ragged (gdr_forward_varlen): q, k, v, g, beta hold the N
    sequences end to end in their token axis with a leading 1, h0 / ht are
    [N, Hv, Dk, Dv]; ``max_seqlen`` bounds the lengths (read from the
    offsets when not given)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype)
    for t, n in ((g, "g"), (beta, "beta"), (h0, "h0")):
        _check(t, n, torch.float32)
    o = torch.empty((B, T, Hv, Dv), dtype=out_dtype, device=q.device)
    B0, T0 = B, T
    if cu_seqlens is not None:  # ragged batch: q [1, rows, Hk, Dk], one state per sequence
        B, T = _ragged_dims(q, cu_seqlens, max_seqlen)
    _check_shapes(B0, T0, Hk, Hv, Dk, Dv, B, channelwise,
                  dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, ht=ht if ht is not True and ht is not None else None))
    prob = make_problem(B, T, Hk, Hv, Dk, Dv, q.dtype, out_dtype, use_qk_l2norm,
                        channelwise, algo, chunk_size, fused_gates, save_for_backward)
    keep = save_for_backward and gdr_keeps_chunks(prob)
    if save_for_backward and not keep:  # the library ignores the flag here: call without it
        prob.flags &= ~GDR_SAVE_CHUNKS
    if ht is True:
        ht = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
    _check(ht, "ht", torch.float32)
    ws = _workspace(gdr_forward_workspace(prob), q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
            _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if cu_seqlens is not None:
        st = lib().gdr_forward_varlen(ctypes.byref(prob), _ptr(cu_seqlens), *args)
    else:
        st = lib().gdr_forward(ctypes.byref(prob), *args)
    if st != GDR_OK:
        raise GdrError(st, "gdr_forward")
    if save_for_backward:
        return o, ht, SavedChunks(ws if keep else None, _save_key(prob), keep)
    return o, ht


def gdr_forward_noalloc(q, k, v, g, beta, h0=None, *, o=None, ht=None, use_qk_l2norm=True, channelwise=False,
                        algo="auto", chunk_size=0, out_dtype=torch.float32, stream=None, fused_gates=False):
    """gdr_forward with the library's fixed device scratch as workspace (the
    C call allocates nothing).  ``o`` and ``ht`` may be given (then nothing is
    allocated here either: ``ht`` may be ``h0``); otherwise they are created.
    Returns (o, ht)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype)
    for t, n in ((g, "g"), (beta, "beta"), (h0, "h0")):
        _check(t, n, torch.float32)
    if o is None:
        o = torch.empty((B, T, Hv, Dv), dtype=out_dtype, device=q.device)
    if ht is None:
        ht = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
    _check(o, "o", out_dtype)
    _check(ht, "ht", torch.float32)
    _check_shapes(B, T, Hk, Hv, Dk, Dv, B, channelwise, dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, ht=ht))
    if tuple(o.shape) != (B, T, Hv, Dv):
        raise ValueError(f"o has shape {tuple(o.shape)}, expected {(B, T, Hv, Dv)}")
    prob = make_problem(B, T, Hk, Hv, Dk, Dv, q.dtype, out_dtype, use_qk_l2norm, channelwise, algo, chunk_size,
                        fused_gates, False)
    st = lib().gdr_forward_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                   _ptr(o), _ptr(ht), _stream(stream))
    if st != GDR_OK:
        raise GdrError(st, "gdr_forward_noalloc")
    return o, ht


def gdr_backward(q, k, v, g, beta, h0, dout, dht=None, *, use_qk_l2norm=True,
                 channelwise=False, algo="auto", chunk_size=0,
                 out_dtype=torch.float32, want_dh0=True, stream=None, fused_gates=False,
                 saved=None, cu_seqlens=None, max_seqlen=None):
    """Returns (dq, dk, dv, dg, dbeta, dh0); dh0 is None if not wanted.  With
    ``fused_gates`` g and beta are pre-activations and dg, dbeta are the
    gradients with respect to them.  ``saved`` is what the forward of the
    same problem and inputs returned with ``save_for_backward``.
    ``cu_seqlens`` / ``max_seqlen`` as for ``gdr_forward``
    (gdr_backward_varlen)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(t, n, q.dtype)
    for t, n in ((g, "g"), (beta, "beta"), (h0, "h0"), (dht, "dht")):
        _check(t, n, torch.float32)
    dev = q.device
    dq = torch.empty((B, T, Hk, Dk), dtype=out_dtype, device=dev)
    dk = torch.empty((B, T, Hk, Dk), dtype=out_dtype, device=dev)
    dv = torch.empty((B, T, Hv, Dv), dtype=out_dtype, device=dev)
    dg = torch.empty(g.shape, dtype=torch.float32, device=dev)
    dbeta = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    B0, T0 = B, T
    if cu_seqlens is not None:
        B, T = _ragged_dims(q, cu_seqlens, max_seqlen)
    _check_shapes(B0, T0, Hk, Hv, Dk, Dv, B, channelwise,
                  dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, dout=dout, dht=dht))
    prob = make_problem(B, T, Hk, Hv, Dk, Dv, q.dtype, out_dtype, use_qk_l2norm,
                        channelwise, algo, chunk_size, fused_gates, saved is not None)
    if saved is not None and saved.key != _save_key(prob):
        raise ValueError("saved chunks belong to a different problem")
    if saved is not None and not saved.kept:  # nothing was kept: the stateless VJP
        prob.flags &= ~GDR_SAVE_CHUNKS
        saved = None
    dh0 = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=dev) if want_dh0 else None
    nws = gdr_backward_workspace(prob)
    if saved is not None:  # the forward's images and chunk states
        if nws > 0 and (saved.ws is None or saved.ws.numel() < nws):
            raise ValueError("saved chunks hold a workspace smaller than the backward needs")
        ws = saved.ws
    else:
        ws = _workspace(nws, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(dout), _ptr(dht),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
            _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if cu_seqlens is not None:
        st = lib().gdr_backward_varlen(ctypes.byref(prob), _ptr(cu_seqlens), *args)
    else:
        st = lib().gdr_backward(ctypes.byref(prob), *args)
    if st != GDR_OK:
        raise GdrError(st, "gdr_backward")
    return dq, dk, dv, dg, dbeta, dh0
