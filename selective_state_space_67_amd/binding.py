"""ctypes binding of libssmscan.so (declared in include/ssm_scan.h).

Argument marshalling only: the functions below read shapes, dtypes, device
pointers and the current HIP stream from torch tensors, fill the C parameter
structs and call the library. Every step of the computation runs in the
library's HIP kernels; there is no fallback of any kind. If the library is
missing (not built) the first call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libssmscan.so"

SSM_F32 = 0
SSM_BF16 = 1
SSM_DISC_DELTA_B = 0
SSM_DISC_ZOH = 1
SSM_STATE_REAL = 0
SSM_STATE_COMPLEX = 1

STATUS_NAMES = {
    0: "SSM_OK", 1: "SSM_ERR_NULL_POINTER", 2: "SSM_ERR_BAD_SHAPE", 3: "SSM_ERR_BAD_DTYPE",
    4: "SSM_ERR_MISALIGNED", 5: "SSM_ERR_UNSUPPORTED", 6: "SSM_ERR_WORKSPACE", 7: "SSM_ERR_ALIAS",
    8: "SSM_ERR_HIP",
}


class SsmError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), detail))


class ScanParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("u", ctypes.c_void_p), ("dt_raw", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p),
        ("Dskip", ctypes.c_void_p), ("z", ctypes.c_void_p), ("reset", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("out", ctypes.c_void_p), ("h_last", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_segments", ctypes.c_int32), ("discretization", ctypes.c_int32),
        ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p), ("conv_state_in", ctypes.c_void_p),
        ("conv_state_out", ctypes.c_void_p), ("conv_width", ctypes.c_int32), ("state_kind", ctypes.c_int32),
    ]


class UpdateParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("h", ctypes.c_void_p), ("u", ctypes.c_void_p), ("dt_raw", ctypes.c_void_p),
        ("z", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("Dskip", ctypes.c_void_p), ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("conv_state", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
        ("conv_b", ctypes.c_void_p), ("conv_width", ctypes.c_int32), ("discretization", ctypes.c_int32),
        ("state_kind", ctypes.c_int32), ("reserved1", ctypes.c_int32),
    ]


class BwdParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
        ("u", ctypes.c_void_p), ("dt_raw", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p),
        ("Dskip", ctypes.c_void_p), ("z", ctypes.c_void_p), ("reset", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("dh_last", ctypes.c_void_p),
        ("du", ctypes.c_void_p), ("d_dt_raw", ctypes.c_void_p), ("dz", ctypes.c_void_p),
        ("dA", ctypes.c_void_p), ("dBm", ctypes.c_void_p), ("dCm", ctypes.c_void_p),
        ("dDskip", ctypes.c_void_p), ("d_dt_bias", ctypes.c_void_p), ("dh0", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p), ("conv_state_in", ctypes.c_void_p),
        ("dconv_w", ctypes.c_void_p), ("dconv_b", ctypes.c_void_p), ("dconv_state_in", ctypes.c_void_p),
        ("conv_width", ctypes.c_int32), ("discretization", ctypes.c_int32),
        ("state_kind", ctypes.c_int32), ("reserved1", ctypes.c_int32),
    ]


EXPORTS = ("ssm_scan_workspace_size", "ssm_scan_fwd", "ssm_scan_fwd_noalloc", "ssm_scan_fwd_wavefront",
           "ssm_scan_aggregate_workspace_size",
           "ssm_scan_aggregate",
           "ssm_state_update", "ssm_scan_bwd_workspace_size", "ssm_scan_bwd", "ssm_status_string", "ssm_last_error",
           "ssm_version", "ssm_abi_struct_size")

_lib = None


def library_path() -> str:
    return os.environ.get("SSM_SCAN_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libssmscan.so (once) and check the struct layouts against it."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError("libssmscan.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(ScanParams), ctypes.POINTER(ctypes.c_size_t)]
    lib.ssm_scan_workspace_size.restype = ctypes.c_int
    lib.ssm_scan_fwd.argtypes = [ctypes.POINTER(ScanParams), vp]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanParams), vp]
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_scan_fwd_wavefront.argtypes = [ctypes.POINTER(ScanParams), vp]
    lib.ssm_scan_fwd_wavefront.restype = ctypes.c_int
    lib.ssm_scan_aggregate_workspace_size.argtypes = [ctypes.POINTER(ScanParams), ctypes.POINTER(ctypes.c_size_t)]
    lib.ssm_scan_aggregate_workspace_size.restype = ctypes.c_int
    lib.ssm_scan_aggregate.argtypes = [ctypes.POINTER(ScanParams), vp, vp, vp]
    lib.ssm_scan_aggregate.restype = ctypes.c_int
    lib.ssm_state_update.argtypes = [ctypes.POINTER(UpdateParams), vp]
    lib.ssm_state_update.restype = ctypes.c_int
    lib.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdParams), ctypes.POINTER(ctypes.c_size_t)]
    lib.ssm_scan_bwd_workspace_size.restype = ctypes.c_int
    lib.ssm_scan_bwd.argtypes = [ctypes.POINTER(BwdParams), vp]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_status_string.argtypes = [ctypes.c_int32]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_last_error.argtypes = []
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_version.argtypes = []
    lib.ssm_version.restype = ctypes.c_int32
    lib.ssm_abi_struct_size.argtypes = [ctypes.c_int32]
    lib.ssm_abi_struct_size.restype = ctypes.c_size_t
    if lib.ssm_abi_struct_size(0) != ctypes.sizeof(ScanParams) or \
            lib.ssm_abi_struct_size(1) != ctypes.sizeof(UpdateParams) or \
            lib.ssm_abi_struct_size(2) != ctypes.sizeof(BwdParams):
        raise ImportError("libssmscan.so struct layout does not match this binding")
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise SsmError(status, _lib.ssm_last_error().decode(errors="replace"))


def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, shape, name, dtype=None):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))


def _stream(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _scan_params(u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, out, h_last, out_dtype,
                 num_segments, conv_w=None, conv_b=None, conv_state_in=None, conv_state_out=None, zoh=False,
                 cplx=False):
    import torch

    Bt, D, L = u.shape
    N = A.shape[1]
    c2 = (2,) if cplx else ()  # complex tensors carry a trailing (re, im) axis
    _need(u, (Bt, D, L), "u")
    _need(dt_raw, (Bt, D, L), "dt_raw", u.dtype)
    _need(A, (D, N) + c2, "A", torch.float32)
    _need(Bm, (Bt, L, N) + c2, "Bm", u.dtype)
    if Cm is not None:
        _need(Cm, (Bt, L, N) + c2, "Cm", u.dtype)
    if dt_bias is not None:
        _need(dt_bias, (D,), "dt_bias", torch.float32)
    if Dskip is not None:
        _need(Dskip, (D,), "Dskip", torch.float32)
    if z is not None:
        _need(z, (Bt, D, L), "z", u.dtype)
    if reset is not None:
        _need(reset, (Bt, L), "reset", torch.uint8)
    if h0 is not None:
        _need(h0, (Bt, D, N) + c2, "h0", torch.float32)
    if out is not None:
        _need(out, (Bt, D, L), "out")
    if h_last is not None:
        _need(h_last, (Bt, D, N) + c2, "h_last", torch.float32)
    p = ScanParams()
    p.batch, p.dim, p.seqlen, p.dstate = Bt, D, L, N
    p.in_dtype = _dtype_code(u)
    p.out_dtype = _dtype_code(out) if out is not None else (SSM_F32 if out_dtype is None
                                                            else _dtype_code(torch.empty(0, dtype=out_dtype)))
    p.u, p.dt_raw, p.dt_bias, p.A = _ptr(u), _ptr(dt_raw), _ptr(dt_bias), _ptr(A)
    p.Bm, p.Cm, p.Dskip, p.z = _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z)
    p.reset, p.h0, p.out, p.h_last = _ptr(reset), _ptr(h0), _ptr(out), _ptr(h_last)
    p.num_segments = int(num_segments)
    p.discretization = SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B
    p.state_kind = SSM_STATE_COMPLEX if cplx else SSM_STATE_REAL
    if conv_w is not None:
        K = conv_w.shape[1]
        _need(conv_w, (D, K), "conv_w", torch.float32)
        if conv_b is not None:
            _need(conv_b, (D,), "conv_b", torch.float32)
        for t, name in ((conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
            if t is not None:
                _need(t, (Bt, D, K - 1), name, torch.float32)
        p.conv_w, p.conv_b = _ptr(conv_w), _ptr(conv_b)
        p.conv_state_in, p.conv_state_out = _ptr(conv_state_in), _ptr(conv_state_out)
        p.conv_width = K
    return p


def ssm_scan_aggregate(u, dt_raw, A, Bm, *, dt_bias=None, reset=None, conv_w=None, conv_b=None, conv_state_in=None,
                       zoh=False, complex_state=False, num_segments=0, P=None, H=None, workspace=None, stream=None):
    """Affine aggregate of the sequence: returns (P, H), (B, D, N) float32
    ((B, D, N, 2) with complex_state), such that the scan maps an entering
    state h to P h + H. Shards of one long sequence are scanned by folding the
    preceding shards' aggregates into h0 (see include/ssm_scan.h)."""
    import torch

    lib = load_library()
    Bt, D, _ = u.shape
    N = A.shape[1]
    shape = (Bt, D, N, 2) if complex_state else (Bt, D, N)
    P = torch.empty(shape, dtype=torch.float32, device=u.device) if P is None else P
    H = torch.empty(shape, dtype=torch.float32, device=u.device) if H is None else H
    _need(P, shape, "P", torch.float32)
    _need(H, shape, "H", torch.float32)
    p = _scan_params(u, dt_raw, A, Bm, None, dt_bias, None, None, reset, None, None, None, None, num_segments,
                     conv_w, conv_b, conv_state_in, None, zoh, complex_state)
    n = ctypes.c_size_t(0)
    _check(lib.ssm_scan_aggregate_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    if n.value and (workspace is None or workspace.numel() * workspace.element_size() < n.value):
        workspace = torch.empty(int(n.value), dtype=torch.uint8, device=u.device)
    if n.value:
        p.workspace = _ptr(workspace)
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.ssm_scan_aggregate(ctypes.byref(p), _ptr(P), _ptr(H), _stream(stream, u.device)))
    return P, H


def prepare_aggregate(u, dt_raw, A, Bm, *, dt_bias=None, reset=None, conv_w=None, conv_b=None, conv_state_in=None,
                      zoh=False, complex_state=False, num_segments=0, P=None, H=None, stream=None):
    """Marshal the arguments of ssm_scan_aggregate once; returns a no-argument
    callable that enqueues the same call again and returns (P, H)."""
    import torch

    lib = load_library()
    Bt, D, _ = u.shape
    N = A.shape[1]
    shape = (Bt, D, N, 2) if complex_state else (Bt, D, N)
    P = torch.empty(shape, dtype=torch.float32, device=u.device) if P is None else P
    H = torch.empty(shape, dtype=torch.float32, device=u.device) if H is None else H
    _need(P, shape, "P", torch.float32)
    _need(H, shape, "H", torch.float32)
    p = _scan_params(u, dt_raw, A, Bm, None, dt_bias, None, None, reset, None, None, None, None, num_segments,
                     conv_w, conv_b, conv_state_in, None, zoh, complex_state)
    n = ctypes.c_size_t(0)
    _check(lib.ssm_scan_aggregate_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=u.device)
    if n.value:
        p.workspace = _ptr(ws)
        p.workspace_bytes = int(n.value)
    st = _stream(stream, u.device)
    fn = lib.ssm_scan_aggregate
    pref, pp, hp = ctypes.byref(p), _ptr(P), _ptr(H)

    def call():
        _check(fn(pref, pp, hp, st))
        return P, H

    call.keep = ((u, dt_raw, A, Bm, dt_bias, reset, conv_w, conv_b, conv_state_in, ws), p)
    return call


def ssm_scan_workspace_size(u, A, *, num_segments=0, out_dtype=None):
    """Workspace bytes ssm_scan_fwd needs for inputs shaped like u (B,D,L) and A (D,N)."""
    import torch

    lib = load_library()
    p = ScanParams()
    p.batch, p.dim, p.seqlen = u.shape
    p.dstate = A.shape[1]
    p.in_dtype = _dtype_code(u)
    p.out_dtype = SSM_F32 if out_dtype in (None, torch.float32) else SSM_BF16
    p.num_segments = int(num_segments)
    n = ctypes.c_size_t(0)
    _check(lib.ssm_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def ssm_scan_fwd(u, dt_raw, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, reset=None, h0=None,
                 out=None, h_last=None, out_dtype=None, workspace=None, num_segments=0, conv_w=None, conv_b=None,
                 conv_state_in=None, conv_state_out=None, zoh=False, complex_state=False, stream=None):
    """Selective scan over the whole sequence; returns ``out`` (B, D, L).

    With conv_w (D, K <= 4) float32, u is the input of a causal depthwise
    conv1d + SiLU stage whose output feeds the scan (conv_b (D,),
    conv_state_in / conv_state_out (B, D, K-1) float32 optional). zoh=True
    selects the exact zero-order-hold input coefficient (e^{delta A} - 1) / A.
    complex_state=True selects the complex diagonal state: A (D, N, 2),
    Bm, Cm (B, L, N, 2) and h0, h_last (B, D, N, 2) then hold (re, im) pairs.

    u, dt_raw, z: (B, D, L) float32 or bfloat16; A: (D, N) float32;
    Bm, Cm: (B, L, N) same dtype as u; dt_bias, Dskip: (D,) float32;
    reset: (B, L) uint8; h0, h_last: (B, D, N) float32. ``out`` is allocated
    (float32 unless ``out_dtype`` says bfloat16) when not given, and so is the
    workspace the library asks for. Runs on ``stream`` (default: the current
    torch stream of u's device).
    """
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(u.shape, dtype=out_dtype or torch.float32, device=u.device)
    p = _scan_params(u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, out, h_last, out_dtype,
                     num_segments, conv_w, conv_b, conv_state_in, conv_state_out, zoh, complex_state)
    n = ctypes.c_size_t(0)
    _check(lib.ssm_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    if n.value:
        if workspace is None or workspace.numel() * workspace.element_size() < n.value:
            workspace = torch.empty(int(n.value), dtype=torch.uint8, device=u.device)
        p.workspace = _ptr(workspace)
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.ssm_scan_fwd(ctypes.byref(p), _stream(stream, u.device)))
    return out


def ssm_scan_fwd_noalloc(u, dt_raw, A, Bm, Cm, *, out, dt_bias=None, Dskip=None, z=None, reset=None, h0=None,
                         h_last=None, num_segments=0, conv_w=None, conv_b=None, conv_state_in=None,
                         conv_state_out=None, zoh=False, complex_state=False, stream=None):
    """ssm_scan_fwd through the allocation-free entry point: the caller passes
    every output (``out`` is required), nothing is allocated here, and a scan
    that splits the sequence uses the library's own per-device scratch
    (include/ssm_scan.h, ssm_scan_fwd_noalloc). Returns ``out``."""
    lib = load_library()
    p = _scan_params(u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, out, h_last, None,
                     num_segments, conv_w, conv_b, conv_state_in, conv_state_out, zoh, complex_state)
    _check(lib.ssm_scan_fwd_noalloc(ctypes.byref(p), _stream(stream, u.device)))
    return out


def ssm_scan_fwd_wavefront(u, dt_raw, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, reset=None, h0=None,
                           out=None, h_last=None, out_dtype=None, stream=None):
    """The same forward as a chunked associative scan with a DPP wavefront scan
    inside each 64-step chunk (include/ssm_scan.h, ssm_scan_fwd_wavefront): N = 16,
    real state, delta B coefficient, no conv stage. Returns ``out``."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(u.shape, dtype=out_dtype or torch.float32, device=u.device)
    p = _scan_params(u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, out, h_last, out_dtype,
                     0, None, None, None, None, False, False)
    _check(lib.ssm_scan_fwd_wavefront(ctypes.byref(p), _stream(stream, u.device)))
    return out


def prepare_scan(u, dt_raw, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, reset=None, h0=None, out=None,
                 h_last=None, out_dtype=None, num_segments=0, conv_w=None, conv_b=None, conv_state_in=None,
                 conv_state_out=None, zoh=False, complex_state=False, wavefront=False, stream=None):
    """Marshal the arguments of ssm_scan_fwd once; returns a no-argument callable
    that enqueues the same scan again (same tensors, same stream) each time it is
    called. The tensors must stay alive and unchanged in shape while it is used.
    wavefront=True calls ssm_scan_fwd_wavefront instead (no workspace)."""
    import torch

    lib = load_library()
    if out is None:
        out = torch.empty(u.shape, dtype=out_dtype or torch.float32, device=u.device)
    p = _scan_params(u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, out, h_last, out_dtype,
                     num_segments, conv_w, conv_b, conv_state_in, conv_state_out, zoh, complex_state)
    n = ctypes.c_size_t(0)
    if not wavefront:
        _check(lib.ssm_scan_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    keep = [u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, out, h_last, conv_w, conv_b, conv_state_in,
            conv_state_out]
    if n.value:
        ws = torch.empty(int(n.value), dtype=torch.uint8, device=u.device)
        keep.append(ws)
        p.workspace = _ptr(ws)
        p.workspace_bytes = int(n.value)
    st = _stream(stream, u.device)
    fn = lib.ssm_scan_fwd_wavefront if wavefront else lib.ssm_scan_fwd
    pref = ctypes.byref(p)

    def call():
        _check(fn(pref, st))
        return out

    call.keep = (keep, p)
    return call


def prepare_state_update(h, u, dt_raw, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, out=None,
                         out_dtype=None, zoh=False, complex_state=False, stream=None):
    """Marshal the arguments of ssm_state_update once; returns a no-argument
    callable that enqueues the same decode step again each time it is called
    (updating h in place every time)."""
    import torch

    lib = load_library()
    Bt, D, N = h.shape[:3]
    if out is None:
        out = torch.empty((Bt, D), dtype=out_dtype or torch.float32, device=u.device)
    p = _update_params(h, u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, out, zoh=zoh, cplx=complex_state)
    st = _stream(stream, u.device)
    fn = lib.ssm_state_update
    pref = ctypes.byref(p)

    def call():
        _check(fn(pref, st))
        return out

    call.keep = ((h, u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, out), p)
    return call


def _update_params(h, u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, out, conv_w=None, conv_b=None, conv_state=None,
                   zoh=False, cplx=False):
    import torch

    Bt, D, N = h.shape[:3]
    c2 = (2,) if cplx else ()  # complex tensors carry a trailing (re, im) axis
    _need(h, (Bt, D, N) + c2, "h", torch.float32)
    _need(u, (Bt, D), "u")
    _need(dt_raw, (Bt, D), "dt_raw", u.dtype)
    _need(A, (D, N) + c2, "A", torch.float32)
    _need(Bm, (Bt, N) + c2, "Bm", u.dtype)
    _need(Cm, (Bt, N) + c2, "Cm", u.dtype)
    if z is not None:
        _need(z, (Bt, D), "z", u.dtype)
    if dt_bias is not None:
        _need(dt_bias, (D,), "dt_bias", torch.float32)
    if Dskip is not None:
        _need(Dskip, (D,), "Dskip", torch.float32)
    _need(out, (Bt, D), "out")
    p = UpdateParams()
    p.batch, p.dim, p.dstate = Bt, D, N
    p.in_dtype, p.out_dtype = _dtype_code(u), _dtype_code(out)
    p.h, p.u, p.dt_raw, p.z = _ptr(h), _ptr(u), _ptr(dt_raw), _ptr(z)
    p.dt_bias, p.A, p.Dskip = _ptr(dt_bias), _ptr(A), _ptr(Dskip)
    p.Bm, p.Cm, p.out = _ptr(Bm), _ptr(Cm), _ptr(out)
    p.discretization = SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B
    p.state_kind = SSM_STATE_COMPLEX if cplx else SSM_STATE_REAL
    if conv_w is not None:
        K = conv_w.shape[1]
        _need(conv_w, (D, K), "conv_w", torch.float32)
        if conv_b is not None:
            _need(conv_b, (D,), "conv_b", torch.float32)
        if K > 1:
            _need(conv_state, (Bt, D, K - 1), "conv_state", torch.float32)
        p.conv_w, p.conv_b, p.conv_state, p.conv_width = _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), K
    return p


def ssm_state_update(h, u, dt_raw, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, out=None,
                     out_dtype=None, conv_w=None, conv_b=None, conv_state=None, zoh=False, complex_state=False,
                     stream=None):
    """Decode step: updates h (B, D, N) float32 in place and returns out (B, D).

    With conv_w (D, K), u is this step's conv input and conv_state
    (B, D, K-1) float32 is shifted in place. complex_state=True: h (B, D, N, 2),
    A (D, N, 2) and Bm, Cm (B, N, 2) hold (re, im) pairs."""
    import torch

    lib = load_library()
    Bt, D, N = h.shape[:3]
    if out is None:
        out = torch.empty((Bt, D), dtype=out_dtype or torch.float32, device=u.device)
    p = _update_params(h, u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, out, conv_w, conv_b, conv_state, zoh,
                       complex_state)
    _check(lib.ssm_state_update(ctypes.byref(p), _stream(stream, u.device)))
    return out


def _bwd_params(u, dt_raw, A, Bm, Cm, dout, dt_bias, Dskip, z, reset, h0, dh_last, grads, conv=None, zoh=False,
                cplx=False):
    import torch

    Bt, D, L = u.shape
    N = A.shape[1]
    _scan_params(u, dt_raw, A, Bm, Cm, dt_bias, Dskip, z, reset, h0, None, None, None, 0,
                 cplx=cplx)  # input checks
    _need(dout, (Bt, D, L), "dout", u.dtype)
    c2 = (2,) if cplx else ()  # complex tensors carry a trailing (re, im) axis
    if dh_last is not None:
        _need(dh_last, (Bt, D, N) + c2, "dh_last", torch.float32)
    shapes = dict(du=(Bt, D, L), d_dt_raw=(Bt, D, L), dz=(Bt, D, L), dA=(D, N) + c2, dBm=(Bt, L, N) + c2,
                  dCm=(Bt, L, N) + c2, dDskip=(D,), d_dt_bias=(D,), dh0=(Bt, D, N) + c2)
    for k, t in grads.items():
        if t is not None and k in shapes:
            _need(t, shapes[k], k)
    p = BwdParams()
    p.batch, p.dim, p.seqlen, p.dstate = Bt, D, L, N
    p.in_dtype = _dtype_code(u)
    p.grad_dtype = _dtype_code(grads["du"])
    p.u, p.dt_raw, p.dt_bias, p.A = _ptr(u), _ptr(dt_raw), _ptr(dt_bias), _ptr(A)
    p.Bm, p.Cm, p.Dskip, p.z = _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z)
    p.reset, p.h0, p.dout, p.dh_last = _ptr(reset), _ptr(h0), _ptr(dout), _ptr(dh_last)
    p.discretization = SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B
    p.state_kind = SSM_STATE_COMPLEX if cplx else SSM_STATE_REAL
    for k, t in grads.items():
        if k in ("dconv_w", "dconv_b", "dconv_state_in"):
            continue
        setattr(p, k, _ptr(t))
    if conv is not None and conv[0] is not None:
        conv_w, conv_b, conv_state_in = conv
        K = conv_w.shape[1]
        _need(conv_w, (D, K), "conv_w", torch.float32)
        if conv_b is not None:
            _need(conv_b, (D,), "conv_b", torch.float32)
        if conv_state_in is not None:
            _need(conv_state_in, (Bt, D, K - 1), "conv_state_in", torch.float32)
        p.conv_w, p.conv_b, p.conv_state_in, p.conv_width = _ptr(conv_w), _ptr(conv_b), _ptr(conv_state_in), K
        p.dconv_w, p.dconv_b = _ptr(grads.get("dconv_w")), _ptr(grads.get("dconv_b"))
        p.dconv_state_in = _ptr(grads.get("dconv_state_in"))
    return p


def _bwd_grads(u, A, Bm, z, grad_dtype, want_dD, want_dbias, want_dh0, cplx=False):
    import torch

    Bt, D, L = u.shape
    N = A.shape[1]
    dev = u.device
    gd = grad_dtype or torch.float32
    f32 = torch.float32
    c2 = (2,) if cplx else ()
    return dict(du=torch.empty((Bt, D, L), dtype=gd, device=dev),
                d_dt_raw=torch.empty((Bt, D, L), dtype=gd, device=dev),
                dz=torch.empty((Bt, D, L), dtype=gd, device=dev) if z is not None else None,
                dA=torch.empty((D, N) + c2, dtype=f32, device=dev),
                dBm=torch.empty((Bt, L, N) + c2, dtype=f32, device=dev),
                dCm=torch.empty((Bt, L, N) + c2, dtype=f32, device=dev),
                dDskip=torch.empty((D,), dtype=f32, device=dev) if want_dD else None,
                d_dt_bias=torch.empty((D,), dtype=f32, device=dev) if want_dbias else None,
                dh0=torch.empty((Bt, D, N) + c2, dtype=f32, device=dev) if want_dh0 else None)


def ssm_scan_bwd(u, dt_raw, A, Bm, Cm, dout, *, dt_bias=None, Dskip=None, z=None, reset=None, h0=None,
                 dh_last=None, grad_dtype=None, want_dDskip=True, want_d_dt_bias=True, want_dh0=True,
                 conv_w=None, conv_b=None, conv_state_in=None, zoh=False, complex_state=False, workspace=None,
                 stream=None):
    """Backward pass of ssm_scan_fwd for the same inputs and the output gradient dout.

    Returns a dict with du, d_dt_raw, dz (None without z) in ``grad_dtype``
    (float32 by default), and float32 dA, dBm, dCm, dDskip, d_dt_bias, dh0
    (the last three None when not asked for). dh_last (B, D, N) float32 is the
    gradient reaching h_last (None = 0). The workspace is allocated when not
    given or too small. With conv_w (D, K), u is the conv input and the dict
    also holds dconv_w (D, K), dconv_b (D,) and dconv_state_in (B, D, K-1).
    complex_state=True: the complex-state scan; A, Bm, Cm, h0, dh_last and
    the gradients dA, dBm, dCm, dh0 carry a trailing (re, im) axis, each
    gradient holding dL/dRe and dL/dIm.
    """
    import torch

    lib = load_library()
    grads = _bwd_grads(u, A, Bm, z, grad_dtype, want_dDskip, want_d_dt_bias, want_dh0, complex_state)
    if conv_w is not None:
        Bt, D, _ = u.shape
        K = conv_w.shape[1]
        grads["dconv_w"] = torch.empty((D, K), dtype=torch.float32, device=u.device)
        grads["dconv_b"] = torch.empty((D,), dtype=torch.float32, device=u.device)
        grads["dconv_state_in"] = (torch.empty((Bt, D, K - 1), dtype=torch.float32, device=u.device)
                                   if K > 1 else None)
    p = _bwd_params(u, dt_raw, A, Bm, Cm, dout, dt_bias, Dskip, z, reset, h0, dh_last, grads,
                    (conv_w, conv_b, conv_state_in), zoh, complex_state)
    n = ctypes.c_size_t(0)
    _check(lib.ssm_scan_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    if workspace is None or workspace.numel() * workspace.element_size() < n.value:
        workspace = torch.empty(int(n.value), dtype=torch.uint8, device=u.device)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.ssm_scan_bwd(ctypes.byref(p), _stream(stream, u.device)))
    return grads


def prepare_scan_bwd(u, dt_raw, A, Bm, Cm, dout, *, dt_bias=None, Dskip=None, z=None, reset=None, h0=None,
                     dh_last=None, grad_dtype=None, conv_w=None, conv_b=None, conv_state_in=None, zoh=False,
                     complex_state=False, stream=None):
    """Marshal the arguments of ssm_scan_bwd once; returns a no-argument callable
    that enqueues the same backward pass again each time it is called and
    returns the gradient dict (the same tensors every time)."""
    import torch

    lib = load_library()
    grads = _bwd_grads(u, A, Bm, z, grad_dtype, True, True, True, complex_state)
    if conv_w is not None:
        Bt, D, _ = u.shape
        K = conv_w.shape[1]
        grads["dconv_w"] = torch.empty((D, K), dtype=torch.float32, device=u.device)
        grads["dconv_b"] = torch.empty((D,), dtype=torch.float32, device=u.device)
        grads["dconv_state_in"] = (torch.empty((Bt, D, K - 1), dtype=torch.float32, device=u.device)
                                   if K > 1 else None)
    p = _bwd_params(u, dt_raw, A, Bm, Cm, dout, dt_bias, Dskip, z, reset, h0, dh_last, grads,
                    (conv_w, conv_b, conv_state_in), zoh, complex_state)
    n = ctypes.c_size_t(0)
    _check(lib.ssm_scan_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    ws = torch.empty(int(n.value), dtype=torch.uint8, device=u.device)
    p.workspace = _ptr(ws)
    p.workspace_bytes = int(n.value)
    st = _stream(stream, u.device)
    fn = lib.ssm_scan_bwd
    pref = ctypes.byref(p)

    def call():
        _check(fn(pref, st))
        return grads

    call.keep = ((u, dt_raw, A, Bm, Cm, dout, dt_bias, Dskip, z, reset, h0, dh_last, conv_w, conv_b, conv_state_in,
                  ws), p)
    return call
