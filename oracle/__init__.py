"""Selective-scan oracle: plain sequential float64 evaluation on the CPU.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package. The product path (the
HIP library and its Python binding) never imports it, and the two share no
code: the only module both sides use is the seeded input generator, which holds
none of the method's arithmetic.

The arithmetic lives in ``ssm_oracle.c`` (C, libm, OpenMP over independent
rows); this module compiles it with gcc, widens inputs to float64 and calls it.
Every input is widened exactly (bf16 bit patterns and float32 both convert to
float64 without rounding), so the oracle sees the same values the GPU sees.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

MAX_N = 1024


def build(force: bool = False) -> str:
    """Compile ssm_oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall", "-Wextra",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def library_path() -> str:
    """liboracle.so, or the build named by SSM_ORACLE_LIBRARY (the sanitizer tier's instrumented copy)."""
    return os.environ.get("SSM_ORACLE_LIBRARY", _LIB)


def _load():
    global _lib
    if _lib is None:
        path = library_path()
        if path == _LIB:
            build()
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_scan_rows.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p, p, p, p, p, p, p,
                                         ctypes.c_int, ctypes.c_int]
        lib.oracle_scan_rows.restype = None
        lib.oracle_state_update.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p, p, p,
                                            ctypes.c_int, ctypes.c_int]
        lib.oracle_state_update.restype = None
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_scan_bwd_rows.argtypes = [i64, i64, i64, i64, i64] + [p] * 23 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_scan_bwd_rows.restype = ctypes.c_int
        lib.oracle_scan_cplx_rows.argtypes = [i64, i64, i64] + [p] * 14 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_scan_cplx_rows.restype = None
        lib.oracle_scan_cplx_bwd_rows.argtypes = [i64, i64, i64, i64, i64] + [p] * 23 + [ctypes.c_int] * 2
        lib.oracle_scan_cplx_bwd_rows.restype = ctypes.c_int
        lib.oracle_conv_silu_rows.argtypes = [i64, i64, i64] + [p] * 10 + [ctypes.c_int]
        lib.oracle_conv_silu_rows.restype = None
        lib.oracle_conv_silu_bwd_rows.argtypes = [i64, i64, i64, i64] + [p] * 12 + [ctypes.c_int]
        lib.oracle_conv_silu_bwd_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def scan_rows(rows_b, rows_d, u_rows, dt_rows, A, Bm, Cm, *, z_rows=None, dt_bias=None,
              Dskip=None, reset=None, h0_rows=None, want_h_last=False, zoh=False, nthreads=0):
    """Run the recurrence on selected (b, d) rows over the full sequence.

    rows_b, rows_d : (R,) int   batch and channel of each row
    u_rows, dt_rows, z_rows : (R, L) values of that row (any float dtype)
    A : (D, N); Bm, Cm : (B, L, N); dt_bias, Dskip : (D,) or None
    reset : (B, L) bool/uint8 or None; h0_rows : (R, N) or None
    Returns out (R, L) float64 and, if asked, h_last (R, N).
    """
    lib = _load()
    rows_b = np.ascontiguousarray(np.asarray(rows_b, dtype=np.int64))
    rows_d = np.ascontiguousarray(np.asarray(rows_d, dtype=np.int64))
    u_rows, dt_rows, z_rows = _f64(u_rows), _f64(dt_rows), _f64(z_rows)
    A, Bm, Cm = _f64(A), _f64(Bm), _f64(Cm)
    dt_bias, Dskip, h0_rows = _f64(dt_bias), _f64(Dskip), _f64(h0_rows)
    R, L = u_rows.shape
    N = A.shape[1]
    if N > MAX_N:
        raise ValueError("oracle supports N <= %d" % MAX_N)
    Bt = Bm.shape[0]
    assert dt_rows.shape == (R, L) and Bm.shape == (Bt, L, N) and Cm.shape == (Bt, L, N)
    assert rows_b.shape == (R,) and rows_d.shape == (R,)
    if z_rows is not None:
        assert z_rows.shape == (R, L)
    if h0_rows is not None:
        assert h0_rows.shape == (R, N)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
        assert reset.shape == (Bt, L)
    out = np.empty((R, L), dtype=np.float64)
    h_last = np.empty((R, N), dtype=np.float64) if want_h_last else None
    lib.oracle_scan_rows(R, L, N, _ptr(rows_b), _ptr(rows_d), _ptr(u_rows), _ptr(dt_rows),
                         _ptr(z_rows), _ptr(dt_bias), _ptr(A), _ptr(Dskip), _ptr(Bm), _ptr(Cm),
                         _ptr(reset), _ptr(h0_rows), _ptr(out), _ptr(h_last), int(bool(zoh)), int(nthreads))
    return (out, h_last) if want_h_last else out


def conv_silu(x, w, *, bias=None, reset=None, state_in=None, want_pre=False, want_state=False, nthreads=0):
    """Causal depthwise conv1d (width K = w.shape[1]) then SiLU over x (B, D, L).

    w: (D, K); bias: (D,); reset: (B, L); state_in: (B, D, K-1), the inputs
    before the sequence (oldest first). Returns u (B, D, L), plus the
    pre-activation and the final conv state (B, D, K-1) when asked for.
    """
    lib = _load()
    x, w, bias, state_in = _f64(x), _f64(w), _f64(bias), _f64(state_in)
    Bt, D, L = x.shape
    K = w.shape[1]
    assert w.shape == (D, K) and K >= 1
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
    rb, rd = np.divmod(np.arange(Bt * D, dtype=np.int64), D)
    u = np.empty((Bt, D, L))
    pre = np.empty((Bt, D, L)) if want_pre else None
    st = np.empty((Bt, D, max(K - 1, 0))) if want_state else None
    if state_in is not None:
        assert state_in.shape == (Bt, D, K - 1)
    lib.oracle_conv_silu_rows(Bt * D, L, K, _ptr(rb), _ptr(rd), _ptr(x), _ptr(w), _ptr(bias), _ptr(reset),
                              _ptr(state_in), _ptr(pre), _ptr(u), _ptr(st) if K > 1 else None, int(nthreads))
    res = [u]
    if want_pre:
        res.append(pre)
    if want_state:
        res.append(st)
    return res[0] if len(res) == 1 else tuple(res)


def conv_silu_bwd(x, w, du, pre, *, reset=None, state_in=None, nthreads=0):
    """Gradients of sum(du * conv_silu(x)) for x, w, bias and state_in.

    Returns dict dx (B, D, L), dw (D, K), dbias (D,), dstate_in (B, D, K-1).
    """
    lib = _load()
    x, w, du, pre, state_in = _f64(x), _f64(w), _f64(du), _f64(pre), _f64(state_in)
    Bt, D, L = x.shape
    K = w.shape[1]
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
    rb, rd = np.divmod(np.arange(Bt * D, dtype=np.int64), D)
    out = dict(dx=np.empty((Bt, D, L)), dw=np.empty((D, K)), dbias=np.empty(D),
               dstate_in=np.empty((Bt, D, max(K - 1, 0))))
    rc = lib.oracle_conv_silu_bwd_rows(Bt * D, L, K, D, _ptr(rb), _ptr(rd), _ptr(x), _ptr(w), _ptr(reset),
                                       _ptr(state_in), _ptr(pre), _ptr(du), _ptr(out["dx"]), _ptr(out["dw"]),
                                       _ptr(out["dbias"]), _ptr(out["dstate_in"]) if K > 1 else None,
                                       int(nthreads))
    if rc != 0:
        raise MemoryError("oracle conv backward: scratch allocation failed")
    return out


def scan(u, dt_raw, A, Bm, Cm, *, z=None, dt_bias=None, Dskip=None, reset=None, h0=None,
         want_h_last=False, conv_w=None, conv_b=None, conv_state=None, want_conv_state=False, zoh=False,
         nthreads=0):
    """Full scan. u, dt_raw, z: (B, D, L); h0: (B, D, N). Returns out (B, D, L).

    With conv_w (D, K) the scan input is silu(causal_conv1d(u)) (see conv_silu);
    conv_state (B, D, K-1) is the input before the sequence, and
    want_conv_state also returns the final conv state (after h_last).
    """
    if conv_w is not None:
        u, cst = conv_silu(u, conv_w, bias=conv_b, reset=reset, state_in=conv_state, want_state=True,
                           nthreads=nthreads)
        res = scan(u, dt_raw, A, Bm, Cm, z=z, dt_bias=dt_bias, Dskip=Dskip, reset=reset, h0=h0,
                   want_h_last=want_h_last, zoh=zoh, nthreads=nthreads)
        if not want_conv_state:
            return res
        return (res + (cst,)) if want_h_last else (res, cst)
    u = np.asarray(u)
    Bt, D, L = u.shape
    N = np.asarray(A).shape[1]
    rb, rd = np.divmod(np.arange(Bt * D, dtype=np.int64), D)
    res = scan_rows(rb, rd, u.reshape(Bt * D, L), np.asarray(dt_raw).reshape(Bt * D, L), A, Bm, Cm,
                    z_rows=None if z is None else np.asarray(z).reshape(Bt * D, L),
                    dt_bias=dt_bias, Dskip=Dskip, reset=reset,
                    h0_rows=None if h0 is None else np.asarray(h0).reshape(Bt * D, N),
                    want_h_last=want_h_last, zoh=zoh, nthreads=nthreads)
    if want_h_last:
        out, hl = res
        return out.reshape(Bt, D, L), hl.reshape(Bt, D, N)
    return res.reshape(Bt, D, L)


def scan_aggregate(u, dt_raw, A, Bm, *, dt_bias=None, reset=None, conv_w=None, conv_b=None, conv_state=None,
                   zoh=False, complex_state=False, nthreads=0):
    """Affine aggregate (P, H) of a whole sequence: the scan maps the entering
    state h to P h + H per (b, d, n). By that definition, H is the final
    state from h0 = 0 and P is the final state from h0 = 1 minus H (C plays
    no part in the state, so it is zero here). A is (D, N) real or complex;
    returns float64 (or complex128) arrays (B, D, N)."""
    if conv_w is not None:
        u = conv_silu(u, conv_w, bias=conv_b, reset=reset, state_in=conv_state, nthreads=nthreads)
    u = np.asarray(u)
    Bt, D, L = u.shape
    N = np.asarray(A).shape[1]
    Cz = np.zeros((Bt, L, N), dtype=np.complex128 if complex_state else np.float64)
    run = scan_cplx if complex_state else scan
    one = np.ones((Bt, D, N), dtype=np.complex128 if complex_state else np.float64)
    _, H = run(u, dt_raw, A, Bm, Cz, dt_bias=dt_bias, reset=reset, want_h_last=True, zoh=zoh, nthreads=nthreads)
    _, H1 = run(u, dt_raw, A, Bm, Cz, dt_bias=dt_bias, reset=reset, h0=one, want_h_last=True, zoh=zoh,
                nthreads=nthreads)
    return H1 - H, H


def state_update(h, u, dt_raw, A, Bm, Cm, *, z=None, dt_bias=None, Dskip=None, conv_w=None, conv_b=None,
                 conv_state=None, zoh=False, nthreads=0):
    """Decode step. h: (B, D, N); u, dt_raw, z: (B, D); Bm, Cm: (B, N).

    Returns (out (B, D), h_new (B, D, N)); the input h is not modified. With
    conv_w (D, K), u is the conv input of this step and conv_state (B, D, K-1)
    holds the previous K-1 inputs (oldest first, zeros when None): the step
    input is silu(conv_b + sum_k conv_w[:, k] * window[k]) over the window
    (state, u), and (out, h_new, new conv state) is returned.
    """
    if conv_w is not None:
        conv_w = _f64(conv_w)
        x = _f64(u)
        Bt, D = x.shape
        K = conv_w.shape[1]
        st = np.zeros((Bt, D, K - 1)) if conv_state is None else _f64(conv_state)
        window = np.concatenate([st, x[:, :, None]], axis=2)
        pre = np.einsum("bdk,dk->bd", window, conv_w) + (0.0 if conv_b is None else _f64(conv_b)[None, :])
        uc = pre / (1.0 + np.exp(-pre))
        out, h_new = state_update(h, uc, dt_raw, A, Bm, Cm, z=z, dt_bias=dt_bias, Dskip=Dskip, zoh=zoh,
                                  nthreads=nthreads)
        return out, h_new, np.ascontiguousarray(window[:, :, 1:])
    lib = _load()
    h_new = np.array(h, dtype=np.float64, copy=True, order="C")
    u, dt_raw, z = _f64(u), _f64(dt_raw), _f64(z)
    A, Bm, Cm, dt_bias, Dskip = _f64(A), _f64(Bm), _f64(Cm), _f64(dt_bias), _f64(Dskip)
    Bt, D, N = h_new.shape
    if N > MAX_N:
        raise ValueError("oracle supports N <= %d" % MAX_N)
    assert u.shape == (Bt, D) and dt_raw.shape == (Bt, D) and A.shape == (D, N)
    assert Bm.shape == (Bt, N) and Cm.shape == (Bt, N)
    out = np.empty((Bt, D), dtype=np.float64)
    lib.oracle_state_update(Bt, D, N, _ptr(h_new), _ptr(u), _ptr(dt_raw), _ptr(z), _ptr(dt_bias),
                            _ptr(A), _ptr(Dskip), _ptr(Bm), _ptr(Cm), _ptr(out), int(bool(zoh)), int(nthreads))
    return out, h_new


def scan_bwd(u, dt_raw, A, Bm, Cm, dout, *, z=None, dt_bias=None, Dskip=None, reset=None, h0=None,
             dh_last=None, conv_w=None, conv_b=None, conv_state=None, zoh=False, nthreads=0):
    """Gradients of sum(dout * out) + sum(dh_last * h_last) for the full scan.

    u, dt_raw, z, dout: (B, D, L); A: (D, N); Bm, Cm: (B, L, N); dt_bias, Dskip: (D,);
    reset: (B, L); h0, dh_last: (B, D, N). Returns a dict of float64 arrays:
    du, d_dt_raw (B, D, L), dz (B, D, L) or None, dA (D, N), dD, d_dt_bias (D,),
    dB, dC (B, L, N) and dh0 (B, D, N). dD and d_dt_bias are the gradients with
    respect to those parameters whether or not they were given (None acts as 0).
    With conv_w, u is the conv input: du is its gradient, and dconv_w (D, K),
    dconv_b (D,) and dconv_state (B, D, K-1) are added.
    """
    if conv_w is not None:
        uc, pre = conv_silu(u, conv_w, bias=conv_b, reset=reset, state_in=conv_state, want_pre=True,
                            nthreads=nthreads)
        g = scan_bwd(uc, dt_raw, A, Bm, Cm, dout, z=z, dt_bias=dt_bias, Dskip=Dskip, reset=reset, h0=h0,
                     dh_last=dh_last, zoh=zoh, nthreads=nthreads)
        cg = conv_silu_bwd(u, conv_w, g["du"], pre, reset=reset, state_in=conv_state, nthreads=nthreads)
        g["du"] = cg["dx"]
        g["dconv_w"], g["dconv_b"], g["dconv_state"] = cg["dw"], cg["dbias"], cg["dstate_in"]
        return g
    lib = _load()
    u, dt_raw, z, dout = _f64(u), _f64(dt_raw), _f64(z), _f64(dout)
    A, Bm, Cm = _f64(A), _f64(Bm), _f64(Cm)
    dt_bias, Dskip, h0, dh_last = _f64(dt_bias), _f64(Dskip), _f64(h0), _f64(dh_last)
    Bt, D, L = u.shape
    N = A.shape[1]
    assert dt_raw.shape == (Bt, D, L) and dout.shape == (Bt, D, L) and A.shape == (D, N)
    assert Bm.shape == (Bt, L, N) and Cm.shape == (Bt, L, N)
    for x in (z,):
        assert x is None or x.shape == (Bt, D, L)
    for x in (h0, dh_last):
        assert x is None or x.shape == (Bt, D, N)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
        assert reset.shape == (Bt, L)
    rb, rd = np.divmod(np.arange(Bt * D, dtype=np.int64), D)
    out = dict(du=np.empty((Bt, D, L)), d_dt_raw=np.empty((Bt, D, L)),
               dz=None if z is None else np.empty((Bt, D, L)), dA=np.empty((D, N)),
               dD=np.empty(D), d_dt_bias=np.empty(D), dB=np.empty((Bt, L, N)),
               dC=np.empty((Bt, L, N)), dh0=np.empty((Bt, D, N)))
    rc = lib.oracle_scan_bwd_rows(
        Bt * D, L, N, Bt, D, _ptr(rb), _ptr(rd), _ptr(u), _ptr(dt_raw), _ptr(z), _ptr(dt_bias),
        _ptr(A), _ptr(Dskip), _ptr(Bm), _ptr(Cm), _ptr(reset), _ptr(h0), _ptr(dout), _ptr(dh_last),
        _ptr(out["du"]), _ptr(out["d_dt_raw"]), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(out["dD"]),
        _ptr(out["d_dt_bias"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dh0"]), int(bool(zoh)), int(nthreads))
    if rc != 0:
        raise MemoryError("oracle backward: scratch allocation failed")
    return out


def _interleave(x):
    """complex array -> float64 array with a trailing (re, im) axis."""
    if x is None:
        return None
    x = np.asarray(x, dtype=np.complex128)
    return np.ascontiguousarray(np.stack([x.real, x.imag], axis=-1))


def scan_cplx(u, dt_raw, A, Bm, Cm, *, z=None, dt_bias=None, Dskip=None, reset=None, h0=None,
              want_h_last=False, zoh=False, nthreads=0):
    """Full scan with a complex diagonal state (the S4D-Lin variant).

    u, dt_raw, z: (B, D, L) real; A: (D, N) complex; Bm, Cm: (B, L, N) complex;
    h0: (B, D, N) complex or None. Returns out (B, D, L) float64 (the gated real
    part of the read-out) and, if asked, h_last (B, D, N) complex128. zoh=True:
    the input coefficient is (e^{delta A} - 1) / A instead of delta.
    """
    lib = _load()
    u, dt_raw, z = _f64(u), _f64(dt_raw), _f64(z)
    dt_bias, Dskip = _f64(dt_bias), _f64(Dskip)
    Ai, Bi, Ci, h0i = _interleave(A), _interleave(Bm), _interleave(Cm), _interleave(h0)
    Bt, D, L = u.shape
    N = Ai.shape[1]
    if N > MAX_N:
        raise ValueError("oracle supports N <= %d" % MAX_N)
    assert dt_raw.shape == (Bt, D, L) and Ai.shape == (D, N, 2)
    assert Bi.shape == (Bt, L, N, 2) and Ci.shape == (Bt, L, N, 2)
    assert z is None or z.shape == (Bt, D, L)
    assert h0i is None or h0i.shape == (Bt, D, N, 2)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
        assert reset.shape == (Bt, L)
    rb, rd = np.divmod(np.arange(Bt * D, dtype=np.int64), D)
    out = np.empty((Bt, D, L))
    hl = np.empty((Bt, D, N, 2)) if want_h_last else None
    lib.oracle_scan_cplx_rows(Bt * D, L, N, _ptr(rb), _ptr(rd), _ptr(u), _ptr(dt_raw), _ptr(z), _ptr(dt_bias),
                              _ptr(Ai), _ptr(Dskip), _ptr(Bi), _ptr(Ci), _ptr(reset), _ptr(h0i), _ptr(out),
                              _ptr(hl), int(bool(zoh)), int(nthreads))
    if want_h_last:
        return out, hl[..., 0] + 1j * hl[..., 1]
    return out


def state_update_cplx(h, u, dt_raw, A, Bm, Cm, *, z=None, dt_bias=None, Dskip=None, zoh=False, nthreads=0):
    """Decode step with a complex state: one step of scan_cplx from h.

    h: (B, D, N) complex; u, dt_raw, z: (B, D); A: (D, N) complex; Bm, Cm: (B, N)
    complex. Returns (out (B, D), h_new (B, D, N) complex128).
    """
    u = _f64(u)
    Bt, D = u.shape
    out, h_new = scan_cplx(u[:, :, None], _f64(dt_raw)[:, :, None], A, np.asarray(Bm)[:, None, :],
                           np.asarray(Cm)[:, None, :], z=None if z is None else _f64(z)[:, :, None],
                           dt_bias=dt_bias, Dskip=Dskip, h0=h, want_h_last=True, zoh=zoh, nthreads=nthreads)
    return out[:, :, 0], h_new


def scan_cplx_bwd(u, dt_raw, A, Bm, Cm, dout, *, z=None, dt_bias=None, Dskip=None, reset=None, h0=None,
                  dh_last=None, zoh=False, nthreads=0):
    """Gradients of sum(dout * out) + sum(Re dh_last Re h_last + Im dh_last Im h_last)
    for the complex-state scan (scan_cplx, zoh as there). Gradients of complex
    inputs are dL/dRe + i dL/dIm. Returns a dict: du, d_dt_raw, dz (B, D, L)
    (dz None without z), dA (D, N) complex, dD, d_dt_bias (D,), dB, dC
    (B, L, N) complex and dh0 (B, D, N) complex."""
    lib = _load()
    u, dt_raw, z, dout = _f64(u), _f64(dt_raw), _f64(z), _f64(dout)
    dt_bias, Dskip = _f64(dt_bias), _f64(Dskip)
    Ai, Bi, Ci, h0i, dhi = (_interleave(v) for v in (A, Bm, Cm, h0, dh_last))
    Bt, D, L = u.shape
    N = Ai.shape[1]
    assert dt_raw.shape == (Bt, D, L) and dout.shape == (Bt, D, L) and Ai.shape == (D, N, 2)
    assert Bi.shape == (Bt, L, N, 2) and Ci.shape == (Bt, L, N, 2)
    assert z is None or z.shape == (Bt, D, L)
    for v in (h0i, dhi):
        assert v is None or v.shape == (Bt, D, N, 2)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
        assert reset.shape == (Bt, L)
    rb, rd = np.divmod(np.arange(Bt * D, dtype=np.int64), D)
    out = dict(du=np.empty((Bt, D, L)), d_dt_raw=np.empty((Bt, D, L)),
               dz=None if z is None else np.empty((Bt, D, L)), dA=np.empty((D, N, 2)), dD=np.empty(D),
               d_dt_bias=np.empty(D), dB=np.empty((Bt, L, N, 2)), dC=np.empty((Bt, L, N, 2)),
               dh0=np.empty((Bt, D, N, 2)))
    rc = lib.oracle_scan_cplx_bwd_rows(
        Bt * D, L, N, Bt, D, _ptr(rb), _ptr(rd), _ptr(u), _ptr(dt_raw), _ptr(z), _ptr(dt_bias), _ptr(Ai),
        _ptr(Dskip), _ptr(Bi), _ptr(Ci), _ptr(reset), _ptr(h0i), _ptr(dout), _ptr(dhi), _ptr(out["du"]),
        _ptr(out["d_dt_raw"]), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(out["dD"]), _ptr(out["d_dt_bias"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dh0"]), int(bool(zoh)), int(nthreads))
    if rc != 0:
        raise MemoryError("oracle complex backward: scratch allocation failed")
    for k in ("dA", "dB", "dC", "dh0"):
        out[k] = out[k][..., 0] + 1j * out[k][..., 1]
    return out
