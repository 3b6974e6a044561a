"""Seeded synthetic inputs for the selective scan, shared by tests, bench and smoke.

This module only draws random numbers and stores them in the two input formats
(float32, or bfloat16 bit patterns rounded to nearest-even). It holds none of
the scan's arithmetic; both the HIP path and the CPU oracle receive the same
stored values from here.

Recipe (one numpy PCG64 stream per workload, ``np.random.default_rng(seed)``),
draws in this order, all in float64 before the cast to the storage dtype:

  u, dt_raw, z  ~ N(0, 1), shape (B, D, L)
  Bm, Cm        ~ N(0, 1), shape (B, L, N)
  y_d           = exp(U[ln lo, ln hi]) per channel; dt_bias[d] = ln(expm1(y_d))
                  (the inverse of softplus, so softplus(dt_bias) = y_d), float32
  document lengths (packed workloads only): integers U{64..1024} drawn per batch
                  row until the row is covered; reset = 1 at each document's
                  first step (t = 0 included), the last document cut at L.
  A[d, n] = -(n + 1) (S4D-Real, float32), Dskip = 1 (float32), h0 = none.

The decode workload uses the same draws at (B, D) / (B, N) plus an initial
state h ~ N(0, 1) in float32, drawn last.

Complex-state workloads (the S4D-Lin variant) draw u, dt_raw, z as above, then
the real and the imaginary parts of Bm and of Cm, each N(0, 1) with shape
(B, L, N) (order: Bm.re, Bm.im, Cm.re, Cm.im), then dt_bias and resets as
above; A[d, n] = -1/2 + i n (S4D-Lin) and Dskip = 1. Complex values are stored
as a trailing (re, im) axis. Decode adds h (re, im) ~ N(0, 1), drawn last.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"


def to_bf16_bits(x) -> np.ndarray:
    """Round float values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs here are finite.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def store(x, dtype: str) -> np.ndarray:
    """Cast float64 draws to the storage format of ``dtype``."""
    if dtype == F32:
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if dtype == BF16:
        return to_bf16_bits(x)
    raise ValueError(dtype)


def widen(x) -> np.ndarray:
    """Stored values as float64 (exact for both storage formats)."""
    if x is None:
        return None
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


# The five workloads: shapes, dtypes, the dt_bias range and the seed of each.
WORKLOADS = [
    dict(name="tiny-fp32", B=1, D=64, L=256, N=16, dtype=F32, dt_lo=1e-3, dt_hi=1e-1, packed=False, seed=0),
    dict(name="mamba130m-layer", B=8, D=1536, L=2048, N=16, dtype=BF16, dt_lo=1e-3, dt_hi=1e-1,
         packed=False, seed=1),
    dict(name="mamba2.8b-layer", B=4, D=5120, L=2048, N=16, dtype=BF16, dt_lo=1e-3, dt_hi=1e-1,
         packed=False, seed=2),
    dict(name="long-genomics", B=1, D=256, L=131072, N=16, dtype=BF16, dt_lo=1e-3, dt_hi=1e-2,
         packed=False, seed=3),
    dict(name="packed-docs-n128", B=2, D=2048, L=4096, N=128, dtype=BF16, dt_lo=1e-3, dt_hi=1e-1,
         packed=True, seed=4),
]
DECODE = dict(name="decode-n128", B=64, D=2048, N=128, dtype=BF16, dt_lo=1e-3, dt_hi=1e-1, seed=5)


def dt_bias_draw(rng, D, lo, hi):
    y = np.exp(rng.uniform(np.log(lo), np.log(hi), size=D))
    return np.log(np.expm1(y)).astype(np.float32)


def doc_resets(rng, B, L, lo=64, hi=1024):
    """Reset mask (B, L) uint8 for rows packed with documents of random length."""
    reset = np.zeros((B, L), dtype=np.uint8)
    for b in range(B):
        t = 0
        while t < L:
            reset[b, t] = 1
            t += int(rng.integers(lo, hi + 1))
    return reset


def s4d_real_A(D, N):
    return np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)))


def make_scan_inputs(B, D, L, N, dtype=F32, seed=0, dt_lo=1e-3, dt_hi=1e-1, packed=False,
                     with_z=True, dskip="ones"):
    """Inputs of one scan workload in storage format (numpy, host).

    dskip: "ones" (D = 1), "normal" (an extra N(0,1) draw after everything else)
    or None (no skip term).
    """
    rng = np.random.default_rng(seed)
    u = store(rng.standard_normal((B, D, L)), dtype)
    dt_raw = store(rng.standard_normal((B, D, L)), dtype)
    z = store(rng.standard_normal((B, D, L)), dtype)
    Bm = store(rng.standard_normal((B, L, N)), dtype)
    Cm = store(rng.standard_normal((B, L, N)), dtype)
    dt_bias = dt_bias_draw(rng, D, dt_lo, dt_hi)
    reset = doc_resets(rng, B, L) if packed else None
    if dskip == "ones":
        Dskip = np.ones(D, dtype=np.float32)
    elif dskip == "normal":
        Dskip = rng.standard_normal(D).astype(np.float32)
    else:
        Dskip = None
    return dict(u=u, dt_raw=dt_raw, z=z if with_z else None, Bm=Bm, Cm=Cm, dt_bias=dt_bias,
                A=s4d_real_A(D, N), Dskip=Dskip, reset=reset, dtype=dtype)


def workload(name: str) -> dict:
    """The workload called ``name`` (shapes, dtype, dt_bias range, seed)."""
    for w in WORKLOADS:
        if w["name"] == name:
            return dict(w)
    raise KeyError(name)


def workload_inputs(name: str, **overrides):
    """Stored inputs of the workload called ``name`` (its own seed)."""
    c = workload(name)
    c.update(overrides)
    return make_scan_inputs(c["B"], c["D"], c["L"], c["N"], dtype=c["dtype"], seed=c["seed"], dt_lo=c["dt_lo"],
                            dt_hi=c["dt_hi"], packed=c["packed"])


def make_scan_inputs_device(B, D, L, N, device, seed=0, dt_lo=1e-3, dt_hi=1e-1):
    """Bfloat16 scan inputs drawn on ``device``, for sizes too large to draw on
    the host. u, dt_raw, z (B, D, L), then Bm, Cm (B, L, N), each N(0, 1) from
    torch's generator on that device seeded with ``seed``, in that order, and
    rounded to bfloat16 (nearest even); dt_bias is the host draw of
    make_scan_inputs (numpy stream ``seed``); A is S4D-Real and Dskip = 1.
    Returns a dict of device tensors (u, dt_raw, z, Bm, Cm) and numpy arrays
    (dt_bias, A, Dskip)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

    x = dict(u=draw((B, D, L)), dt_raw=draw((B, D, L)), z=draw((B, D, L)), Bm=draw((B, L, N)), Cm=draw((B, L, N)))
    x.update(dt_bias=dt_bias_draw(np.random.default_rng(seed), D, dt_lo, dt_hi), A=s4d_real_A(D, N),
             Dskip=np.ones(D, dtype=np.float32), dtype=BF16)
    return x


def s4d_lin_A(D, N):
    """A[d, n] = -1/2 + i n as (D, N, 2) float32 (re, im) pairs."""
    A = np.empty((D, N, 2), dtype=np.float32)
    A[..., 0] = -0.5
    A[..., 1] = np.arange(N, dtype=np.float32)[None, :]
    return A


def make_cplx_inputs(B, D, L, N, dtype=F32, seed=0, dt_lo=1e-3, dt_hi=1e-1, packed=False, with_z=True):
    """Inputs of one complex-state scan workload in storage format (numpy, host)."""
    rng = np.random.default_rng(seed)
    u = store(rng.standard_normal((B, D, L)), dtype)
    dt_raw = store(rng.standard_normal((B, D, L)), dtype)
    z = store(rng.standard_normal((B, D, L)), dtype)
    parts = [rng.standard_normal((B, L, N)) for _ in range(4)]
    Bm = store(np.stack(parts[:2], axis=-1), dtype)
    Cm = store(np.stack(parts[2:], axis=-1), dtype)
    dt_bias = dt_bias_draw(rng, D, dt_lo, dt_hi)
    reset = doc_resets(rng, B, L) if packed else None
    return dict(u=u, dt_raw=dt_raw, z=z if with_z else None, Bm=Bm, Cm=Cm, dt_bias=dt_bias,
                A=s4d_lin_A(D, N), Dskip=np.ones(D, dtype=np.float32), reset=reset, dtype=dtype)


def make_cplx_decode_inputs(B, D, N, dtype=BF16, seed=5, dt_lo=1e-3, dt_hi=1e-1, with_z=True):
    rng = np.random.default_rng(seed)
    u = store(rng.standard_normal((B, D)), dtype)
    dt_raw = store(rng.standard_normal((B, D)), dtype)
    z = store(rng.standard_normal((B, D)), dtype)
    parts = [rng.standard_normal((B, N)) for _ in range(4)]
    Bm = store(np.stack(parts[:2], axis=-1), dtype)
    Cm = store(np.stack(parts[2:], axis=-1), dtype)
    dt_bias = dt_bias_draw(rng, D, dt_lo, dt_hi)
    h = rng.standard_normal((B, D, N, 2)).astype(np.float32)
    return dict(u=u, dt_raw=dt_raw, z=z if with_z else None, Bm=Bm, Cm=Cm, dt_bias=dt_bias,
                A=s4d_lin_A(D, N), Dskip=np.ones(D, dtype=np.float32), h=h, dtype=dtype)


def as_complex(x):
    """A (..., 2) (re, im) array (float32 or bf16 bits) as complex128, exactly."""
    if x is None:
        return None
    w = widen(x)
    return w[..., 0] + 1j * w[..., 1]


def make_decode_inputs(B, D, N, dtype=BF16, seed=5, dt_lo=1e-3, dt_hi=1e-1, with_z=True):
    rng = np.random.default_rng(seed)
    u = store(rng.standard_normal((B, D)), dtype)
    dt_raw = store(rng.standard_normal((B, D)), dtype)
    z = store(rng.standard_normal((B, D)), dtype)
    Bm = store(rng.standard_normal((B, N)), dtype)
    Cm = store(rng.standard_normal((B, N)), dtype)
    dt_bias = dt_bias_draw(rng, D, dt_lo, dt_hi)
    h = rng.standard_normal((B, D, N)).astype(np.float32)
    return dict(u=u, dt_raw=dt_raw, z=z if with_z else None, Bm=Bm, Cm=Cm, dt_bias=dt_bias,
                A=s4d_real_A(D, N), Dskip=np.ones(D, dtype=np.float32), h=h, dtype=dtype)


def decode_inputs(**overrides):
    c = dict(DECODE)
    c.update(overrides)
    return make_decode_inputs(c["B"], c["D"], c["N"], dtype=c["dtype"], seed=c["seed"],
                              dt_lo=c["dt_lo"], dt_hi=c["dt_hi"])


def to_torch(x, device):
    """A stored array as a torch tensor on ``device`` (bf16 bits become bfloat16)."""
    import torch

    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if not x.flags.writeable:
        x = x.copy()
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)
