"""GPU parity of the sequence aggregate (ssm_scan_aggregate) against the oracle,
and the sharded scan it enables.

The oracle's aggregate is pinned by the closed form of the decay product, the
one-step value, composition of halves and the sharded scan
(test_oracle_aggregate_pins.py).

Tolerances.
- H is the final state of a scan from a zero state: the forward's bound,
  tol (1 + |ref|) with tol = 1e-5 (float32 inputs) or 2e-3 (bfloat16), plus
  the complex path's phase term (test_cplx_gpu.py) for the complex state.
- P = exp(A S), S = the sum of delta over the sequence. The kernel sums delta
  in float32: a relative error of at most (L + 2) 2^-24 in S (sequential
  summation, first order), which multiplies |A S| in the exponent; plus a few
  ulps for exp2 and A log2 e. So |P - ref| <= |ref| (|A| S (L + 2) + 8) 2^-24
  + 1e-7.
"""
import numpy as np
import pytest

import oracle
from selective_state_space_67_amd import workloads as wl

from gpu_helpers import TOL, device, to_dev
from test_cplx_gpu import phase_bound

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def gpu_aggregate(x, cplx, zoh=False, num_segments=0, conv=None):
    import torch

    from selective_state_space_67_amd import ssm_scan_aggregate

    dev = device()
    t = {k: to_dev(x[k], dev) for k in ("u", "dt_raw", "Bm", "dt_bias", "A", "reset")}
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    w, cb, st = conv if conv else (None, None, None)
    P, H = ssm_scan_aggregate(t["u"], t["dt_raw"], t["A"], t["Bm"], dt_bias=t["dt_bias"], reset=t["reset"],
                              zoh=zoh, complex_state=cplx, num_segments=num_segments, conv_w=f32(w),
                              conv_b=f32(cb), conv_state_in=f32(st))
    torch.cuda.synchronize()
    P, H = P.cpu().numpy().astype(np.float64), H.cpu().numpy().astype(np.float64)
    if cplx:
        P, H = P[..., 0] + 1j * P[..., 1], H[..., 0] + 1j * H[..., 1]
    return P, H


def ref_aggregate(x, cplx, zoh=False, conv=None):
    w, cb, st = conv if conv else (None, None, None)
    A = wl.as_complex(x["A"]) if cplx else x["A"]
    Bm = wl.as_complex(x["Bm"]) if cplx else wl.widen(x["Bm"])
    return oracle.scan_aggregate(wl.widen(x["u"]), wl.widen(x["dt_raw"]), A, Bm, dt_bias=x["dt_bias"],
                                 reset=x["reset"], conv_w=w, conv_b=cb, conv_state=st, zoh=zoh, complex_state=cplx)


def check(x, got, ref, cplx, zoh=False, conv=None, what=""):
    P, H = got
    rP, rH = ref
    dt = wl.widen(x["dt_raw"])
    D, L = dt.shape[1], dt.shape[2]
    bias = np.zeros(D) if x["dt_bias"] is None else x["dt_bias"].astype(np.float64)
    xx = dt + bias[None, :, None]
    S = (np.maximum(xx, 0) + np.log1p(np.exp(-np.abs(xx)))).sum(axis=2)     # (B, D)
    A = wl.as_complex(x["A"]) if cplx else x["A"]
    pbound = np.abs(rP) * (np.abs(A)[None] * S[:, :, None] * (L + 2) + 8) * U32 + 1e-7
    perr = np.abs(P - rP)
    assert np.all(perr <= pbound), "%s P: worst %.3g of bound" % (what, float(np.max(perr / pbound)))
    hb = TOL[x["dtype"]] * (1 + np.abs(rH))
    if cplx:
        xs = dict(x)
        if conv:
            xs["u"] = oracle.conv_silu(wl.widen(x["u"]), conv[0], bias=conv[1], reset=x["reset"], state_in=conv[2])
        xs["z"] = None
        xs["Cm"] = np.zeros_like(x["Bm"])
        hb = hb + phase_bound(xs, None, zoh)[1]
    herr = np.abs(H - rH)
    assert np.all(herr <= hb), "%s H: worst %.3g of bound" % (what, float(np.max(herr / hb)))
    print(what, "P %.3f H %.3f" % (float(np.max(perr / pbound)), float(np.max(herr / hb))), flush=True)


@pytest.mark.parametrize("cplx", [False, True])
@pytest.mark.parametrize("N", [1, 16, 64, 128])
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_aggregate(cplx, N, dtype):
    make = wl.make_cplx_inputs if cplx else wl.make_scan_inputs
    x = make(2, 24, 500, N, dtype, seed=300 + N, packed=True)
    x["reset"][0, :] = 0                     # row 0 has no reset: P is not zero there
    got = gpu_aggregate(x, cplx)
    check(x, got, ref_aggregate(x, cplx), cplx, what="N=%d %s cplx=%s" % (N, dtype, cplx))


@pytest.mark.parametrize("cplx", [False, True])
@pytest.mark.parametrize("nseg", [1, 3, 8])
def test_aggregate_pieces_zoh_conv(cplx, nseg):
    """The library's own pieces (folded in order), the zero-order hold and the conv stage."""
    make = wl.make_cplx_inputs if cplx else wl.make_scan_inputs
    x = make(1, 40, 3000, 16, wl.F32, seed=320 + nseg, dt_lo=1e-3, dt_hi=1e-2)
    x["reset"] = np.zeros((1, 3000), np.uint8)
    rng = np.random.default_rng(nseg)
    conv = ((rng.standard_normal((40, 4)) * 0.5).astype(np.float32), (rng.standard_normal(40) * 0.2).astype(np.float32),
            rng.standard_normal((1, 40, 3)).astype(np.float32))
    for zoh, cv in ((False, None), (True, conv)):
        got = gpu_aggregate(x, cplx, zoh=zoh, num_segments=nseg, conv=cv)
        check(x, got, ref_aggregate(x, cplx, zoh=zoh, conv=cv), cplx, zoh=zoh, conv=cv,
              what="pieces=%d zoh=%s cplx=%s" % (nseg, zoh, cplx))


def test_sharded_scan_at_the_long_genomics_shard():
    """The long-genomics sequence (1 x 256 x 131072, N = 16) cut into 8 shards of
    16384 steps, one GPU's share each: every shard's aggregate on the GPU, the
    fold h <- P h + H between shards (the part a collective would carry), and
    every shard's scan with h0 = that state; the outputs of 32 sampled
    channels against the oracle's scan of the whole sequence."""
    import torch

    from selective_state_space_67_amd import ssm_scan_aggregate, ssm_scan_fwd

    cfg = wl.workload("long-genomics")
    x = wl.workload_inputs("long-genomics")
    dev = device()
    t = {k: to_dev(x[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    shards, Ls = 8, cfg["L"] // 8
    h = torch.zeros((B, D, N), dtype=torch.float32, device=dev)
    outs = []
    for s in range(shards):
        sl = slice(s * Ls, (s + 1) * Ls)
        u, dt, z = (t[k][:, :, sl].contiguous() for k in ("u", "dt_raw", "z"))
        Bm, Cm = t["Bm"][:, sl].contiguous(), t["Cm"][:, sl].contiguous()
        outs.append(ssm_scan_fwd(u, dt, t["A"], Bm, Cm, dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=z,
                                 h0=h.clone()))
        P, H = ssm_scan_aggregate(u, dt, t["A"], Bm, dt_bias=t["dt_bias"])
        h = torch.addcmul(H, P, h)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).cpu().numpy().astype(np.float64)
    ds = np.sort(np.random.default_rng(33).choice(D, 32, replace=False))
    w = wl.widen
    ref = oracle.scan_rows(np.zeros(32, np.int64), ds, w(x["u"][0, ds]), w(x["dt_raw"][0, ds]), x["A"], w(x["Bm"]),
                           w(x["Cm"]), z_rows=w(x["z"][0, ds]), dt_bias=x["dt_bias"], Dskip=x["Dskip"])
    err = np.abs(got[0, ds] - ref)
    bound = TOL[cfg["dtype"]] * (1 + np.abs(ref))
    assert np.all(err <= bound), float(np.max(err / bound))
    print("sharded long-genomics: worst err/bound %.3f" % float(np.max(err / bound)), flush=True)
