"""GPU parity of the exact zero-order-hold discretisation against the oracle.

The oracle's ZOH is pinned by ODE integration, the continuous steady state
and finite differences (test_oracle_zoh_pins.py). Tolerances are the forward's
(1e-5 (1 + |ref|) with float32 inputs, 2e-3 (1 + |ref|) with bf16) and the
backward's (1e-4 (rms + |ref|)). The kernel evaluates the coefficient
(e^{delta A} - 1) / A from e^{delta A} where |delta A| >= 1/16 and by a
series below, so the cases below use step sizes that put delta*A on both sides.
"""
import numpy as np
import pytest

import oracle
from selective_state_space_67_amd import workloads as wl

from gpu_helpers import assert_close, device, to_dev

pytestmark = pytest.mark.gpu


def case(B, D, L, N, dtype, seed, packed=False, dt_lo=1e-3, dt_hi=3e-1, conv=False):
    x = wl.make_scan_inputs(B, D, L, N, dtype, seed=seed, dt_lo=dt_lo, dt_hi=dt_hi, packed=packed)
    rng = np.random.default_rng(seed + 5)
    x["Dskip"] = rng.standard_normal(D).astype(np.float32)
    x["A"][:, 0] = 0.0 if N > 1 else x["A"][:, 0]   # A = 0: the coefficient's limit delta
    x["conv_w"] = (rng.standard_normal((D, 4)) * 0.5).astype(np.float32) if conv else None
    x["dout"] = wl.store(rng.standard_normal((B, D, L)), dtype)
    return x


def run_fwd(x, num_segments=0):
    import torch

    from selective_state_space_67_amd import ssm_scan_fwd

    dev = device()
    t = {k: to_dev(x[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset")}
    cw = None if x["conv_w"] is None else torch.from_numpy(x["conv_w"]).to(dev)
    Bt, D, N = x["u"].shape[0], x["u"].shape[1], x["A"].shape[1]
    hl = torch.empty((Bt, D, N), dtype=torch.float32, device=dev)
    out = ssm_scan_fwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"], Dskip=t["Dskip"],
                       z=t["z"], reset=t["reset"], h_last=hl, num_segments=num_segments, conv_w=cw, zoh=True)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), hl.cpu().numpy().astype(np.float64)


def ref_fwd(x):
    w = wl.widen
    return oracle.scan(w(x["u"]), w(x["dt_raw"]), x["A"], w(x["Bm"]), w(x["Cm"]), z=w(x["z"]), dt_bias=x["dt_bias"],
                       Dskip=x["Dskip"], reset=x["reset"], conv_w=x["conv_w"], want_h_last=True, zoh=True)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("N", [1, 16, 32, 64, 128, 256])
def test_zoh_forward(dtype, N):
    x = case(2, 20, 260, N, dtype, 700 + N, packed=True)
    got, hl = run_fwd(x)
    ref, rhl = ref_fwd(x)
    assert_close(got, ref, dtype, what="out N=%d" % N)
    assert_close(hl, rhl, dtype, what="h_last N=%d" % N)


@pytest.mark.parametrize("dtype,B,D,L,nseg", [(wl.F32, 2, 37, 1000, 0), (wl.BF16, 1, 16, 4000, 3)])
def test_zoh_forward_sixteen_states(dtype, B, D, L, nseg):
    # N = 16, even L, no resets: the 16-state kernel's zero-order-hold variant,
    # with a partial channel group, and pieces joined by aggregates. Every
    # state decays here (A = 0 would make state 0 a plain running sum over the
    # whole sequence, whose float32 rounding outgrows the float32 tolerance
    # after a few hundred steps in any kernel); small step sizes still put
    # delta*A below 1/16, where the coefficient is the series.
    x = case(B, D, L, 16, dtype, 900 + D)
    x["A"][:, 0] = -1.0
    got, hl = run_fwd(x, num_segments=nseg)
    ref, rhl = ref_fwd(x)
    assert_close(got, ref, dtype, what="out")
    assert_close(hl, rhl, dtype, what="h_last")


def test_zoh_forward_split_and_conv():
    x = case(1, 32, 5000, 16, wl.BF16, 9, dt_lo=1e-3, dt_hi=1e-2, conv=True)
    got, _ = run_fwd(x, num_segments=4)
    ref, _ = ref_fwd(x)
    assert_close(got, ref, wl.BF16)


@pytest.mark.parametrize("N", [128, 12])
def test_zoh_decode(N):
    import torch

    from selective_state_space_67_amd import ssm_state_update

    dev = device()
    y = wl.make_decode_inputs(4, 64, N, dtype=wl.F32, seed=N, dt_hi=0.5)
    y["A"][:3] = 0.0
    t = {k: wl.to_torch(y[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    h = torch.from_numpy(y["h"]).to(dev)
    o = ssm_state_update(h, t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"], Dskip=t["Dskip"],
                         z=t["z"], zoh=True)
    torch.cuda.synchronize()
    ro, rh = oracle.state_update(y["h"], y["u"], y["dt_raw"], y["A"], y["Bm"], y["Cm"], z=y["z"],
                                 dt_bias=y["dt_bias"], Dskip=y["Dskip"], zoh=True)
    assert_close(o.cpu().numpy(), ro, wl.F32, what="out")
    assert_close(h.cpu().numpy(), rh, wl.F32, what="h")


KEYS = dict(du="du", d_dt_raw="d_dt_raw", dz="dz", dA="dA", dBm="dB", dCm="dC", dDskip="dD", d_dt_bias="d_dt_bias",
            dh0="dh0", dconv_w="dconv_w", dconv_b="dconv_b")


@pytest.mark.parametrize("dtype,N,conv", [(wl.F32, 16, False), (wl.BF16, 16, True), (wl.BF16, 64, False),
                                          (wl.F32, 128, False), (wl.BF16, 200, False)])
def test_zoh_backward(dtype, N, conv):
    import torch

    from selective_state_space_67_amd import ssm_scan_bwd

    x = case(2, 24, 300, N, dtype, 800 + N, packed=True, conv=conv)
    dev = device()
    t = {k: to_dev(x[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset", "dout")}
    cw = None if x["conv_w"] is None else torch.from_numpy(x["conv_w"]).to(dev)
    g = ssm_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], t["dout"], dt_bias=t["dt_bias"],
                     Dskip=t["Dskip"], z=t["z"], reset=t["reset"], conv_w=cw, zoh=True)
    torch.cuda.synchronize()
    w = wl.widen
    r = oracle.scan_bwd(w(x["u"]), w(x["dt_raw"]), x["A"], w(x["Bm"]), w(x["Cm"]), w(x["dout"]), z=w(x["z"]),
                        dt_bias=x["dt_bias"], Dskip=x["Dskip"], reset=x["reset"], conv_w=x["conv_w"], zoh=True)
    for gk, rk in KEYS.items():
        if g.get(gk) is None or r.get(rk) is None:
            continue
        o, ref = g[gk].float().cpu().numpy().astype(np.float64), r[rk]
        bound = 1e-4 * (np.sqrt(np.mean(ref * ref)) + np.abs(ref)) + 1e-30
        ratio = np.abs(o - ref) / bound
        assert np.all(ratio <= 1), "%s: worst %.3g of the bound at %s" % (gk, ratio.max(), np.argmax(ratio))
