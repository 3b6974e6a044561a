"""Pins of the complex-state backward oracle (oracle.scan_cplx_bwd).

The gradients are the chain rule through the complex recurrence; what pins
them here, independently of that code:
- central finite differences of the loss sum(dout * out) + <dh_last, h_last>
  (h_last's real and imaginary parts weighted separately), evaluated with the
  forward oracle, for every input: the real ones (u, dt_raw, z, D, dt_bias)
  and the real and imaginary parts of the complex ones (A, B, C, h0), on a
  small problem with resets, an initial state and a gate;
- zero imaginary parts reproduce the real backward oracle (pinned by its own
  finite differences), with zero imaginary parts in every complex gradient;
- both with the delta B input coefficient and with the exact zero-order hold.
"""
import numpy as np
import pytest

import oracle


def cplx(rng, *shape):
    return rng.standard_normal(shape) + 1j * rng.standard_normal(shape)


def problem(seed, with_z=True):
    rng = np.random.default_rng(seed)
    Bt, D, L, N = 2, 2, 9, 3
    x = dict(u=rng.standard_normal((Bt, D, L)), dt_raw=rng.standard_normal((Bt, D, L)) - 0.5,
             z=rng.standard_normal((Bt, D, L)) if with_z else None,
             A=-rng.uniform(0.2, 1.0, (D, N)) + 1j * rng.uniform(-3, 3, (D, N)),
             Bm=cplx(rng, Bt, L, N), Cm=cplx(rng, Bt, L, N), Dskip=rng.standard_normal(D),
             dt_bias=rng.standard_normal(D) * 0.5, h0=cplx(rng, Bt, D, N))
    reset = np.zeros((Bt, L), np.uint8)
    reset[1, 4] = 1
    reset[0, 0] = 1
    x["reset"] = reset
    dout = rng.standard_normal((Bt, D, L))
    dh_last = cplx(rng, Bt, D, N)
    return x, dout, dh_last


def loss(x, dout, dh_last, zoh=False):
    out, hl = oracle.scan_cplx(x["u"], x["dt_raw"], x["A"], x["Bm"], x["Cm"], z=x["z"], dt_bias=x["dt_bias"],
                               Dskip=x["Dskip"], reset=x["reset"], h0=x["h0"], want_h_last=True, zoh=zoh)
    return float(np.sum(dout * out) + np.sum(dh_last.real * hl.real + dh_last.imag * hl.imag))


def grads(x, dout, dh_last, zoh=False):
    return oracle.scan_cplx_bwd(x["u"], x["dt_raw"], x["A"], x["Bm"], x["Cm"], dout, z=x["z"],
                                dt_bias=x["dt_bias"], Dskip=x["Dskip"], reset=x["reset"], h0=x["h0"],
                                dh_last=dh_last, zoh=zoh)


def fd(x, dout, dh_last, key, part, eps=1e-6, zoh=False):
    """Central differences of the loss over every element of x[key] (part: 'real' or 'imag')."""
    base = x[key]
    res = np.zeros(base.shape)
    for idx in np.ndindex(base.shape):
        vals = []
        for sgn in (1, -1):
            y = dict(x)
            arr = np.array(base, dtype=complex if part == "imag" or np.iscomplexobj(base) else float, copy=True)
            arr[idx] += sgn * eps * (1j if part == "imag" else 1.0)
            y[key] = arr
            vals.append(loss(y, dout, dh_last, zoh))
        res[idx] = (vals[0] - vals[1]) / (2 * eps)
    return res


GRAD_OF = dict(u="du", dt_raw="d_dt_raw", z="dz", Dskip="dD", dt_bias="d_dt_bias", A="dA", Bm="dB", Cm="dC",
               h0="dh0")


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("key", ["u", "dt_raw", "z", "Dskip", "dt_bias", "A", "Bm", "Cm", "h0"])
def test_finite_differences(key, zoh):
    x, dout, dh_last = problem(3)
    g = grads(x, dout, dh_last, zoh)[GRAD_OF[key]]
    parts = ("real", "imag") if np.iscomplexobj(x[key]) else ("real",)
    for part in parts:
        num = fd(x, dout, dh_last, key, part, zoh=zoh)
        got = g.real if part == "real" else g.imag
        scale = np.max(np.abs(num)) + 1e-12
        np.testing.assert_allclose(got, num, rtol=2e-5, atol=2e-6 * scale, err_msg="%s %s" % (key, part))


def test_without_gate():
    x, dout, dh_last = problem(4, with_z=False)
    g = grads(x, dout, dh_last)
    assert g["dz"] is None
    num = fd(x, dout, dh_last, "u", "real")
    np.testing.assert_allclose(g["du"], num, rtol=2e-5, atol=1e-7)


@pytest.mark.parametrize("zoh", [False, True])
def test_real_case_is_the_real_backward(zoh):
    rng = np.random.default_rng(5)
    Bt, D, L, N = 2, 4, 50, 6
    u, dt, z, dout = (rng.standard_normal((Bt, D, L)) for _ in range(4))
    A = -rng.uniform(0.5, 3, (D, N))
    Bm, Cm = rng.standard_normal((Bt, L, N)), rng.standard_normal((Bt, L, N))
    h0, dhl = rng.standard_normal((Bt, D, N)), rng.standard_normal((Bt, D, N))
    Dsk, bias = rng.standard_normal(D), rng.standard_normal(D)
    reset = (rng.uniform(size=(Bt, L)) < 0.08).astype(np.uint8)
    gc = oracle.scan_cplx_bwd(u, dt, A + 0j, Bm + 0j, Cm + 0j, dout, z=z, dt_bias=bias, Dskip=Dsk, reset=reset,
                              h0=h0 + 0j, dh_last=dhl + 0j, zoh=zoh)
    gr = oracle.scan_bwd(u, dt, A, Bm, Cm, dout, z=z, dt_bias=bias, Dskip=Dsk, reset=reset, h0=h0, dh_last=dhl,
                         zoh=zoh)
    for k in ("du", "d_dt_raw", "dz", "dD", "d_dt_bias"):
        np.testing.assert_allclose(gc[k], gr[k], rtol=1e-12, atol=1e-12, err_msg=k)
    for k in ("dA", "dB", "dC", "dh0"):
        np.testing.assert_allclose(gc[k].real, gr[k], rtol=1e-12, atol=1e-12, err_msg=k)
        assert np.all(gc[k].imag == 0), k


def test_zoh_small_A_series_branch():
    """|delta A| below 1e-3, where d phi/dA comes from its series: finite
    differences of the A gradient, and of delta's."""
    x, dout, dh_last = problem(6)
    x["A"] = x["A"] * 1e-5
    g = grads(x, dout, dh_last, zoh=True)
    for key in ("A", "dt_raw"):
        parts = ("real", "imag") if key == "A" else ("real",)
        for part in parts:
            num = fd(x, dout, dh_last, key, part, eps=1e-7 if key == "A" else 1e-6, zoh=True)
            got = g[GRAD_OF[key]].real if part == "real" else g[GRAD_OF[key]].imag
            scale = np.max(np.abs(num)) + 1e-12
            np.testing.assert_allclose(got, num, rtol=2e-5, atol=2e-6 * scale, err_msg="%s %s" % (key, part))


@pytest.mark.parametrize("cplx", [False, True])
def test_zoh_series_meets_closed_form(cplx):
    """d phi/dA switches from its series to the closed form at |delta A| = 1e-3:
    on a one-step problem whose A gradient is conj(d phi/dA) exactly, the two
    sides of the switch agree to 1e-11 (a wrong series coefficient shows up
    at 1e-7)."""
    delta = 0.37
    x = np.log(np.expm1(delta))                       # dt_raw with softplus = delta
    one = np.ones((1, 1, 1))
    res = []
    for f in (1.0 - 1e-9, 1.0 + 1e-9):
        mag = 1e-3 / delta * f
        A = np.array([[mag * np.exp(0.7j)]]) if cplx else np.array([[-mag]])
        if cplx:
            g = oracle.scan_cplx_bwd(one, one * x, A, np.ones((1, 1, 1)) + 0j, np.ones((1, 1, 1)) + 0j, one,
                                     zoh=True)
        else:
            g = oracle.scan_bwd(one, one * x, A, np.ones((1, 1, 1)), np.ones((1, 1, 1)), one, zoh=True)
        res.append(complex(g["dA"][0, 0]))
    assert abs(res[0] - res[1]) <= 1e-11 * abs(res[0]), res
