"""Coefficients of the sine and cosine polynomials in cplx_device.h.

sin(w r) ~ r (S1 + S3 x + S5 x^2 + S7 x^3) and cos(w r) ~ 1 + x (C2 + C4 x + C6 x^2 + C8 x^3),
x = r^2, for |r| <= 1/8 revolution, w = 2 pi rounded to float32. Each is a weighted least-squares
fit on Chebyshev nodes whose weights are raised where the error is largest (iteratively, toward
equal ripple): relative error for the sine, absolute for the cosine. The fit runs in float64; the
coefficients are then rounded to float32. The script prints them and the error of evaluating the
polynomials in float32 (Horner with fused multiply-adds, emulated in float64 and rounded), next to
the same evaluation of the Taylor series of degree 9 and 10.

Usage: python rotation_coefficients.py
"""
import numpy as np

W = float(np.float32(2.0 * np.pi))
R = 0.125


def _nodes(n=4000):
    t = np.cos(np.pi * (np.arange(n) + 0.5) / n)
    return np.concatenate([(t + 1.0) / 2.0 * R, [R]])


def _reweighted_lstsq(A, f, w0, err, iters=30):
    w = w0.copy()
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(A * w[:, None], f * w, rcond=None)
        e = np.abs(err(c))
        w = w * (1.0 + 20.0 * e / e.max())
    return c, np.abs(err(c)).max()


def fit():
    r = _nodes()
    x = r * r
    s_true, c_true = np.sin(W * r), np.cos(W * r)
    As = np.stack([r * x**j for j in range(4)], 1)
    s, s_err = _reweighted_lstsq(As, s_true, 1.0 / np.abs(s_true), lambda c: (As @ c - s_true) / s_true)
    Ac = np.stack([x**(j + 1) for j in range(4)], 1)
    c, c_err = _reweighted_lstsq(Ac, c_true - 1.0, np.ones_like(r), lambda k: Ac @ k - (c_true - 1.0))
    return s.astype(np.float32), c.astype(np.float32), s_err, c_err


def _fma(a, b, c):
    return (np.float64(a) * np.float64(b) + np.float64(c)).astype(np.float32)


def _horner(x, coefs):
    v = np.full_like(x, coefs[-1])
    for k in coefs[-2::-1]:
        v = _fma(x, v, np.float32(k))
    return v


def float32_errors(s, c):
    r = np.linspace(-R, R, 200001).astype(np.float32)
    x = (r * r).astype(np.float32)
    sn = (r * _horner(x, s)).astype(np.float64)
    cs = _fma(x, _horner(x, c), np.float32(1.0)).astype(np.float64)
    rs, rc = np.sin(W * r.astype(np.float64)), np.cos(W * r.astype(np.float64))
    mag = np.sqrt(sn * sn + cs * cs) - 1.0
    return np.abs(sn - rs).max(), np.abs(cs - rc).max(), mag.mean()


if __name__ == "__main__":
    s, c, s_err, c_err = fit()
    for name, v in zip(("kS1", "kS3", "kS5", "kS7"), s):
        print("%s = %r" % (name, float(v)))
    for name, v in zip(("kC2", "kC4", "kC6", "kC8"), c):
        print("%s = %r" % (name, float(v)))
    print("fit error (float64): sin %.3g relative, cos %.3g absolute" % (s_err, c_err))
    p2 = W * W
    taylor_s = np.float32([W, -W * p2 / 6, W * p2**2 / 120, -W * p2**3 / 5040, W * p2**4 / 362880])
    taylor_c = np.float32([-p2 / 2, p2**2 / 24, -p2**3 / 720, p2**4 / 40320, -p2**5 / 3628800])
    for name, ss, cc in (("fitted, degree 7 / 8", s, c), ("Taylor, degree 9 / 10", taylor_s, taylor_c)):
        es, ec, mb = float32_errors(ss, cc)
        print("%s: float32 evaluation error sin %.3g, cos %.3g; mean of |e^(i w r)| - 1: %.3g" % (name, es, ec, mb))
