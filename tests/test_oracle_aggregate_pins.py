"""Pins of the oracle's sequence aggregate (oracle.scan_aggregate).

The aggregate (P, H) is defined by the scan's affine map h_last = P h0 + H.
What pins it, apart from that definition:
- P is the product of the decays, exp(A sum_t delta_t), and 0 when a reset
  lies in the sequence (real and complex A, either input coefficient);
- one step: H = delta u B (and (e^{delta A} - 1)/A u B with the zero-order hold);
- composition: the aggregates of two halves compose to the whole's,
  P = P2 P1, H = P2 H1 + H2, with the conv stage's state handed over;
- the sharded scan: shards scanned with h0 folded from the preceding shards'
  aggregates reproduce the full scan's outputs.
"""
import numpy as np
import pytest

import oracle


def softplus(x):
    return np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))


def case(seed, Bt=2, D=3, L=40, N=4, cplx=False):
    rng = np.random.default_rng(seed)
    u, dt = rng.standard_normal((Bt, D, L)), rng.standard_normal((Bt, D, L)) - 1.0
    bias = rng.standard_normal(D) * 0.3
    if cplx:
        A = -rng.uniform(0.2, 1.0, (D, N)) + 1j * rng.uniform(-4, 4, (D, N))
        Bm = rng.standard_normal((Bt, L, N)) + 1j * rng.standard_normal((Bt, L, N))
    else:
        A = -rng.uniform(0.2, 2.0, (D, N))
        Bm = rng.standard_normal((Bt, L, N))
    return u, dt, A, Bm, bias


@pytest.mark.parametrize("cplx", [False, True])
@pytest.mark.parametrize("zoh", [False, True])
def test_decay_product_closed_form(cplx, zoh):
    u, dt, A, Bm, bias = case(1, cplx=cplx)
    reset = np.zeros((2, 40), np.uint8)
    reset[1, 17] = 1
    P, _ = oracle.scan_aggregate(u, dt, A, Bm, dt_bias=bias, reset=reset, zoh=zoh, complex_state=cplx)
    S = softplus(dt + bias[None, :, None]).sum(axis=2)            # (B, D)
    want = np.exp(A[None] * S[:, :, None])
    want[1] = 0.0                                                  # row 1 meets a reset
    np.testing.assert_allclose(P, want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("cplx", [False, True])
def test_one_step(cplx):
    u, dt, A, Bm, bias = case(2, L=1, cplx=cplx)
    delta = softplus(dt[:, :, 0] + bias[None])[:, :, None]        # (B, D, 1)
    _, H = oracle.scan_aggregate(u, dt, A, Bm, dt_bias=bias, complex_state=cplx)
    np.testing.assert_allclose(H, delta * u[:, :, :1] * Bm[:, None, 0, :], rtol=1e-13, atol=1e-15)
    _, Hz = oracle.scan_aggregate(u, dt, A, Bm, dt_bias=bias, zoh=True, complex_state=cplx)
    coef = np.expm1(delta * A[None]) / A[None]
    np.testing.assert_allclose(Hz, coef * u[:, :, :1] * Bm[:, None, 0, :], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("cplx", [False, True])
@pytest.mark.parametrize("K", [0, 4])
def test_halves_compose(cplx, K):
    u, dt, A, Bm, bias = case(3, L=64, cplx=cplx)
    rng = np.random.default_rng(4)
    reset = (rng.uniform(size=(2, 64)) < 0.05).astype(np.uint8)
    conv = {}
    if K:
        conv = dict(conv_w=rng.standard_normal((3, K)) * 0.5, conv_b=rng.standard_normal(3) * 0.2,
                    conv_state=rng.standard_normal((2, 3, K - 1)))
    P, H = oracle.scan_aggregate(u, dt, A, Bm, dt_bias=bias, reset=reset, complex_state=cplx, **conv)
    k = 27
    c1, c2 = dict(conv), dict(conv)
    if K:
        c2["conv_state"] = u[:, :, k - (K - 1):k]                  # the first half's last K-1 inputs
        # a reset inside the carried window hides the inputs before it
        for b in range(2):
            for j in range(K - 1):
                if reset[b, k - (K - 1) + j + 1:k + 1].any():
                    c2["conv_state"][b, :, j] = 0.0
    P1, H1 = oracle.scan_aggregate(u[:, :, :k], dt[:, :, :k], A, Bm[:, :k], dt_bias=bias, reset=reset[:, :k],
                                   complex_state=cplx, **c1)
    P2, H2 = oracle.scan_aggregate(u[:, :, k:], dt[:, :, k:], A, Bm[:, k:], dt_bias=bias, reset=reset[:, k:],
                                   complex_state=cplx, **c2)
    np.testing.assert_allclose(P, P2 * P1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(H, P2 * H1 + H2, rtol=1e-11, atol=1e-12)


def test_sharded_scan_reproduces_the_full_scan():
    rng = np.random.default_rng(6)
    Bt, D, L, N, shards = 2, 3, 90, 5, 4
    u, dt, A, Bm, bias = case(6, Bt, D, L, N)
    Cm, z = rng.standard_normal((Bt, L, N)), rng.standard_normal((Bt, D, L))
    Dsk, h0 = rng.standard_normal(D), rng.standard_normal((Bt, D, N))
    reset = (rng.uniform(size=(Bt, L)) < 0.04).astype(np.uint8)
    full = oracle.scan(u, dt, A, Bm, Cm, z=z, dt_bias=bias, Dskip=Dsk, reset=reset, h0=h0)
    cuts = [0, 17, 40, 71, L]
    h = h0
    for s in range(shards):
        a, b = cuts[s], cuts[s + 1]
        sl = np.s_[:, :, a:b]
        part = oracle.scan(u[sl], dt[sl], A, Bm[:, a:b], Cm[:, a:b], z=z[sl], dt_bias=bias, Dskip=Dsk,
                           reset=reset[:, a:b], h0=h)
        np.testing.assert_allclose(part, full[sl], rtol=1e-12, atol=1e-12)
        P, H = oracle.scan_aggregate(u[sl], dt[sl], A, Bm[:, a:b], dt_bias=bias, reset=reset[:, a:b])
        h = P * h + H
