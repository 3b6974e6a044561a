"""Pins of the complex-state oracle (oracle.scan_cplx), independent of its code.

The complex diagonal state is the S4D-Lin variant: its initialisation
A = -1/2 + i n is on "Technical analysis: Mamba selective state spaces",
section 4.1, and section 5.3 says a complex state keeps phase information.
The pages define nothing else about it; the reading (complex A, B, C and h,
real delta and u, the real part of sum_n C h) is the one stated in the
oracle's header. What pins it here:

- a brute-force materialised form: each output is the real part of the sum
  over earlier steps s of C_t (prod_{s<r<=t} exp(delta_r A)) delta_s B_s u_s,
  built from products of decays with numpy complex arithmetic, no recurrence;
- the real special case: zero imaginary parts give the real scan, which has
  its own pins;
- constant inputs: the complex geometric series in closed form;
- pure rotation (Re A = 0, B = 0): h_t = exp(i w S_t) h0 with S_t the running
  sum of delta, which fixes the sign of the phase;
- a conjugate pair of states reads out twice the real part of one of them.

With the exact zero-order hold (input coefficient (e^{delta A} - 1) / A), each
step equals a DOP853 integration of the complex system h' = A h + B u over the
step; constant inputs reach the continuous fixed point -B u / A exactly; A = 0
gives the delta B form bit for bit, a real A the real ZOH oracle, and a tiny
delta A the delta B form to 1e-10 (no cancellation in e^{delta A} - 1).
"""
import numpy as np
import pytest

import oracle


def softplus(x):
    return np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))


def silu(x):
    return x / (1 + np.exp(-x))


def cplx(rng, *shape):
    return rng.standard_normal(shape) + 1j * rng.standard_normal(shape)


def brute_force(u, dt_raw, A, Bm, Cm, z, dt_bias, Dskip, reset, h0):
    Bt, D, L = u.shape
    out = np.zeros((Bt, D, L))
    for b in range(Bt):
        for d in range(D):
            delta = softplus(dt_raw[b, d] + dt_bias[d])
            a = np.exp(delta[:, None] * A[d][None, :])          # (L, N)
            if reset is not None:
                a[reset[b] != 0] = 0.0                           # a reset at r clears h_{r-1}
            for t in range(L):
                acc = np.zeros(A.shape[1], dtype=complex)
                acc += np.prod(a[:t + 1], axis=0) * h0[b, d]
                for s in range(t + 1):
                    acc += np.prod(a[s + 1:t + 1], axis=0) * delta[s] * Bm[b, s] * u[b, d, s]
                y = np.sum(Cm[b, t] * acc).real + Dskip[d] * u[b, d, t]
                out[b, d, t] = y * silu(z[b, d, t])
    return out


def test_brute_force_materialised_form():
    rng = np.random.default_rng(11)
    Bt, D, L, N = 2, 3, 14, 4
    u, dt_raw, z = (rng.standard_normal((Bt, D, L)) for _ in range(3))
    A = -rng.uniform(0.1, 1.0, (D, N)) + 1j * rng.uniform(-3, 3, (D, N))
    Bm, Cm, h0 = cplx(rng, Bt, L, N), cplx(rng, Bt, L, N), cplx(rng, Bt, D, N)
    dt_bias, Dskip = rng.standard_normal(D) - 1, rng.standard_normal(D)
    reset = np.zeros((Bt, L), np.uint8)
    reset[0, 5] = reset[1, 0] = reset[1, 9] = 1
    got = oracle.scan_cplx(u, dt_raw, A, Bm, Cm, z=z, dt_bias=dt_bias, Dskip=Dskip, reset=reset, h0=h0)
    ref = brute_force(u, dt_raw, A, Bm, Cm, z, dt_bias, Dskip, reset, h0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_real_case_is_the_real_scan():
    rng = np.random.default_rng(12)
    Bt, D, L, N = 2, 5, 60, 8
    u, dt_raw, z = (rng.standard_normal((Bt, D, L)) for _ in range(3))
    A = -rng.uniform(0.5, 4, (D, N))
    Bm, Cm, h0 = rng.standard_normal((Bt, L, N)), rng.standard_normal((Bt, L, N)), rng.standard_normal((Bt, D, N))
    dt_bias, Dskip = rng.standard_normal(D), rng.standard_normal(D)
    reset = (rng.uniform(size=(Bt, L)) < 0.05).astype(np.uint8)
    got, hl = oracle.scan_cplx(u, dt_raw, A + 0j, Bm + 0j, Cm + 0j, z=z, dt_bias=dt_bias, Dskip=Dskip,
                               reset=reset, h0=h0 + 0j, want_h_last=True)
    ref, rhl = oracle.scan(u, dt_raw, A, Bm, Cm, z=z, dt_bias=dt_bias, Dskip=Dskip, reset=reset, h0=h0,
                           want_h_last=True)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hl.real, rhl, rtol=1e-13, atol=1e-13)
    assert np.all(hl.imag == 0)


def test_constant_inputs_geometric_series():
    # Constant delta, B, C, u: h_t = a^(t+1) h0 + b (1 - a^(t+1)) / (1 - a) with
    # a = exp(delta A), b = delta B u.
    L, N = 3000, 5
    delta = 0.03
    x = np.log(np.expm1(delta))              # softplus(x) = delta
    A = (-0.5 + 1j * np.arange(N))[None, :]  # the S4D-Lin initialisation
    Bv = np.array([1 + 2j, -0.5 + 0.1j, 0.3j, 2.0, -1 - 1j])
    Cv = np.array([0.5 - 1j, 1j, 2.0, -0.7 + 0.2j, 1 + 1j])
    h0 = np.array([1j, -2.0, 0.5 + 0.5j, 0.0, 3 - 1j])[None, None, :]
    uval, dsk = 0.8, 0.25
    u = np.full((1, 1, L), uval)
    dt_raw = np.full((1, 1, L), x)
    Bm = np.broadcast_to(Bv, (1, L, N))
    Cm = np.broadcast_to(Cv, (1, L, N))
    got, hl = oracle.scan_cplx(u, dt_raw, A, Bm, Cm, Dskip=np.array([dsk]), h0=h0, want_h_last=True)
    a = np.exp(delta * A[0])
    b = delta * Bv * uval
    t = np.arange(L)[:, None]
    h = a ** (t + 1) * h0[0, 0] + b * (1 - a ** (t + 1)) / (1 - a)
    ref = (h * Cv).sum(axis=1).real + dsk * uval
    np.testing.assert_allclose(got[0, 0], ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hl[0, 0], h[-1], rtol=1e-10, atol=1e-12)


def test_pure_rotation_fixes_the_phase_sign():
    # Re A = 0 and B = 0: h_t = exp(i w S_t) h0, S_t = sum_{r<=t} delta_r.
    rng = np.random.default_rng(13)
    L, w = 200, 1.7
    dt_raw = rng.standard_normal((1, 2, L))
    A = np.array([[1j * w], [1j * w]])
    Bm = np.zeros((1, L, 1), complex)
    Cm = np.ones((1, L, 1), complex)
    Cm_i = np.full((1, L, 1), 1j)
    h0 = np.ones((1, 2, 1), complex)
    u = rng.standard_normal((1, 2, L))
    S = np.cumsum(softplus(dt_raw[0]), axis=1)
    out = oracle.scan_cplx(u, dt_raw, A, Bm, Cm, h0=h0)
    np.testing.assert_allclose(out[0], np.cos(w * S), atol=1e-12)
    out = oracle.scan_cplx(u, dt_raw, A, Bm, Cm_i, h0=h0)
    np.testing.assert_allclose(out[0], -np.sin(w * S), atol=1e-12)    # Re(i e^{i wS}) = -sin(wS)


def test_conjugate_pair_doubles_the_real_part():
    rng = np.random.default_rng(14)
    Bt, D, L = 2, 3, 80
    u, dt_raw = rng.standard_normal((Bt, D, L)), rng.standard_normal((Bt, D, L))
    A1 = -rng.uniform(0.1, 1, (D, 1)) + 1j * rng.uniform(0, 5, (D, 1))
    B1, C1 = cplx(rng, Bt, L, 1), cplx(rng, Bt, L, 1)
    single = oracle.scan_cplx(u, dt_raw, A1, B1, C1)
    pair = oracle.scan_cplx(u, dt_raw, np.concatenate([A1, A1.conj()], 1), np.concatenate([B1, B1.conj()], 2),
                            np.concatenate([C1, C1.conj()], 2))
    np.testing.assert_allclose(pair, 2 * single, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("with_z", [False, True])
def test_decode_steps_reproduce_the_scan(with_z):
    rng = np.random.default_rng(15)
    Bt, D, L, N = 2, 4, 30, 6
    u, dt_raw, z = (rng.standard_normal((Bt, D, L)) for _ in range(3))
    A = -0.5 + 1j * np.arange(N)[None, :].repeat(D, 0)
    Bm, Cm, h0 = cplx(rng, Bt, L, N), cplx(rng, Bt, L, N), cplx(rng, Bt, D, N)
    dt_bias, Dskip = rng.standard_normal(D), rng.standard_normal(D)
    zz = z if with_z else None
    ref, rhl = oracle.scan_cplx(u, dt_raw, A, Bm, Cm, z=zz, dt_bias=dt_bias, Dskip=Dskip, h0=h0,
                                want_h_last=True)
    h = h0
    for t in range(L):
        o, h = oracle.state_update_cplx(h, u[:, :, t], dt_raw[:, :, t], A, Bm[:, t], Cm[:, t],
                                        z=None if zz is None else zz[:, :, t], dt_bias=dt_bias, Dskip=Dskip)
        np.testing.assert_allclose(o, ref[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h, rhl, rtol=1e-12, atol=1e-12)


# ---- exact zero-order hold with a complex state ----

def test_zoh_steps_equal_ode_integration():
    """Each step is the exact solution of h' = A h + B u over delta with B, u held."""
    import scipy.integrate

    rng = np.random.default_rng(21)
    D, L, N = 2, 6, 3
    u = rng.standard_normal((1, D, L))
    dt = rng.standard_normal((1, D, L))
    A = -rng.uniform(0.2, 2.0, (D, N)) + 1j * rng.uniform(-6, 6, (D, N))
    Bm, Cm, h0 = cplx(rng, 1, L, N), cplx(rng, 1, L, N), cplx(rng, 1, D, N)
    out, hl = oracle.scan_cplx(u, dt, A, Bm, Cm, h0=h0, want_h_last=True, zoh=True)
    for d in range(D):
        h = h0[0, d].copy()
        for t in range(L):
            delta = softplus(dt[0, d, t])
            rhs = lambda s, y, t=t: A[d] * y + Bm[0, t] * u[0, d, t]
            h = scipy.integrate.solve_ivp(rhs, (0.0, delta), h, method="DOP853", rtol=1e-12, atol=1e-14).y[:, -1]
            np.testing.assert_allclose(out[0, d, t], np.sum(Cm[0, t] * h).real, rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(hl[0, d], h, rtol=1e-9, atol=1e-11)


def test_zoh_steady_state_and_limits():
    # constant inputs: h -> -B u / A exactly, whatever the step
    D, L, N = 3, 4000, 3
    A = np.array([[-0.5 + 2j, -1.0 - 0.5j, -2.0 + 7j]] * D)
    Bv = np.array([0.3 - 1j, -1.2, 0.7 + 0.4j])
    u = np.full((1, D, L), 1.7)
    dt = np.broadcast_to(np.array([-2.0, 0.0, 1.5])[None, :, None], (1, D, L)).copy()
    _, hl = oracle.scan_cplx(u, dt, A, np.broadcast_to(Bv, (1, L, N)), np.zeros((1, L, N), complex),
                             want_h_last=True, zoh=True)
    np.testing.assert_allclose(hl[0], np.broadcast_to(-Bv * 1.7 / A[0], (D, N)), rtol=1e-11)
    # A = 0 gives the delta B form exactly; a real A gives the real ZOH oracle
    rng = np.random.default_rng(22)
    u, dt = rng.standard_normal((2, 3, 40)), rng.standard_normal((2, 3, 40))
    Bm, Cm = rng.standard_normal((2, 40, 4)), rng.standard_normal((2, 40, 4))
    A0 = np.zeros((3, 4), complex)
    np.testing.assert_array_equal(oracle.scan_cplx(u, dt, A0, Bm + 0j, Cm + 0j, zoh=True),
                                  oracle.scan_cplx(u, dt, A0, Bm + 0j, Cm + 0j, zoh=False))
    Ar = -rng.uniform(0.1, 3, (3, 4))
    np.testing.assert_allclose(oracle.scan_cplx(u, dt, Ar + 0j, Bm + 0j, Cm + 0j, zoh=True),
                               oracle.scan(u, dt, Ar, Bm, Cm, zoh=True), rtol=1e-12, atol=1e-13)
    # small delta A: the coefficient stays accurate (no cancellation in e^{delta A} - 1)
    A_small = np.full((1, 1), -1e-12 + 3e-12j)
    o1 = oracle.scan_cplx(np.ones((1, 1, 3)), np.zeros((1, 1, 3)), A_small, np.ones((1, 3, 1), complex),
                          np.ones((1, 3, 1), complex), zoh=True)
    o0 = oracle.scan_cplx(np.ones((1, 1, 3)), np.zeros((1, 1, 3)), A_small, np.ones((1, 3, 1), complex),
                          np.ones((1, 3, 1), complex), zoh=False)
    np.testing.assert_allclose(o1, o0, rtol=1e-10)
