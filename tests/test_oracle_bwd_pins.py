"""Pins for the oracle's backward pass, independent of its own reverse sweep.

The backward is the gradient of loss = sum(dout * out) + sum(dh_last * h_last).
Each test checks it against something that does not reuse the reverse-sweep
code:
  - central finite differences of the forward oracle (itself pinned by the
    forward tests), element by element for every input on tiny cases, and as
    directional derivatives on multi-hundred-step cases;
  - Euler's identity for homogeneous functions: out and h_last are jointly
    linear in (u, h0), linear in C apart from the skip term, and linear in B
    when h0 = 0, so the gradients' inner products with those inputs must equal
    fixed combinations of the loss;
  - reset isolation: a packed row's gradients equal those of the documents
    scanned on their own.
Random diagonal A, per-channel dt_bias and D, several batch rows and gates are
used so that a transposed index, a dropped term, a wrong sign or a misplaced
reset in the reverse sweep fails at least one test.
"""
import numpy as np
import pytest

import oracle

INPUTS = ["u", "dt_raw", "z", "dt_bias", "A", "Dskip", "Bm", "Cm", "h0"]
GRAD_OF = dict(u="du", dt_raw="d_dt_raw", z="dz", dt_bias="d_dt_bias", A="dA", Dskip="dD",
               Bm="dB", Cm="dC", h0="dh0")


def rand_case(rng, B=2, D=2, L=6, N=3, with_z=True, with_reset=False, with_h0=True):
    c = dict(u=rng.standard_normal((B, D, L)), dt_raw=rng.standard_normal((B, D, L)),
             z=rng.standard_normal((B, D, L)) if with_z else None,
             A=-rng.uniform(0.1, 3.0, size=(D, N)), Bm=rng.standard_normal((B, L, N)),
             Cm=rng.standard_normal((B, L, N)), dt_bias=rng.uniform(-3.0, 1.0, size=D),
             Dskip=rng.standard_normal(D),
             h0=rng.standard_normal((B, D, N)) if with_h0 else None, reset=None)
    if with_reset:
        r = np.zeros((B, L), dtype=np.uint8)
        r[0, 0] = 1           # discards h0 of batch row 0
        r[:, L // 2] = 1      # a document boundary inside every row
        c["reset"] = r
    c["dout"] = rng.standard_normal((B, D, L))
    c["dh_last"] = rng.standard_normal((B, D, N))
    return c


def loss(c):
    out, hl = oracle.scan(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["dt_bias"],
                          Dskip=c["Dskip"], reset=c["reset"], h0=c["h0"], want_h_last=True)
    val = float(np.sum(c["dout"] * out))
    if c["dh_last"] is not None:
        val += float(np.sum(c["dh_last"] * hl))
    return val


def grads(c):
    return oracle.scan_bwd(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], c["dout"], z=c["z"],
                           dt_bias=c["dt_bias"], Dskip=c["Dskip"], reset=c["reset"], h0=c["h0"],
                           dh_last=c["dh_last"])


@pytest.mark.parametrize("with_reset", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_finite_differences_every_element(seed, with_reset):
    rng = np.random.default_rng(100 + seed)
    c = rand_case(rng, with_reset=with_reset)
    g = grads(c)
    for name in INPUTS:
        x = c[name]
        ref = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            eps = 1e-6 * max(1.0, abs(x[idx]))
            keep = x[idx]
            x[idx] = keep + eps
            fp = loss(c)
            x[idx] = keep - eps
            fm = loss(c)
            x[idx] = keep
            ref[idx] = (fp - fm) / (2 * eps)
        got = g[GRAD_OF[name]]
        np.testing.assert_allclose(got, ref, rtol=2e-7, atol=2e-7 * (1 + np.abs(ref).max()),
                                   err_msg=name)


def test_finite_differences_without_gate_h0_or_dh_last():
    rng = np.random.default_rng(7)
    c = rand_case(rng, B=1, D=3, L=5, N=2, with_z=False, with_h0=False)
    c["dh_last"] = None
    g = grads(c)
    assert g["dz"] is None
    for name in ["u", "dt_raw", "A", "Bm", "Cm", "dt_bias", "Dskip"]:
        x = c[name]
        ref = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + 1e-6
            fp = loss(c)
            x[idx] = keep - 1e-6
            fm = loss(c)
            x[idx] = keep
            ref[idx] = (fp - fm) / 2e-6
        np.testing.assert_allclose(g[GRAD_OF[name]], ref, rtol=2e-7, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("with_reset", [False, True])
def test_directional_derivative_long(with_reset):
    """All inputs perturbed together along a random direction, L = 300, N = 16."""
    rng = np.random.default_rng(11)
    c = rand_case(rng, B=2, D=4, L=300, N=16, with_reset=with_reset)
    if with_reset:
        c["reset"] = (rng.uniform(size=(2, 300)) < 0.02).astype(np.uint8)
    g = grads(c)
    dirs = {k: rng.standard_normal(c[k].shape) for k in INPUTS}
    pred = sum(float(np.sum(g[GRAD_OF[k]] * dirs[k])) for k in INPUTS)

    def moved(s):
        m = dict(c)
        for k in INPUTS:
            m[k] = c[k] + s * dirs[k]
        return loss(m)

    eps = 1e-6
    fd = (moved(eps) - moved(-eps)) / (2 * eps)
    assert abs(fd - pred) <= 1e-6 * (1 + abs(pred)), (fd, pred)


@pytest.mark.parametrize("with_reset", [False, True])
def test_homogeneity_identities(with_reset):
    """Euler: for f homogeneous of degree 1 in a group of inputs x, <grad_x f, x> = f."""
    rng = np.random.default_rng(23)
    c = rand_case(rng, B=3, D=8, L=257, N=16, with_reset=with_reset)
    if with_reset:
        c["reset"] = (rng.uniform(size=(3, 257)) < 0.03).astype(np.uint8)
    out, hl = oracle.scan(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["dt_bias"],
                          Dskip=c["Dskip"], reset=c["reset"], h0=c["h0"], want_h_last=True)
    gate = c["z"] / (1 + np.exp(-c["z"]))
    f_out = np.sum(c["dout"] * out)
    f_hl = np.sum(c["dh_last"] * hl)
    skip = np.sum(c["dout"] * gate * c["Dskip"][None, :, None] * c["u"])
    g = grads(c)
    tol = 1e-10 * (abs(f_out) + abs(f_hl) + abs(skip) + 1)
    # (u, h0) jointly: out and h_last are linear in them
    assert abs(np.sum(g["du"] * c["u"]) + np.sum(g["dh0"] * c["h0"]) - (f_out + f_hl)) < tol
    # C: out minus its skip term is linear in C; h_last does not depend on C
    assert abs(np.sum(g["dC"] * c["Cm"]) - (f_out - skip)) < tol
    # D: the skip term is linear in D
    assert abs(np.sum(g["dD"] * c["Dskip"]) - skip) < tol
    # B with h0 = 0: the state, and with it out minus skip and h_last, is linear in B
    c["h0"] = None
    out0, hl0 = oracle.scan(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["dt_bias"],
                            Dskip=c["Dskip"], reset=c["reset"], h0=None, want_h_last=True)
    g0 = grads(c)
    f0 = np.sum(c["dout"] * out0) - skip + np.sum(c["dh_last"] * hl0)
    assert abs(np.sum(g0["dB"] * c["Bm"]) - f0) < 1e-10 * (abs(f0) + 1)


def test_reset_isolates_document_gradients():
    """A packed row's gradients equal those of its documents scanned separately."""
    rng = np.random.default_rng(31)
    L, D, N = 40, 3, 4
    cuts = [0, 9, 10, 27, L]             # documents [0,9), [9,10), [10,27), [27,40)
    c = rand_case(rng, B=1, D=D, L=L, N=N)
    c["reset"] = np.zeros((1, L), dtype=np.uint8)
    c["reset"][0, cuts[:-1]] = 1
    c["dh_last"] = rng.standard_normal((1, D, N))
    g = grads(c)
    assert np.all(g["dh0"] == 0.0)       # the reset at t = 0 discards h0
    acc = dict(dA=0.0, dD=0.0, d_dt_bias=0.0)
    for i, (s, e) in enumerate(zip(cuts[:-1], cuts[1:])):
        last = e == L
        sub = {k: (c[k][..., s:e] if k in ("u", "dt_raw", "z", "dout") else c[k])
               for k in ("u", "dt_raw", "z", "dout", "A", "dt_bias", "Dskip")}
        gs = oracle.scan_bwd(sub["u"], sub["dt_raw"], c["A"], c["Bm"][:, s:e], c["Cm"][:, s:e], sub["dout"],
                             z=sub["z"], dt_bias=c["dt_bias"], Dskip=c["Dskip"], h0=None,
                             dh_last=c["dh_last"] if last else None)
        for k in ("du", "d_dt_raw", "dz"):
            np.testing.assert_allclose(g[k][..., s:e], gs[k], rtol=1e-12, atol=1e-13, err_msg=k)
        for k in ("dB", "dC"):
            np.testing.assert_allclose(g[k][:, s:e], gs[k], rtol=1e-12, atol=1e-13, err_msg=k)
        for k in acc:
            acc[k] = acc[k] + gs[k]
    for k in acc:
        np.testing.assert_allclose(g[k], acc[k], rtol=1e-12, atol=1e-13, err_msg=k)


def test_thread_count_does_not_change_results_beyond_rounding():
    rng = np.random.default_rng(41)
    c = rand_case(rng, B=2, D=16, L=64, N=8, with_reset=True)
    a = oracle.scan_bwd(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], c["dout"], z=c["z"],
                        dt_bias=c["dt_bias"], Dskip=c["Dskip"], reset=c["reset"], h0=c["h0"],
                        dh_last=c["dh_last"], nthreads=1)
    b = oracle.scan_bwd(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], c["dout"], z=c["z"],
                        dt_bias=c["dt_bias"], Dskip=c["Dskip"], reset=c["reset"], h0=c["h0"],
                        dh_last=c["dh_last"], nthreads=4)
    for k in a:
        if a[k] is not None:
            np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-12, err_msg=k)
