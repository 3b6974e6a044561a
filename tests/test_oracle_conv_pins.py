"""Pins for the oracle's causal conv1d + SiLU input stage and its backward.

The conv stage is checked against two library routines (numpy.convolve and
torch's conv1d with left padding K-1, in float64 on the CPU), a closed form for
K = 1, reset isolation, split/resume through the conv state, decode-step
equivalence, and central finite differences of the whole scan for the
gradients of the conv input, weights, bias and initial state.
"""
import numpy as np
import pytest

import oracle


def case(rng, B=2, D=3, L=24, N=3, K=4, reset=False):
    c = dict(x=rng.standard_normal((B, D, L)), dt=rng.standard_normal((B, D, L)), z=rng.standard_normal((B, D, L)),
             A=-rng.uniform(0.1, 2.0, size=(D, N)), Bm=rng.standard_normal((B, L, N)),
             Cm=rng.standard_normal((B, L, N)), bias=rng.uniform(-3, 0, size=D), Dsk=rng.standard_normal(D),
             w=rng.standard_normal((D, K)) * 0.7, cb=rng.standard_normal(D) * 0.3,
             cst=rng.standard_normal((B, D, K - 1)), reset=None)
    if reset:
        r = np.zeros((B, L), np.uint8)
        r[:, L // 3] = 1
        r[0, 0] = 1
        r[1, L - 2] = 1
        c["reset"] = r
    return c


def silu(p):
    return p / (1 + np.exp(-p))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_matches_numpy_convolve(K):
    rng = np.random.default_rng(K)
    x = rng.standard_normal((2, 3, 50))
    w = rng.standard_normal((3, K))
    b = rng.standard_normal(3)
    u = oracle.conv_silu(x, w, bias=b)
    for i in range(2):
        for d in range(3):
            pre = np.convolve(x[i, d], w[d, ::-1])[:50] + b[d]   # library convolution (flips its kernel)
            np.testing.assert_allclose(u[i, d], silu(pre), rtol=1e-13, atol=1e-14)


def test_conv_matches_torch_conv1d_with_state():
    import torch

    rng = np.random.default_rng(9)
    B, D, L, K = 2, 5, 40, 4
    x = rng.standard_normal((B, D, L))
    w = rng.standard_normal((D, K))
    b = rng.standard_normal(D)
    st = rng.standard_normal((B, D, K - 1))
    u, st_out = oracle.conv_silu(x, w, bias=b, state_in=st, want_state=True)
    xt = torch.from_numpy(np.concatenate([st, x], axis=2))
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(b), groups=D)
    np.testing.assert_allclose(u, silu(ref.numpy()), rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(st_out, x[:, :, L - (K - 1):])


def test_width_one_is_pointwise():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 4, 30))
    w = rng.standard_normal((4, 1))
    b = rng.standard_normal(4)
    np.testing.assert_allclose(oracle.conv_silu(x, w, bias=b), silu(w[None, :, 0:1] * x + b[None, :, None]),
                               rtol=1e-14, atol=1e-15)


def test_reset_isolates_documents_in_conv_and_scan():
    rng = np.random.default_rng(5)
    c = case(rng, B=1, L=30)
    cuts = [0, 7, 8, 19, 30]
    reset = np.zeros((1, 30), np.uint8)
    reset[0, cuts[:-1]] = 1
    out = oracle.scan(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["bias"], Dskip=c["Dsk"],
                      reset=reset, conv_w=c["w"], conv_b=c["cb"], conv_state=c["cst"])
    for s, e in zip(cuts[:-1], cuts[1:]):
        part = oracle.scan(c["x"][..., s:e], c["dt"][..., s:e], c["A"], c["Bm"][:, s:e], c["Cm"][:, s:e],
                           z=c["z"][..., s:e], dt_bias=c["bias"], Dskip=c["Dsk"], conv_w=c["w"], conv_b=c["cb"])
        np.testing.assert_allclose(out[..., s:e], part, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("k", [1, 2, 11, 23])
def test_split_resume_through_conv_state(k):
    rng = np.random.default_rng(7)
    c = case(rng)
    kw = dict(z=c["z"], dt_bias=c["bias"], Dskip=c["Dsk"], conv_w=c["w"], conv_b=c["cb"])
    full, hl, cs = oracle.scan(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], h0=None, conv_state=c["cst"],
                               want_h_last=True, want_conv_state=True, **kw)
    a, ha, csa = oracle.scan(c["x"][..., :k], c["dt"][..., :k], c["A"], c["Bm"][:, :k], c["Cm"][:, :k],
                             z=c["z"][..., :k], dt_bias=c["bias"], Dskip=c["Dsk"], conv_w=c["w"], conv_b=c["cb"],
                             conv_state=c["cst"], want_h_last=True, want_conv_state=True)
    b, hb, csb = oracle.scan(c["x"][..., k:], c["dt"][..., k:], c["A"], c["Bm"][:, k:], c["Cm"][:, k:],
                             z=c["z"][..., k:], dt_bias=c["bias"], Dskip=c["Dsk"], conv_w=c["w"], conv_b=c["cb"],
                             h0=ha, conv_state=csa, want_h_last=True, want_conv_state=True)
    np.testing.assert_allclose(np.concatenate([a, b], axis=2), full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hb, hl, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(csb, cs)


def test_decode_steps_reproduce_conv_scan():
    rng = np.random.default_rng(8)
    c = case(rng, L=15)
    ref = oracle.scan(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["bias"], Dskip=c["Dsk"],
                      conv_w=c["w"], conv_b=c["cb"], conv_state=c["cst"])
    h = np.zeros((2, 3, 3))
    st = c["cst"]
    for t in range(15):
        o, h, st = oracle.state_update(h, c["x"][..., t], c["dt"][..., t], c["A"], c["Bm"][:, t], c["Cm"][:, t],
                                       z=c["z"][..., t], dt_bias=c["bias"], Dskip=c["Dsk"], conv_w=c["w"],
                                       conv_b=c["cb"], conv_state=st)
        np.testing.assert_allclose(o, ref[..., t], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("with_reset", [False, True])
def test_finite_differences_conv_inputs(with_reset):
    rng = np.random.default_rng(12 + with_reset)
    c = case(rng, L=14, reset=with_reset)
    dout = rng.standard_normal(c["x"].shape)
    dh_last = rng.standard_normal((2, 3, 3))

    def loss(x, w, cb, cst):
        out, hl = oracle.scan(x, c["dt"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["bias"], Dskip=c["Dsk"],
                              reset=c["reset"], conv_w=w, conv_b=cb, conv_state=cst, want_h_last=True)
        return float(np.sum(dout * out) + np.sum(dh_last * hl))

    g = oracle.scan_bwd(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], dout, z=c["z"], dt_bias=c["bias"],
                        Dskip=c["Dsk"], reset=c["reset"], dh_last=dh_last, conv_w=c["w"], conv_b=c["cb"],
                        conv_state=c["cst"])
    args = dict(x=c["x"], w=c["w"], cb=c["cb"], cst=c["cst"])
    names = dict(x="du", w="dconv_w", cb="dconv_b", cst="dconv_state")
    for name, arr in args.items():
        ref = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + 1e-6
            fp = loss(**args)
            arr[idx] = keep - 1e-6
            fm = loss(**args)
            arr[idx] = keep
            ref[idx] = (fp - fm) / 2e-6
        np.testing.assert_allclose(g[names[name]], ref, rtol=2e-7, atol=2e-7 * (1 + np.abs(ref).max()),
                                   err_msg=name)
