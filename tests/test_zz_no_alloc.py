"""The allocation-free forward entry point (ssm_scan_fwd_noalloc) against
ssm_scan_fwd through the C-ABI: same inputs, same results.

Three calls in a row on one GPU, each smaller than the one before, all of
them split into pieces so that the library's scratch carries the pieces'
aggregates (the second and third calls find the previous call's contents
there). Each result must equal ssm_scan_fwd's bit for bit (the same kernels
run on the same inputs) and lie within the oracle bound of its input type.
"""
import sys

import numpy as np
import pytest

from selective_state_space_67_amd import workloads as wl

from gpu_helpers import assert_close, oracle_full

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_67_amd import load_library

    load_library()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def run_both(x, num_segments, h0=None, cplx=False):
    import torch

    from selective_state_space_67_amd import ssm_scan_fwd, ssm_scan_fwd_noalloc, ssm_scan_workspace_size

    dev = torch.device("cuda:0")
    t = {k: wl.to_torch(x[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset")}
    Bt, D, L = x["u"].shape
    N = x["A"].shape[1]
    c2 = (2,) if cplx else ()
    h0_t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, np.float32)).to(dev)
    ws = ssm_scan_workspace_size(t["u"], t["A"], num_segments=num_segments) if not cplx else None
    out_ref = torch.empty((Bt, D, L), dtype=torch.float32, device=dev)
    hl_ref = torch.empty((Bt, D, N) + c2, dtype=torch.float32, device=dev)
    ssm_scan_fwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"],
                 reset=t["reset"], h0=h0_t, out=out_ref, h_last=hl_ref, num_segments=num_segments,
                 complex_state=cplx)
    out = torch.full((Bt, D, L), float("nan"), dtype=torch.float32, device=dev)
    hl = torch.full((Bt, D, N) + c2, float("nan"), dtype=torch.float32, device=dev)
    ssm_scan_fwd_noalloc(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], out=out, dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=t["z"], reset=t["reset"], h0=h0_t, h_last=hl,
                         num_segments=num_segments, complex_state=cplx)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), hl.cpu().numpy(), out_ref.cpu().numpy(), hl_ref.cpu().numpy(), ws)


def test_noalloc_matches_the_forward_on_consecutive_calls():
    import oracle

    # 1: bf16, 32 channels x 20000 steps; the planner splits the sequence itself
    x = wl.make_scan_inputs(1, 32, 20000, 16, dtype=wl.BF16, seed=61)
    log("no-alloc call 1: 1 x 32 x 20000, N = 16, bf16, automatic split")
    out, hl, out_ref, hl_ref, ws = run_both(x, 0)
    assert ws > 0, "this case must split the sequence"
    np.testing.assert_array_equal(out, out_ref)
    np.testing.assert_array_equal(hl, hl_ref)
    assert_close(out, oracle_full(x), wl.BF16)

    # 2: smaller, float32, resets and an initial state, 5 pieces
    x = wl.make_scan_inputs(2, 20, 3000, 16, dtype=wl.F32, seed=62)
    x["reset"] = wl.doc_resets(np.random.default_rng(63), 2, 3000, lo=200, hi=900)
    h0 = np.random.default_rng(64).standard_normal((2, 20, 16)).astype(np.float32)
    log("no-alloc call 2: 2 x 20 x 3000, N = 16, float32, resets, h0, 5 pieces")
    out, hl, out_ref, hl_ref, ws = run_both(x, 5, h0=h0)
    assert ws > 0
    np.testing.assert_array_equal(out, out_ref)
    np.testing.assert_array_equal(hl, hl_ref)
    ref, hl_o = oracle_full(x, h0=h0, want_h_last=True)
    assert_close(out, ref, wl.F32)
    assert_close(hl, hl_o, wl.F32, what="h_last")

    # 3: smaller still, the complex diagonal state, 3 pieces
    xc = wl.make_cplx_inputs(1, 16, 600, 16, wl.F32, seed=65, dt_lo=1e-3, dt_hi=1e-2)
    log("no-alloc call 3: 1 x 16 x 600, N = 16 complex, float32, 3 pieces")
    out, hl, out_ref, hl_ref, _ = run_both(xc, 3, cplx=True)
    np.testing.assert_array_equal(out, out_ref)
    np.testing.assert_array_equal(hl, hl_ref)
    w = wl.widen
    ref = oracle.scan_cplx(w(xc["u"]), w(xc["dt_raw"]), wl.as_complex(xc["A"]), wl.as_complex(xc["Bm"]),
                           wl.as_complex(xc["Cm"]), z=w(xc["z"]), dt_bias=xc["dt_bias"], Dskip=xc["Dskip"])
    assert np.all(np.isfinite(out))
    # steps of at most 1e-2 keep the decay's phase error small at N = 16: the
    # float32 bound with a tenfold margin for it
    assert np.max(np.abs(out - ref) / (1.0 + np.abs(ref))) < 1e-4
