"""Benchmark of the selective-scan forward on one MI355X.

One step = one ssm_scan_fwd call over the Mamba-130M-shaped layer workload
(batch 8, 1536 channels, 2048 steps, N = 16; bf16 inputs, float32 state,
arithmetic and output), inputs resident in HBM. Prints one JSON line:

  value        whole-job throughput in scan elements (B*D*L*N) per second over
               the K timed steps (wall clock, synchronised on both sides)
  hbm_gbps     algorithmic HBM bytes per step / time per step
  roofline     the scan kernel against the bound that limits it: the vector
               ALU, whose peak is 256 CUs x 64 lanes x 2.4 GHz = 39.3e12 float32
               lane-operations per second (no packed float32; a transcendental
               counts twice), measured with HIP events on the launch stream;
               `traffic` is the HBM byte count from the rocprofv3 counter runs
               recorded under profiles/ (null when the kernel source changed
               since they were taken)
  cold_cache   the same launch after a 1 GiB write that evicts L2 and MALL
  decode       the single-token decode step (batch 64, 2048 channels, N = 128),
               warm (repeated steps) and with cold caches
  backward     ssm_scan_bwd on the same workload with a random output gradient
               (checkpoint sweep, reverse sweep and reduction, back to back)
  conv_stage   the same forward and backward with the fused causal conv1d
               (width 4) + SiLU input stage, u being the conv input
  zoh          the same forward and backward with the exact zero-order-hold
               input coefficient (e^{delta A} - 1) / A in place of delta
  complex_state the complex diagonal state (S4D-Lin A) at the same shape:
               forward, forward with the zero-order hold, backward, decode
  sequence_shard one of 8 shards of the long-genomics sequence: its aggregate
               and its scan from a carried state
  cpu_baseline the float64 oracle on the host cores over the same workload,
               whole passes repeated until about 10 s of CPU work

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# Vector ALU issue rate of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic ALU work of the scan in fp32 lane-operations (an FMA is one; a
# transcendental counts the two issue slots it occupies):
#   per (b, d, t, n): exp(delta*A) (2) + delta*A (1) + B*delta*u (1)
#                     + state FMA (1) + C.h FMA (1)                     = 6
#   per (b, d, t):    softplus = exp, log (4) + 5 ops; silu = exp, rcp (4)
#                     + 2 ops; delta*u, D*u + y, gate (3)               = 18
OPS_PER_ELEMENT = 6.0
OPS_PER_ROW_STEP = 18.0
# Backward, per (b, d, t, n): the forward step again (6) and the adjoint:
# g FMA, a*h, g*(a*h), dA FMA, S1 FMA, S2 FMA, Y FMA, g*delta*u, dy*h,
# a*g (10) = 16; per (b, d, t): softplus (9), sigmoid (4), silu and silu' (8),
# du, d dt_raw, dz, dD and d dt_bias (8) = 29.
BWD_OPS_PER_ELEMENT = 16.0
BWD_OPS_PER_ROW_STEP = 29.0
SCAN_SOURCES = ["selective_state_space_67_amd/csrc/scan_fwd_kernel.h",
                "selective_state_space_67_amd/csrc/scan_fwd.hip",
                "selective_state_space_67_amd/csrc/device_math.h"]
COUNTERS_DIR = os.path.join(ROOT, "profiles")


def scan_source_hash() -> str:
    h = hashlib.sha256()
    for p in SCAN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary of this
    workload, if the kernel source is unchanged since it was taken."""
    path = os.path.join(COUNTERS_DIR, "scan_counters_%s.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != scan_source_hash():
        return None
    return float(t.group(1))


def algorithmic_bytes(B, D, L, N, s_in, s_out, reset=False, h0=False, h_last=False):
    """HBM bytes the scan must move: u, dt_raw, z, B, C, A, D, dt_bias, [reset], out, [h0, h_last]."""
    b = 3 * B * D * L * s_in + 2 * B * L * N * s_in + 4 * D * N + 8 * D + B * D * L * s_out
    if reset:
        b += B * L
    if h0:
        b += 4 * B * D * N
    if h_last:
        b += 4 * B * D * N
    return b


def backward_bytes(B, D, L, N, s_in, s_grad, reset=False):
    """HBM bytes the backward must move: u, dt_raw, z, dout and B, C read once;
    du, d dt_raw, dz and dB, dC written once; the small parameters and their
    gradients."""
    return (4 * B * D * L * s_in + 2 * B * L * N * s_in + 3 * B * D * L * s_grad + 2 * B * L * N * 4
            + 2 * (4 * D * N + 8 * D) + (B * L if reset else 0))


def decode_bytes(B, D, N, s_in, s_out):
    return 8 * B * D * N + 3 * B * D * s_in + 2 * B * N * s_in + 4 * D * N + 8 * D + B * D * s_out


def percentile(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--workload", default="mamba130m-layer",
                    help="workload name: mamba130m-layer (the default and the headline); tiny-fp32, "
                         "mamba2.8b-layer, long-genomics and packed-docs-n128 print their own line for reference")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the launches timed after an L2/MALL-evicting write")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (for counter calibration runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_67_amd import load_library
    from selective_state_space_67_amd import binding
    from selective_state_space_67_amd import workloads as wl

    load_library()
    dev = torch.device("cuda:0")
    cfg = wl.workload(args.workload)
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    x = wl.workload_inputs(args.workload)
    t = {k: wl.to_torch(x[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset")}
    out = torch.empty((B, D, L), dtype=torch.float32, device=dev)
    call = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                Dskip=t["Dskip"], z=t["z"], reset=t["reset"], out=out)
    s_in = 4 if cfg["dtype"] == wl.F32 else 2
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # K timed steps, back to back.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps

    # Per-launch kernel time with HIP events on the launch stream.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    launch_s = float(np.mean(launch_ms)) / 1e3

    # Cold caches: a 1 GiB write before each launch, outside the timed events.
    cold = []
    if not args.no_cold:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for i in range(min(args.steps, 50)):
            scratch.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            cold.append(e0.elapsed_time(e1))
        del scratch

    if args.copy_calibration:
        src = torch.ones(1 << 27, dtype=torch.float32, device=dev)   # 512 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    elements = B * D * L * N
    abytes = algorithmic_bytes(B, D, L, N, s_in, 4, reset=x["reset"] is not None)
    ops = OPS_PER_ELEMENT * elements + OPS_PER_ROW_STEP * B * D * L
    achieved = ops / launch_s / 1e12
    traffic = recorded_traffic(cfg["name"])

    # Decode step at its workload size.
    y = wl.decode_inputs()
    td = {k: wl.to_torch(y[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    hd = torch.from_numpy(y["h"]).to(dev)
    od = torch.empty((y["h"].shape[0], y["h"].shape[1]), dtype=torch.float32, device=dev)

    dec = binding.prepare_state_update(hd, td["u"], td["dt_raw"], td["A"], td["Bm"], td["Cm"],
                                       dt_bias=td["dt_bias"], Dskip=td["Dskip"], z=td["z"], out=od)
    for _ in range(5):
        dec()
    # back-to-back launches between one event pair: the mean GPU time per step
    dsteps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(dsteps):
        dec()
    e1.record(stream)
    e1.synchronize()
    dms = [e0.elapsed_time(e1) / dsteps]
    Bd, Dd, Nd = y["h"].shape
    dbytes = decode_bytes(Bd, Dd, Nd, 2, 4)
    dsec = float(np.median(dms)) / 1e3
    # Repeated steps keep the 67 MB state in the last-level cache; a decode
    # loop over many layers would not. Cold: a 1 GiB write before each launch.
    dcold = []
    if not args.no_cold:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for i in range(min(args.steps, 50)):
            scratch.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dec()
            e1.record(stream)
            e1.synchronize()
            dcold.append(e0.elapsed_time(e1))
        del scratch

    # A launch-bound decode loop (one sequence of the Mamba-130M layer shape,
    # 32 tokens): prepared launches one by one, against the same 32 steps
    # captured once in a HIP graph and replayed.
    y1 = wl.make_decode_inputs(1, 1536, 16, dtype=wl.BF16, seed=5)
    t1 = {k: wl.to_torch(y1[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    h1 = torch.from_numpy(y1["h"]).to(dev)
    loop = binding.prepare_state_update(h1, t1["u"], t1["dt_raw"], t1["A"], t1["Bm"], t1["Cm"], dt_bias=t1["dt_bias"],
                                        Dskip=t1["Dskip"], z=t1["z"])
    tokens = 32

    def eager_loop():
        for _ in range(tokens):
            loop()

    for _ in range(3):
        eager_loop()
    torch.cuda.synchronize()
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    l0.record(stream)
    for _ in range(10):
        eager_loop()
    l1.record(stream)
    l1.synchronize()
    eager_tok = l0.elapsed_time(l1) / (10 * tokens) / 1e3
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        gl = binding.prepare_state_update(h1, t1["u"], t1["dt_raw"], t1["A"], t1["Bm"], t1["Cm"],
                                          dt_bias=t1["dt_bias"], Dskip=t1["Dskip"], z=t1["z"])
        gl()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gcap = binding.prepare_state_update(h1, t1["u"], t1["dt_raw"], t1["A"], t1["Bm"], t1["Cm"],
                                            dt_bias=t1["dt_bias"], Dskip=t1["Dskip"], z=t1["z"])
        for _ in range(tokens):
            gcap()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    l0.record(stream)
    for _ in range(10):
        graph.replay()
    l1.record(stream)
    l1.synchronize()
    graph_tok = l0.elapsed_time(l1) / (10 * tokens) / 1e3
    del graph, gcap, gl, loop, t1, h1, y1

    # Backward pass on the same workload.
    rng = np.random.default_rng(1234)
    dout = wl.to_torch(wl.store(rng.standard_normal((B, D, L)), cfg["dtype"]), dev)
    bwd = binding.prepare_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dout, dt_bias=t["dt_bias"],
                                   Dskip=t["Dskip"], z=t["z"], reset=t["reset"])
    for _ in range(3):
        bwd()
    bsteps = max(5, min(args.steps, 20))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(bsteps):
        bwd()
    e1.record(stream)
    e1.synchronize()
    bsec = e0.elapsed_time(e1) / bsteps / 1e3
    bbytes = backward_bytes(B, D, L, N, s_in, 4, reset=x["reset"] is not None)
    bops = BWD_OPS_PER_ELEMENT * elements + BWD_OPS_PER_ROW_STEP * B * D * L

    # Fused conv1d (width 4) + SiLU input stage, forward and backward.
    rc = np.random.default_rng(4321)
    cw = torch.from_numpy((rc.standard_normal((D, 4)) * 0.5).astype(np.float32)).to(dev)
    cb = torch.from_numpy((rc.standard_normal(D) * 0.2).astype(np.float32)).to(dev)
    fconv = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                 Dskip=t["Dskip"], z=t["z"], reset=t["reset"], conv_w=cw, conv_b=cb)
    bconv = binding.prepare_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dout, dt_bias=t["dt_bias"],
                                     Dskip=t["Dskip"], z=t["z"], reset=t["reset"], conv_w=cw, conv_b=cb)

    def timed(fn, n):
        for _ in range(3):
            fn()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(n):
            fn()
        s1.record(stream)
        s1.synchronize()
        return s0.elapsed_time(s1) / n / 1e3

    csec_f = timed(fconv, max(5, min(args.steps, 50)))
    csec_b = timed(bconv, bsteps)
    del fconv, bconv

    # Exact zero-order hold.
    fzoh = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                Dskip=t["Dskip"], z=t["z"], reset=t["reset"], zoh=True)
    bzoh = binding.prepare_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dout, dt_bias=t["dt_bias"],
                                    Dskip=t["Dskip"], z=t["z"], reset=t["reset"], zoh=True)
    zsec_f = timed(fzoh, max(5, min(args.steps, 50)))
    zsec_b = timed(bzoh, bsteps)
    del bwd, dout, fzoh, bzoh

    # Complex diagonal state (S4D-Lin A = -1/2 + i n) at the same shape, and its decode step.
    xc = wl.make_cplx_inputs(B, D, L, N, cfg["dtype"], seed=cfg["seed"], dt_lo=cfg["dt_lo"],
                             dt_hi=cfg["dt_hi"], packed=cfg["packed"])
    tc = {k: wl.to_torch(xc[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset")}
    fcx = binding.prepare_scan(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], dt_bias=tc["dt_bias"],
                               Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True)
    xsec_f = timed(fcx, max(5, min(args.steps, 30)))
    fcz = binding.prepare_scan(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], dt_bias=tc["dt_bias"],
                               Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True, zoh=True)
    xsec_z = timed(fcz, max(5, min(args.steps, 30)))
    doutc = wl.to_torch(wl.store(np.random.default_rng(4242).standard_normal((B, D, L)), cfg["dtype"]), dev)
    bcx = binding.prepare_scan_bwd(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], doutc, dt_bias=tc["dt_bias"],
                                   Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True)
    xsec_b = timed(bcx, bsteps)
    bcz = binding.prepare_scan_bwd(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], doutc, dt_bias=tc["dt_bias"],
                                   Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True, zoh=True)
    xsec_bz = timed(bcz, bsteps)
    del fcx, fcz, bcx, bcz, doutc, tc, xc
    yc = wl.make_cplx_decode_inputs(Bd, Dd, Nd, wl.BF16, seed=5)
    tdc = {k: wl.to_torch(yc[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    hdc = torch.from_numpy(yc["h"]).to(dev)
    dcx = binding.prepare_state_update(hdc, tdc["u"], tdc["dt_raw"], tdc["A"], tdc["Bm"], tdc["Cm"],
                                       dt_bias=tdc["dt_bias"], Dskip=tdc["Dskip"], z=tdc["z"], complex_state=True)
    xsec_d = timed(dcx, 50)
    # state (B, D, N, 2) read and written, plus the per-row inputs, complex B, C and A
    xdbytes = 16 * Bd * Dd * Nd + 3 * Bd * Dd * 2 + 2 * Bd * Nd * 2 * 2 + 8 * Dd * Nd + 8 * Dd + Bd * Dd * 4
    del dcx, tdc, hdc, yc

    # One GPU's share of the long-genomics sequence split 8 ways: the shard's
    # aggregate (what the other shards need) and its scan from a carried state.
    c3 = wl.workload("long-genomics")
    Ls = c3["L"] // 8
    xs = wl.make_scan_inputs(c3["B"], c3["D"], Ls, c3["N"], c3["dtype"], seed=3, dt_lo=c3["dt_lo"], dt_hi=c3["dt_hi"])
    ts = {k: wl.to_torch(xs[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    h0s = torch.zeros((c3["B"], c3["D"], c3["N"]), dtype=torch.float32, device=dev)
    fsh = binding.prepare_scan(ts["u"], ts["dt_raw"], ts["A"], ts["Bm"], ts["Cm"], dt_bias=ts["dt_bias"],
                               Dskip=ts["Dskip"], z=ts["z"], h0=h0s)
    Pa = torch.empty_like(h0s)
    Ha = torch.empty_like(h0s)
    agg = binding.prepare_aggregate(ts["u"], ts["dt_raw"], ts["A"], ts["Bm"], dt_bias=ts["dt_bias"], P=Pa, H=Ha)
    ssec_a = timed(agg, 20)
    ssec_f = timed(fsh, 20)
    shard_elems = c3["B"] * c3["D"] * Ls * c3["N"]
    del fsh, agg, ts, xs, h0s, Pa, Ha

    result = {
        # value is the element rate; the achieved HBM rate and its fraction of
        # peak are hbm_gbps and hbm_frac_of_peak below
        "metric": "selective-scan elements/s (B\u00b7D\u00b7L\u00b7N) and achieved HBM GB/s vs peak, 1 GPU",
        "value": elements / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s scan: B=%d D=%d L=%d N=%d, %s u/dt/z/B/C, fp32 A/D/dt_bias/state/out, "
                               "silu gate, %s" % (cfg["name"], B, D, L, N, cfg["dtype"],
                                                  "document resets" if cfg["packed"] else "no reset"),
                   "global_batch": B, "seq_len": L, "d_inner": D, "d_state": N, "parallelism": "none"},
        "hbm_gbps": abytes / wall / 1e9,
        "hbm_frac_of_peak": abytes / wall / 1e9 / HBM_PEAK_GBPS,
        "roofline": {
            "kernel": "scan_kernel<NPL=%d, %s, %s>" % (max(1, (N + 15) // 16), cfg["dtype"],
                                                       "reset" if cfg["packed"] else "no reset"),
            "bound": "alu",
            "achieved": achieved,
            "peak": ALU_PEAK_TOPS,
            "unit": "TOP/s (fp32 VALU lane-ops; transcendental = 2)",
            "frac": achieved / ALU_PEAK_TOPS,
            "traffic": traffic,
            "launch_ms_mean": launch_s * 1e3,
            "launch_ms_median": float(np.median(launch_ms)), "launch_ms_p10": percentile(launch_ms, 10),
            "launch_ms_p90": percentile(launch_ms, 90),
            "algorithmic_bytes": abytes,
            "algorithmic_ops": ops,
            "hbm_gbps_at_launch_time": abytes / launch_s / 1e9,
        },
        "cold_cache": None if not cold else {
            "launch_ms_median": float(np.median(cold)), "launch_ms_p10": percentile(cold, 10),
            "launch_ms_p90": percentile(cold, 90), "hbm_gbps": abytes / (float(np.median(cold)) / 1e3) / 1e9},
        "decode": {"workload": "state update B=64 D=2048 N=128, bf16 inputs, fp32 state",
                   "note": "launch_ms_mean / hbm_gbps: steps repeated on one state, which can stay in the "
                           "last-level cache; cold_cache: the state read from HBM, as in a model whose layers' "
                           "states do not fit the caches",
                   "launch_ms_mean": dsec * 1e3, "algorithmic_bytes": dbytes,
                   "hbm_gbps": dbytes / dsec / 1e9, "hbm_frac": dbytes / dsec / 1e9 / HBM_PEAK_GBPS,
                   "cold_cache": None if not dcold else {
                       "launch_ms_median": float(np.median(dcold)),
                       "hbm_gbps": dbytes / (float(np.median(dcold)) / 1e3) / 1e9,
                       "hbm_frac": dbytes / (float(np.median(dcold)) / 1e3) / 1e9 / HBM_PEAK_GBPS}},
        "decode_loop": {"workload": "32 decode steps of one sequence, B=1 D=1536 N=16, bf16 inputs",
                        "eager_us_per_token": eager_tok * 1e6, "hip_graph_us_per_token": graph_tok * 1e6},
        "backward": {"workload": "ssm_scan_bwd on the same inputs, %s dout, fp32 gradients" % cfg["dtype"],
                     "ms_per_call": bsec * 1e3, "elements_per_s": elements / bsec,
                     "algorithmic_bytes": bbytes, "hbm_gbps": bbytes / bsec / 1e9,
                     "algorithmic_ops": bops, "alu_frac": bops / bsec / 1e12 / ALU_PEAK_TOPS,
                     "vs_forward": bsec / launch_s},
        "conv_stage": {"workload": "the same scan with u = silu(causal depthwise conv1d of width 4 + bias)",
                       "fwd_ms": csec_f * 1e3, "fwd_vs_plain_forward": csec_f / launch_s,
                       "fwd_elements_per_s": elements / csec_f, "bwd_ms": csec_b * 1e3,
                       "bwd_vs_plain_backward": csec_b / bsec,
                       "hbm_bytes_saved_by_fusion": B * D * L * (s_in + 4)},
        "zoh": {"workload": "the same scan with Bbar = (e^{delta A} - 1) / A * B",
                "fwd_ms": zsec_f * 1e3, "fwd_vs_plain_forward": zsec_f / launch_s,
                "fwd_elements_per_s": elements / zsec_f, "bwd_ms": zsec_b * 1e3,
                "bwd_vs_plain_backward": zsec_b / bsec},
        "complex_state": {"workload": "the same shape with a complex diagonal state: A = -1/2 + i n (S4D-Lin), "
                                      "complex B, C (re, im pairs), y = Re(C h)",
                          "fwd_ms": xsec_f * 1e3, "fwd_vs_plain_forward": xsec_f / launch_s,
                          "fwd_elements_per_s": elements / xsec_f,
                          "zoh_fwd_ms": xsec_z * 1e3,
                          "bwd_ms": xsec_b * 1e3, "bwd_vs_complex_forward": xsec_b / xsec_f,
                          "bwd_elements_per_s": elements / xsec_b, "zoh_bwd_ms": xsec_bz * 1e3,
                          "decode_workload": "state update B=64 D=2048 N=128 complex, bf16 inputs, fp32 state",
                          "decode_ms": xsec_d * 1e3, "decode_algorithmic_bytes": xdbytes,
                          "decode_hbm_gbps": xdbytes / xsec_d / 1e9},
        "sequence_shard": {"workload": "one of 8 shards of the long-genomics sequence: B=1 D=256 L=%d N=16, "
                                       "bf16; the all-gather and fold of the aggregates between devices is "
                                       "not built" % Ls,
                           "aggregate_ms": ssec_a * 1e3, "scan_from_carried_state_ms": ssec_f * 1e3,
                           "elements_per_s": shard_elems / (ssec_a + ssec_f)},
    }

    if not args.no_cpu:
        import oracle

        # The whole workload, every row, through the oracle (inputs widened to
        # float64 before the clock starts).
        w = wl.widen
        rows = np.arange(B * D)
        rb, rd = rows // D, rows % D
        u64, dt64, z64 = (w(x[k]).reshape(B * D, L) for k in ("u", "dt_raw", "z"))
        Bm64, Cm64 = w(x["Bm"]), w(x["Cm"])
        threads = oracle.max_threads()

        def run_oracle():
            return oracle.scan_rows(rb, rd, u64, dt64, x["A"], Bm64, Cm64, z_rows=z64, dt_bias=x["dt_bias"],
                                    Dskip=x["Dskip"], reset=x["reset"])

        # Whole-workload passes until about 10 s of CPU work (at most 200).
        c0 = time.perf_counter()
        ref = run_oracle()
        reps = 1
        while time.perf_counter() - c0 < 10.0 and reps < 200:
            run_oracle()
            reps += 1
        total = time.perf_counter() - c0
        csec = total / reps
        got = out.reshape(B * D, L).cpu().numpy().astype(np.float64)
        tol = 1e-5 if cfg["dtype"] == wl.F32 else 2e-3
        margin = float(np.max(np.abs(got - ref) / (tol * (1.0 + np.abs(ref)))))
        result["cpu_baseline"] = {"value": elements / csec, "unit": "elements/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": "the full workload (all %d rows x %d steps x %d states), "
                                            "float64, OpenMP over rows; %d passes, %.2f s each, %.1f s in all"
                                            % (B * D, L, N, reps, csec, total)}
        result["parity_vs_oracle"] = {"rows": int(B * D), "max_err_over_bound": margin,
                                      "bound": "%g*(1+|ref|)" % tol}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
