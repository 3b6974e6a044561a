"""Benchmark of the selective-scan forward on one MI355X.

One step = one ssm_scan_fwd call over the Mamba-130M-shaped layer workload
(batch 8, 1536 channels, 2048 steps, N = 16; bf16 inputs, float32 state,
arithmetic and output), inputs resident in HBM. Before each timed launch a
1 GiB read of another buffer evicts the L2 caches and the last-level (MALL)
cache, outside the launch's HIP event pair, so every timed launch reads its
inputs from HBM. (A read leaves the caches holding clean lines; a write would
leave a gigabyte of dirty lines whose write-back the timed launch would pay.)
Prints one JSON line:

  value        elements (B*D*L*N) per second at the median timed launch
  ms_per_step  that median launch time; warm figures (back-to-back launches
               with caches holding the inputs) are reported under "warm"
  roofline     the dominant kernel (the 16-state full pass) against both of
               its ceilings, with HIP events on the launch stream:
                 hbm: algorithmic bytes per launch / mean launch time against
                      8 TB/s (and against the measured device-copy ceiling)
                 alu: float32 vector lane-operations per launch / mean launch
                      time against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz =
                      39.3e12 (no packed float32; a transcendental counts the
                      two issue slots it occupies)
               `bound` is whichever fraction is larger; `traffic` is the HBM
               byte count per launch from the rocprofv3 counter runs recorded
               under profiles/ (null once the kernel source has changed)
  hbm_ceiling  a 1 GiB device copy and a 1 GiB read (sum) on the same GPU
  length_sweep the forward at L = 256 .. 131072 with 2 x 2048 channels
               (device-drawn bf16 inputs): elements/s per L and the number of
               pieces the planner cut the sequence into (a check that the
               cost is linear in L)
  decode       the single-token decode step (batch 64, 2048 channels, N = 128),
               repeated steps and with cold caches
  backward, conv_stage, zoh, complex_state, sequence_shard, decode_loop:
               the other entry points and options at the same shape
  cpu_baseline the float64 oracle on the host cores over the whole workload
               (every row), whole passes repeated for about 10 s, with the CPU
               model, the core count, and a single-thread run of the tiny
               float32 workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workload NAME]
                       [--only forward|decode|backward] [--no-extras]
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
SCAN_SOURCES = ["selective_state_space_67_amd/csrc/scan_fwd_n16.hip",
                "selective_state_space_67_amd/csrc/scan_fwd_kernel.h",
                "selective_state_space_67_amd/csrc/scan_fwd.hip",
                "selective_state_space_67_amd/csrc/device_math.h"]
COUNTERS_DIR = os.path.join(ROOT, "profiles")
EVICT_BYTES = 1 << 30


def scan_source_hash() -> str:
    h = hashlib.sha256()
    for p in SCAN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary of this
    workload, if the kernel source is unchanged since it was taken."""
    path = os.path.join(COUNTERS_DIR, "scan_forward_%s.md" % workload)
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


def kernel_label(N, dtype, packed, L):
    """Name of the kernel the full pass of this workload launches."""
    tiles = [(16, "1, 1"), (32, "1, 2"), (64, "1, 4"), (128, "2, 4"), (256, "4, 4")]
    reset = "reset" if packed else "no reset"
    if N == 16 and L % 2 == 0:
        return "scan16_kernel<%s, %s>" % (dtype, reset)
    tile = next(t for n, t in tiles if N <= n)
    return "scan_kernel<Tile<%s>, %s, %s, full pass>" % (tile, dtype, reset)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class Timer:
    """HIP event pairs on one stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def launches(self, fn, n, evict=None):
        """Per-launch times (ms) of n launches; with `evict`, a cache-evicting
        read of that buffer runs before each launch, outside its event pair."""
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:
            if evict is not None:
                evict.sum()
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        t.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    def mean(self, fn, n, pre=3):
        """Mean time (s) of n back-to-back launches between one event pair."""
        t = self.torch
        for _ in range(pre):
            fn()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(n):
            fn()
        e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n / 1e3


def measure_forward(args, torch, binding, wl, timer, evict):
    dev = torch.device("cuda:0")
    cfg = wl.workload(args.workload)
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    x = wl.workload_inputs(args.workload)
    t = {k: wl.to_torch(x[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset")}
    out = torch.empty((B, D, L), dtype=torch.float32, device=dev)
    call = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                Dskip=t["Dskip"], z=t["z"], reset=t["reset"], out=out)
    s_in = 4 if cfg["dtype"] == wl.F32 else 2
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # K timed steps, each launch after a cache-evicting write (wall clock
    # around the whole loop, synchronised on both sides; one GPU, no barrier)
    w0 = time.perf_counter()
    cold = timer.launches(call, args.steps, evict=evict)
    wall = time.perf_counter() - w0
    # warm: back-to-back launches, the caches holding what the last launch left
    warm_mean = timer.mean(call, args.steps)
    warm = timer.launches(call, min(args.steps, 50))
    elements = B * D * L * N
    return dict(cfg=cfg, x=x, t=t, out=out, call=call, s_in=s_in, cold=cold, wall=wall, warm_mean=warm_mean,
                warm=warm, elements=elements)


def measure_wavefront(torch, binding, timer, f, evict, steps):
    """The same forward through ssm_scan_fwd_wavefront (a DPP wavefront scan of
    the affine pairs inside each 64-step chunk, carry across chunks), timed
    like the headline: cold launches, median."""
    cfg, t = f["cfg"], f["t"]
    if cfg["N"] != 16:
        return None
    out = torch.empty_like(f["out"])
    call = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                Dskip=t["Dskip"], z=t["z"], reset=t["reset"], out=out, wavefront=True)
    for _ in range(3):
        call()
    cold = timer.launches(call, steps, evict=evict)
    torch.cuda.synchronize()
    return dict(cold=cold, out=out)


def hbm_ceiling(torch, timer):
    dev = torch.device("cuda:0")
    src = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_s = timer.mean(lambda: dst.copy_(src), 10)
    read_s = timer.mean(lambda: src.sum(), 10)
    del src, dst
    return {"copy_gbps": 2 * EVICT_BYTES / copy_s / 1e9, "read_gbps": EVICT_BYTES / read_s / 1e9,
            "what": "a 1 GiB device copy (bytes read + written) and a 1 GiB float32 sum (bytes read), "
                    "mean of 10 launches"}


def length_sweep(torch, binding, wl, timer):
    """The forward at several sequence lengths with 2 x 2048 channels, N = 16."""
    from selective_state_space_67_amd import ssm_scan_workspace_size

    dev = torch.device("cuda:0")
    B, D, N = 2, 2048, 16
    res = []
    for L in (256, 1024, 4096, 16384, 65536, 131072):
        x = wl.make_scan_inputs_device(B, D, L, N, dev, seed=99)
        A = torch.from_numpy(x["A"]).to(dev)
        bias = torch.from_numpy(x["dt_bias"]).to(dev)
        Dk = torch.from_numpy(x["Dskip"]).to(dev)
        out = torch.empty((B, D, L), dtype=torch.float32, device=dev)
        call = binding.prepare_scan(x["u"], x["dt_raw"], A, x["Bm"], x["Cm"], dt_bias=bias, Dskip=Dk, z=x["z"],
                                    out=out)
        ws = ssm_scan_workspace_size(x["u"], A)
        pieces = 1 + ws // (2 * B * D * N * 4)
        n = max(3, min(50, int(2e6 // L)))
        sec = timer.mean(call, n)
        res.append({"L": L, "pieces": int(pieces), "us_per_call": sec * 1e6, "elements_per_s": B * D * L * N / sec})
        del x, out, call
    return {"workload": "B=2 D=2048 N=16, bf16 inputs drawn on the device, z and D, no resets; "
                        "mean of back-to-back launches", "points": res}


def measure_decode(torch, binding, wl, timer, evict):
    dev = torch.device("cuda:0")
    y = wl.decode_inputs()
    td = {k: wl.to_torch(y[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    hd = torch.from_numpy(y["h"]).to(dev)
    od = torch.empty((y["h"].shape[0], y["h"].shape[1]), dtype=torch.float32, device=dev)
    dec = binding.prepare_state_update(hd, td["u"], td["dt_raw"], td["A"], td["Bm"], td["Cm"],
                                       dt_bias=td["dt_bias"], Dskip=td["Dskip"], z=td["z"], out=od)
    warm_s = timer.mean(dec, 50, pre=5)
    cold = timer.launches(dec, 50, evict=evict)
    Bd, Dd, Nd = y["h"].shape
    dbytes = decode_bytes(Bd, Dd, Nd, 2, 4)
    cold_s = float(np.median(cold)) / 1e3
    # ceiling: torch's in-place add on a float32 tensor of the state's size
    # (the same state bytes read and written), timed the same way
    probe = torch.zeros_like(hd)
    ceil_s = float(np.median(timer.launches(lambda: probe.add_(1.0), 50, evict=evict))) / 1e3
    del probe
    return {"workload": "state update B=64 D=2048 N=128, bf16 inputs, fp32 state",
            "note": "cold_cache: the state read from HBM (a 1 GiB read before each launch), as in a model whose "
                    "layers' states do not fit the caches; warm: steps repeated on one state, which can stay in "
                    "the last-level cache",
            "algorithmic_bytes": dbytes,
            "cold_cache": {"launch_ms_median": cold_s * 1e3, "launch_ms_p10": percentile(cold, 10),
                           "launch_ms_p90": percentile(cold, 90), "hbm_gbps": dbytes / cold_s / 1e9,
                           "hbm_frac": dbytes / cold_s / 1e9 / HBM_PEAK_GBPS},
            "warm": {"launch_ms_mean": warm_s * 1e3, "hbm_gbps": dbytes / warm_s / 1e9,
                     "hbm_frac": dbytes / warm_s / 1e9 / HBM_PEAK_GBPS},
            "inplace_ceiling": {"what": "torch in-place add on a float32 tensor of the state's size, cold cache "
                                        "like the step (state bytes read and written once)",
                                "launch_ms_median": ceil_s * 1e3, "gbps": 2 * hd.numel() * 4 / ceil_s / 1e9,
                                "step_over_ceiling": cold_s / ceil_s}}


def decode_loop(torch, binding, wl, timer):
    """A launch-bound decode loop (one sequence of the Mamba-130M layer shape,
    32 tokens): prepared launches one by one, against the same 32 steps
    captured once in a HIP graph and replayed."""
    dev = torch.device("cuda:0")
    stream = timer.stream
    y1 = wl.make_decode_inputs(1, 1536, 16, dtype=wl.BF16, seed=5)
    t1 = {k: wl.to_torch(y1[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    h1 = torch.from_numpy(y1["h"]).to(dev)
    tokens = 32

    def prep():
        return binding.prepare_state_update(h1, t1["u"], t1["dt_raw"], t1["A"], t1["Bm"], t1["Cm"],
                                            dt_bias=t1["dt_bias"], Dskip=t1["Dskip"], z=t1["z"])

    loop = prep()

    def eager_loop():
        for _ in range(tokens):
            loop()

    eager_tok = timer.mean(eager_loop, 10) / tokens
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        prep()()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gcap = prep()
        for _ in range(tokens):
            gcap()
    graph_tok = timer.mean(graph.replay, 10) / tokens
    del graph, gcap
    return {"workload": "32 decode steps of one sequence, B=1 D=1536 N=16, bf16 inputs",
            "eager_us_per_token": eager_tok * 1e6, "hip_graph_us_per_token": graph_tok * 1e6}


def measure_backward(torch, binding, wl, timer, f, steps):
    dev = torch.device("cuda:0")
    cfg, t, s_in, elements = f["cfg"], f["t"], f["s_in"], f["elements"]
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    rng = np.random.default_rng(1234)
    dout = wl.to_torch(wl.store(rng.standard_normal((B, D, L)), cfg["dtype"]), dev)
    bwd = binding.prepare_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dout, dt_bias=t["dt_bias"],
                                   Dskip=t["Dskip"], z=t["z"], reset=t["reset"])
    bsteps = max(5, min(steps, 20))
    bsec = timer.mean(bwd, bsteps)
    bbytes = backward_bytes(B, D, L, N, s_in, 4, reset=t["reset"] is not None)
    bops = BWD_OPS_PER_ELEMENT * elements + BWD_OPS_PER_ROW_STEP * B * D * L
    return dout, bsec, {"workload": "ssm_scan_bwd on the same inputs, %s dout, fp32 gradients" % cfg["dtype"],
                        "ms_per_call": bsec * 1e3, "elements_per_s": elements / bsec,
                        "algorithmic_bytes": bbytes, "hbm_gbps": bbytes / bsec / 1e9,
                        "algorithmic_ops": bops, "alu_frac": bops / bsec / 1e12 / ALU_PEAK_TOPS}


def measure_extras(torch, binding, wl, timer, f, dout, bsec, fwd_s, steps):
    dev = torch.device("cuda:0")
    cfg, t, s_in, elements = f["cfg"], f["t"], f["s_in"], f["elements"]
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    bsteps = max(5, min(steps, 20))
    res = {}
    # fused conv1d (width 4) + SiLU input stage, forward and backward
    rc = np.random.default_rng(4321)
    cw = torch.from_numpy((rc.standard_normal((D, 4)) * 0.5).astype(np.float32)).to(dev)
    cb = torch.from_numpy((rc.standard_normal(D) * 0.2).astype(np.float32)).to(dev)
    fconv = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                 Dskip=t["Dskip"], z=t["z"], reset=t["reset"], conv_w=cw, conv_b=cb)
    bconv = binding.prepare_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dout, dt_bias=t["dt_bias"],
                                     Dskip=t["Dskip"], z=t["z"], reset=t["reset"], conv_w=cw, conv_b=cb)
    csec_f = timer.mean(fconv, max(5, min(steps, 50)))
    csec_b = timer.mean(bconv, bsteps)
    res["conv_stage"] = {"workload": "the same scan with u = silu(causal depthwise conv1d of width 4 + bias)",
                         "fwd_ms": csec_f * 1e3, "fwd_vs_plain_forward": csec_f / fwd_s,
                         "fwd_elements_per_s": elements / csec_f, "bwd_ms": csec_b * 1e3,
                         "bwd_vs_plain_backward": csec_b / bsec,
                         "hbm_bytes_saved_by_fusion": B * D * L * (s_in + 4)}
    del fconv, bconv
    # exact zero-order hold
    fzoh = binding.prepare_scan(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                Dskip=t["Dskip"], z=t["z"], reset=t["reset"], zoh=True)
    bzoh = binding.prepare_scan_bwd(t["u"], t["dt_raw"], t["A"], t["Bm"], t["Cm"], dout, dt_bias=t["dt_bias"],
                                    Dskip=t["Dskip"], z=t["z"], reset=t["reset"], zoh=True)
    zsec_f = timer.mean(fzoh, max(5, min(steps, 50)))
    zsec_b = timer.mean(bzoh, bsteps)
    res["zoh"] = {"workload": "the same scan with Bbar = (e^{delta A} - 1) / A * B",
                  "fwd_ms": zsec_f * 1e3, "fwd_vs_plain_forward": zsec_f / fwd_s,
                  "fwd_elements_per_s": elements / zsec_f, "bwd_ms": zsec_b * 1e3,
                  "bwd_vs_plain_backward": zsec_b / bsec}
    del fzoh, bzoh
    # complex diagonal state (S4D-Lin A = -1/2 + i n) at the same shape, and its decode step
    xc = wl.make_cplx_inputs(B, D, L, N, cfg["dtype"], seed=cfg["seed"], dt_lo=cfg["dt_lo"],
                             dt_hi=cfg["dt_hi"], packed=cfg["packed"])
    tc = {k: wl.to_torch(xc[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip", "reset")}
    fcx = binding.prepare_scan(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], dt_bias=tc["dt_bias"],
                               Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True)
    xsec_f = timer.mean(fcx, max(5, min(steps, 30)))
    fcz = binding.prepare_scan(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], dt_bias=tc["dt_bias"],
                               Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True, zoh=True)
    xsec_z = timer.mean(fcz, max(5, min(steps, 30)))
    doutc = wl.to_torch(wl.store(np.random.default_rng(4242).standard_normal((B, D, L)), cfg["dtype"]), dev)
    bcx = binding.prepare_scan_bwd(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], doutc, dt_bias=tc["dt_bias"],
                                   Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True)
    xsec_b = timer.mean(bcx, bsteps)
    bcz = binding.prepare_scan_bwd(tc["u"], tc["dt_raw"], tc["A"], tc["Bm"], tc["Cm"], doutc, dt_bias=tc["dt_bias"],
                                   Dskip=tc["Dskip"], z=tc["z"], reset=tc["reset"], complex_state=True, zoh=True)
    xsec_bz = timer.mean(bcz, bsteps)
    del fcx, fcz, bcx, bcz, doutc, tc, xc
    yc = wl.make_cplx_decode_inputs(64, 2048, 128, wl.BF16, seed=5)
    tdc = {k: wl.to_torch(yc[k], dev) for k in ("u", "dt_raw", "z", "Bm", "Cm", "dt_bias", "A", "Dskip")}
    hdc = torch.from_numpy(yc["h"]).to(dev)
    dcx = binding.prepare_state_update(hdc, tdc["u"], tdc["dt_raw"], tdc["A"], tdc["Bm"], tdc["Cm"],
                                       dt_bias=tdc["dt_bias"], Dskip=tdc["Dskip"], z=tdc["z"], complex_state=True)
    xsec_d = timer.mean(dcx, 50)
    evict = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
    xcold_d = float(np.median(timer.launches(dcx, 30, evict=evict))) / 1e3
    del evict
    Bd, Dd, Nd = 64, 2048, 128
    # state (B, D, N, 2) read and written, plus the per-row inputs, complex B, C and A
    xdbytes = 16 * Bd * Dd * Nd + 3 * Bd * Dd * 2 + 2 * Bd * Nd * 2 * 2 + 8 * Dd * Nd + 8 * Dd + Bd * Dd * 4
    del dcx, tdc, hdc, yc
    res["complex_state"] = {
        "workload": "the same shape with a complex diagonal state: A = -1/2 + i n (S4D-Lin), complex B, C "
                    "(re, im pairs), y = Re(C h)",
        "fwd_ms": xsec_f * 1e3, "fwd_vs_plain_forward": xsec_f / fwd_s, "fwd_elements_per_s": elements / xsec_f,
        "zoh_fwd_ms": xsec_z * 1e3, "bwd_ms": xsec_b * 1e3, "bwd_vs_complex_forward": xsec_b / xsec_f,
        "bwd_elements_per_s": elements / xsec_b, "zoh_bwd_ms": xsec_bz * 1e3,
        "decode_workload": "state update B=64 D=2048 N=128 complex, bf16 inputs, fp32 state",
        "decode_ms": xsec_d * 1e3, "decode_algorithmic_bytes": xdbytes, "decode_hbm_gbps": xdbytes / xsec_d / 1e9,
        "decode_cold_ms_median": xcold_d * 1e3, "decode_cold_hbm_gbps": xdbytes / xcold_d / 1e9}
    # one GPU's share of the long-genomics sequence split 8 ways: the shard's
    # aggregate (what the other shards need) and its scan from a carried state
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
    ssec_a = timer.mean(agg, 20)
    ssec_f = timer.mean(fsh, 20)
    shard_elems = c3["B"] * c3["D"] * Ls * c3["N"]
    res["sequence_shard"] = {
        "workload": "one of 8 shards of the long-genomics sequence: B=1 D=256 L=%d N=16, bf16; the all-gather "
                    "and fold of the aggregates between devices is not built" % Ls,
        "aggregate_ms": ssec_a * 1e3, "scan_from_carried_state_ms": ssec_f * 1e3,
        "elements_per_s": shard_elems / (ssec_a + ssec_f)}
    return res


def cpu_baseline(wl, f):
    """The float64 oracle over the whole workload, every row, passes repeated
    until about 10 s of CPU work (at most 200), plus a single-thread run of the
    tiny float32 workload."""
    import oracle

    cfg, x, out, elements = f["cfg"], f["x"], f["out"], f["elements"]
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    w = wl.widen
    rows = np.arange(B * D)
    rb, rd = rows // D, rows % D
    u64, dt64, z64 = (w(x[k]).reshape(B * D, L) for k in ("u", "dt_raw", "z"))
    Bm64, Cm64 = w(x["Bm"]), w(x["Cm"])
    threads = oracle.max_threads()

    def run_oracle():
        return oracle.scan_rows(rb, rd, u64, dt64, x["A"], Bm64, Cm64, z_rows=z64, dt_bias=x["dt_bias"],
                                Dskip=x["Dskip"], reset=x["reset"])

    c0 = time.perf_counter()
    ref = run_oracle()
    reps = 1
    while time.perf_counter() - c0 < 10.0 and reps < 200:
        run_oracle()
        reps += 1
    total = time.perf_counter() - c0
    csec = total / reps
    # single thread, tiny float32 workload (1 x 64 x 256 x 16), about 2 s of passes
    xt = wl.workload_inputs("tiny-fp32")
    te = 64 * 256 * 16
    s0 = time.perf_counter()
    n1 = 0
    while time.perf_counter() - s0 < 2.0:
        oracle.scan(xt["u"], xt["dt_raw"], xt["A"], xt["Bm"], xt["Cm"], z=xt["z"], dt_bias=xt["dt_bias"],
                    Dskip=xt["Dskip"], nthreads=1)
        n1 += 1
    t1 = (time.perf_counter() - s0) / n1
    got = out.reshape(B * D, L).cpu().numpy().astype(np.float64)
    tol = 1e-5 if cfg["dtype"] == wl.F32 else 2e-3
    margin = float(np.max(np.abs(got - ref) / (tol * (1.0 + np.abs(ref)))))
    base = {"value": elements / csec, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": "the full workload (all %d rows x %d steps x %d states), float64, OpenMP over rows on "
                      "%d threads; %d passes, %.2f s each, %.1f s in all" % (B * D, L, N, threads, reps, csec, total),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "single_thread_tiny_fp32": {"elements_per_s": te / t1, "passes": n1,
                                        "workload": "tiny-fp32: 1 x 64 x 256 x 16, one thread"}}
    parity = {"rows": int(B * D), "max_err_over_bound": margin, "bound": "%g*(1+|ref|)" % tol}
    return base, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other entry points and options (backward, conv, zoh, complex, shard, sweep)")
    ap.add_argument("--only", choices=("forward", "decode", "backward", "wavefront"), default=None,
                    help="run just this entry point's timed launches (for profiler runs); prints no JSON line")
    ap.add_argument("--workload", default="mamba130m-layer",
                    help="workload name: mamba130m-layer (the default and the headline); tiny-fp32, "
                         "mamba2.8b-layer, long-genomics and packed-docs-n128 print their own line for reference")
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
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    evict = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device=dev)

    if args.copy_calibration:
        src = torch.ones(1 << 27, dtype=torch.float32, device=dev)   # 512 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only == "decode":
        measure_decode(torch, binding, wl, timer, evict)
        print("decode timed", flush=True)
        return
    f = measure_forward(args, torch, binding, wl, timer, evict)
    if args.only == "forward":
        print("forward timed: median %.1f us" % (np.median(f["cold"]) * 1e3), flush=True)
        return
    if args.only == "backward":
        measure_backward(torch, binding, wl, timer, f, args.steps)
        print("backward timed", flush=True)
        return
    if args.only == "wavefront":
        wf = measure_wavefront(torch, binding, timer, f, evict, args.steps)
        print("wavefront timed: median %.1f us" % (np.median(wf["cold"]) * 1e3), flush=True)
        return

    cfg, elements = f["cfg"], f["elements"]
    B, D, L, N = cfg["B"], cfg["D"], cfg["L"], cfg["N"]
    cold_s = float(np.median(f["cold"])) / 1e3
    cold_mean_s = float(np.mean(f["cold"])) / 1e3
    warm_s = float(np.mean(f["warm"])) / 1e3
    abytes = algorithmic_bytes(B, D, L, N, f["s_in"], 4, reset=f["x"]["reset"] is not None)
    ops = OPS_PER_ELEMENT * elements + OPS_PER_ROW_STEP * B * D * L
    ceiling = hbm_ceiling(torch, timer)
    hbm_achieved = abytes / cold_mean_s / 1e9
    alu_achieved = ops / cold_mean_s / 1e12
    hbm = {"achieved": hbm_achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": hbm_achieved / HBM_PEAK_GBPS,
           "frac_of_copy_ceiling": hbm_achieved / ceiling["copy_gbps"], "algorithmic_bytes_per_launch": abytes}
    alu = {"achieved": alu_achieved, "peak": ALU_PEAK_TOPS, "unit": "T lane-op/s (fp32 VALU; transcendental = 2)",
           "frac": alu_achieved / ALU_PEAK_TOPS, "algorithmic_ops_per_launch": ops}
    top = alu if alu["frac"] >= hbm["frac"] else hbm
    roofline = {
        "kernel": kernel_label(N, cfg["dtype"], cfg["packed"], L),
        "bound": "alu" if top is alu else "hbm",
        "achieved": top["achieved"], "peak": top["peak"], "unit": top["unit"], "frac": top["frac"],
        "traffic": recorded_traffic(cfg["name"]),
        "launch_ms_mean": cold_mean_s * 1e3, "launch_ms_median": cold_s * 1e3,
        "launch_ms_p10": percentile(f["cold"], 10), "launch_ms_p90": percentile(f["cold"], 90),
        "timed_launches": len(f["cold"]),
        "hbm": hbm, "alu": alu,
    }
    result = {
        "metric": "selective-scan elements/s (B·D·L·N) and achieved HBM GB/s vs peak, 1 GPU",
        "value": elements / cold_s,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": cold_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s scan: B=%d D=%d L=%d N=%d, %s u/dt/z/B/C, fp32 A/D/dt_bias/state/out, "
                               "silu gate, %s" % (cfg["name"], B, D, L, N, cfg["dtype"],
                                                  "document resets" if cfg["packed"] else "no reset"),
                   "input_dtype": cfg["dtype"], "global_batch": B, "seq_len": L, "d_inner": D, "d_state": N,
                   "parallelism": "none"},
        "timing": "value and ms_per_step: median of the K timed launches (HIP events on the launch stream), "
                  "each after a 1 GiB cache-evicting read outside its event pair; wall_s_timed_region: the "
                  "wall clock of those K steps, evicting reads included",
        "wall_s_timed_region": f["wall"],
        "hbm_gbps": abytes / cold_s / 1e9,
        "hbm_frac_of_peak": abytes / cold_s / 1e9 / HBM_PEAK_GBPS,
        "roofline": roofline,
        "warm": {"launch_ms_mean": warm_s * 1e3, "back_to_back_ms_mean": f["warm_mean"] * 1e3,
                 "elements_per_s": elements / warm_s, "hbm_gbps": abytes / warm_s / 1e9},
        "hbm_ceiling": ceiling,
    }
    wf = measure_wavefront(torch, binding, timer, f, evict, min(args.steps, 50)) if not args.no_extras else None
    if wf is not None:
        wf_s = float(np.median(wf["cold"])) / 1e3
        result["wavefront_scan"] = {
            "workload": "the same forward through ssm_scan_fwd_wavefront: one wave per (b, d), one step per lane, "
                        "a DPP scan of the affine pairs inside each 64-step chunk, carry across chunks",
            "launch_ms_median": wf_s * 1e3, "elements_per_s": elements / wf_s,
            "vs_forward": wf_s / cold_s,
            "max_abs_diff_vs_forward": float((wf["out"] - f["out"]).abs().max().item()),
        }
        del wf
    result["decode"] = measure_decode(torch, binding, wl, timer, evict)
    del evict
    if not args.no_extras:
        result["length_sweep"] = length_sweep(torch, binding, wl, timer)
        result["decode_loop"] = decode_loop(torch, binding, wl, timer)
        dout, bsec, result["backward"] = measure_backward(torch, binding, wl, timer, f, args.steps)
        result["backward"]["vs_forward"] = bsec / cold_mean_s
        result.update(measure_extras(torch, binding, wl, timer, f, dout, bsec, cold_mean_s, args.steps))
    if not args.no_cpu:
        result["cpu_baseline"], result["parity_vs_oracle"] = cpu_baseline(wl, f)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
