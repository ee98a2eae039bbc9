"""Benchmark of the S6 selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one forward scan (softplus Delta, discretisation, recurrence, C-contraction, D skip, SiLU gate, final
state: one fused launch) over the Mamba-2.8B-layer-shaped workload: batch 4, d_inner 5120, L 4096, N 16, bf16 I/O,
fp32 state, seeded synthetic inputs already resident in HBM.  Prints one JSON line.  Also reported, outside `value`:
the backward pass over the same workload (one ssm_scan_bwd call: every gradient, states recomputed, bf16 dy and
per-step gradients), the single-token decode step (batch 256, d_inner 5120, 64 steps with fresh inputs) and the fp64
CPU oracle timed on the host cores over the same step (a reported baseline; its output also gates parity of the timed
step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
VALU_PEAK_TFLOPS = 78.6          # non-packed fp32 FMA: 256 CU x 4 SIMD x 16 lanes x 2 FLOP x 2.4 GHz
TRANS_SLOTS = 2                  # issue cost of v_exp/v_log/v_rcp in FMA slots on gfx950 (half rate)


def scan_algorithmic_bytes(b, D, L, N, io_bytes=2, gate=True, dskip=True):
    """x, dt, (z), y once; B, C once per batch; A, dt_bias, (Dskip) once; h_final once (fp32)."""
    seq = b * D * L * io_bytes * (3 + (1 if gate else 0))
    bc = 2 * b * N * L * io_bytes
    par = D * N * 4 + D * 4 + (D * 4 if dskip else 0)
    return seq + bc + par + b * D * N * 4


def scan_algorithmic_flops(b, D, L, N, gate=True, dskip=True):
    """fp32 work per (b, d, t) in FMA-slot units x 2 FLOP:
    per state n: Delta*A (1), exp (2 slots), (Delta x)*B (1), h = a h + b (1 FMA), y += C h (1 FMA)  -> 6 slots;
    per element: dt + bias (1), softplus = exp + log + rcp (6) + 5 ops, Delta*x (1), D*x (1), silu = exp + rcp (4)
    + 3 ops.  Each slot is counted as 2 FLOP so that the figure compares with the 78.6 TFLOP/s FMA peak."""
    per_elem = 6 * N + 1 + 11 + 1 + (1 if dskip else 0) + (7 if gate else 0)
    return 2.0 * per_elem * b * D * L


def complex_algorithmic_flops(b, D, L, N, gate=True, dskip=True):
    """Complex-A forward per (b, d, t) in FMA-slot units x 2: per state Delta*Re(A), exp (2), sin + cos (4),
    (Delta x) B (2), the complex update (4), Re(C h) (2) and its sum (1) = 16; per element as the real scan (25)."""
    per_elem = 16 * N + 1 + 11 + 1 + (1 if dskip else 0) + (7 if gate else 0)
    return 2.0 * per_elem * b * D * L


def conv_algorithmic_flops(b, D, L, width=4):
    """The causal convolution + SiLU in front of the scan, per (b, d, t): width FMAs, SiLU = exp + rcp (4 slots) + 2."""
    return 2.0 * (width + 6) * b * D * L


def bwd_algorithmic_flops(b, D, L, N, gate=True, dskip=True):
    """fp32 work of the backward per (b, d, t), in FMA-slot units x 2 FLOP (same convention as the forward).
    Per state n: zero-start chunk pass 8 (Delta*A, exp 2, (Delta x)*B, h FMA, decay product, C*ds, lambda FMA);
    recomputation 5 (Delta*A, exp 2, (Delta x)*B, h FMA); adjoint 2 (g += C ds, g *= a); dA 3 (a h_prev, g u,
    += Delta); dx / dDelta terms 2 (g B, A g u) and their sums over n 2; dB / dC 2 FMA; with the gate C h and its sum 2.
    Per element: softplus twice (11 each), sigmoid(u) 4, silu twice (7 each), dz 4, dx / dDelta / du 4."""
    per_n = 8 + 5 + 2 + 3 + 4 + 2 + (2 if gate else 0)
    per_elem = 11 * 2 + 4 + (7 * 2 + 4 if gate else 0) + 4 + (2 if dskip else 0)
    return 2.0 * (per_n * N + per_elem) * b * D * L


def bwd_algorithmic_bytes(b, D, L, N, io_bytes=2, gate=True, dskip=True):
    """Inputs read twice (x, dt, z, dy by the chunk pass and the main pass), B and C twice, per-step gradients
    written once, dB / dC / dA / dD / dbias / dh0 written once (fp32)."""
    seq_in = b * D * L * io_bytes * (3 + (1 if gate else 0))
    seq_out = b * D * L * io_bytes * (2 + (1 if gate else 0))
    bc = 2 * b * N * L * io_bytes
    return 2 * seq_in + seq_out + 2 * bc + 2 * b * N * L * 4 + D * N * 4 * 2 + D * 4 * 4 + b * D * N * 4


def decode_algorithmic_bytes(b, D, N, io_bytes=2, gate=True, dskip=True):
    return (b * D * N * 4 * 2 + b * D * io_bytes * (3 + (1 if gate else 0)) + 2 * b * N * io_bytes + D * N * 4
            + D * 4 * (2 if dskip else 1))


def ssd_algorithmic_bytes(b, L, H, P, G, N, y_bytes=2, gate=True, h_final=True):
    """SSD layer: x (and z) read and y written once, dt read, B and C read once per group, h_final written (fp32),
    A / dt_bias / Dskip per head."""
    seq = b * L * H * P
    return (seq * 2 * (2 if gate else 1) + seq * y_bytes + b * L * H * 2 + 2 * b * L * G * N * 2
            + (b * H * P * N * 4 if h_final else 0) + 3 * H * 4)


def ssd_algorithmic_flops(b, L, H, P, G, N, Q=64):
    """FLOPs of the chunked dual form (one multiply-add = 2): per batch, chunk and group C B^T (2 Q^2 N); per batch,
    chunk and head the masked product M x over the lower triangle (Q (Q+1) P), C S_prev (2 Q N P) and the state
    update (2 Q N P)."""
    nc = -(-L // Q)
    return b * nc * (G * 2 * Q * Q * N + H * (Q * (Q + 1) * P + 4 * Q * N * P))


# the source files each kernel is built from (its translation unit and the headers it includes)
KERNEL_SOURCES = (("scan_kernel", ("common.hpp", "scan_fwd.hpp", "ssm_scan.hip")),
                  ("decode_kernel", ("common.hpp", "scan_fwd.hpp", "ssm_scan.hip")),
                  ("bwd_", ("common.hpp", "ssm_scan_bwd.hip")),
                  ("ssd_", ("common.hpp", "ssm_ssd.hip")),
                  ("complex_", ("common.hpp", "ssm_complex_scan.hip")),
                  ("conv1d_", ("common.hpp", "scan_fwd.hpp", "ssm_conv_scan.hip")))


def ssd_decode_algorithmic_bytes(b, H, P, G, N, io_bytes=2, gate=True):
    """One SSD decode step: the fp32 state read and written, x (and z) read and y written, dt, B, C, per-head
    parameters."""
    return (2 * b * H * P * N * 4 + b * H * P * io_bytes * (3 if gate else 2) + b * H * io_bytes
            + 2 * b * G * N * io_bytes + 3 * H * 4)


def src_hash(kernel_key):
    """Hash of the sources a kernel is built from: a counter record taken on other sources is stale."""
    files = next(f for prefix, f in KERNEL_SOURCES if kernel_key.startswith(prefix))
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_57_amd", "csrc")
    for name in files:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def ssd_traffic(nseg):
    """HBM bytes of one ssm_ssd_fwd call on the 2.7B layer: the full pass, plus the zero-start pass when the
    sequence is split into L-segments; None unless every record involved is current."""
    full = measured_traffic("ssd_fwd_kernel mamba2-2.7b-layer")
    if nseg <= 1 or full is None:
        return full
    zero = measured_traffic("ssd_fwd_kernel zero-start mamba2-2.7b-layer")
    return None if zero is None else full + zero


def measured_traffic(kernel_key):
    """HBM bytes per launch (read + written) from the committed rocprofv3 counter record, if it was taken on the
    current kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    for line in lines:
        if line.startswith("#") or "|" not in line:
            continue
        f = [x.strip() for x in line.split("|")]
        if len(f) == 4 and f[0] == kernel_key:
            if f[1] != src_hash(kernel_key):
                return None
            return int(f[2]) + int(f[3])
    return None


def host_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-complex", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (torch) five times: the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE readings")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the scan shards over channels with no communication, so a multi-GPU "
              "figure is the one-GPU figure at a smaller d_inner; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import selective_state_space_57_amd as ssm
    from selective_state_space_57_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": src.numel() * 4,
                          "copy_calibration_bytes_written_per_launch": dst.numel() * 4}), flush=True)
        return

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    w = I.WORKLOADS[2]
    b, D, L, N = w.batch, w.dim, w.seqlen, w.dstate
    host = I.scan_inputs(w)
    d = {k: up(v) for k, v in host.items()}
    y = torch.empty((b, D, L), dtype=torch.bfloat16, device=dev)
    hf = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    p = ssm.make_params(b, D, L, N, ssm.SSM_BF16, ssm.SSM_BF16)
    nseg = ssm.plan_segments(p)
    ws_n = ssm.workspace_bytes(p)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], dt_bias=d["dt_bias"], Dskip=d["Dskip"], z=d["z"],
                     y=y, h_final=hf, workspace=ws if ws_n else None, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    ms = ev0.elapsed_time(ev1) / args.steps

    elems = b * D * L
    value = elems / (ms * 1e-3)
    nbytes = scan_algorithmic_bytes(b, D, L, N)
    flops = scan_algorithmic_flops(b, D, L, N)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    kernel_key = "scan_kernel<bf16,bf16,euler,gate,dskip> mamba2.8b-layer"

    out = {
        "metric": "scan elements/s (B*D*L), Mamba-2.8B-layer-shaped forward selective scan",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the Mamba-2.8B layer workload)",
        "config": {"workload": "mamba2.8b-layer", "batch": b, "d_inner": D, "seqlen": L, "d_state": N,
                   "io": "bf16", "state": "f32", "gate": True, "dskip": True, "disc": "euler-b", "segments": nseg},
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBps": gbs, "frac_of_8TBps": gbs / HBM_PEAK_GBS},
        "roofline": {"bound": "alu", "achieved": tflops, "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / VALU_PEAK_TFLOPS, "traffic": measured_traffic(kernel_key),
                     "kernel": kernel_key, "algorithmic_flops": flops},
        "host_wall_ms_timed_region": wall_ms,
    }

    # ---- context: what a plain device-to-device copy reaches here (1 GiB, read + written, timed after the scan)
    cp_src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * cp_src.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    out["hbm"]["copy_ceiling_GBps"] = copy_gbs
    out["hbm"]["frac_of_copy_ceiling"] = gbs / copy_gbs
    del cp_src, cp_dst

    # ---- context: single launches with the 256 MB Infinity Cache evicted before each (512 MB written by a fill
    # kernel on the same stream), median and 10th / 90th percentiles; `value` above is the mean of back-to-back steps
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    cold = []
    for i in range(20):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold.sort()
    out["cold"] = {"launches": len(cold), "median_ms": cold[len(cold) // 2], "p10_ms": cold[len(cold) // 10],
                   "p90_ms": cold[(9 * len(cold)) // 10], "elements_per_s_at_median": elems / (cold[len(cold) // 2] * 1e-3),
                   "flush": "512 MB written by a fill kernel before each launch"}

    # ---- the same forward with the block's causal convolution (width 4) + SiLU fused in front of the scan
    if not args.no_conv:
        from selective_state_space_57_amd import _abi
        cvp = I.conv_params(w, 4)
        cw, cb = up(cvp["conv_w"]), up(cvp["conv_b"])
        conv = _abi.make_conv(cw.data_ptr(), 4, cb.data_ptr(), 0, 0, 1)
        cargs = (d["x"].data_ptr(), d["dt"].data_ptr(), d["dt_bias"].data_ptr(), d["A"].data_ptr(),
                 d["B"].data_ptr(), d["C"].data_ptr(), d["Dskip"].data_ptr(), d["z"].data_ptr(), 0, y.data_ptr(),
                 hf.data_ptr(), ws.data_ptr() if ws_n else 0, ws_n, stream.cuda_stream)

        def cstep():
            st = _abi.conv_scan_fwd_raw(p, conv, *cargs)
            if st:
                _abi.check(st)

        for _ in range(5):
            cstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            cstep()
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / args.steps
        cfl = flops + conv_algorithmic_flops(b, D, L, 4)
        out["conv_scan"] = {"workload": "mamba2.8b-layer + causal conv1d (width 4) + SiLU", "ms_per_step": cms,
                            "elements_per_s": elems / (cms * 1e-3), "overhead_vs_scan": cms / ms - 1.0,
                            "algorithmic_flops": cfl, "achieved_TFLOPs": cfl / (cms * 1e-3) / 1e12,
                            "frac_of_valu_peak": cfl / (cms * 1e-3) / 1e12 / VALU_PEAK_TFLOPS,
                            "algorithmic_bytes": nbytes + D * 4 * 5,
                            "note": "x is read once and the convolved sequence never goes to memory; a separate "
                                    "convolution kernel would add a write and a read of it (2 x 168 MB in bf16)"}
        # the convolution on its own (recompute of u for training) and its backward, bf16 in and out
        uu = torch.empty((b, D, L), dtype=torch.bfloat16, device=dev)
        gdx = torch.empty((b, D, L), dtype=torch.bfloat16, device=dev)
        gdw = torch.empty((D, 4), dtype=torch.float32, device=dev)
        gdb = torch.empty((D,), dtype=torch.float32, device=dev)

        def kfwd():
            _abi.check(_abi.conv1d_fwd_raw(p, conv, d["x"].data_ptr(), uu.data_ptr(), stream.cuda_stream))

        def kbwd():
            _abi.check(_abi.conv1d_bwd_raw(p, conv, d["x"].data_ptr(), uu.data_ptr(), 0, gdx.data_ptr(),
                                           gdw.data_ptr(), gdb.data_ptr(), 0, stream.cuda_stream))

        ctimes = {}
        for name, fn in (("fwd", kfwd), ("bwd", kbwd)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ctimes[name] = e0.elapsed_time(e1) / args.steps
        cby = {"fwd": 2 * elems * 2, "bwd": 3 * elems * 2}   # x read + u written; x, du read + dx written (bf16)
        for name in ("fwd", "bwd"):
            gbs_ = cby[name] / (ctimes[name] * 1e-3) / 1e9
            out["conv_scan"]["conv1d_" + name] = {
                "ms": ctimes[name], "algorithmic_bytes": cby[name],
                "roofline": {"bound": "hbm", "achieved": gbs_, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs_ / HBM_PEAK_GBS,
                             "traffic": measured_traffic("conv1d_%s_kernel<bf16,bf16,4> mamba2.8b-layer" % name)}}
        del uu, gdx

    # ---- complex diagonal A (S4D-Lin) on the same shape: complex B, C and state
    if not args.no_complex:
        from selective_state_space_57_amd import _abi
        hc = I.complex_inputs(w)
        A2, B2, C2 = up(hc["A"]), up(hc["B"]), up(hc["C"])
        hfc = torch.empty((b, D, N, 2), dtype=torch.float32, device=dev)
        xargs = (d["x"].data_ptr(), d["dt"].data_ptr(), d["dt_bias"].data_ptr(), A2.data_ptr(), B2.data_ptr(),
                 C2.data_ptr(), d["Dskip"].data_ptr(), d["z"].data_ptr(), 0, y.data_ptr(), hfc.data_ptr(),
                 stream.cuda_stream)

        def xstep():
            st = _abi.complex_scan_fwd_raw(p, *xargs)
            if st:
                _abi.check(st)

        for _ in range(3):
            xstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nx = max(1, args.steps // 4)
        e0.record(stream)
        for _ in range(nx):
            xstep()
        e1.record(stream)
        torch.cuda.synchronize()
        xms = e0.elapsed_time(e1) / nx
        xfl = complex_algorithmic_flops(b, D, L, N)
        out["complex_scan"] = {"workload": "mamba2.8b-layer shape, complex diagonal A (S4D-Lin), complex B, C",
                               "ms_per_step": xms, "elements_per_s": elems / (xms * 1e-3),
                               "ratio_to_real_scan": xms / ms, "algorithmic_flops": xfl,
                               "achieved_TFLOPs": xfl / (xms * 1e-3) / 1e12,
                               "frac_of_valu_peak": xfl / (xms * 1e-3) / 1e12 / VALU_PEAK_TFLOPS}

    # ---- Mamba-2 SSD layer (scalar A per head, N = 128) at the Mamba-2 2.7B layer shape, bf16 matrix cores
    if not args.no_ssd:
        from selective_state_space_57_amd import _abi
        sw = I.SSD_WORKLOADS[1]
        sb, sL, sH, sP, sG, sN = sw.batch, sw.seqlen, sw.nheads, sw.headdim, sw.ngroups, sw.dstate
        hs = I.ssd_inputs(sw)
        sd = {k: up(v) for k, v in hs.items()}
        ys = torch.empty((sb, sL, sH, sP), dtype=torch.bfloat16, device=dev)
        hfs = torch.empty((sb, sH, sP, sN), dtype=torch.float32, device=dev)
        spar = _abi.make_ssd_params(sb, sL, sH, sP, sG, sN, ssm.SSM_BF16, ssm.SSM_BF16)
        snseg = _abi.ssd_plan_segments(spar)
        sws_n = _abi.ssd_workspace_bytes(spar)
        sws = torch.empty(max(sws_n, 1), dtype=torch.uint8, device=dev)
        sargs = (sd["x"].data_ptr(), sd["dt"].data_ptr(), sd["dt_bias"].data_ptr(), sd["A"].data_ptr(),
                 sd["B"].data_ptr(), sd["C"].data_ptr(), sd["Dskip"].data_ptr(), sd["z"].data_ptr(), 0,
                 ys.data_ptr(), hfs.data_ptr(), sws.data_ptr() if sws_n else 0, sws_n, stream.cuda_stream)

        def sstep():
            st = _abi.ssd_fwd_raw(spar, *sargs)
            if st:
                _abi.check(st)

        for _ in range(5):
            sstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            sstep()
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / args.steps
        sby = ssd_algorithmic_bytes(sb, sL, sH, sP, sG, sN)
        sfl = ssd_algorithmic_flops(sb, sL, sH, sP, sG, sN)
        sgbs = sby / (sms * 1e-3) / 1e9
        stf = sfl / (sms * 1e-3) / 1e12
        selem = sb * sL * sH * sP
        out["ssd"] = {"workload": "mamba2-2.7b-layer: batch %d, seqlen %d, %d heads x %d, ngroups %d, d_state %d, "
                                  "bf16 io, gate + D, %d L-segments" % (sb, sL, sH, sP, sG, sN, snseg),
                      "ms_per_step": sms, "elements_per_s": selem / (sms * 1e-3),
                      "ratio_to_s6_scan_same_elements": sms / ms if selem == elems else None,
                      "roofline": {"bound": "hbm", "achieved": sgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": sgbs / HBM_PEAK_GBS, "traffic": ssd_traffic(snseg),
                                   "kernel": "ssd_fwd_kernel<128,bf16,euler,gate,dskip> (+ the zero-start pass "
                                             "over all but the last L-segment)",
                                   "algorithmic_bytes": sby},
                      "mfma": {"algorithmic_flops": sfl, "achieved_TFLOPs": stf, "peak_bf16_TFLOPs": 2500.0,
                               "frac": stf / 2500.0}}
        if not args.no_cpu_baseline:
            # the fp64 SSD oracle on a bounded sample of the same inputs: batch element 0, all heads and steps
            import oracle
            oracle.build(force=False)
            fs = I.as_f64({k: (None if v is None else (v[:1] if k in ("x", "z", "dt", "B", "C") else v))
                           for k, v in hs.items()})
            t0 = time.perf_counter()
            oracle.ssd(fs["x"], fs["dt"], fs["A"], fs["B"], fs["C"], dt_bias=fs["dt_bias"], Dskip=fs["Dskip"],
                       z=fs["z"], nthreads=host_cores())
            cs = time.perf_counter() - t0
            out["ssd"]["cpu_baseline"] = {"value": sL * sH * sP / cs, "unit": "elements/s", "cores": host_cores(),
                                          "kind": "oracle", "seconds": cs,
                                          "sample": "batch element 0 of the layer (1/4 of it), fp64"}
        del sd, ys, hfs, sws

    # ---- Mamba-2 SSD decode: 8 single-token steps with fresh inputs (256 sequences, 80 heads of 64, N = 128)
    if not args.no_ssd and not args.no_decode:
        from selective_state_space_57_amd import _abi
        wsd = I.SSD_WORKLOADS[2]
        db_, dH, dP, dG, dN = wsd.batch, wsd.nheads, wsd.headdim, wsd.ngroups, wsd.dstate
        sstate = torch.from_numpy(I.ssd_inputs(wsd, with_h0=True)["h0"]).to(dev)
        sin = [{k: up(v) for k, v in I.ssd_inputs(wsd, step=s_).items() if k != "h0"} for s_ in range(wsd.decode_steps)]
        ysd = torch.empty((db_, dH, dP), dtype=torch.bfloat16, device=dev)
        pdd = _abi.make_ssd_params(db_, 1, dH, dP, dG, dN, ssm.SSM_BF16, ssm.SSM_BF16)
        sdargs = [(sstate.data_ptr(), q["x"].data_ptr(), q["dt"].data_ptr(), q["dt_bias"].data_ptr(),
                   q["A"].data_ptr(), q["B"].data_ptr(), q["C"].data_ptr(), q["Dskip"].data_ptr(), q["z"].data_ptr(),
                   ysd.data_ptr(), stream.cuda_stream) for q in sin]

        def sdstep(s_):
            st = _abi.ssd_state_update_raw(pdd, *sdargs[s_])
            if st:
                _abi.check(st)

        for s_ in range(2):
            sdstep(s_)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s_ in range(wsd.decode_steps):
            sdstep(s_)
        e1.record(stream)
        torch.cuda.synchronize()
        sdms = e0.elapsed_time(e1) / wsd.decode_steps
        sdby = ssd_decode_algorithmic_bytes(db_, dH, dP, dG, dN)
        out["ssd_decode"] = {"workload": "mamba2-decode-b256: 256 sequences, 80 heads x 64, N = 128, bf16 io",
                             "steps": wsd.decode_steps, "us_per_step": sdms * 1e3,
                             "roofline": {"bound": "hbm", "achieved": sdby / (sdms * 1e-3) / 1e9,
                                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": sdby / (sdms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                          "algorithmic_bytes": sdby,
                                          "traffic": measured_traffic("ssd_decode_kernel mamba2-decode-b256")}}
        del sstate, sin

    # ---- backward over the same workload: bf16 dy in, bf16 dx / ddt / dz out, fp32 parameter gradients
    if not args.no_bwd:
        from selective_state_space_57_amd import _abi
        dy = up(I.cotangents(w)["dy"])
        pb = ssm.make_params(b, D, L, N, ssm.SSM_BF16, ssm.SSM_BF16)
        wsb_n = ssm.bwd_workspace_bytes(pb)
        wsb = torch.empty(wsb_n, dtype=torch.uint8, device=dev)
        bf, f32 = torch.bfloat16, torch.float32
        g = {"dx": torch.empty((b, D, L), dtype=bf, device=dev), "ddt": torch.empty((b, D, L), dtype=bf, device=dev),
             "dz": torch.empty((b, D, L), dtype=bf, device=dev), "dA": torch.empty((D, N), dtype=f32, device=dev),
             "dB": torch.empty((b, N, L), dtype=f32, device=dev), "dC": torch.empty((b, N, L), dtype=f32, device=dev),
             "dD": torch.empty((D,), dtype=f32, device=dev), "db": torch.empty((D,), dtype=f32, device=dev),
             "dh0": torch.empty((b, D, N), dtype=f32, device=dev)}
        bargs = (d["x"].data_ptr(), d["dt"].data_ptr(), d["dt_bias"].data_ptr(), d["A"].data_ptr(),
                 d["B"].data_ptr(), d["C"].data_ptr(), d["Dskip"].data_ptr(), d["z"].data_ptr(), 0, dy.data_ptr(), 0,
                 g["dx"].data_ptr(), g["ddt"].data_ptr(), g["dA"].data_ptr(), g["dB"].data_ptr(), g["dC"].data_ptr(),
                 g["dD"].data_ptr(), g["dz"].data_ptr(), g["db"].data_ptr(), g["dh0"].data_ptr(), wsb.data_ptr(),
                 wsb_n, stream.cuda_stream)

        def bstep():
            st = _abi.scan_bwd_raw(pb, *bargs)
            if st:
                _abi.check(st)

        for _ in range(3):
            bstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.bwd_steps):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / args.bwd_steps
        bfl = bwd_algorithmic_flops(b, D, L, N)
        bby = bwd_algorithmic_bytes(b, D, L, N)
        out["bwd"] = {"workload": "mamba2.8b-layer", "steps": args.bwd_steps, "ms_per_step": bms,
                      "elements_per_s": elems / (bms * 1e-3), "ratio_to_forward": bms / ms,
                      "kernels": "prep + carry + main + 2 reduce (one ssm_scan_bwd call)",
                      "algorithmic_flops": bfl, "achieved_TFLOPs": bfl / (bms * 1e-3) / 1e12,
                      "frac_of_valu_peak": bfl / (bms * 1e-3) / 1e12 / VALU_PEAK_TFLOPS,
                      "algorithmic_bytes": bby, "achieved_GBps": bby / (bms * 1e-3) / 1e9,
                      "workspace_bytes": wsb_n,
                      "main_kernel_traffic": measured_traffic("bwd_main_kernel<bf16,bf16,euler,gate> mamba2.8b-layer")}
        del wsb

    # ---- decode: 64 single-token steps with fresh inputs (batch 256, d_inner 5120)
    if not args.no_decode:
        wd = I.WORKLOADS[4]
        state = torch.from_numpy(I.decode_state(wd)).to(dev)
        steps_in = []
        for s in range(wd.decode_steps):
            hs = I.scan_inputs(wd, step=s)
            steps_in.append({k: up(v) for k, v in hs.items()})
        yd = torch.empty((wd.batch, wd.dim), dtype=torch.bfloat16, device=dev)
        # arguments marshalled once: a decode step is ~20 us of GPU work, so per-call Python checks would otherwise
        # leave the GPU idle between launches and the events would time the host
        from selective_state_space_57_amd import _abi
        pd = ssm.make_params(wd.batch, wd.dim, 1, wd.dstate, ssm.SSM_BF16, ssm.SSM_BF16)
        sh = stream.cuda_stream
        dargs = [(state.data_ptr(), q["x"].data_ptr(), q["dt"].data_ptr(), q["dt_bias"].data_ptr(), q["A"].data_ptr(),
                  q["B"].data_ptr(), q["C"].data_ptr(), q["Dskip"].data_ptr(), q["z"].data_ptr(), yd.data_ptr(), sh)
                 for q in steps_in]

        def dstep(s):
            st = _abi.state_update_raw(pd, *dargs[s])
            if st:
                _abi.check(st)

        for s in range(4):
            dstep(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(wd.decode_steps):
            dstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / wd.decode_steps
        dbytes = decode_algorithmic_bytes(wd.batch, wd.dim, wd.dstate)
        out["decode"] = {"workload": "decode-b256-d5120", "steps": wd.decode_steps, "us_per_step": dms * 1e3,
                         "algorithmic_bytes_per_step": dbytes, "achieved_GBps": dbytes / (dms * 1e-3) / 1e9,
                         "frac_of_8TBps": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_kernel<bf16,bf16,euler,vec> decode-b256-d5120"),
                         "note": "64 consecutive steps, each with its own pre-generated x/dt/z/B/C tensors; the 84 MB "
                                 "fp32 state can be partly served by the 256 MB Infinity Cache"}

    # ---- CPU baseline: the fp64 oracle on the host cores over the same full step; also gates parity
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        y32 = torch.empty((b, D, L), dtype=torch.float32, device=dev)
        ssm.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], dt_bias=d["dt_bias"], Dskip=d["Dskip"], z=d["z"],
                     y=y32, h_final=hf, workspace=ws if ws_n else None, stream=stream)
        torch.cuda.synchronize()
        f = I.as_f64(host)
        oracle.build(force=False)
        t0 = time.perf_counter()
        yr, hr = oracle.scan(f["x"], f["dt"], f["A"], f["B"], f["C"], dt_bias=f["dt_bias"], Dskip=f["Dskip"],
                             z=f["z"], nthreads=cores)
        cpu_s = time.perf_counter() - t0
        yg = y32.cpu().numpy().astype(np.float64)
        rms = float(np.sqrt(np.mean(yr * yr)))
        err = float(np.max(np.abs(yg - yr))) / rms
        herr = float(np.max(np.abs(hf.cpu().numpy() - hr))) / float(np.sqrt(np.mean(hr * hr)))
        out["cpu_baseline"] = {"value": elems / cpu_s, "unit": "elements/s", "cores": cores, "kind": "oracle",
                               "sample": "one full step of the same workload (4 x 5120 x 4096 elements), fp64",
                               "seconds": cpu_s}
        out["parity"] = {"max_abs_err_over_rms_y": err, "h_final_err_over_rms": herr, "tolerance": 3e-3,
                         "pass": bool(err <= 3e-3 and herr <= 3e-3)}
        if not out["parity"]["pass"]:
            print(json.dumps(out))
            print("parity gate failed", file=sys.stderr)
            sys.exit(1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
