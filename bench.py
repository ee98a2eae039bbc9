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
# VALU issue: 256 CU x 4 SIMD x 32 lanes x 2.4 GHz = 7.86e13 lane-slots/s for non-packed fp32, where a slot is one
# add, multiply or FMA per lane (a wave64 FMA issues every 2 cycles on gfx950; packed FP32 is not used).  This is the
# published 157.3 TFLOP/s fp32 vector peak counted in FMAs.  Reported in units of 10^12 lane-slots/s.
VALU_PEAK_TSLOTS = 256 * 4 * 32 * 2.4e9 / 1e12
# Issue cost of one v_exp_f32 / v_log_f32 / v_rcp_f32 in slots.  The issue-rate probe
# (selective_state_space_57_amd/csrc/issue_probe.hip, run by every bench.py call: `issue_rates` in the JSON line)
# measures on MI355X about 2.4 cycles per wave64 FMA and 8.2 per wave64 exp, and an exp interleaved with FMAs in one
# wave, or issued by another wave of the same SIMD, costs the same (no co-issue): 4 slots.  The record is in
# profiles/issue_rates_mi355x.md.
TRANS_SLOTS = 4


def scan_algorithmic_bytes(b, D, L, N, io_bytes=2, gate=True, dskip=True):
    """x, dt, (z), y once; B, C once per batch; A, dt_bias, (Dskip) once; h_final once (fp32)."""
    seq = b * D * L * io_bytes * (3 + (1 if gate else 0))
    bc = 2 * b * N * L * io_bytes
    par = D * N * 4 + D * 4 + (D * 4 if dskip else 0)
    return seq + bc + par + b * D * N * 4


# -|u| log2(e), exp, 1 + v, w - 1, v - (w - 1), 1 - v, log2, x ln 2, fma, max(u, 0), +
SOFTPLUS_SLOTS = 9 + 2 * TRANS_SLOTS
SILU_SLOTS = 3 + 2 * TRANS_SLOTS      # -z log2(e), exp, 1 + e, rcp, z r


def scan_elem_slots(N, gate=True, dskip=True, softplus=True):
    """Algorithmic VALU issue slots of the forward scan per (b, d, t) element (transcendental = TRANS_SLOTS).
    Per state n: Delta*A' (1), exp (TRANS_SLOTS), (Delta x)*B (1), h = a h + b (1 FMA), y += C h (1 FMA);
    per element: dt + bias (1), softplus, Delta*x (1), D*x (1 FMA), silu and the gate's product (1)."""
    per_elem = 1 + (SOFTPLUS_SLOTS if softplus else 0) + 1 + (1 if dskip else 0) + (SILU_SLOTS + 1 if gate else 0)
    return (4 + TRANS_SLOTS) * N + per_elem


def scan_algorithmic_slots(b, D, L, N, gate=True, dskip=True, softplus=True):
    return float(scan_elem_slots(N, gate, dskip, softplus)) * b * D * L


def zoh_elem_slots(N, gate=True, dskip=True, softplus=True):
    """The forward scan under the ZOH rule, per (b, d, t) element: Euler's slots plus, per state, the coefficient
    expm1(Delta A) / A: Delta*A (1), expm1 near 0 as a degree-7 polynomial (7 FMA + 1 multiply), the choice between it
    and exp - 1 (compare, select, subtract: 3), the division by A as a multiply (1), and B*x no longer sharing the
    per-element Delta*x (1)."""
    return scan_elem_slots(N, gate, dskip, softplus) + (1 + 8 + 3 + 1 + 1) * N


def complex_algorithmic_slots(b, D, L, N, gate=True, dskip=True):
    """Complex-A forward per (b, d, t): per state Delta*Re(A), exp, sin + cos (about 18 fused multiply-adds and bit
    operations of the polynomial evaluation with its reduction), (Delta x) B (2), the complex update (4), Re(C h) (2)
    and its sum (1); per element as the real scan."""
    return float((1 + TRANS_SLOTS + 18 + 2 + 4 + 2 + 1) * N + scan_elem_slots(0, gate, dskip)) * b * D * L


def conv_algorithmic_slots(b, D, L, width=4):
    """The causal convolution + SiLU in front of the scan, per (b, d, t): width FMAs, SiLU (7)."""
    return float(width + SILU_SLOTS) * b * D * L


def bwd_algorithmic_slots(b, D, L, N, gate=True, dskip=True):
    """VALU issue slots of the backward per (b, d, t) (same convention as the forward).
    Per state n: zero-start chunk pass (Delta*A, exp, (Delta x)*B, h FMA, decay product, C*ds, lambda FMA);
    recomputation (Delta*A, exp, (Delta x)*B, h FMA); adjoint 2 (g += C ds, g *= a); dA 3 (a h_prev, g u,
    += Delta); dx / dDelta terms 2 (g B, A g u) and their sums over n 2; dB / dC 2 FMA; with the gate C h and its sum 2.
    Per element: softplus twice, sigmoid(u) (exp, add, rcp), silu twice, dz 4, dx / dDelta / du 4."""
    per_n = (6 + TRANS_SLOTS) + (3 + TRANS_SLOTS) + 2 + 3 + 4 + 2 + (2 if gate else 0)
    per_elem = (SOFTPLUS_SLOTS * 2 + 1 + 2 * TRANS_SLOTS + (SILU_SLOTS * 2 + 4 if gate else 0) + 4
                + (2 if dskip else 0))
    return float(per_n * N + per_elem) * b * D * L


def alu_roofline(slots, ms, kernel, traffic=None, extra=None):
    """The ALU roofline object: algorithmic lane-slots per launch / launch time against VALU_PEAK_TSLOTS."""
    ach = slots / (ms * 1e-3) / 1e12
    r = {"bound": "alu", "achieved": ach, "peak": VALU_PEAK_TSLOTS, "unit": "Tslot/s", "frac": ach / VALU_PEAK_TSLOTS,
         "traffic": traffic, "kernel": kernel, "algorithmic_slots": slots,
         "slot_model": "one fp32 add / multiply / FMA per lane = 1 slot, one exp / log / rcp = %d slots (measured "
                       "in issue_rates); peak = 256 CU x 4 SIMD x 32 lanes x 2.4 GHz (non-packed fp32; the 157.3 "
                       "TFLOP/s fp32 vector peak in FMAs)" % TRANS_SLOTS}
    if extra:
        r.update(extra)
    return r


def hbm_roofline(nbytes, ms, traffic=None, kernel=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "kernel": kernel, "algorithmic_bytes": nbytes}


PROBE_KINDS = (("fma", 0), ("exp", 1), ("mix_exp_fma_1_1", 2), ("mix_exp_fma_1_3", 3), ("log", 4), ("rcp", 5),
               ("split_waves_exp_fma", 6), ("mul_dpp_bcast", 7), ("lds_read_b128", 8),
               ("lds_read_b128_row_broadcast", 9), ("lds_write_b32", 10), ("lds_read_b32", 11),
               ("scan_step_dpp", 12), ("scan_step_plain", 13), ("vmem_load_b128", 14),
               ("vmem_load_b128_row_broadcast", 15), ("lds_write_b64", 16), ("lds_write_b128", 17),
               ("scan_step_wave_combine", 18))
# bytes one wave moves per LDS (or vector-memory) instruction of each memory probe kind
PROBE_LDS_BYTES = {8: 64 * 16, 9: 64 * 16, 10: 64 * 4, 11: 64 * 4, 14: 64 * 16, 15: 64 * 16, 16: 64 * 8,
                   17: 64 * 16}


def issue_rates(torch, dev, stream, iters=4000, reps=3):
    """Run the issue-rate probe (libssm57_probe.so): per kernel the lane-operations retired per second, the exp cost
    in FMA slots, whether exps and FMAs overlap, and the shader clock under load (s_memtime over s_memrealtime)."""
    import ctypes
    path = os.path.join(ROOT, "selective_state_space_57_amd", "libssm57_probe.so")
    lib = ctypes.CDLL(path)
    lib.ssm_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ssm_probe_launch.restype = ctypes.c_int
    lib.ssm_probe_ops_per_iter.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int * 3)]
    grid = lib.ssm_probe_grid()
    lanes = grid * 256
    out = torch.empty(lanes, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * grid, dtype=torch.int64, device=dev)
    wall_khz = lib.ssm_probe_wallclock_khz()
    res = {}
    for name, kind in PROBE_KINDS:
        for _ in range(2):
            rc = lib.ssm_probe_launch(kind, iters, out.data_ptr(), clk.data_ptr(), stream.cuda_stream)
            assert rc == 0, ("probe launch", name, rc)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            lib.ssm_probe_launch(kind, iters, out.data_ptr(), clk.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        ops = (ctypes.c_int * 3)()
        lib.ssm_probe_ops_per_iter(kind, ctypes.byref(ops))
        c = clk.view(grid, 2).double()
        ghz = float((c[:, 0] / c[:, 1].clamp(min=1)).median()) * wall_khz * 1e-6 if wall_khz else None
        waves = lanes // 64
        cycles_per_simd = ms * 1e-3 * (ghz or 2.4) * 1e9
        if kind in PROBE_LDS_BYTES:   # LDS bytes per clock per CU
            r = {"ms": ms, "shader_clock_GHz": ghz, "instructions_per_wave": ops[0] * iters,
                 "bytes_per_clock_per_CU": ops[0] * iters * waves * PROBE_LDS_BYTES[kind] / 256 / cycles_per_simd,
                 "cycles_per_wave_instruction_per_CU": cycles_per_simd * 256 / (ops[0] * iters * waves)}
        elif kind in (12, 13, 18):    # SIMD cycles per wave and state step (64 lanes x one state step each)
            r = {"ms": ms, "shader_clock_GHz": ghz,
                 "cycles_per_wave_step": cycles_per_simd * 1024 / (waves * iters * ops[1])}
        else:
            r = {"ms": ms, "fma_lane_ops_per_s": ops[0] * iters * lanes / (ms * 1e-3),
                 "trans_lane_ops_per_s": ops[1] * iters * lanes / (ms * 1e-3), "shader_clock_GHz": ghz,
                 "cycles_per_wave_instruction": cycles_per_simd * 1024 / (waves * iters * (ops[0] + ops[1] + ops[2]))}
        res[name] = r
    t = {k: v["ms"] for k, v in res.items()}
    fma = res["fma"]["fma_lane_ops_per_s"]
    expr = res["exp"]["trans_lane_ops_per_s"]
    summary = {
        "fma_lane_ops_per_s": fma, "exp_lane_ops_per_s": expr,
        "fma_frac_of_issue_peak": fma / (VALU_PEAK_TSLOTS * 1e12),
        "exp_cost_in_fma_slots": fma / expr,
        "log_cost_in_fma_slots": fma / res["log"]["trans_lane_ops_per_s"],
        "rcp_cost_in_fma_slots": fma / res["rcp"]["trans_lane_ops_per_s"],
        # equal work split two ways; 1.0 = the two kinds take turns on one issue port, max/sum = they overlap fully
        "mix_1_1_time_over_sum": t["mix_exp_fma_1_1"] / (t["fma"] + t["exp"]),
        "mix_1_1_time_over_max": t["mix_exp_fma_1_1"] / max(t["fma"], t["exp"]),
        "split_waves_time_over_mean": t["split_waves_exp_fma"] / (0.5 * (t["fma"] + t["exp"])),
        "split_waves_time_over_max_half": t["split_waves_exp_fma"] / (0.5 * max(t["fma"], t["exp"])),
        "mul_dpp_over_fma_rate": res["mul_dpp_bcast"]["fma_lane_ops_per_s"] / fma,
        "cycles_per_wave_instruction": {k: res[k]["cycles_per_wave_instruction"]
                                        for k in ("fma", "exp", "mul_dpp_bcast")},
        "memory_bytes_per_clock_per_CU": {k: res[k]["bytes_per_clock_per_CU"]
                                          for k in ("lds_read_b128", "lds_read_b128_row_broadcast", "lds_read_b32",
                                                    "lds_write_b32",
                                                    "lds_write_b64", "lds_write_b128", "vmem_load_b128",
                                                    "vmem_load_b128_row_broadcast")},
        "scan_step_cycles_per_wave": {k: res[k]["cycles_per_wave_step"]
                                      for k in ("scan_step_dpp", "scan_step_plain", "scan_step_wave_combine")},
        "shader_clock_GHz_under_fma_load": res["fma"]["shader_clock_GHz"],
        "wall_clock_kHz": wall_khz, "iters": iters, "lanes": lanes,
        "kernels": res,
    }
    return summary


def time_launches(torch, stream, fn, n):
    """n back-to-back launches with an event between consecutive ones: (mean ms, sorted per-launch ms)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    return evs[0].elapsed_time(evs[n]) / n, per


SPIN_UP_MS = 150.0


def spin_up(torch, stream, fn, target_ms=SPIN_UP_MS, max_launches=4000):
    """Run fn back to back, untimed, in batches until about target_ms of GPU time have passed (a batch is timed with
    two events; the first launch can include one-time loading, so the batch size follows the latest batch); returns
    the number of launches."""
    done, total, batch = 0, 0.0, 4
    while total < target_ms and done < max_launches:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        total += ms
        done += batch
        per = max(ms / batch, 1e-3)
        batch = max(1, min(max_launches - done, int((target_ms - total) / per) + 1))
    return done


def pct(per):
    """p10 / median / p90 of a sorted list."""
    n = len(per)
    return {"p10_ms": per[n // 10], "median_ms": per[n // 2], "p90_ms": per[min(n - 1, (9 * n) // 10)]}


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
KERNEL_SOURCES = (("scan_kernel<bf16,bf16,euler,gate,dskip,conv>", ("common.hpp", "scan_fwd.hpp", "ssm_conv_scan.hip")),
                  ("scan_kernel", ("common.hpp", "scan_fwd.hpp", "ssm_scan.hip")),
                  ("decode_", ("common.hpp", "scan_fwd.hpp", "ssm_scan.hip")),
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


def bwd_traffic():
    """HBM bytes of one ssm_scan_bwd call on the 2.8B layer: prep, carry and main (the two reductions move under 1% of
    it and have no record); None unless every record is current."""
    parts = [measured_traffic("bwd_%s mamba2.8b-layer" % k)
             for k in ("prep_kernel<bf16,bf16,euler,gate>", "carry_kernel", "main_kernel<bf16,bf16,euler,gate>")]
    return None if any(v is None for v in parts) else sum(parts)


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


# launches timed per workload leg (each leg also does a spin-up and two untimed warm-up launches)
LEG_STEPS = {"tiny-s6-fp32": 100, "mamba130m-layer": 50, "mamba2.8b-layer": 50, "million-length": 10}
# the oracle's bounded sample per workload leg: channels (of b * D, taken from the start) or None for all
LEG_CPU_CHANNELS = {"tiny-s6-fp32": None, "mamba130m-layer": None, "mamba2.8b-layer": None, "million-length": 64}


def workload_leg(torch, np, ssm, I, up, w, dev, stream, steps=None, cpu=True, log=None):
    """Forward scan of one workload as the product runs it (y in the io dtype): per-launch times, elements/s, the HBM
    and ALU roofline fractions, and, with cpu, the fp64 oracle timed on a bounded sample of the same inputs (which
    also checks the fp32-y result on that sample)."""
    b, D, L, N = w.batch, w.dim, w.seqlen, w.dstate
    io_bytes = 4 if w.io == I.F32 else 2
    if log:
        log("workload %s: generating inputs" % w.name)
    host = I.scan_inputs(w)
    d = {k: up(v) for k, v in host.items()}
    ydt = torch.float32 if w.io == I.F32 else torch.bfloat16
    y = torch.empty((b, D, L), dtype=ydt, device=dev)
    hf = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    p = ssm.make_params(b, D, L, N, ssm.io_code(ydt), ssm.io_code(ydt))
    nseg = ssm.plan_segments(p)
    ws_n = ssm.workspace_bytes(p)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    from selective_state_space_57_amd import _abi

    # arguments marshalled once (the binding's per-call checks would leave the GPU idle between short launches)
    sargs = (d["x"].data_ptr(), d["dt"].data_ptr(), d["dt_bias"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(),
             d["C"].data_ptr(), d["Dskip"].data_ptr(), d["z"].data_ptr(), 0, y.data_ptr(), hf.data_ptr(),
             ws.data_ptr() if ws_n else 0, ws_n, stream.cuda_stream)

    def step():
        st = _abi.scan_fwd_raw(p, *sargs)
        if st:
            _abi.check(st)

    spin_up(torch, stream, step)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    n = steps or LEG_STEPS.get(w.name, 20)
    ms, per = time_launches(torch, stream, step, n)
    elems = b * D * L
    nbytes = scan_algorithmic_bytes(b, D, L, N, io_bytes, w.gate, w.dskip)
    slots = scan_algorithmic_slots(b, D, L, N, w.gate, w.dskip)
    io = "f32" if w.io == I.F32 else "bf16"
    key = "scan_kernel<%s,%s,euler,gate,dskip> %s" % (io, io, w.name)
    leg = {"workload": w.name, "batch": b, "d_inner": D, "seqlen": L, "d_state": N, "io": io, "segments": nseg,
           "kernels": ("segments pass + carry + correction pass (one ssm_scan_fwd call)" if nseg > 1 else "scan"),
           "launches": n, "ms_per_step": ms, "warm": pct(per), "elements_per_s": elems / (ms * 1e-3),
           "hbm": hbm_roofline(nbytes, ms, measured_traffic(key), key),
           "roofline": alu_roofline(slots, ms, key, measured_traffic(key))}
    if log:
        log("workload %s: %.4f ms per call (%d segments)" % (w.name, ms, nseg))
    if cpu:
        import oracle
        oracle.build(force=False)
        y32 = torch.empty((b, D, L), dtype=torch.float32, device=dev)
        ssm.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], dt_bias=d["dt_bias"], Dskip=d["Dskip"], z=d["z"],
                     y=y32, h_final=hf, workspace=ws if ws_n else None, stream=stream)
        torch.cuda.synchronize()
        nch = LEG_CPU_CHANNELS.get(w.name)
        sub = dict(host)
        if nch is not None:   # the first nch channels of batch element 0
            for k in ("x", "dt", "z"):
                sub[k] = host[k][:1, :nch]
            for k in ("B", "C"):
                sub[k] = host[k][:1]
            for k in ("A", "dt_bias", "Dskip"):
                sub[k] = host[k][:nch]
            yg = y32[:1, :nch].cpu().numpy().astype(np.float64)
            hg = hf[:1, :nch].cpu().numpy().astype(np.float64)
        else:
            yg = y32.cpu().numpy().astype(np.float64)
            hg = hf.cpu().numpy().astype(np.float64)
        del y32
        f = I.as_f64(sub)
        cores = host_cores()
        t0 = time.perf_counter()
        yr, hr = oracle.scan(f["x"], f["dt"], f["A"], f["B"], f["C"], dt_bias=f["dt_bias"], Dskip=f["Dskip"],
                             z=f["z"], nthreads=cores)
        cs = time.perf_counter() - t0
        ey = float(np.max(np.abs(yg - yr))) / float(np.sqrt(np.mean(yr * yr)))
        eh = float(np.max(np.abs(hg - hr))) / float(np.sqrt(np.mean(hr * hr)))
        tol = 1e-5 if w.io == I.F32 else 3e-3
        leg["cpu_baseline"] = {"value": yr.size / cs, "unit": "elements/s", "cores": cores, "kind": "oracle",
                               "seconds": cs,
                               "sample": ("the whole workload" if nch is None else
                                          "channels 0..%d of batch element 0, all %d steps" % (nch - 1, L)) + ", fp64"}
        leg["parity_on_cpu_sample"] = {"max_abs_err_over_rms_y": ey, "h_final_err_over_rms": eh, "tolerance": tol,
                                       "pass": bool(ey <= tol and eh <= tol), "elements": int(yr.size)}
        if log:
            log("workload %s: oracle %.2f s on %d cores, err y %.2e h %.2e" % (w.name, cs, cores, ey, eh))
    return leg


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
    ap.add_argument("--no-zoh", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=20)
    ap.add_argument("--no-configs", action="store_true", help="skip the legs of the other scan workloads")
    ap.add_argument("--workload", default=None,
                    help="run only the forward scan of this workload (tiny-s6-fp32, mamba130m-layer, "
                         "mamba2.8b-layer, million-length) for a few launches: for profiling")
    ap.add_argument("--issue-rates-only", action="store_true", help="only run the issue-rate probe")
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
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": src.numel() * 4,
                          "copy_calibration_bytes_written_per_launch": dst.numel() * 4}), flush=True)
        return
    if args.issue_rates_only:
        print(json.dumps({"issue_rates": issue_rates(torch, dev, stream)}), flush=True)
        return

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    def log(msg):
        print("bench: " + msg, file=sys.stderr, flush=True)

    if args.workload:
        w = next(w_ for w_ in I.WORKLOADS.values() if w_.name == args.workload and not w_.decode_steps)
        leg = workload_leg(torch, np, ssm, I, up, w, dev, stream, steps=max(1, args.steps), cpu=False, log=log)
        print(json.dumps({"workload_leg": leg}), flush=True)
        return

    w = I.WORKLOADS[2]
    b, D, L, N = w.batch, w.dim, w.seqlen, w.dstate
    log("headline workload %s: generating inputs" % w.name)
    host = I.scan_inputs(w)
    d = {k: up(v) for k, v in host.items()}
    y = torch.empty((b, D, L), dtype=torch.bfloat16, device=dev)
    hf = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    p = ssm.make_params(b, D, L, N, ssm.SSM_BF16, ssm.SSM_BF16)
    nseg = ssm.plan_segments(p)
    ws_n = ssm.workspace_bytes(p)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    from selective_state_space_57_amd import _abi
    # arguments marshalled once: the binding's per-call checks take about as long as the kernel, so timing through
    # it would measure the host (the GPU would idle between launches)
    sargs = (d["x"].data_ptr(), d["dt"].data_ptr(), d["dt_bias"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(),
             d["C"].data_ptr(), d["Dskip"].data_ptr(), d["z"].data_ptr(), 0, y.data_ptr(), hf.data_ptr(),
             ws.data_ptr() if ws_n else 0, ws_n, stream.cuda_stream)

    def step():
        st = _abi.scan_fwd_raw(p, *sargs)
        if st:
            _abi.check(st)

    # Spin-up: the GPU leaves its idle power state only after some tens of milliseconds of load (measured: the first
    # 100 back-to-back launches after a 10-launch warm-up average 0.388 ms, every later 100 0.365-0.369 ms, and after
    # 1 s idle the first 100 again 0.391 ms).  So before the W warm-up steps the same launch runs, untimed, until about
    # SPIN_UP_MS of GPU time have passed; the timed steps then measure the kernel under continuous load.
    spin_n = spin_up(torch, stream, step)
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
    # the same launches, each between two events: per-launch spread (a clock droop under sustained load shows as a
    # rising median over p10)
    _, per_launch = time_launches(torch, stream, step, max(10, args.steps))
    log("headline: %.4f ms per step" % ms)

    elems = b * D * L
    value = elems / (ms * 1e-3)
    nbytes = scan_algorithmic_bytes(b, D, L, N)
    slots = scan_algorithmic_slots(b, D, L, N)
    kernel_key = "scan_kernel<bf16,bf16,euler,gate,dskip> mamba2.8b-layer"
    traffic = measured_traffic(kernel_key)

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
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
                "frac_of_8TBps": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "roofline": hbm_roofline(nbytes, ms, traffic, kernel_key)},
        "roofline": alu_roofline(slots, ms, kernel_key, traffic,
                                 {"hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "slots_per_element": scan_elem_slots(N)}),
        "warm": dict(pct(per_launch), launches=len(per_launch),
                     note="back-to-back launches, an event between consecutive ones"),
        "host_wall_ms_timed_region": wall_ms,
        "spin_up": {"launches": spin_n, "target_ms": SPIN_UP_MS,
                    "note": "untimed launches before the warm-up steps, until the GPU has left its idle power state"},
    }
    log("issue-rate probe")
    out["issue_rates"] = issue_rates(torch, dev, stream)

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
    out["hbm"]["frac_of_copy_ceiling"] = out["hbm"]["achieved_GBps"] / copy_gbs
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

    # ---- the other scan workloads (the tiny fp32 case, the 130M layer, the million-length sequence)
    if not args.no_configs:
        out["workloads"] = {}
        for cfg in (0, 1, 3):
            wk = I.WORKLOADS[cfg]
            out["workloads"][wk.name] = workload_leg(torch, np, ssm, I, up, wk, dev, stream,
                                                     cpu=not args.no_cpu_baseline, log=log)
            torch.cuda.empty_cache()

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

        spin_up(torch, stream, cstep)
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
        csl = slots + conv_algorithmic_slots(b, D, L, 4)
        out["conv_scan"] = {"workload": "mamba2.8b-layer + causal conv1d (width 4) + SiLU", "ms_per_step": cms,
                            "elements_per_s": elems / (cms * 1e-3), "overhead_vs_scan": cms / ms - 1.0,
                            "roofline": alu_roofline(csl, cms, "scan_kernel<bf16,bf16,euler,gate,dskip,conv>",
                                                     measured_traffic("scan_kernel<bf16,bf16,euler,gate,dskip,conv> "
                                                                      "mamba2.8b-layer")),
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
            spin_up(torch, stream, fn)
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

    # ---- the same forward under the ZOH rule, Bbar = expm1(Delta A) / A * B
    if not args.no_zoh:
        from selective_state_space_57_amd import _abi
        pz = ssm.make_params(b, D, L, N, ssm.SSM_BF16, ssm.SSM_BF16, disc=ssm.ZOH)
        zws_n = ssm.workspace_bytes(pz)
        zws = torch.empty(max(zws_n, 1), dtype=torch.uint8, device=dev)
        zargs = sargs[:-3] + (zws.data_ptr() if zws_n else 0, zws_n, stream.cuda_stream)

        def zstep():
            st = _abi.scan_fwd_raw(pz, *zargs)
            if st:
                _abi.check(st)

        spin_up(torch, stream, zstep)
        for _ in range(5):
            zstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            zstep()
        e1.record(stream)
        torch.cuda.synchronize()
        zms = e0.elapsed_time(e1) / args.steps
        zsl = float(zoh_elem_slots(N)) * elems
        out["zoh"] = {"workload": "mamba2.8b-layer, ZOH rule for Bbar", "ms_per_step": zms,
                      "elements_per_s": elems / (zms * 1e-3), "ratio_to_euler": zms / ms,
                      "slots_per_element": zoh_elem_slots(N),
                      "roofline": alu_roofline(zsl, zms, "scan_kernel<bf16,bf16,zoh,gate,dskip> mamba2.8b-layer",
                                               measured_traffic("scan_kernel<bf16,bf16,zoh,gate,dskip> "
                                                                "mamba2.8b-layer"),
                                               {"hbm_frac": nbytes / (zms * 1e-3) / 1e9 / HBM_PEAK_GBS})}
        del zws

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

        spin_up(torch, stream, xstep)
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
        xsl = complex_algorithmic_slots(b, D, L, N)
        out["complex_scan"] = {"workload": "mamba2.8b-layer shape, complex diagonal A (S4D-Lin), complex B, C",
                               "ms_per_step": xms, "elements_per_s": elems / (xms * 1e-3),
                               "ratio_to_real_scan": xms / ms,
                               "roofline": alu_roofline(xsl, xms, "complex_scan_kernel mamba2.8b-layer",
                                                        measured_traffic("complex_scan_kernel mamba2.8b-layer"))}

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

        spin_up(torch, stream, sstep)
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

        spin_up(torch, stream, lambda: sdstep(0))   # (the state's values do not change the timing)
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

        spin_up(torch, stream, bstep)
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
        bsl = bwd_algorithmic_slots(b, D, L, N)
        bby = bwd_algorithmic_bytes(b, D, L, N)
        out["bwd"] = {"workload": "mamba2.8b-layer", "steps": args.bwd_steps, "ms_per_step": bms,
                      "elements_per_s": elems / (bms * 1e-3), "ratio_to_forward": bms / ms,
                      "kernels": "prep + carry + main + 2 reduce (one ssm_scan_bwd call)",
                      "roofline": alu_roofline(bsl, bms, "ssm_scan_bwd (all five kernels)", bwd_traffic()),
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

        # (spin-up on a scratch copy of the state: the timed steps start from the generated one)
        spin_state = state.clone()
        spin_args = (spin_state.data_ptr(),) + dargs[0][1:]
        spin_up(torch, stream, lambda: _abi.state_update_raw(pd, *spin_args))
        del spin_state
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
        dkey = "decode_vec_kernel<bf16,bf16,euler> decode-b256-d5120"
        out["decode"] = {"workload": "decode-b256-d5120", "steps": wd.decode_steps, "us_per_step": dms * 1e3,
                         "algorithmic_bytes_per_step": dbytes, "achieved_GBps": dbytes / (dms * 1e-3) / 1e9,
                         "frac_of_8TBps": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "roofline": hbm_roofline(dbytes, dms, measured_traffic(dkey), dkey),
                         "traffic": measured_traffic(dkey),
                         "note": "64 consecutive steps, each with its own pre-generated x/dt/z/B/C tensors; the 84 MB "
                                 "fp32 state can be partly served by the 256 MB Infinity Cache"}
        # the same 64 steps with each step's inputs first copied on the GPU into fixed buffers, as when the layer's
        # input projection has just produced them (in cache and address translation warm); only the decode launch
        # is timed
        wbuf = {k: torch.empty_like(steps_in[0][k]) for k in ("x", "dt", "z", "B", "C")}
        wargs = (state.data_ptr(), wbuf["x"].data_ptr(), wbuf["dt"].data_ptr(), steps_in[0]["dt_bias"].data_ptr(),
                 steps_in[0]["A"].data_ptr(), wbuf["B"].data_ptr(), wbuf["C"].data_ptr(),
                 steps_in[0]["Dskip"].data_ptr(), wbuf["z"].data_ptr(), yd.data_ptr(), sh)
        wt = []
        for s in range(wd.decode_steps):
            for k in wbuf:
                wbuf[k].copy_(steps_in[s][k])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st_ = _abi.state_update_raw(pd, *wargs)
            e1.record(stream)
            if st_:
                _abi.check(st_)
            wt.append((e0, e1))
        torch.cuda.synchronize()
        wus = sorted(a.elapsed_time(b_) * 1e3 for a, b_ in wt)
        wmed = wus[len(wus) // 2]
        out["decode"]["producer_warm"] = {
            "us_per_step_median": wmed, "us_p10": wus[len(wus) // 10], "us_p90": wus[(9 * len(wus)) // 10],
            "achieved_GBps": dbytes / (wmed * 1e-6) / 1e9, "frac_of_8TBps": dbytes / (wmed * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "each step's x, dt, z, B, C copied on the GPU into fixed buffers just before the step (as a preceding "
                    "projection would leave them); the decode launch alone is timed"}
        del wbuf
        # the same 64 steps (fresh inputs) with the 256 MB Infinity Cache evicted before each (512 MB written by a fill
        # kernel on the stream): the state then comes from HBM rather than from the cache the previous step filled
        flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        ct = []
        for s in range(wd.decode_steps):
            flush.fill_(float(s))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dstep(s)
            e1.record(stream)
            ct.append((e0, e1))
        torch.cuda.synchronize()
        del flush
        cus = sorted(a.elapsed_time(b_) * 1e3 for a, b_ in ct)
        cmed = cus[len(cus) // 2]
        out["decode"]["cold"] = {
            "us_per_step_median": cmed, "us_p10": cus[len(cus) // 10], "us_p90": cus[(9 * len(cus)) // 10],
            "achieved_GBps": dbytes / (cmed * 1e-6) / 1e9, "frac_of_8TBps": dbytes / (cmed * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "flush": "512 MB written by a fill kernel before each step; each step timed alone"}
        if not args.no_cpu_baseline:
            import oracle
            oracle.build(force=False)
            st64 = I.decode_state(wd).astype(np.float64)
            cs = []
            for s_ in range(4):
                f = I.as_f64(I.scan_inputs(wd, step=s_))
                t0 = time.perf_counter()
                _, st64 = oracle.state_update(st64, f["x"], f["dt"], f["A"], f["B"], f["C"], dt_bias=f["dt_bias"],
                                              Dskip=f["Dskip"], z=f["z"], nthreads=host_cores())
                cs.append(time.perf_counter() - t0)
            cps = sorted(cs)[len(cs) // 2]
            out["decode"]["cpu_baseline"] = {"value": cps * 1e6, "unit": "us/step", "cores": host_cores(),
                                             "kind": "oracle", "seconds_per_step": cps,
                                             "sample": "4 steps of the same workload (all 256 x 5120 channels), "
                                                       "median, fp64"}
        del state, steps_in

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
