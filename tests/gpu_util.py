"""Helpers for the GPU parity tests: upload storage arrays, run the HIP path, run the oracle on the same values."""
from __future__ import annotations

import numpy as np

import oracle
from selective_state_space_57_amd import inputs as I

SEQ_KEYS = ("x", "dt", "z")


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch


def to_dev(d: dict) -> dict:
    torch = torch_dev()
    out = {}
    for k, v in d.items():
        if v is None:
            out[k] = None
        elif v.dtype == np.uint16:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).view(torch.bfloat16).cuda()
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()
    return out


def to_np64(t) -> np.ndarray:
    torch = torch_dev()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(dd: dict, disc=0, y_dtype=None, segments=0, softplus=True, h0=None):
    import selective_state_space_57_amd as ssm
    torch = torch_dev()
    y, hf = ssm.scan_fwd(dd["x"], dd["dt"], dd["A"], dd["B"], dd["C"], dt_bias=dd["dt_bias"], Dskip=dd["Dskip"],
                         z=dd["z"], h0=dd["h0"] if h0 is None else h0, y_dtype=y_dtype, disc=disc,
                         softplus=softplus, segments=segments)
    torch.cuda.synchronize()
    return y, hf


def oracle_ref(d: dict, disc=0, softplus=True, chans=None, nthreads=0):
    """Oracle on the exact (rounded) input values; chans = list of (b, d) to compute only those channels."""
    if chans is None:
        f = I.as_f64(d)
        return oracle.scan(f["x"], f["dt"], f["A"], f["B"], f["C"], dt_bias=f["dt_bias"], Dskip=f["Dskip"],
                           z=f["z"], h0=f["h0"], disc=disc, softplus=softplus, nthreads=nthreads)
    ys, hs = [], []
    f64 = lambda a: None if a is None else I.to_f64(a)
    for (bi, di) in chans:
        sl = lambda a: None if a is None else f64(a[bi:bi + 1, di:di + 1])
        y, h = oracle.scan(sl(d["x"]), sl(d["dt"]), f64(d["A"][di:di + 1]), f64(d["B"][bi:bi + 1]),
                           f64(d["C"][bi:bi + 1]),
                           dt_bias=None if d["dt_bias"] is None else f64(d["dt_bias"][di:di + 1]),
                           Dskip=None if d["Dskip"] is None else f64(d["Dskip"][di:di + 1]), z=sl(d["z"]),
                           h0=sl(d["h0"]), disc=disc, softplus=softplus, nthreads=nthreads)
        ys.append(y[0, 0])
        hs.append(h[0, 0])
    return np.stack(ys), np.stack(hs)


def rel_max(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / rms(ref)."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def bf16_rne(a: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(I.f32_to_bf16_bits(np.asarray(a, np.float32)))


# tolerances, max |got - ref| / rms(ref): fp32 I/O 1e-5 (fp32 rounding of the recurrence, which grows at most with
# the decay memory, about 1e3 steps times 2^-24); bf16 I/O with fp32 state 3e-3, measured with fp32 y (rounding y to
# bf16 alone moves it by up to 2^-8 |y|, so bf16 y is instead checked bit-equal to the rounded fp32 y)
TOL_F32 = 1e-5
TOL_BF16 = 3e-3


def tol_for(io: str) -> float:
    return TOL_F32 if io == I.F32 else TOL_BF16


def sample_channels(b, D, k, seed=0):
    r = np.random.default_rng(seed)
    ch = {(0, 0), (b - 1, D - 1), (0, D - 1), (b - 1, 0)}
    while len(ch) < min(k, b * D):
        ch.add((int(r.integers(b)), int(r.integers(D))))
    return sorted(ch)
