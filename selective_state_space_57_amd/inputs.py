"""Seeded synthetic inputs for the selective scan (shared by the tests, the benchmark and the oracle's callers).

This module holds no part of the scan's arithmetic: it draws random numbers, rounds them to the storage dtype and
converts storage formats.  Nothing here imports the HIP binding or the oracle.

Workloads (sizes b, D, L, N) follow the Mamba paper's settings: N = 16 states per channel (paper section 4.5/4.6
ablations, state dimension 16), d_inner = E * d_model with E = 2 (section 3.4), layer shapes of the 130M and 2.8B
models, million-length sequences as in the DNA and audio experiments (sections 4.3-4.4), and large-batch recurrent
decode (section 4.5).  Initialisations follow section 3.6: A from S4D-Real, A_n = -(n+1), and the Delta bias drawn as
softplus^-1 of a value log-uniform in a range around [0.001, 0.1].

Recipe:
  * every tensor k of workload `cfg` at decode step `step` is drawn in flattened chunks of 2**24 elements, chunk i
    from numpy's default_rng(SeedSequence(57, spawn_key=(cfg, step, k, i)));
  * tensor order k: 0 x, 1 Delta*, 2 bias, 3 A-jitter, 4 B, 5 C, 6 Dskip, 7 z, 8 h0/state, 9 dy, 10 dh_final
    (the cotangents fed to the backward pass), 11 conv weight, 12 conv bias, 13 conv state (the causal convolution
    in front of the scan: weight and bias U(-1/sqrt(width), 1/sqrt(width)), the default init of a 1-D convolution
    with one input channel per group; state N(0, 1)), 14 imaginary part of B, 15 imaginary part of C, 16 imaginary
    part of h0 and 17 the jitter of A's imaginary part (the complex-A variant; A is S4D-Lin, A_n = -1/2 + n i, with
    the same N(0, a_jitter) jitter on both parts);
  * normals are numpy float32 standard normals; log-uniforms are exp(uniform(log lo, log hi)) in float64;
  * Delta-logit = softplus^-1(Delta*) - bias[d], with softplus^-1(v) = log(expm1(v)), rounded to the io dtype;
  * bf16 values are rounded to nearest-even from float32 (float64 -> float32 -> bf16 for float64 sources).

Mamba-2 SSD workloads (SSDWorkload: batch, seqlen, nheads H, headdim P, ngroups G, dstate N) use the same tensor
order and seeding with their own workload ids: 0 x (b, L, H, P), 1 Delta* (b, L, H), 2 bias (H), 3 A (H): minus a
log-uniform value in [1, 16] (the range S4D-Real's -(n+1) spans for N = 16, one scalar per head), 4 B and 5 C
(b, L, G, N), 6 Dskip (H), 7 z (b, L, H, P), 8 h0 (b, H, P, N).  Delta-logit = softplus^-1(Delta*) - bias[h].
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np

CHUNK = 1 << 24
SEED = 57

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    io: str                 # "f32" or "bf16" for x, dt, B, C, z (and y)
    delta_lo: float
    delta_hi: float
    a_jitter: float         # std of the N(0, s) jitter added to A = -(n+1); 0 = exact S4D-Real
    gate: bool = True
    dskip: bool = True
    decode_steps: int = 0   # > 0: single-token decode workload, seqlen ignored
    cfg_id: int = 0

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    0: Workload("tiny-s6-fp32", 1, 64, 256, 16, F32, 1e-3, 1e-1, 0.0, cfg_id=0),
    1: Workload("mamba130m-layer", 8, 1536, 2048, 16, BF16, 1e-3, 1e-1, 0.1, cfg_id=1),
    2: Workload("mamba2.8b-layer", 4, 5120, 4096, 16, BF16, 1e-3, 1e-1, 0.1, cfg_id=2),
    3: Workload("million-length", 1, 512, 1 << 20, 16, BF16, 1e-4, 1e-1, 0.1, cfg_id=3),
    4: Workload("decode-b256-d5120", 256, 5120, 1, 16, BF16, 1e-3, 1e-1, 0.1, decode_steps=64, cfg_id=4),
}


@dataclasses.dataclass(frozen=True)
class SSDWorkload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    io: str
    delta_lo: float
    delta_hi: float
    gate: bool = True
    dskip: bool = True
    decode_steps: int = 0
    cfg_id: int = 100

    @property
    def elements(self) -> int:
        """b * D * L with D = nheads * headdim channels (the same count as the S6 workloads)."""
        return self.batch * self.nheads * self.headdim * self.seqlen

    def replace(self, **kw) -> "SSDWorkload":
        return dataclasses.replace(self, **kw)


# Mamba-2 2.7B (close reading, Mamba-2 paragraph): d_model 2560, expand 2 -> 5120 channels = 80 heads of 64, N = 128,
# one group; the layer is run at the same batch and length as the Mamba-2.8B S6 layer above.
SSD_WORKLOADS = {
    0: SSDWorkload("tiny-ssd", 1, 200, 4, 64, 1, 128, BF16, 1e-3, 1e-1, cfg_id=100),
    1: SSDWorkload("mamba2-2.7b-layer", 4, 4096, 80, 64, 1, 128, BF16, 1e-3, 1e-1, cfg_id=101),
    2: SSDWorkload("mamba2-decode-b256", 256, 1, 80, 64, 1, 128, BF16, 1e-3, 1e-1, decode_steps=8, cfg_id=102),
}


def _rng(cfg: int, step: int, k: int, i: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=(cfg, step, k, i)))


def _chunks(n):
    for i, s in enumerate(range(0, n, CHUNK)):
        yield i, s, min(n, s + CHUNK)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _fill(n, fn):
    """Run fn(i, s, e) for every chunk; chunks are seeded independently, so the order does not matter."""
    ch = list(_chunks(n))
    if len(ch) <= 1:
        for c in ch:
            fn(*c)
        return
    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda c: fn(*c), ch))


def _normal(cfg, step, k, n) -> np.ndarray:
    out = np.empty(n, np.float32)

    def f(i, s, e):
        out[s:e] = _rng(cfg, step, k, i).standard_normal(e - s, dtype=np.float32)
    _fill(n, f)
    return out


def _loguniform_chunk(cfg, step, k, i, m, lo, hi) -> np.ndarray:
    v = _rng(cfg, step, k, i).uniform(np.log(lo), np.log(hi), m)
    np.exp(v, out=v)
    return v


def _loguniform(cfg, step, k, n, lo, hi) -> np.ndarray:
    out = np.empty(n, np.float64)
    for i, s, e in _chunks(n):
        out[s:e] = _loguniform_chunk(cfg, step, k, i, e - s, lo, hi)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even), returned as uint16 bit patterns.  Finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a: np.ndarray, io: str) -> np.ndarray:
    """float32/float64 values -> storage array (float32, or uint16 bf16 bits)."""
    a32 = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a32) if io == BF16 else np.ascontiguousarray(a32)


def to_f64(a: np.ndarray, io: str | None = None) -> np.ndarray:
    """Storage array -> exact float64 values."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _softplus_inv(v: np.ndarray) -> np.ndarray:
    # inverse of log(1 + e^u): u = log(e^v - 1); used only to place the drawn Delta values, not part of the scan
    return np.log(np.expm1(v))


def _storage_empty(n, io):
    return np.empty(n, np.uint16 if io == BF16 else np.float32)


def _normal_storage(cfg, step, k, n, io) -> np.ndarray:
    out = _storage_empty(n, io)

    def f(i, s, e):
        out[s:e] = to_storage(_rng(cfg, step, k, i).standard_normal(e - s, dtype=np.float32), io)
    _fill(n, f)
    return out


def scan_inputs(w: Workload, step: int = 0, with_h0: bool = False) -> dict:
    """Inputs for ssm_scan_fwd (or one decode step when w.decode_steps > 0, with seqlen = 1 squeezed away).

    Returns a dict of storage arrays: x, dt, z (b, D, L); B, C (b, N, L); A (D, N) f32; dt_bias, Dskip (D,) f32;
    h0 (b, D, N) f32 or None.  For decode workloads the sequence tensors are (b, D) and (b, N).
    """
    b, D, N = w.batch, w.dim, w.dstate
    L = 1 if w.decode_steps else w.seqlen
    c = w.cfg_id
    io = w.io
    nx = b * D * L
    # the bias is a per-channel parameter: drawn once (decode step 0) and reused by every step
    bias = _softplus_inv(_loguniform(c, 0, 2, D, w.delta_lo, w.delta_hi)).astype(np.float32)
    base = -(np.arange(N, dtype=np.float64) + 1.0)
    if w.a_jitter > 0:
        jit = _normal(c, 0, 3, D * N).astype(np.float64).reshape(D, N) * w.a_jitter
        A = np.minimum(base[None, :] + jit, -1e-4)
    else:
        A = np.broadcast_to(base, (D, N)).copy()
    A = A.astype(np.float32)
    x = _normal_storage(c, step, 0, nx, io)
    dt = _storage_empty(nx, io)
    bias64 = bias.astype(np.float64)

    def fdt(i, s, e):
        v = _loguniform_chunk(c, step, 1, i, e - s, w.delta_lo, w.delta_hi)   # Delta*
        np.expm1(v, out=v)                                                   # softplus^-1(Delta*) ...
        np.log(v, out=v)
        if L >= 64:                                                          # ... minus the channel's bias
            for r in range(s // L, (e - 1) // L + 1):
                v[max(s, r * L) - s:min(e, (r + 1) * L) - s] -= bias64[r % D]
        else:
            v -= bias64[(np.arange(s, e, dtype=np.int64) // L) % D]
        dt[s:e] = to_storage(v, io)
    _fill(nx, fdt)
    Bm = _normal_storage(c, step, 4, b * N * L, io)
    Cm = _normal_storage(c, step, 5, b * N * L, io)
    Dskip = _normal(c, 0, 6, D) if w.dskip else None
    z = _normal_storage(c, step, 7, nx, io) if w.gate else None
    shp = (b, D) if w.decode_steps else (b, D, L)
    bshp = (b, N) if w.decode_steps else (b, N, L)
    out = {
        "x": x.reshape(shp),
        "dt": dt.reshape(shp),
        "dt_bias": bias,
        "A": A,
        "B": Bm.reshape(bshp),
        "C": Cm.reshape(bshp),
        "Dskip": None if Dskip is None else Dskip.astype(np.float32),
        "z": None if z is None else z.reshape(shp),
        "h0": None,
    }
    if with_h0:
        out["h0"] = _normal(c, 0, 8, b * D * N).reshape(b, D, N)
    return out


def cotangents(w: Workload, step: int = 0, io: str | None = None, with_dh_final: bool = False) -> dict:
    """Cotangents for the backward pass: dy (b, D, L) N(0, 1) in storage dtype `io` (default: the workload's) and,
    optionally, dh_final (b, D, N) f32 N(0, 1)."""
    b, D, N, L = w.batch, w.dim, w.dstate, w.seqlen
    c = w.cfg_id
    dy = _normal_storage(c, step, 9, b * D * L, io or w.io).reshape(b, D, L)
    dhf = _normal(c, step, 10, b * D * N).reshape(b, D, N) if with_dh_final else None
    return {"dy": dy, "dh_final": dhf}


def random_small_cotangents(seed: int, b: int, D: int, L: int, N: int, io: str = F32, dh_final=False) -> dict:
    """Cotangents matching random_small(seed, ...)."""
    w = Workload("small", b, D, L, N, io, 1e-3, 1e-1, 0.0, cfg_id=1000 + seed)
    return cotangents(w, io=io, with_dh_final=dh_final)


def conv_params(w: Workload, width: int = 4, with_state: bool = False) -> dict:
    """Causal convolution parameters for workload w: weight (D, width), bias (D,), state (b, D, width-1) or None."""
    c, D = w.cfg_id, w.dim
    bound = 1.0 / np.sqrt(width)
    wt = (_rng(c, 0, 11, 0).uniform(-bound, bound, D * width)).astype(np.float32).reshape(D, width)
    bias = _rng(c, 0, 12, 0).uniform(-bound, bound, D).astype(np.float32)
    st = _normal(c, 0, 13, w.batch * D * (width - 1)).reshape(w.batch, D, width - 1) if with_state else None
    return {"conv_w": wt, "conv_b": bias, "conv_state": st}


def random_small_conv(seed: int, b: int, D: int, N: int, width: int = 4, with_state: bool = False) -> dict:
    """Convolution parameters matching random_small(seed, ...)."""
    w = Workload("small", b, D, 1, N, F32, 1e-3, 1e-1, 0.0, cfg_id=1000 + seed)
    return conv_params(w, width, with_state)


def complex_inputs(w: Workload, step: int = 0, with_h0: bool = False) -> dict:
    """Inputs of the complex-A scan: x, dt, z, dt_bias, Dskip as scan_inputs; A (D, N, 2) f32 S4D-Lin; B, C
    (b, N, L, 2) in storage dtype (real parts = scan_inputs' B, C); h0 (b, D, N, 2) f32 or None.  Decode workloads
    drop the seqlen axis as in scan_inputs."""
    d = scan_inputs(w, step, with_h0=False)
    b, D, N = w.batch, w.dim, w.dstate
    L = 1 if w.decode_steps else w.seqlen
    c, io = w.cfg_id, w.io
    nbc = b * N * L
    re = -0.5 + (_normal(c, 0, 3, D * N).astype(np.float64).reshape(D, N) * w.a_jitter if w.a_jitter > 0 else 0.0)
    im = np.arange(N, dtype=np.float64)[None, :] + (
        _normal(c, 0, 17, D * N).astype(np.float64).reshape(D, N) * w.a_jitter if w.a_jitter > 0 else 0.0)
    A = np.stack([np.minimum(re, -1e-4) * np.ones((D, N)), im * np.ones((D, N))], axis=-1).astype(np.float32)
    bshp = (b, N) if w.decode_steps else (b, N, L)
    Bi = _normal_storage(c, step, 14, nbc, io).reshape(bshp)
    Ci = _normal_storage(c, step, 15, nbc, io).reshape(bshp)
    d["A"] = A
    d["B"] = np.ascontiguousarray(np.stack([d["B"], Bi], axis=-1))
    d["C"] = np.ascontiguousarray(np.stack([d["C"], Ci], axis=-1))
    if with_h0:
        d["h0"] = np.stack([_normal(c, 0, 8, b * D * N).reshape(b, D, N), _normal(c, 0, 16, b * D * N).reshape(b, D, N)],
                           axis=-1).astype(np.float32)
    return d


def complex_as_oracle(d: dict) -> dict:
    """Storage dict of complex_inputs -> oracle arguments (float64 / complex128)."""
    f = {k: (None if v is None else to_f64(v)) for k, v in d.items()}
    for k in ("A", "B", "C", "h0"):
        if f.get(k) is not None:
            f[k] = f[k][..., 0] + 1j * f[k][..., 1]
    return f


def decode_state(w: Workload) -> np.ndarray:
    """Initial decode state (b, D, N) f32, N(0, 1)."""
    return _normal(w.cfg_id, 0, 8, w.batch * w.dim * w.dstate).reshape(w.batch, w.dim, w.dstate)


def random_small(seed: int, b: int, D: int, L: int, N: int, io: str = F32, delta=(1e-3, 1e-1), a_jitter=0.1,
                 gate=True, dskip=True, bias=True, h0=False) -> dict:
    """Small random case for parity sweeps (odd sizes, optional parts switched off)."""
    w = Workload("small", b, D, L, N, io, delta[0], delta[1], a_jitter, gate, dskip, cfg_id=1000 + seed)
    d = scan_inputs(w, with_h0=h0)
    if not bias:
        # fold the bias into the logit so that the same Delta values are produced without a bias vector
        lg = to_f64(d["dt"]) + d["dt_bias"].astype(np.float64)[None, :, None]
        d["dt"] = to_storage(lg, io)
        d["dt_bias"] = None
    return d


def ssd_inputs(w: SSDWorkload, step: int = 0, with_h0: bool = False) -> dict:
    """Inputs of the SSD layer as storage arrays: x, z (b, L, H, P); dt (b, L, H); B, C (b, L, G, N); A, dt_bias,
    Dskip (H,) f32; h0 (b, H, P, N) f32 or None.  Decode workloads drop the L axis."""
    b, H, P, G, N = w.batch, w.nheads, w.headdim, w.ngroups, w.dstate
    L = 1 if w.decode_steps else w.seqlen
    c, io = w.cfg_id, w.io
    bias = _softplus_inv(_loguniform(c, 0, 2, H, w.delta_lo, w.delta_hi)).astype(np.float32)
    A = (-_loguniform(c, 0, 3, H, 1.0, 16.0)).astype(np.float32)
    nx = b * L * H * P
    ndt = b * L * H
    x = _normal_storage(c, step, 0, nx, io)
    bias64 = bias.astype(np.float64)
    dt = _storage_empty(ndt, io)

    def fdt(i, s0, e):
        v = _loguniform_chunk(c, step, 1, i, e - s0, w.delta_lo, w.delta_hi)
        np.expm1(v, out=v)
        np.log(v, out=v)
        v -= bias64[np.arange(s0, e, dtype=np.int64) % H]
        dt[s0:e] = to_storage(v, io)
    _fill(ndt, fdt)
    Bm = _normal_storage(c, step, 4, b * L * G * N, io)
    Cm = _normal_storage(c, step, 5, b * L * G * N, io)
    Dskip = _normal(c, 0, 6, H).astype(np.float32) if w.dskip else None
    z = _normal_storage(c, step, 7, nx, io) if w.gate else None
    pre = (b,) if w.decode_steps else (b, L)
    out = {"x": x.reshape(pre + (H, P)), "dt": dt.reshape(pre + (H,)), "dt_bias": bias, "A": A,
           "B": Bm.reshape(pre + (G, N)), "C": Cm.reshape(pre + (G, N)), "Dskip": Dskip,
           "z": None if z is None else z.reshape(pre + (H, P)), "h0": None}
    if with_h0:
        out["h0"] = _normal(c, 0, 8, b * H * P * N).reshape(b, H, P, N)
    return out


def random_small_ssd(seed: int, b: int, L: int, H: int, P: int, G: int, N: int, io: str = BF16, gate=True,
                     dskip=True, bias=True, h0=False, delta=(1e-3, 1e-1)) -> dict:
    """Small random SSD case for parity sweeps (odd lengths, optional parts switched off)."""
    w = SSDWorkload("small-ssd", b, L, H, P, G, N, io, delta[0], delta[1], gate, dskip, cfg_id=2000 + seed)
    d = ssd_inputs(w, with_h0=h0)
    if not bias:
        lg = to_f64(d["dt"]) + d["dt_bias"].astype(np.float64)
        d["dt"] = to_storage(lg, io)
        d["dt_bias"] = None
    return d


def as_f64(d: dict) -> dict:
    """Storage dict -> float64 dict for the oracle."""
    return {k: (None if v is None else to_f64(v)) for k, v in d.items()}
