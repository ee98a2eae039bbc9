"""GPU parity of the backward scan (ssm_scan_bwd) against the fp64 oracle's scan_bwd.

The oracle's backward is pinned by central finite differences of the pinned forward (tests/test_oracle_pins.py).
Errors are max |gpu - oracle| / rms(oracle) per gradient tensor.  Tolerances: fp32 cotangents give fp32 gradients
whose only error is fp32 rounding in the recomputation, the adjoint recurrence and the fixed-order sums (TOL_BWD);
bf16 cotangents return bf16 gradients, which add one bf16 rounding (TOL_BF16, as for the forward's bf16 output).
"""
import numpy as np
import pytest

import oracle
import selective_state_space_57_amd as ssm
from selective_state_space_57_amd import inputs as I
import gpu_util as G

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-4
KEYS = {"dx": "dx", "ddt": "ddt", "dz": "dz", "dA": "dA", "dB": "dB", "dC": "dC", "dDskip": "dD",
        "ddt_bias": "ddt_bias", "dh0": "dh0"}


def run_bwd(dd, ct, disc=0, softplus=True):
    torch = G.torch_dev()
    g = ssm.scan_bwd(dd["x"], dd["dt"], dd["A"], dd["B"], dd["C"], ct["dy"], dt_bias=dd["dt_bias"],
                     Dskip=dd["Dskip"], z=dd["z"], h0=dd["h0"], dh_final=ct["dh_final"], disc=disc,
                     softplus=softplus)
    torch.cuda.synchronize()
    return g


def oracle_bwd(d, ct, disc=0, softplus=True):
    f, c = I.as_f64(d), I.as_f64(ct)
    return oracle.scan_bwd(f["x"], f["dt"], f["A"], f["B"], f["C"], c["dy"], dt_bias=f["dt_bias"], Dskip=f["Dskip"],
                           z=f["z"], h0=f["h0"], dh_final=c["dh_final"], disc=disc, softplus=softplus)


def compare(got, ref, tol, label=""):
    errs = {}
    for k, rk in KEYS.items():
        if got.get(k) is None:
            continue
        errs[k] = G.rel_max(G.to_np64(got[k]), ref[rk])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, (label, bad, tol)
    return errs


def check_case(seed, b, D, L, N, io="f32", disc=0, gate=True, dskip=True, bias=True, h0=False, dhf=False,
               softplus=True, positive_dt=False):
    d = I.random_small(seed, b, D, L, N, io=io, gate=gate, dskip=dskip, bias=bias, h0=h0)
    if positive_dt:  # Delta = dt directly, positive
        r = np.random.default_rng(seed)
        d["dt"] = I.to_storage(np.exp(r.uniform(np.log(1e-3), np.log(0.5), d["x"].shape)), io)
    ct = I.random_small_cotangents(seed, b, D, L, N, io=I.F32, dh_final=dhf)
    g = run_bwd(G.to_dev(d), G.to_dev(ct), disc=disc, softplus=softplus)
    ref = oracle_bwd(d, ct, disc=disc, softplus=softplus)
    return compare(g, ref, TOL_BWD, (seed, b, D, L, N, io, disc))


@pytest.mark.parametrize("seed,b,D,L,N,io,disc,gate,dskip,bias,h0,dhf", [
    (1, 1, 16, 64, 16, "f32", 0, True, True, True, False, False),     # one chunk, one workgroup
    (2, 2, 5, 1, 16, "f32", 0, True, True, True, True, True),         # a single step
    (3, 2, 17, 100, 16, "f32", 0, True, True, True, True, True),      # ragged channels and steps
    (4, 1, 3, 257, 5, "bf16", 0, True, True, True, False, True),      # N = 5, five chunks
    (5, 3, 40, 130, 1, "f32", 1, True, True, True, True, False),      # ZOH, N = 1
    (6, 2, 33, 200, 16, "f32", 1, False, False, False, True, True),   # ZOH without gate / skip / bias
    (7, 2, 21, 191, 16, "bf16", 1, True, True, True, True, True),     # ZOH, bf16 inputs
    (8, 1, 64, 256, 16, "f32", 0, False, True, True, False, False),   # no gate
    (9, 4, 7, 15, 16, "bf16", 0, True, False, True, True, False),     # shorter than a block
])
def test_bwd_random_cases(seed, b, D, L, N, io, disc, gate, dskip, bias, h0, dhf):
    check_case(seed, b, D, L, N, io, disc, gate, dskip, bias, h0, dhf)


@pytest.mark.parametrize("disc", [0, 1])
def test_bwd_no_softplus(disc):
    check_case(20 + disc, 2, 19, 150, 16, "f32", disc, bias=False, h0=True, dhf=True, softplus=False,
               positive_dt=True)


def test_bwd_several_quads_per_wave():
    # 2 x 64 chunks and 19 channel groups of 16: the planner gives each workgroup two quads per wave, so the dB / dC
    # tiles accumulate across channel quads before the reduction
    p = ssm.make_params(2, 300, 4096, 16, ssm.SSM_F32)
    assert ssm.bwd_workspace_bytes(p) > 0
    check_case(30, 2, 300, 4096, 16, "f32", 0, h0=True, dhf=True)


def test_bwd_tiny_workload():
    w = I.WORKLOADS[0]
    d = I.scan_inputs(w, with_h0=True)
    ct = I.cotangents(w, with_dh_final=True)
    g = run_bwd(G.to_dev(d), G.to_dev(ct))
    compare(g, oracle_bwd(d, ct), TOL_BWD, "tiny")


def test_bwd_deterministic():
    torch = G.torch_dev()
    d = I.random_small(40, 2, 37, 301, 16, io="bf16", h0=True)
    ct = I.random_small_cotangents(40, 2, 37, 301, 16, io="bf16", dh_final=True)
    dd, dc = G.to_dev(d), G.to_dev(ct)
    g1 = run_bwd(dd, dc)
    g2 = run_bwd(dd, dc)
    for k in KEYS:
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_bf16_gradients_are_rne_of_fp32():
    # the same bf16 cotangent passed as bf16 (bf16 gradients) and as its exact fp32 value (fp32 gradients): the kernel
    # arithmetic is identical, so the bf16 outputs must be the round-to-nearest-even of the fp32 ones
    torch = G.torch_dev()
    d = I.random_small(41, 2, 37, 301, 16, io="bf16", h0=True)
    ct = I.random_small_cotangents(41, 2, 37, 301, 16, io="bf16", dh_final=True)
    dd, dc = G.to_dev(d), G.to_dev(ct)
    g16 = run_bwd(dd, dc)
    dc32 = dict(dc, dy=dc["dy"].to(torch.float32))
    g32 = run_bwd(dd, dc32)
    for k in ("dx", "ddt", "dz"):
        want = G.bf16_rne(g32[k].cpu().numpy())
        assert np.array_equal(g16[k].to(torch.float32).cpu().numpy(), want), k
    for k in ("dA", "dB", "dC", "dDskip", "ddt_bias", "dh0"):
        assert torch.equal(g16[k], g32[k]), k


@pytest.mark.parametrize("cfg", [1, 2])
def test_bwd_full_size(cfg):
    """Full layer size (the 130M and 2.8B layers), the launch configuration the benchmark times, dy and dh_final
    seeded normals everywhere: every gradient tensor against the oracle's backward on the whole layer."""
    w = I.WORKLOADS[cfg]
    d = I.scan_inputs(w, with_h0=True)
    ct = I.cotangents(w, io=I.F32, with_dh_final=True)
    g = run_bwd(G.to_dev(d), G.to_dev(ct))
    ref = oracle_bwd(d, ct)
    errs = compare(g, ref, TOL_BWD, w.name)
    print("%s backward errors:" % w.name, {k: "%.1e" % e for k, e in errs.items()}, flush=True)


@pytest.mark.parametrize("cfg,ndim", [(1, 6), (2, 6)])
def test_bwd_full_size_sampled(cfg, ndim):
    """Full layer size, the launch configuration the benchmark times.  The backward is linear in dy, so with dy zero
    outside a sample of channels (all batches of `ndim` channels) every gradient is that of the sample alone: dB / dC
    in full and the per-channel gradients of the sample are checked against the oracle run on the sample, and every
    other channel's gradients must be exactly zero."""
    torch = G.torch_dev()
    w = I.WORKLOADS[cfg]
    d = I.scan_inputs(w, with_h0=True)
    ct = I.cotangents(w, io=I.F32, with_dh_final=True)
    r = np.random.default_rng(cfg)
    chans = np.unique(np.concatenate([[0, w.dim - 1], r.choice(w.dim, ndim - 2, replace=False)]))
    mask = np.zeros(w.dim, bool)
    mask[chans] = True
    ct["dy"][:, ~mask] = 0
    ct["dh_final"][:, ~mask] = 0
    g = run_bwd(G.to_dev(d), G.to_dev(ct))
    sub = {k: (None if v is None else (v[:, chans] if k in ("x", "dt", "z", "h0") else
                                       (v[chans] if k in ("A", "dt_bias", "Dskip") else v)))
           for k, v in d.items()}
    sct = {"dy": ct["dy"][:, chans], "dh_final": ct["dh_final"][:, chans]}
    ref = oracle_bwd(sub, sct)
    got = {}
    for k in KEYS:
        a = G.to_np64(g[k])
        if k in ("dB", "dC"):
            got[k] = a
            continue
        axis = 1 if k in ("dx", "ddt", "dz", "dh0") else 0
        rest = np.delete(a, chans, axis=axis)
        assert not np.any(rest), (k, "non-zero gradient outside the sampled channels")
        got[k] = np.take(a, chans, axis=axis)
    errs = {k: G.rel_max(got[k], ref[rk]) for k, rk in KEYS.items()}
    assert all(e <= TOL_BWD for e in errs.values()), errs


def test_bwd_million_length_sampled():
    """The million-step layer (1 x 512 x 2^20, 16,384 chunks) at full size, with dy and dh_final non-zero only on
    three channels (seeded normals; the backward is linear in them): those channels' gradients and the full dB / dC
    against the oracle run on the three channels, every other channel's gradients exactly zero."""
    torch = G.torch_dev()
    w = I.WORKLOADS[3]
    print("million-length backward: generating inputs", flush=True)
    d = I.scan_inputs(w, with_h0=True)
    chans = np.array([0, 301, w.dim - 1])
    r = np.random.default_rng(33)
    dy = np.zeros((w.batch, w.dim, w.seqlen), np.float32)
    dy[:, chans] = r.standard_normal((w.batch, len(chans), w.seqlen), dtype=np.float32)
    dhf = np.zeros((w.batch, w.dim, w.dstate), np.float32)
    dhf[:, chans] = r.standard_normal((w.batch, len(chans), w.dstate), dtype=np.float32)
    print("million-length backward: GPU", flush=True)
    g = run_bwd(G.to_dev(d), G.to_dev({"dy": dy, "dh_final": dhf}))
    sub = {k: (None if v is None else (v[:, chans] if k in ("x", "dt", "z", "h0") else
                                       (v[chans] if k in ("A", "dt_bias", "Dskip") else v)))
           for k, v in d.items()}
    print("million-length backward: oracle on %d channels" % len(chans), flush=True)
    ref = oracle_bwd(sub, {"dy": dy[:, chans], "dh_final": dhf[:, chans]})
    errs = {}
    for k, rk in KEYS.items():
        a = G.to_np64(g[k])
        if k not in ("dB", "dC"):
            axis = 1 if k in ("dx", "ddt", "dz", "dh0") else 0
            assert not np.any(np.delete(a, chans, axis=axis)), (k, "non-zero gradient outside the sampled channels")
            a = np.take(a, chans, axis=axis)
        errs[k] = G.rel_max(a, ref[rk])
    print("million-length backward errors:", {k: "%.1e" % e for k, e in errs.items()}, flush=True)
    assert all(e <= TOL_BWD for e in errs.values()), errs
