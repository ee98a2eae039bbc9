"""GPU parity of the S6 scan and decode step in the method's limiting cases, through the C ABI, against the fp64
oracle and, where a closed form exists, against that closed form computed here in fp64:

* zero-order hold with some A[d, n] exactly 0 (the input coefficient's limit expm1(Delta A) / A -> Delta; tutorial
  "离散化"), mixed with decaying states, on the mask-free full-tile path and on ragged tiles;
* Delta -> 0 (the paper's section 3.5.2: a small Delta keeps the state and ignores the input): softplus off with
  Delta = 1e-12, and softplus on with logits of -40, where h stays h0 and y = (C h0 + D x) silu(z);
* the softplus tails, logits of +-40 and 700 mixed into ordinary ones (700 resets the state exactly: exp(700 A)
  underflows to 0, section 3.5.2 "reset");
* Theorem 1 (paper section 3.5.1; close reading "核心创新"): N = 1, A = -1, B = C = 1, zero-order hold, no D and no
  gate turn the scan into the gated recurrence h_t = (1 - g_t) h_{t-1} + g_t x_t with g_t = sigmoid(dt_t + bias).

Tolerances as in the other parity tests: max |got - ref| / rms(ref) <= 1e-5 for fp32 inputs, 3e-3 for bf16 inputs
with fp32 y; the softplus-tails test scales the fp32 bar with the dynamic range its resets create (stated there).
"""
import numpy as np
import pytest

import oracle
import selective_state_space_57_amd as ssm
from selective_state_space_57_amd import inputs as I
import gpu_util as G

pytestmark = pytest.mark.gpu

ZOH = 1

# (b, D, L, N): full tiles (16 channels x 64-step chunks, N = 16: the mask-free path) and ragged ones
SHAPES = [(2, 32, 256, 16), (3, 19, 77, 16), (1, 45, 130, 5)]


def _scan_vs_oracle(d, io, disc=0, softplus=True, segments=0, tol=None):
    torch = G.torch_dev()
    dd = G.to_dev(d)
    y, hf = G.run_gpu(dd, disc=disc, y_dtype=torch.float32, softplus=softplus, segments=segments)
    yr, hr = G.oracle_ref(d, disc=disc, softplus=softplus)
    yg, hg = G.to_np64(y), G.to_np64(hf)
    tol = G.tol_for(io) if tol is None else tol
    ey, eh = G.rel_max(yg, yr), G.rel_max(hg, hr)
    assert ey <= tol, ("y", ey, tol)
    assert eh <= tol, ("h_final", eh, tol)
    return yg, hg, yr, hr


def _decode_vs_oracle(d, io, disc=0, softplus=True, steps=None, tol=None):
    """Run the sequence step by step through ssm_state_update and compare every step's y and the final state."""
    torch = G.torch_dev()
    dd = G.to_dev(d)
    f = I.as_f64(d)
    L = d["x"].shape[2]
    steps = L if steps is None else min(steps, L)
    state = dd["h0"].clone()
    ref = f["h0"].copy()
    tol = G.tol_for(io) if tol is None else tol
    for t in range(steps):
        sl = lambda k: dd[k][:, :, t].contiguous()
        y = ssm.state_update(state, sl("x"), sl("dt"), dd["A"], sl("B"), sl("C"), dt_bias=dd["dt_bias"],
                             Dskip=dd["Dskip"], z=None if dd["z"] is None else sl("z"), y_dtype=torch.float32,
                             disc=disc, softplus=softplus)
        fz = None if f["z"] is None else f["z"][:, :, t]
        yr, ref = oracle.state_update(ref, f["x"][:, :, t], f["dt"][:, :, t], f["A"], f["B"][:, :, t],
                                      f["C"][:, :, t], dt_bias=f["dt_bias"], Dskip=f["Dskip"], z=fz, disc=disc,
                                      softplus=softplus)
        assert G.rel_max(G.to_np64(y), yr) <= tol, ("decode y at step", t)
    assert G.rel_max(G.to_np64(state), ref) <= tol, "decode state"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%dx%dxN%d" % s for s in SHAPES])
def test_zoh_with_zero_A_entries(io, shape):
    b, D, L, N = shape
    d = I.random_small(300 + D, b, D, L, N, io=io, h0=True)
    A = d["A"].copy()
    A[:, ::3] = 0.0            # every third state of every channel does not decay
    A[D // 2] = 0.0            # and one channel not at all
    d["A"] = A
    _scan_vs_oracle(d, io, disc=ZOH)
    _scan_vs_oracle(d, io, disc=ZOH, segments=3)
    _decode_vs_oracle(d, io, disc=ZOH, steps=24)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_hold_delta_1e_12(io):
    # softplus off, Delta = 1e-12: exp(Delta A) rounds to 1 in fp32 and Delta B x is ~1e-12, so h stays h0
    b, D, L, N = 2, 32, 256, 16
    d = I.random_small(310, b, D, L, N, io=io, bias=False, h0=True)
    d["dt"] = I.to_storage(np.full(d["x"].shape, 1e-12), io)
    for disc in (0, ZOH):
        yg, hg, yr, hr = _scan_vs_oracle(d, io, disc=disc, softplus=False)
        # closed form: y_t = (sum_n C_n(t) h0_n + D x_t) silu(z_t), h_final = h0
        f = I.as_f64(d)
        ch = np.einsum("bnl,bdn->bdl", f["C"], f["h0"])
        pre = ch + f["Dskip"][None, :, None] * f["x"]
        yc = pre * f["z"] / (1.0 + np.exp(-f["z"]))
        assert G.rel_max(yg, yc) <= 1e-5, "hold: y = (C h0 + D x) silu(z)"
        assert G.rel_max(hg, f["h0"]) <= 1e-6, "hold: h_final = h0"
    _decode_vs_oracle(d, io, softplus=False, steps=16)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES[:2], ids=["%dx%dx%dxN%d" % s for s in SHAPES[:2]])
def test_softplus_tails(io, shape):
    # logits of -40 (Delta = 4e-18: hold), +40 (Delta = 40: near-total decay) and 700 (Delta = 700: exp(Delta A)
    # underflows to 0, the state restarts from the current input) at random places among ordinary logits
    b, D, L, N = shape
    d = I.random_small(320 + D, b, D, L, N, io=io, bias=False, h0=True)
    r = np.random.default_rng(321)
    lg = I.to_f64(d["dt"])
    pick = r.random(lg.shape)
    lg = np.where(pick < 0.04, -40.0, lg)
    lg = np.where((pick >= 0.04) & (pick < 0.06), 40.0, lg)
    lg = np.where((pick >= 0.06) & (pick < 0.07), 700.0, lg)
    d["dt"] = I.to_storage(lg, io)
    # A logit of 700 restarts the state at 700 B x, so for the next few hundred steps the state and y carry values up
    # to ~40x rms(y).  fp32 rounding of the recurrence is relative to the magnitude carried (about 2^-24 per step over
    # the decay memory), so for fp32 inputs the bar relative to rms(y) scales with that range: 3e-5.  (A plain fp32
    # recurrence in numpy, one rounding per operation, is 0.94e-5 of rms(y) from the oracle on the 2 x 32 x 256 case.)
    tol = 3e-5 if io == "f32" else G.TOL_BF16
    for disc in (0, ZOH):
        _scan_vs_oracle(d, io, disc=disc, tol=tol)
        _decode_vs_oracle(d, io, disc=disc, steps=32, tol=tol)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_theorem1_gated_rnn(io):
    # N = 1, A = -1, B = C = 1, zero-order hold, no D, no gate, softplus Delta:
    # exp(-Delta) = 1 - sigmoid(u) and expm1(-Delta) / -1 = sigmoid(u), u = dt + bias
    b, D, L, N = 2, 37, 1000, 1
    d = I.random_small(330, b, D, L, N, io=io, gate=False, dskip=False, h0=True)
    d["A"] = np.full((D, 1), -1.0, np.float32)
    d["B"] = I.to_storage(np.ones((b, 1, L)), io)
    d["C"] = I.to_storage(np.ones((b, 1, L)), io)
    yg, hg, _, _ = _scan_vs_oracle(d, io, disc=ZOH)
    f = I.as_f64(d)
    u = f["dt"] + f["dt_bias"][None, :, None]
    g = 1.0 / (1.0 + np.exp(-u))
    h = f["h0"][:, :, 0].copy()
    yc = np.empty_like(f["x"])
    for t in range(L):
        h = (1.0 - g[:, :, t]) * h + g[:, :, t] * f["x"][:, :, t]
        yc[:, :, t] = h
    tol = G.tol_for(io)
    assert G.rel_max(yg, yc) <= tol, "Theorem 1: y = gated RNN"
    assert G.rel_max(hg[:, :, 0], h) <= tol, "Theorem 1: final state"
    _decode_vs_oracle(d, io, disc=ZOH, steps=40)
