"""Independent checks that pin the fp64 oracle to what the pages and the mathematics fix.

Each check takes an oracle object (``oracle.Oracle``) and raises AssertionError on disagreement.  None of them
re-types the oracle's step loop: each computes the expected value by a different route (a convolution kernel, a
gated RNN, cumulative sums, a tree scan, a hand-worked example, an algebraic identity).

Sources (cited by page title and section):
  * Mamba paper (arXiv 2312.00752), Chinese translation on gitcode.csdn.net: section 2 (discretisation, recurrence
    (2), convolution (3), LTI, diagonal structure), section 3.3.2 (scan), section 3.5 (Theorem 1, selection effects:
    boundary reset with Delta -> inf, ignoring inputs with Delta -> 0), section 3.6 (S4D-Real A, Delta bias init).
  * "Mamba" tutorial on docs.ifdog.com: sections on ZOH discretisation (diagonal case), S4's convolution view
    (K = [CB, CAB, CA^2B, ...]), softplus, the associative combine of the parallel scan, SiLU gate of the block.
  * Close reading on alishangtian.com: statement of Theorem 1 (N = 1, A = -1 gives a gated RNN).
"""
from __future__ import annotations

import math
import numpy as np

EULER_B, ZOH = 0, 1


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence(5757, spawn_key=(seed,)))


def _case(seed, b=2, D=3, L=23, N=4, gate=True, dskip=True, h0=True, drange=(1e-3, 1.5)):
    r = _rng(seed)
    x = r.standard_normal((b, D, L))
    # logits whose softplus covers [drange]: u = log(expm1(delta))
    delta = np.exp(r.uniform(np.log(drange[0]), np.log(drange[1]), (b, D, L)))
    bias = r.uniform(-0.5, 0.5, D)
    dt = np.log(np.expm1(delta)) - bias[None, :, None]
    A = -(np.arange(N) + 1.0)[None, :] * np.exp(r.uniform(-0.3, 0.3, (D, N)))
    B = r.standard_normal((b, N, L))
    C = r.standard_normal((b, N, L))
    Dk = r.standard_normal(D) if dskip else None
    z = r.standard_normal((b, D, L)) if gate else None
    H0 = r.standard_normal((b, D, N)) if h0 else None
    return dict(x=x, dt=dt, dt_bias=bias, A=A, B=B, C=C, Dskip=Dk, z=z, h0=H0)


def _softplus_lib(u):
    # library route, independent of the oracle's max(u,0)+log1p(exp(-|u|)) form
    return np.logaddexp(0.0, u)


def _coef(delta, A, disc):
    """B-bar / B for the two discretisation rules (tutorial ZOH formula, diagonal case; Euler = Delta)."""
    if disc == EULER_B:
        return delta
    with np.errstate(invalid="ignore", divide="ignore"):
        c = np.expm1(delta * A) / A
    return np.where(A == 0.0, delta, c)


def _silu(z):
    return z * (1.0 / (1.0 + np.exp(-z)))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, float(np.max(np.abs(b)))))


# ---------------------------------------------------------------------------------------------------------------
# P1: LTI case equals the convolution y = K * x with K_k = sum_n C_n Abar_n^k Bbar_n (+ D x)  (paper section 2,
#     equations (2)-(3); tutorial "卷积视角与 FFT 并行").  Brute force O(L^2).
def pin_lti_convolution(orc, disc, N=4, L=40, seed=1):
    r = _rng(100 + seed + 10 * disc + N)
    D = 3
    u = r.uniform(-3, 1, D)                   # one Delta logit per channel, constant in time
    A = -(np.arange(N) + 1.0)[None, :] * np.exp(r.uniform(-0.2, 0.2, (D, N)))
    Bv = r.standard_normal(N)
    Cv = r.standard_normal(N)
    Dk = r.standard_normal(D)
    x = r.standard_normal((1, D, L))
    dt = np.repeat(u[None, :, None], L, axis=2)
    Bm = np.repeat(Bv[None, :, None], L, axis=2)
    Cm = np.repeat(Cv[None, :, None], L, axis=2)
    y, _ = orc.scan(x, dt, A, Bm, Cm, Dskip=Dk, disc=disc)
    delta = _softplus_lib(u)
    exp_y = np.zeros((1, D, L))
    for d in range(D):
        Ab = np.exp(delta[d] * A[d])
        Bb = _coef(delta[d], A[d], disc) * Bv
        K = np.array([np.sum(Cv * Ab ** k * Bb) for k in range(L)])
        exp_y[0, d] = np.convolve(x[0, d], K)[:L] + Dk[d] * x[0, d]
    assert _rel(y, exp_y) < 1e-12, ("P1", disc, N, _rel(y, exp_y))


# P2: Theorem 1 (paper section 3.5.1; alishangtian statement): N = 1, A = -1, B = C = 1, ZOH, Delta = softplus(u)
#     gives h_t = (1 - g_t) h_{t-1} + g_t x_t with g_t = sigmoid(u_t).
def pin_theorem1(orc, L=57, seed=2):
    r = _rng(200 + seed)
    D = 4
    x = r.standard_normal((1, D, L))
    u = r.uniform(-6, 6, (1, D, L))
    h0 = r.standard_normal((1, D, 1))
    y, hf = orc.scan(x, u, -np.ones((D, 1)), np.ones((1, 1, L)), np.ones((1, 1, L)), h0=h0, disc=ZOH)
    g = 1.0 / (1.0 + np.exp(-u))
    h = h0[0, :, 0].copy()
    exp_y = np.zeros_like(x)
    for t in range(L):
        h = (1 - g[0, :, t]) * h + g[0, :, t] * x[0, :, t]
        exp_y[0, :, t] = h
    assert np.max(np.abs(y - exp_y)) < 1e-13 * max(1.0, np.max(np.abs(exp_y))), ("P2", np.max(np.abs(y - exp_y)))
    assert np.max(np.abs(hf[0, :, 0] - h)) < 1e-13


# P3: splitting the sequence and handing over the state equals the single pass (constant-size recurrent state,
#     paper section 1 (ii)).
def pin_split(orc, disc, seed=3):
    c = _case(300 + seed + disc, L=37)
    y, hf = orc.scan(**c, disc=disc)
    cut = 1 + seed % 30
    s1 = {k: (v[..., :cut] if k in ("x", "dt", "B", "C", "z") and v is not None else v) for k, v in c.items()}
    s2 = {k: (v[..., cut:] if k in ("x", "dt", "B", "C", "z") and v is not None else v) for k, v in c.items()}
    y1, h1 = orc.scan(**s1, disc=disc)
    s2["h0"] = h1
    y2, h2 = orc.scan(**s2, disc=disc)
    assert _rel(np.concatenate([y1, y2], axis=2), y) < 1e-13, "P3 y"
    assert _rel(h2, hf) < 1e-13, "P3 h_final"


# P4: the materialised (cumulative-sum) form.  With S_t = sum_{r<=t} Delta_r,
#     h_t,n = sum_{s<=t} exp(A_n (S_t - S_s)) Bbar_{s,n} x_s + exp(A_n S_t) h0_n   (the expanded state of shape
#     (B, L, D, N) that paper section 3.3 describes and never materialises on the GPU).
def pin_materialised(orc, disc, seed=4):
    c = _case(400 + seed + disc, b=2, D=2, L=19, N=3)
    y, hf = orc.scan(**c, disc=disc)
    b, D, L = c["x"].shape
    N = c["A"].shape[1]
    delta = _softplus_lib(c["dt"] + c["dt_bias"][None, :, None])
    S = np.cumsum(delta, axis=2)
    exp_y = np.zeros_like(c["x"])
    exp_h = np.zeros((b, D, N))
    for bi in range(b):
        for d in range(D):
            A = c["A"][d]
            H = np.zeros((L, N))
            for t in range(L):
                acc = np.exp(A * S[bi, d, t]) * c["h0"][bi, d]
                for s in range(t + 1):
                    bb = _coef(delta[bi, d, s], A, disc) * c["B"][bi, :, s] * c["x"][bi, d, s]
                    acc = acc + np.exp(A * (S[bi, d, t] - S[bi, d, s])) * bb
                H[t] = acc
            yy = np.sum(c["C"][bi].T * H, axis=1) + c["Dskip"][d] * c["x"][bi, d]
            exp_y[bi, d] = yy * _silu(c["z"][bi, d])
            exp_h[bi, d] = H[-1]
    assert _rel(y, exp_y) < 1e-10, ("P4 y", _rel(y, exp_y))
    assert _rel(hf, exp_h) < 1e-10, ("P4 h", _rel(hf, exp_h))


# P5: associativity.  The parallel scan's combine (a1, b1) o (a2, b2) = (a2 a1, a2 b1 + b2) (tutorial, "硬件感知的
#     并行扫描"), applied as Hillis-Steele and as a chunked two-level scan, reproduces the oracle's states.
def _combine(p, q):
    return q[0] * p[0], q[0] * p[1] + q[1]


def pin_associative(orc, disc, seed=5):
    c = _case(500 + seed + disc, b=1, D=2, L=29, N=3, gate=False, dskip=False)
    y, hf = orc.scan(**c, disc=disc)
    delta = _softplus_lib(c["dt"] + c["dt_bias"][None, :, None])[0]
    L = delta.shape[1]
    for d in range(2):
        A = c["A"][d]
        a = np.exp(delta[d][:, None] * A[None, :])                                          # (L, N)
        bb = _coef(delta[d][:, None], A[None, :], disc) * c["B"][0].T * c["x"][0, d][:, None]
        # Hillis-Steele inclusive scan
        pa, pb = a.copy(), bb.copy()
        k = 1
        while k < L:
            na, nb = pa.copy(), pb.copy()
            for t in range(k, L):
                na[t], nb[t] = _combine((pa[t - k], pb[t - k]), (pa[t], pb[t]))
            pa, pb = na, nb
            k *= 2
        H = pa * c["h0"][0, d][None, :] + pb
        assert _rel(H[-1], hf[0, d]) < 1e-13, "P5 Hillis-Steele h_final"
        assert _rel(np.sum(c["C"][0].T * H, axis=1), y[0, d]) < 1e-12, "P5 Hillis-Steele y"
        # chunked: per-chunk aggregates, exclusive scan of aggregates, replay
        cs = 1 + (seed + d) % 7
        carry = (np.ones(a.shape[1]), c["h0"][0, d].copy())
        H2 = np.zeros_like(H)
        for s0 in range(0, L, cs):
            agg = (np.ones(a.shape[1]), np.zeros(a.shape[1]))
            for t in range(s0, min(L, s0 + cs)):
                agg = _combine(agg, (a[t], bb[t]))
                tot = _combine(carry, agg)
                H2[t] = tot[1]
            carry = _combine(carry, agg)
        assert _rel(H2, H) < 1e-13, "P5 chunked"


# P6: linearity in (x, h0) when Delta, B, C are fixed and the gate is off (recurrence (2) is linear).
def pin_linearity(orc, disc, seed=6):
    c1 = _case(600 + seed + disc, gate=False)
    c2 = _case(650 + seed + disc, gate=False)
    al, be = 0.7, -1.3
    mix = dict(c1)
    mix["x"] = al * c1["x"] + be * c2["x"]
    mix["h0"] = al * c1["h0"] + be * c2["h0"]
    c2s = dict(c1)
    c2s["x"], c2s["h0"] = c2["x"], c2["h0"]
    y1, h1 = orc.scan(**c1, disc=disc)
    y2, h2 = orc.scan(**c2s, disc=disc)
    ym, hm = orc.scan(**mix, disc=disc)
    assert _rel(ym, al * y1 + be * y2) < 1e-12, "P6 y"
    assert _rel(hm, al * h1 + be * h2) < 1e-12, "P6 h"


# P7: selection effects (paper section 3.5.2): a huge Delta at t* resets the state, so outputs from t* on do not
#     depend on anything before t*; a vanishing Delta keeps the state and ignores the input.
def pin_reset_hold(orc, disc, seed=7):
    c = _case(700 + seed + disc, L=30)
    ts = 11
    c["dt"] = c["dt"].copy()
    c["dt"][:, :, ts] = 1e4
    y, hf = orc.scan(**c, disc=disc)
    c2 = dict(c)
    r = _rng(750 + seed)
    c2["x"] = c["x"].copy()
    c2["x"][:, :, :ts] = r.standard_normal(c["x"][:, :, :ts].shape)
    c2["h0"] = r.standard_normal(c["h0"].shape)
    y2, hf2 = orc.scan(**c2, disc=disc)
    assert np.array_equal(y[:, :, ts:], y2[:, :, ts:]), "P7 reset"
    assert np.array_equal(hf, hf2), "P7 reset h"
    assert not np.allclose(y[:, :, :ts], y2[:, :, :ts]), "P7 reset sanity"
    # hold: Delta = 1e-12 (softplus off) => h ~ h0, y ~ (C.h0 + D x) silu(z)
    c3 = dict(c)
    c3["dt"] = np.full_like(c["dt"], 1e-12)
    c3["dt_bias"] = None
    y3, hf3 = orc.scan(**c3, disc=disc, softplus=False)
    exp = (np.einsum("bnl,bdn->bdl", c["C"], c["h0"]) + c["Dskip"][None, :, None] * c["x"]) * _silu(c["z"])
    assert np.max(np.abs(y3 - exp)) < 1e-9, "P7 hold y"
    assert np.max(np.abs(hf3 - c["h0"])) < 1e-9, "P7 hold h"


# P8: ZOH vs Euler for B: one step from h0 = 0 with x = B = C = 1 gives y_ZOH / y_Euler = expm1(Delta A)/(Delta A),
#     which tends to 1 + Delta A / 2 as Delta -> 0 (tutorial ZOH formula, diagonal case).
def pin_zoh_euler(orc):
    for u, a in [(-8.0, -1.0), (-2.0, -3.5), (0.5, -0.25), (3.0, -16.0), (-20.0, -1.0)]:
        args = (np.ones((1, 1, 1)), np.full((1, 1, 1), u), np.full((1, 1), a), np.ones((1, 1, 1)), np.ones((1, 1, 1)))
        yz, _ = orc.scan(*args, disc=ZOH)
        ye, _ = orc.scan(*args, disc=EULER_B)
        delta = math.log1p(math.exp(u)) if u < 30 else u
        ratio = math.expm1(delta * a) / (delta * a)
        with np.errstate(divide="ignore", invalid="ignore"):   # a broken oracle may give 0 / 0; it then fails here
            got = yz[0, 0, 0] / ye[0, 0, 0]
        assert abs(got - ratio) < 1e-14, ("P8", u, a)
        if delta < 1e-3:
            assert abs(ratio - (1 + delta * a / 2)) < (delta * a) ** 2 + 4e-16
    # A == 0 takes the limit Delta * B
    args = (np.ones((1, 1, 1)), np.zeros((1, 1, 1)), np.zeros((1, 1)), np.ones((1, 1, 1)), np.ones((1, 1, 1)))
    yz, _ = orc.scan(*args, disc=ZOH)
    assert abs(yz[0, 0, 0] - math.log(2.0)) < 1e-15


# P9: decode == scan: L single-token steps equal one scan of length L started from the same state.
def pin_decode_scan(orc, disc, seed=9):
    c = _case(900 + seed + disc, L=13)
    y, hf = orc.scan(**c, disc=disc)
    st = c["h0"].copy()
    for t in range(c["x"].shape[2]):
        yt, st = orc.state_update(st, c["x"][:, :, t], c["dt"][:, :, t], c["A"], c["B"][:, :, t], c["C"][:, :, t],
                                  dt_bias=c["dt_bias"], Dskip=c["Dskip"], z=c["z"][:, :, t], disc=disc)
        assert _rel(yt, y[:, :, t]) < 1e-14, "P9 y"
    assert _rel(st, hf) < 1e-14, "P9 state"
    # decode reduces to Theorem 1's gated RNN as well (independent of the scan entry point)
    r = _rng(990 + seed)
    u = r.uniform(-5, 5, (1, 3))
    xv = r.standard_normal((1, 3))
    s0 = r.standard_normal((1, 3, 1))
    yd, s1 = orc.state_update(s0, xv, u, -np.ones((3, 1)), np.ones((1, 1)), np.ones((1, 1)), disc=ZOH)
    g = 1 / (1 + np.exp(-u))
    assert np.max(np.abs(yd - ((1 - g) * s0[:, :, 0] + g * xv))) < 1e-14, "P9 theorem-1 decode"


# Worked examples computed by hand from the definitions (tests/golden/worked_examples.txt).
def pin_worked_examples(orc, rows):
    for row in rows:
        disc = EULER_B if row["disc"] == "euler" else ZOH
        N = 1
        args = dict(x=np.full((1, 1, 1), row["x"]), dt=np.full((1, 1, 1), row["u"]), A=np.full((1, N), row["A"]),
                    B=np.full((1, N, 1), row["B"]), C=np.full((1, N, 1), row["C"]),
                    Dskip=None if row["D"] is None else np.array([row["D"]]),
                    z=None if row["z"] is None else np.full((1, 1, 1), row["z"]), h0=np.full((1, 1, N), row["h0"]))
        y, hf = orc.scan(**args, disc=disc)
        assert abs(y[0, 0, 0] - row["y"]) < 1e-14 * max(1, abs(row["y"])), (row["name"], y[0, 0, 0], row["y"])
        assert abs(hf[0, 0, 0] - row["h"]) < 1e-14 * max(1, abs(row["h"])), (row["name"], hf[0, 0, 0], row["h"])


# P10: backward = central finite differences of the (pinned) forward oracle, for every input element.  The loss is
#      sum(dy * y) + sum(dh_final * h_final) with random weights; every gradient the backward returns is checked.
def pin_bwd_finite_differences(orc, disc, seed=10):
    c = _case(1000 + seed + disc, b=2, D=3, L=9, N=4)
    r = _rng(1100 + seed + disc)
    if disc == ZOH:
        c["A"] = c["A"].copy()
        c["A"][0, 0] = 0.0      # A == 0 limit
        c["A"][1, 1] = -6e-4    # |Delta A| just under 1e-3: series branch of the A-derivative, where its terms matter
        c["A"][2, 2] = -1e-5    # tiny |Delta A|
    dy = r.standard_normal(c["x"].shape)
    dhf = r.standard_normal(c["h0"].shape)
    g = orc.scan_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], dy, dt_bias=c["dt_bias"], Dskip=c["Dskip"], z=c["z"],
                     h0=c["h0"], dh_final=dhf, disc=disc)

    def loss(cc):
        y, hf = orc.scan(**cc, disc=disc)
        return float(np.sum(dy * y) + np.sum(dhf * hf))

    names = {"x": "dx", "dt": "ddt", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "Dskip": "dD", "dt_bias": "ddt_bias",
             "h0": "dh0"}
    for key, gk in names.items():
        base = c[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            cp = dict(c)
            v = base.copy()
            v[idx] = base[idx] + eps
            cp[key] = v
            lp = loss(cp)
            v[idx] = base[idx] - eps
            lm = loss(cp)
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - g[gk])) / max(1.0, float(np.max(np.abs(fd))))
        assert err < 2e-6, ("P10", disc, gk, err)


# P11: causal depthwise conv1d (then SiLU).  The convolution against numpy.convolve (an independent implementation)
#      over the zero- or state-padded sequence, every width 1..4; SiLU against closed forms.
def pin_conv_numpy(orc, seed=11):
    r = _rng(seed)
    for K in (1, 2, 3, 4):
        b, D, L = 2, 3, 37
        x = r.standard_normal((b, D, L))
        w = r.standard_normal((D, K))
        bias = r.standard_normal(D)
        st = r.standard_normal((b, D, K - 1)) if K > 1 else None
        u, so = orc.conv1d(x, w, bias=bias, state_in=st, silu=False)
        for bi in range(b):
            for d in range(D):
                pad = st[bi, d] if st is not None else np.zeros(0)
                ref = np.convolve(np.concatenate([pad, x[bi, d]]), w[d][::-1], "valid") + bias[d]
                assert np.max(np.abs(ref - u[bi, d])) < 1e-12, ("P11", K)
                if K > 1:
                    assert np.array_equal(so[bi, d], x[bi, d, L - (K - 1):]), ("P11 state", K)
    # SiLU: w = 0, bias = ln 3 -> sigmoid = 3/4, u = 0.75 ln 3; bias = -ln 3 -> u = -0.25 ln 3; bias = 0 -> 0
    w = np.zeros((3, 4))
    for bv, want in ((np.log(3.0), 0.75 * np.log(3.0)), (-np.log(3.0), -0.25 * np.log(3.0)), (0.0, 0.0)):
        u, _ = orc.conv1d(np.ones((1, 3, 5)), w, bias=np.full(3, bv), silu=True)
        assert np.max(np.abs(u - want)) < 1e-15, ("P11 silu", bv)


# P12: streaming: the convolution of a sequence equals the convolution of its two halves, the second continuing from
#      the first's state; a sequence shorter than the state shifts the state (closed form).
def pin_conv_split(orc, seed=12):
    r = _rng(seed)
    x = r.standard_normal((2, 4, 50))
    w = r.standard_normal((4, 4))
    bias = r.standard_normal(4)
    st = r.standard_normal((2, 4, 3))
    u, so = orc.conv1d(x, w, bias=bias, state_in=st)
    u1, s1 = orc.conv1d(x[:, :, :21], w, bias=bias, state_in=st)
    u2, s2 = orc.conv1d(x[:, :, 21:], w, bias=bias, state_in=s1)
    assert np.max(np.abs(np.concatenate([u1, u2], axis=2) - u)) < 1e-14, "P12"
    assert np.array_equal(s2, so), "P12 state"
    u3, s3 = orc.conv1d(x[:, :, :1], w, bias=bias, state_in=st)
    assert np.array_equal(s3, np.concatenate([st[:, :, 1:], x[:, :, :1]], axis=2)), "P12 short"


# P13: complex diagonal A (Mamba paper section 3.6, S4D-Lin).  (a) real inputs reduce to the (pinned) real oracle,
#      both rules; (b) LTI case = convolution with K_k = Re(sum_n C_n Abar_n^k Bbar_n) built from numpy complex powers
#      (brute force), both rules; (c) conjugating A, B, C, h0 leaves y unchanged and conjugates h_final; (d) an
#      impulse through a pure rotation (A = i w, N = 1, Delta = dt fixed): y_t = Delta cos(w Delta t); (e) L decode
#      steps = one scan.
def pin_conv_bwd_finite_differences(orc, seed=15):
    """Backward of the causal convolution (+ SiLU) = central differences of the (pinned) forward, element by element,
    for x, the taps, the bias and the incoming window, loss sum(du u) + sum(dstate_out state_out); also a sequence
    shorter than the window (the returned window then still holds part of the incoming one)."""
    r = _rng(seed)
    for (b, D, L, K, silu) in ((2, 3, 11, 4, True), (1, 2, 9, 3, False), (2, 2, 2, 4, True), (1, 3, 6, 1, True)):
        x = r.standard_normal((b, D, L))
        w = r.standard_normal((D, K)) * 0.7
        bias = r.standard_normal(D)
        st = r.standard_normal((b, D, K - 1))
        du = r.standard_normal((b, D, L))
        dso = r.standard_normal((b, D, K - 1))
        g = orc.conv1d_bwd(x, w, du, bias=bias, state_in=st, dstate_out=dso, silu=silu)

        def loss(x_, w_, b_, s_):
            u, so = orc.conv1d(x_, w_, b_, s_, silu=silu)
            return float(np.sum(u * du) + np.sum(so * dso))

        eps = 1e-6
        for name, arr, key in (("x", x, "dx"), ("w", w, "dw"), ("bias", bias, "dbias"), ("state", st, "dstate_in")):
            if arr.size == 0:
                continue
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                args = {"x": x, "w": w, "bias": bias, "state": st}
                ap, am = arr.copy(), arr.copy()
                ap[idx] += eps
                am[idx] -= eps
                args[name] = ap
                lp = loss(args["x"], args["w"], args["bias"], args["state"])
                args[name] = am
                lm = loss(args["x"], args["w"], args["bias"], args["state"])
                num[idx] = (lp - lm) / (2 * eps)
            err = float(np.max(np.abs(num - g[key]))) / max(1.0, float(np.max(np.abs(num))))
            assert err < 1e-7, ("conv bwd", name, b, D, L, K, silu, err)


def pin_complex(orc, seed=13):
    r = _rng(seed)
    b, D, L, N = 2, 3, 24, 4
    x = r.standard_normal((b, D, L))
    dt = r.uniform(-3.0, 0.5, (b, D, L))
    bias = r.uniform(-0.5, 0.5, D)
    Are = -r.uniform(0.3, 2.0, (D, N))
    Aim = r.uniform(-4.0, 4.0, (D, N))
    Bre, Bim = r.standard_normal((b, N, L)), r.standard_normal((b, N, L))
    Cre, Cim = r.standard_normal((b, N, L)), r.standard_normal((b, N, L))
    Dk = r.standard_normal(D)
    z = r.standard_normal((b, D, L))
    h0 = r.standard_normal((b, D, N)) + 1j * r.standard_normal((b, D, N))
    for disc in (EULER_B, ZOH):
        # (a)
        y1, h1 = orc.scan(x, dt, Are, Bre, Cre, dt_bias=bias, Dskip=Dk, z=z, h0=h0.real, disc=disc)
        y2, h2 = orc.complex_scan(x, dt, Are + 0j, Bre + 0j, Cre + 0j, dt_bias=bias, Dskip=Dk, z=z, h0=h0.real + 0j,
                                  disc=disc)
        assert np.max(np.abs(y1 - y2)) < 1e-12 and np.max(np.abs(h1 - h2)) < 1e-12, ("P13a", disc)
        # (b) LTI: constant Delta per channel, constant B, C
        A = Are + 1j * Aim
        Bc = (Bre[:, :, :1] + 1j * Bim[:, :, :1]) * np.ones((1, 1, L))
        Cc = (Cre[:, :, :1] + 1j * Cim[:, :, :1]) * np.ones((1, 1, L))
        dtc = np.repeat(dt[:, :, :1], L, axis=2)
        y, _ = orc.complex_scan(x, dtc, A, Bc, Cc, Dskip=Dk, disc=disc)
        for bi in range(b):
            for d in range(D):
                delta = np.log1p(np.exp(dtc[bi, d, 0]))
                ab = np.exp(delta * A[d])
                coef = delta if disc == EULER_B else (ab - 1.0) / A[d]
                bb = coef * Bc[bi, :, 0]
                K = np.array([np.sum(Cc[bi, :, 0] * ab ** k * bb).real for k in range(L)])
                ref = np.array([np.sum(K[:t + 1][::-1] * x[bi, d, :t + 1]) for t in range(L)]) + Dk[d] * x[bi, d]
                assert np.max(np.abs(ref - y[bi, d])) < 1e-10, ("P13b", disc)
        # (c)
        B = Bre + 1j * Bim
        C = Cre + 1j * Cim
        ya, ha = orc.complex_scan(x, dt, A, B, C, dt_bias=bias, Dskip=Dk, z=z, h0=h0, disc=disc)
        yb, hb = orc.complex_scan(x, dt, A.conj(), B.conj(), C.conj(), dt_bias=bias, Dskip=Dk, z=z, h0=h0.conj(),
                                  disc=disc)
        assert np.max(np.abs(ya - yb)) < 1e-12 and np.max(np.abs(ha - hb.conj())) < 1e-12, ("P13c", disc)
        # (e)
        st = h0.copy()
        for t in range(L):
            yd, st = orc.complex_state_update(st, x[:, :, t], dt[:, :, t], A, B[:, :, t], C[:, :, t], dt_bias=bias,
                                              Dskip=Dk, z=z[:, :, t], disc=disc)
            assert np.max(np.abs(yd - ya[:, :, t])) < 1e-12, ("P13e", disc, t)
        assert np.max(np.abs(st - ha)) < 1e-12, ("P13e state", disc)
    # (d)
    w, delta, T = 0.7, 0.3, 40
    xi = np.zeros((1, 1, T))
    xi[0, 0, 0] = 1.0
    y, _ = orc.complex_scan(xi, np.full((1, 1, T), delta), np.array([[1j * w]]), np.ones((1, 1, T)) + 0j,
                            np.ones((1, 1, T)) + 0j, softplus=False)
    assert np.max(np.abs(y[0, 0] - delta * np.cos(w * delta * np.arange(T)))) < 1e-13, "P13d"


def _ssd_case(seed, b=2, L=37, H=4, P=3, G=2, N=5):
    r = _rng(seed)
    x = r.standard_normal((b, L, H, P))
    dt = r.uniform(-4.0, 1.0, (b, L, H))
    bias = r.uniform(-0.5, 0.5, H)
    A = -r.uniform(0.2, 3.0, H)
    A[1] = 0.0                       # the A == 0 limit of the zero-order hold
    B = r.standard_normal((b, L, G, N))
    C = r.standard_normal((b, L, G, N))
    Dk = r.standard_normal(H)
    z = r.standard_normal((b, L, H, P))
    h0 = r.standard_normal((b, H, P, N))
    return dict(x=x, dt=dt, dt_bias=bias, A=A, B=B, C=C, Dskip=Dk, z=z, h0=h0)


def _ssd_as_s6(orc, c, disc, g, hpg):
    """The heads of group g as S6 channels d = (head, column): A repeated over the state, B and C of the group."""
    b, L, H, P = c["x"].shape
    N = c["B"].shape[3]
    hs = slice(g * hpg, (g + 1) * hpg)
    x = c["x"][:, :, hs, :].transpose(0, 2, 3, 1).reshape(b, hpg * P, L)
    z = c["z"][:, :, hs, :].transpose(0, 2, 3, 1).reshape(b, hpg * P, L)
    dt = np.repeat(c["dt"][:, :, hs].transpose(0, 2, 1), P, axis=1)
    A = np.repeat(c["A"][hs], P)[:, None] * np.ones((1, N))
    bias = np.repeat(c["dt_bias"][hs], P)
    Dk = np.repeat(c["Dskip"][hs], P)
    h0 = c["h0"][:, hs].reshape(b, hpg * P, N)
    y, hf = orc.scan(x, dt, A, c["B"][:, :, g, :].transpose(0, 2, 1), c["C"][:, :, g, :].transpose(0, 2, 1),
                     dt_bias=bias, Dskip=Dk, z=z, h0=h0, disc=disc)
    return y.reshape(b, hpg, P, L).transpose(0, 3, 1, 2), hf.reshape(b, hpg, P, N)


def pin_ssd(orc, seed=14):
    """Mamba-2 SSD layer (close reading, section on Mamba-2/SSD; tutorial, "Mamba-2 与结构化对偶性"):
    (a) it is the S6 recurrence with the head's scalar A on every state entry and the group's B, C;
    (b) it equals the masked quadratic form y = (L o C B^T)(coef x) + D x with L[t,s] = exp(A (cum_t - cum_s)),
        cum = cumulative sum of Delta, plus the h0 term exp(A cum_t) C_t h0^T, computed with cumulative sums and
        one matrix product per head (the attention-like dual of the recurrence);
    (c) a split sequence with the state handed over equals one pass; (d) decode steps equal the scan."""
    c = _ssd_case(seed)
    b, L, H, P = c["x"].shape
    G, N = c["B"].shape[2], c["B"].shape[3]
    hpg = H // G
    for disc in (EULER_B, ZOH):
        y, hf = orc.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], dt_bias=c["dt_bias"], Dskip=c["Dskip"], z=c["z"],
                        h0=c["h0"], disc=disc)
        # (a)
        for g in range(G):
            ys, hs = _ssd_as_s6(orc, c, disc, g, hpg)
            assert np.max(np.abs(ys - y[:, :, g * hpg:(g + 1) * hpg])) < 1e-12, ("P14a y", disc, g)
            assert np.max(np.abs(hs - hf[:, g * hpg:(g + 1) * hpg])) < 1e-12, ("P14a h", disc, g)
        # (b)
        delta = _softplus_lib(c["dt"] + c["dt_bias"][None, None, :])            # (b, L, H)
        for bi in range(b):
            for h in range(H):
                a, g = c["A"][h], h // hpg
                dl = delta[bi, :, h]
                cum = np.cumsum(dl)
                coef = _coef(dl, np.full(L, a), disc)
                Lm = np.tril(np.exp(a * (cum[:, None] - cum[None, :])))
                Bg, Cg = c["B"][bi, :, g, :], c["C"][bi, :, g, :]
                xh = c["x"][bi, :, h, :]                                          # (L, P)
                ssm = (Lm * (Cg @ Bg.T)) @ (coef[:, None] * xh) + np.exp(a * cum)[:, None] * (Cg @ c["h0"][bi, h].T)
                ref = (ssm + c["Dskip"][h] * xh) * _silu(c["z"][bi, :, h, :])
                assert _rel(y[bi, :, h, :], ref) < 1e-11, ("P14b y", disc, bi, h)
                wts = np.exp(a * (cum[-1] - cum)) * coef
                href = (xh * wts[:, None]).T @ Bg + np.exp(a * cum[-1]) * c["h0"][bi, h]
                assert _rel(hf[bi, h], href) < 1e-11, ("P14b h", disc, bi, h)
        # (c)
        L1 = 15
        part = {k: c[k] for k in ("dt_bias", "Dskip", "A")}
        y1, h1 = orc.ssd(c["x"][:, :L1], c["dt"][:, :L1], B=c["B"][:, :L1], C=c["C"][:, :L1], z=c["z"][:, :L1],
                         h0=c["h0"], disc=disc, **part)
        y2, h2 = orc.ssd(c["x"][:, L1:], c["dt"][:, L1:], B=c["B"][:, L1:], C=c["C"][:, L1:], z=c["z"][:, L1:], h0=h1,
                         disc=disc, **part)
        assert np.max(np.abs(np.concatenate([y1, y2], axis=1) - y)) < 1e-12, ("P14c y", disc)
        assert np.max(np.abs(h2 - hf)) < 1e-12, ("P14c h", disc)
        # (d)
        st = c["h0"]
        for t in range(L):
            yd, st = orc.ssd_state_update(st, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                                          dt_bias=c["dt_bias"], Dskip=c["Dskip"], z=c["z"][:, t], disc=disc)
            assert np.max(np.abs(yd - y[:, t])) < 1e-12, ("P14d", disc, t)
        assert np.max(np.abs(st - hf)) < 1e-12, ("P14d state", disc)


def _checks(orc, worked_rows):
    checks = [("worked", lambda: pin_worked_examples(orc, worked_rows)), ("theorem1", lambda: pin_theorem1(orc)),
              ("zoh_euler", lambda: pin_zoh_euler(orc))]
    for disc in (EULER_B, ZOH):
        for N in (1, 4, 16):
            checks.append(("lti_N%d_disc%d" % (N, disc), lambda disc=disc, N=N: pin_lti_convolution(orc, disc, N=N)))
        checks += [("split_%d" % disc, lambda disc=disc: pin_split(orc, disc)),
                   ("materialised_%d" % disc, lambda disc=disc: pin_materialised(orc, disc)),
                   ("associative_%d" % disc, lambda disc=disc: pin_associative(orc, disc)),
                   ("linearity_%d" % disc, lambda disc=disc: pin_linearity(orc, disc)),
                   ("reset_hold_%d" % disc, lambda disc=disc: pin_reset_hold(orc, disc)),
                   ("decode_scan_%d" % disc, lambda disc=disc: pin_decode_scan(orc, disc)),
                   ("bwd_fd_%d" % disc, lambda disc=disc: pin_bwd_finite_differences(orc, disc))]
    checks += [("conv_numpy", lambda: pin_conv_numpy(orc)), ("conv_split", lambda: pin_conv_split(orc)),
               ("conv_bwd_fd", lambda: pin_conv_bwd_finite_differences(orc)),
               ("complex", lambda: pin_complex(orc)), ("ssd", lambda: pin_ssd(orc))]
    return checks


def _run(fn):
    try:
        fn()
        return None
    except Exception as e:  # noqa: BLE001 -- a mutant may also crash or raise
        return repr(e)[:200]


def all_pins(orc, worked_rows):
    """Run every pin; returns a list of (name, error-or-None)."""
    return [(name, _run(fn)) for name, fn in _checks(orc, worked_rows)]


def first_failure(orc, worked_rows, prefer=()):
    """Run the pins until one fails, those whose names start with one of `prefer` first; returns (name, error), or
    None when every pin passes.  A planted mistake has to fail one pin, and which one does not matter."""
    checks = _checks(orc, worked_rows)
    first = [c for c in checks if c[0].startswith(tuple(prefer))] if prefer else []
    for name, fn in first + [c for c in checks if c not in first]:
        err = _run(fn)
        if err is not None:
            return name, err
    return None
