"""CPU tests: the fp64 oracle against its pins (closed forms, identities, hand-worked examples), and a mutation
test showing that plausible mistakes planted in the oracle's source are caught by at least one pin."""
import os
import re
import tempfile

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")


def load_worked():
    rows = []
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        num = lambda s: None if s == "-" else float(s)
        rows.append(dict(name=f[0], disc=f[1], u=num(f[2]), A=num(f[3]), B=num(f[4]), C=num(f[5]), x=num(f[6]),
                         h0=num(f[7]), D=num(f[8]), z=num(f[9]), y=num(f[10]), h=num(f[11])))
    return rows


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle()


def test_worked_examples(orc):
    pins.pin_worked_examples(orc, load_worked())


def test_theorem1(orc):
    pins.pin_theorem1(orc)


def test_zoh_euler_ratio(orc):
    pins.pin_zoh_euler(orc)


@pytest.mark.parametrize("disc", [pins.EULER_B, pins.ZOH])
@pytest.mark.parametrize("N", [1, 4, 16])
def test_lti_convolution(orc, disc, N):
    pins.pin_lti_convolution(orc, disc, N=N)


@pytest.mark.parametrize("disc", [pins.EULER_B, pins.ZOH])
@pytest.mark.parametrize("name", ["split", "materialised", "associative", "linearity", "reset_hold", "decode_scan"])
def test_identity(orc, name, disc):
    getattr(pins, "pin_" + name)(orc, disc)


@pytest.mark.parametrize("disc", [pins.EULER_B, pins.ZOH])
def test_backward_finite_differences(orc, disc):
    pins.pin_bwd_finite_differences(orc, disc)


def test_backward_without_optional_parts(orc):
    # no gate / D / bias / h0 / dh_final: dz is zero, dD is the gradient at D = 0 (sum of dy * x), and the rest still
    # matches differences
    r = np.random.default_rng(3)
    x = r.standard_normal((1, 2, 7)); dt = r.uniform(-3, 1, (1, 2, 7)); A = -np.array([[1.0, 2.0], [0.5, 3.0]])
    B = r.standard_normal((1, 2, 7)); C = r.standard_normal((1, 2, 7)); dy = r.standard_normal((1, 2, 7))
    g = orc.scan_bwd(x, dt, A, B, C, dy)
    assert not np.any(g["dz"]) and np.all(np.isfinite(g["dh0"]))
    assert np.allclose(g["dD"], np.sum(dy * x, axis=(0, 2)), rtol=1e-13, atol=1e-13)
    y0, _ = orc.scan(x, dt, A, B, C)
    eps = 1e-6
    xp = x.copy(); xp[0, 1, 3] += eps
    xm = x.copy(); xm[0, 1, 3] -= eps
    fd = (np.sum(dy * orc.scan(xp, dt, A, B, C)[0]) - np.sum(dy * orc.scan(xm, dt, A, B, C)[0])) / (2 * eps)
    assert abs(fd - g["dx"][0, 1, 3]) < 1e-7


def test_conv_numpy(orc):
    pins.pin_conv_numpy(orc)


def test_conv_backward_finite_differences(orc):
    pins.pin_conv_bwd_finite_differences(orc)


def test_conv_split(orc):
    pins.pin_conv_split(orc)


def test_complex_a(orc):
    pins.pin_complex(orc)


def test_ssd(orc):
    pins.pin_ssd(orc)


def test_softplus_tails(orc):
    # Delta for very negative / positive logits: log1p(e^u) ~ e^u and ~ u + e^-u (no cancellation, no overflow).
    u = np.array([-40.0, -12.0, 0.0, 12.0, 40.0, 700.0])
    x = np.ones((1, 1, 6))
    # N = 1, A tiny so Abar ~ 1 and h after each step accumulates Delta; use one step per channel instead
    for i, uu in enumerate(u):
        y, _ = orc.scan(np.ones((1, 1, 1)), np.full((1, 1, 1), uu), np.full((1, 1), -1e-300), np.ones((1, 1, 1)),
                        np.ones((1, 1, 1)))
        exp = np.logaddexp(0.0, uu)
        assert abs(y[0, 0, 0] - exp) <= 1e-15 * max(1.0, exp), (uu, y[0, 0, 0], exp)


def test_all_pins_run_and_pass(orc):
    """The mutation test below runs the same list of pins (first_failure and all_pins share it): every entry must be
    (name, None) for the true oracle, and every family of pins must be in it (a check that is listed but never run
    would make the mutation test vacuous)."""
    res = pins.all_pins(orc, load_worked())
    assert all(isinstance(k, str) and e is None for k, e in res), [r for r in res if r[1] is not None]
    names = {k for k, _ in res}
    for must in ("worked", "theorem1", "zoh_euler", "split_0", "bwd_fd_1", "conv_numpy", "conv_split", "conv_bwd_fd",
                 "complex", "ssd"):
        assert must in names, must


# Mutation test: each planted mistake is a regex substitution on oracle_scan.c; every mutant must fail a pin.
MUTANTS = [
    ("drop_dskip", r"if \(has_D\) y \+= Dv \* xv;", "if (has_D) y += 0.0 * xv;"),
    ("gate_wrong_sign", r"zv / \(1\.0 \+ exp\(-zv\)\)", "zv / (1.0 + exp(zv))"),
    ("abar_sign", r"exp\(delta \* An\)", "exp(-delta * An)"),
    ("abar_missing_delta", r"double abar = exp\(delta \* An\);", "double abar = exp(An);"),
    ("euler_no_delta", r"coef = delta;\n    \} else", "coef = 1.0;\n    } else"),
    ("zoh_no_div", r"expm1\(delta \* An\) / An", "expm1(delta * An)"),
    ("softplus_plain", r"return u > 0\.0 \? u \+ log1p\(exp\(-u\)\) : log1p\(exp\(u\)\);", "return u;"),
    ("softplus_pos_branch", r"u \+ log1p\(exp\(-u\)\)", "log1p(exp(-u))"),
    ("bias_ignored", r"double u = dtv \+ bias;", "double u = dtv;"),
    ("y_before_update", r"h\[n\] = abar \* h\[n\] \+ coef \* Bt\[n \* Bstride\] \* xv;\n    y \+= Ct\[n \* Cstride\] \* h\[n\];",
     "y += Ct[n * Cstride] * h[n];\n    h[n] = abar * h[n] + coef * Bt[n * Bstride] * xv;"),
    ("B_C_swapped", r"coef \* Bt\[n \* Bstride\]", "coef * Ct[n * Cstride]"),
    ("h0_ignored", r"h\[n\] = h0 \? h0\[ch \* dstate \+ n\] : 0\.0;", "h[n] = 0.0;"),
    ("B_wrong_batch", r"const double\* Bb = B \+ b \* dstate \* seqlen;", "const double* Bb = B;"),
    ("A_wrong_row", r"A \+ d \* dstate, Bb \+ t", "A, Bb + t"),
    ("x_time_shift", r"yr\[t\] = step\(dstate, disc, use_softplus, xr\[t\]",
     "yr[t] = step(dstate, disc, use_softplus, xr[t > 0 ? t - 1 : 0]"),
    ("hfinal_zero", r"h_final\[ch \* dstate \+ n\] = h\[n\];", "h_final[ch * dstate + n] = 0.0;"),
    ("decode_bias_ignored", r"dt\[ch\], dt_bias \? dt_bias\[d\] : 0\.0", "dt[ch], 0.0"),
    ("bwd_no_decay_term", r"dDelta \+= g\[n\] \* \(dcoef_dd \* Bv \* xv \+ hprev \* abar \* An\);",
     "dDelta += g[n] * (dcoef_dd * Bv * xv);"),
    ("bwd_no_skip_dx", r"double dDelta = 0\.0, dxv = ds \* Dv;", "double dDelta = 0.0, dxv = 0.0;"),
    ("bwd_dC_uses_hprev", r"dC\[b \* N \* L \+ n \* L \+ t\] \+= ds \* hcur;", "dC[b * N * L + n * L + t] += ds * hprev;"),
    ("bwd_adjoint_not_decayed", r"g\[n\] \*= abar;", "g[n] *= 1.0;"),
    ("bwd_softplus_derivative", r"dDelta \* sigm\(u\)", "dDelta * sigm(-u)"),
    ("bwd_silu_derivative", r"\(sg \* \(1\.0 \+ zv \* \(1\.0 - sg\)\)\)", "sg"),
    ("bwd_zoh_dA_series", r"0\.5 \+ e \* \(1\.0 / 3\.0", "0.5 + e * (1.0 / 2.0"),
    ("conv_taps_reversed", r"acc \+= w\[d \* K \+ k\] \* xv;", "acc += w[d * K + (K - 1 - k)] * xv;"),
    ("conv_state_ignored", r"const double xv = tau >= 0 \? xr\[tau\] : \(st \? st\[S \+ tau\] : 0\.0\);",
     "const double xv = tau >= 0 ? xr[tau] : 0.0;"),
    ("conv_bias_dropped", r"double acc = bias \? bias\[d\] : 0\.0;", "double acc = 0.0;"),
    ("conv_state_out_shift", r"const int64_t tau = seqlen - S \+ i;", "const int64_t tau = seqlen - S + i - 1;"),
    ("conv_sigmoid_not_silu", r"use_silu \? acc / \(1\.0 \+ exp\(-acc\)\)", "use_silu ? 1.0 / (1.0 + exp(-acc))"),
    ("complex_rotation_sign", r"h\[2 \* n \+ 1\] = abr \* hi \+ abi \* hr \+ bbi;", "h[2 * n + 1] = abr * hi - abi * hr + bbi;"),
    ("complex_output_sign", r"y \+= Ct\[n \* bstride\] \* h\[2 \* n\] - Ct", "y += Ct[n * bstride] * h[2 * n] + Ct"),
    ("complex_zoh_division", r"ci = \(ei \* ar - er \* ai\) / den;", "ci = (ei * ar + er * ai) / den;"),
    ("complex_cos_sin_swapped", r"abr = mag \* cos\(ang\), abi = mag \* sin\(ang\)", "abr = mag * sin(ang), abi = mag * cos(ang)"),
    ("conv_bwd_silu_derivative", r"g \*= sg \* \(1\.0 \+ pre \* \(1\.0 - sg\)\);", "g *= sg;"),
    ("conv_bwd_window_out_ignored", r"for \(int64_t i = 0; i < S; \+\+i\) de\[L \+ i\] \+= dstate_out\[bd \* S \+ i\];",
     "for (int64_t i = 0; i < S; ++i) de[L + i] += 0.0;"),
    ("conv_bwd_taps_flipped", r"de\[t \+ k\] \+= w\[d \* K \+ k\] \* g;", "de[t + k] += w[d * K + (K - 1 - k)] * g;"),
    ("conv_bwd_dw_shift", r"sw\[k\] \+= g \* e\[t \+ k\];", "sw[k] += g * e[t + (k > 0 ? k - 1 : 0)];"),
    ("ssd_group_index", r"g = h / hpg", "g = h % G"),
    ("ssd_abar_sign", r"const double abar = exp\(delta \* Ah\);", "const double abar = exp(-delta * Ah);"),
    ("ssd_euler_no_delta", r"coef = disc == 0 \? delta :", "coef = disc == 0 ? 1.0 :"),
    ("ssd_zoh_no_div", r"expm1\(delta \* Ah\) / Ah", "expm1(delta * Ah)"),
    ("ssd_dskip_head", r"acc \+= Dskip\[h\] \* xv;", "acc += Dskip[0] * xv;"),
    ("ssd_y_before_update", r"S\[n\] = abar \* S\[n\] \+ coef \* Bt\[n\] \* xv;\n        acc \+= Ct\[n\] \* S\[n\];",
     "acc += Ct[n] * S[n];\n        S[n] = abar * S[n] + coef * Bt[n] * xv;"),
    ("ssd_h0_ignored", r"S\[n\] = h0 \? h0\[ch \* N \+ n\] : 0\.0;", "S[n] = 0.0;"),
    ("ssd_B_time_shift", r"const double\* Bt = B \+ \(\(b \* seqlen \+ t\)", "const double* Bt = B + ((b * seqlen + (t > 0 ? t - 1 : 0))"),
    ("ssd_decode_bias", r"const double u = dt\[b \* H \+ h\] \+ \(dt_bias \? dt_bias\[h\] : 0\.0\);",
     "const double u = dt[b * H + h];"),
    ("ssd_x_head0", r"const double xv = x\[row \* P \+ p\];", "const double xv = x[(row - h) * P + p];"),
    # decode-only code paths of the complex and SSD layers
    ("complex_decode_dskip_dropped", r"if \(Dskip\) yv \+= Dskip\[d\] \* x\[bd\];", "if (Dskip) yv += 0.0;"),
    ("complex_decode_gate_dropped", r"if \(z\) yv \*= z\[bd\] / \(1\.0 \+ exp\(-z\[bd\]\)\);", "if (z) yv *= 1.0;"),
    ("ssd_decode_gate_sign", r"if \(z\) acc \*= z\[i\] / \(1\.0 \+ exp\(-z\[i\]\)\);",
     "if (z) acc *= z[i] / (1.0 + exp(z[i]));"),
    ("ssd_decode_zoh_no_div", r"expm1\(delta \* Ah\) / Ah\);(\s+const double\* Bt = B \+ \(b \* G)",
     r"expm1(delta * Ah));\1"),
    ("bwd_dB_no_coef", r"dB\[b \* N \* L \+ n \* L \+ t\] \+= g\[n\] \* coef \* xv;",
     "dB[b * N * L + n * L + t] += g[n] * xv;"),
    ("bwd_dA_decay_no_delta", r"hprev \* abar \* delta\);", "hprev * abar);"),
    ("bwd_dD_ignores_gate", r"accD \+= ds \* xv;", "accD += dyv * xv;"),
    ("bwd_dz_no_preactivation", r"dz\[ch \* L \+ t\] = dyv \* S\[t\] \* ", "dz[ch * L + t] = dyv * "),
    ("bwd_dbias_dropped", r"if \(ddt_bias\) ddt_bias\[d\] = sb;", "if (ddt_bias) ddt_bias[d] = 0.0;"),
    ("bwd_dh0_zero", r"dh0\[ch \* N \+ n\] = g\[n\];", "dh0[ch * N + n] = 0.0;"),
    ("conv_bwd_dbias_dropped", r"if \(dbias\) dbias\[d\] = sb;", "if (dbias) dbias[d] = 0.0;"),
    # the SSD decode's own copies of lines the scan shares (the patterns above rewrite both)
    ("ssd_decode_group_index", r"const int64_t g = h / hpg;(\s+const double Ah = A\[h\];\s+const double u = dt\[b \* H)",
     r"const int64_t g = h % G;\1"),
    ("ssd_decode_abar_sign", r"const double abar = exp\(delta \* Ah\);(\s+const double coef = disc == 0 \? delta : "
     r"\(Ah == 0\.0 \? delta : expm1\(delta \* Ah\) / Ah\);\s+const double\* Bt = B \+ \(b \* G \+ g\) \* N;)",
     r"const double abar = exp(-delta * Ah);\1"),
    ("ssd_decode_C_from_B", r"const double\* Ct = C \+ \(b \* G \+ g\) \* N;", "const double* Ct = B + (b * G + g) * N;"),
]


# the pins a mistake in each part of the oracle is likely to fail, tried first (every pin is tried before a mutant
# counts as uncaught)
PREFER = (("conv_bwd", ("conv_bwd_fd",)), ("conv", ("conv_numpy", "conv_split")), ("complex", ("complex",)),
          ("ssd", ("ssd",)), ("bwd", ("bwd_fd",)), ("decode", ("decode_scan",)))


@pytest.mark.parametrize("name,pat,rep", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, pat, rep):
    src = oracle.source_text()
    mutated, n = re.subn(pat, rep, src)
    assert n >= 1, "mutation pattern %s no longer matches the oracle source" % name
    prefer = next((p for k, p in PREFER if name.startswith(k)), ())
    with tempfile.TemporaryDirectory() as td:
        lib = oracle.compile_variant(mutated, os.path.join(td, "mut_%s.so" % name))
        caught = pins.first_failure(oracle.Oracle(lib), load_worked(), prefer)
    assert caught is not None, "mutant %s passed every pin" % name
