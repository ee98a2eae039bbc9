"""Fits the sine and cosine polynomials of sincos_cw (ssm_complex_scan.hip) on |r| <= pi/4.

Minimax approximation by Lawson's algorithm (iteratively reweighted least squares) in fp64, in powers of u = r^2:
sin r = r (1 + c1 u + c2 u^2 + c3 u^3) and cos r = 1 + d1 u + d2 u^2 + d3 u^3 + d4 u^4.  Prints the coefficients
rounded to float32, the fit's own error, and the worst error of a float32 evaluation with one rounding per fused
multiply-add (in units in the last place of the result), next to the Taylor series one term longer.
Run: python3 sincos_fit.py
"""
import numpy as np

R = np.pi / 4
r = np.concatenate([np.cos(np.linspace(0, np.pi / 2, 4001)) * R, np.linspace(0, R, 4001)])
u = r * r


def lawson(target, deg, iters=60):
    """c_1..c_deg minimising max |1 + sum_j c_j u^j - target| over the nodes (Lawson's reweighting)."""
    w = np.ones_like(u)
    for _ in range(iters):
        a = np.stack([u ** j for j in range(1, deg + 1)], 1) * w[:, None]
        c, *_ = np.linalg.lstsq(a, (target - 1.0) * w, rcond=None)
        err = 1.0 + sum(c[j - 1] * u ** j for j in range(1, deg + 1)) - target
        w = w * (1 + 10 * np.abs(err) / np.abs(err).max())
        w /= w.mean()
    return c, np.abs(err).max()


sin_over_r = np.where(r > 0, np.sin(r) / np.where(r > 0, r, 1.0), 1.0)
cs, es = lawson(sin_over_r, 3)
cc, ec = lawson(np.cos(r), 4)
f32 = np.float32
cs32, cc32 = [f32(v) for v in cs], [f32(v) for v in cc]
print("sin r / r - 1: relative error %.2e; float32 coefficients %s" % (es, ["%.9e" % v for v in cs32]))
print("cos r - 1:     absolute error %.2e; float32 coefficients %s" % (ec, ["%.9e" % v for v in cc32]))


def fma32(a, b, c):
    return f32(np.float64(a) * np.float64(b) + np.float64(c))


def ulps(v, ref):
    return abs(float(v) - ref) / float(np.spacing(f32(max(abs(ref), 1e-30))))


worst = {"fit sin": 0.0, "fit cos": 0.0, "taylor sin": 0.0, "taylor cos": 0.0}
for x in np.linspace(-R, R, 28571).astype(np.float32):
    x2 = f32(x * x)
    xs, xc = np.sin(float(x)), np.cos(float(x))
    p = fma32(x2, cs32[2], cs32[1]); p = fma32(x2, p, cs32[0])
    worst["fit sin"] = max(worst["fit sin"], ulps(fma32(f32(x * x2), p, x), xs))
    p = fma32(x2, cc32[3], cc32[2]); p = fma32(x2, p, cc32[1]); p = fma32(x2, p, cc32[0])
    worst["fit cos"] = max(worst["fit cos"], ulps(fma32(x2, p, f32(1)), xc))
    p = fma32(x2, f32(1 / 362880), f32(-1 / 5040)); p = fma32(x2, p, f32(1 / 120)); p = fma32(x2, p, f32(-1 / 6))
    worst["taylor sin"] = max(worst["taylor sin"], ulps(fma32(f32(x * x2), p, x), xs))
    p = fma32(x2, f32(-1 / 3628800), f32(1 / 40320)); p = fma32(x2, p, f32(-1 / 720)); p = fma32(x2, p, f32(1 / 24))
    p = fma32(x2, p, f32(-0.5))
    worst["taylor cos"] = max(worst["taylor cos"], ulps(fma32(x2, p, f32(1)), xc))
print("float32 evaluation, worst error in ulps:", ", ".join("%s %.2f" % kv for kv in worst.items()))
