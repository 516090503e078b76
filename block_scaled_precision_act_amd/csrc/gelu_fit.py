"""Derives the GELU coefficients in mx_epilogue.h (gelu_f32); run it to reproduce them.

erfc(z) = t exp(-z^2 + Q(t)),  t = 1 / (1 + p z),  z >= 0: the form of the erfcc routine of
Numerical Recipes (Press et al., 2nd ed., section 6.2).  With p = 0.4, Q is a degree-4
polynomial fitted to log(exp(z^2) erfc(z)) - log(t) by least squares on dense samples of z,
reweighted towards the largest errors so that the maximum error shrinks (|error of Q| is the
relative error of erfc).  The kernel evaluates exp in base 2, so the coefficients are printed
multiplied by log2(e), with -1 (the factor 1/2 of Phi(-|x|) = erfc(z) / 2) and +32 (a 2^32
pre-scale that keeps the value normal) added to the constant term.
"""
import numpy as np
from scipy.special import erfcx

P, DEGREE = 0.4, 4


def fit(p=P, n=DEGREE, iters=30):
    z = np.concatenate([np.linspace(0, 12, 200001), np.geomspace(12, 1e4, 2000)])
    t = 1 / (1 + p * z)
    target = np.log(erfcx(z)) - np.log(t)          # erfcx(z) = exp(z^2) erfc(z)
    w = np.ones_like(t)
    V = np.vander(t, n + 1, increasing=True)
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * w[:, None], target * w, rcond=None)
        e = V @ c - target
        w = w * (1 + 4 * np.abs(e) / np.abs(e).max())
        w /= w.mean()
    return c, np.abs(V @ c - target).max()


if __name__ == "__main__":
    c, err = fit()
    k = c * np.log2(np.e)
    k[0] += 32.0 - 1.0
    print(f"max |error of Q| = relative error of erfc: {err:.3g}")
    print("p / sqrt 2:", "%.9g" % np.float32(P / np.sqrt(2.0)))
    print("-log2(e) / 2:", "%.9g" % np.float32(-np.log2(np.e) / 2))
    print("coefficients, constant term first:", ["%.9g" % np.float32(v) for v in k])
