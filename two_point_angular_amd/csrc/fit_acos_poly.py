"""Fit the polynomial of the fp32 arccos core and write gc_acos_poly.h.

The pair kernel evaluates, for a = |x| in [0, 1],

    acos(a) ~= sqrt(1 - a) * P(a),

with P a degree-6 polynomial minimising max |P(a) - acos(a)/sqrt(1 - a)| over [0, 1]
(a linear-programming minimax fit on a dense grid, with the coefficients rounded to fp32
one at a time and the rest refitted).  The
ratio acos(a)/sqrt(1 - a) is smooth on [0, 1] (it tends to sqrt(2) at a = 1), so a
low-degree polynomial suffices; sqrt(1 - a) carries the square-root behaviour of acos
at a = 1.  This is the same square-root-times-polynomial form as the handbook
approximation that the page's fast path uses (section "L4: fast acos, with an
asterisk"), refitted here to a higher degree because the page's degree-3 version moves
counts between bins.

The header records the coefficients (as exact fp32 hex literals) and two measured
errors that the kernel's guard relies on:
  * FIT_ERR: max |P(a) - acos(a)/sqrt(1-a)| in fp64 with the fp32-rounded coefficients;
  * CORE_ERR: max |q - (pi/2 - acos(a))| over every fp32 a in [0, 1] of the fp32 core
    q = fma(-sqrt(1-a), P(a), pi/2), evaluated with emulated fp32 arithmetic
    (--exhaustive; otherwise on a 2^24-point grid).

Usage: python fit_acos_poly.py [--exhaustive]
"""
import argparse
import os

import numpy as np
from scipy.optimize import linprog

DEGREE = 6
HERE = os.path.dirname(os.path.abspath(__file__))


def target(a):
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    m = a < 1.0
    out[m] = np.arccos(a[m]) / np.sqrt(1.0 - a[m])
    out[~m] = np.sqrt(2.0)
    return out


def _lp_correction(V, resid):
    """Minimax LP for d with V d ~= resid; the residual is normalised to unit size first,
    because the solver's absolute tolerances (~1e-7) are as large as the errors fitted."""
    scale = float(np.max(np.abs(resid))) or 1.0
    r = resid / scale
    n = V.shape[1]
    c = np.zeros(n + 1)
    c[-1] = 1.0
    A = np.vstack([np.hstack([V, -np.ones((len(r), 1))]), np.hstack([-V, -np.ones((len(r), 1))])])
    b = np.concatenate([r, -r])
    res = linprog(c, A_ub=A, b_ub=b, bounds=[(None, None)] * n + [(0, None)], method="highs")
    if not res.success:
        raise RuntimeError(res.message)
    return res.x[:n] * scale


def _fit_free(a, g, degree, fixed, passes=4):
    """Minimax power-series coefficients of P with fixed[k] (not None) held at that value."""
    n = degree + 1
    V = np.vander(a, n, increasing=True)
    free = [k for k in range(n) if fixed[k] is None]
    coef = np.array([0.0 if f is None else f for f in fixed])
    for _ in range(passes):
        resid = g - V @ coef
        d = _lp_correction(V[:, free], resid)
        coef[free] += d
    return coef


def fit(degree=DEGREE):
    """Minimax fit, then fp32 rounding one coefficient at a time (lowest order first), each
    time re-solving the still-free coefficients, so the rounding error is absorbed."""
    a = np.unique(np.concatenate([np.linspace(0.0, 1.0, 20001), 1.0 - np.logspace(-14, -1, 2000)]))
    g = target(a)
    fixed = [None] * (degree + 1)
    coef = _fit_free(a, g, degree, fixed)
    for k in range(degree + 1):
        fixed[k] = float(np.float32(coef[k]))
        if k < degree:
            coef = _fit_free(a, g, degree, fixed)
    return np.array(fixed, dtype=np.float64)


def _compose(mono_u):
    # P(u) with u = 2a - 1, expanded in powers of a
    out = np.zeros(len(mono_u))
    base = np.array([1.0])
    lin = np.array([-1.0, 2.0])
    for k, ck in enumerate(mono_u):
        out[: len(base)] += ck * base
        base = np.polynomial.polynomial.polymul(base, lin)
    return out


def f32(x):
    return np.float32(x)


def fma32(a, b, c):
    """fp32 fma emulated in fp64 (exact product of two fp32, one fp64 add, round to fp32)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def core_q(a32, coef32):
    """q = fma(-sqrt(1 - a), P(a), pi/2) in emulated fp32 (correctly rounded sqrt)."""
    y = (np.float32(1.0) - a32).astype(np.float32)
    s = np.sqrt(y.astype(np.float64)).astype(np.float32)
    p = np.full_like(a32, coef32[-1])
    for ck in coef32[-2::-1]:
        p = fma32(p, a32, np.full_like(a32, ck))
    return fma32(-s, p, np.full_like(a32, np.float32(np.pi / 2)))


def measure(coef32, exhaustive=False):
    fit_a = np.linspace(0.0, 1.0, 2_000_001)
    p64 = np.polynomial.polynomial.polyval(fit_a, coef32.astype(np.float64))
    fit_err = float(np.max(np.abs(p64 - target(fit_a))))
    worst = 0.0
    if exhaustive:
        lo = np.float32(0.0).view(np.uint32)
        hi = np.float32(1.0).view(np.uint32)
        step = 1 << 24
        for start in range(int(lo), int(hi) + 1, step):
            bits = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
            a32 = bits.view(np.float32)
            q = core_q(a32, coef32)
            err = np.abs(q.astype(np.float64) - (np.pi / 2 - np.arccos(a32.astype(np.float64))))
            worst = max(worst, float(err.max()))
    else:
        a32 = np.linspace(0.0, 1.0, 1 << 24).astype(np.float32)
        q = core_q(a32, coef32)
        worst = float(np.max(np.abs(q.astype(np.float64) - (np.pi / 2 - np.arccos(a32.astype(np.float64))))))
    return fit_err, worst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--exhaustive", action="store_true")
    args = ap.parse_args()
    where = "every fp32 a in [0,1]" if args.exhaustive else "2^24-point grid"
    lines = ["// Generated by fit_acos_poly.py -- do not edit.", "#pragma once"]
    for degree, prefix in ((DEGREE, "GC_ACOS"),):
        coef32 = fit(degree).astype(np.float32)
        fit_err, core_err = measure(coef32, args.exhaustive)
        lines += [
            "// acos(a) ~= sqrt(1 - a) * P(a) for a in [0, 1]; P minimax (degree %d)." % degree,
            "// FIT_ERR:  max |P(a) - acos(a)/sqrt(1-a)| with these fp32 coefficients = %.3e" % fit_err,
            "// CORE_ERR: max |fma(-sqrt(1-a), P(a), pi/2) - (pi/2 - acos(a))| in fp32, %s = %.3e rad"
            % (where, core_err),
            "#define %s_DEGREE %d" % (prefix, degree),
            "#define %s_FIT_ERR %.6e" % (prefix, fit_err),
            "#define %s_CORE_ERR %.6e" % (prefix, core_err),
        ]
        for k, ck in enumerate(coef32):
            lines.append("#define %s_C%d %sf  /* %.9e */" % (prefix, k, float(ck).hex(), float(ck)))
    path = os.path.join(HERE, "gc_acos_poly.h")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
