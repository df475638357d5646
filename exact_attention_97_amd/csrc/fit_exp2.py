"""Fit the polynomial used by the kernels' software exp2.

2^x is split as 2^n * 2^f with n = floor(x) and f = x - n in [0, 1); 2^f is
replaced by p(f) = 1 + c1 f + c2 f^2 + c3 f^3.  p(0) = 1 is imposed so that
exp2(0) is exactly 1 (a row's own maximum then contributes exactly one).
The remaining coefficients minimise the maximum relative error on [0, 1)
by a linear-programming minimax fit on a dense grid (scipy.optimize.linprog),
then the float32-rounded coefficients are re-evaluated in float32 Horner
form.  Run: python fit_exp2.py  (prints the constants of exp2_poly in
device_common.hpp; tests/test_oracle.py checks that the header holds them).
"""

import numpy as np
from scipy.optimize import linprog


def fit(degree=3, npts=20001):
    f = np.linspace(0.0, 1.0, npts)
    t = np.exp2(f)
    # unknowns: c1..c_deg, e ; minimise e subject to |(1 + sum c_k f^k) / t - 1| <= e
    cols = [f**k / t for k in range(1, degree + 1)]
    a_ub = []
    b_ub = []
    for sgn in (1.0, -1.0):
        a = np.stack([sgn * c for c in cols] + [-np.ones_like(f)], axis=1)
        a_ub.append(a)
        b_ub.append(sgn * (1.0 - 1.0 / t))
    res = linprog(np.r_[np.zeros(degree), 1.0], A_ub=np.vstack(a_ub), b_ub=np.concatenate(b_ub),
                  bounds=[(None, None)] * degree + [(0, None)], method="highs")
    assert res.success
    return res.x[:degree], res.x[degree]


def eval_f32(c, f):
    f = f.astype(np.float32)
    c = [np.float32(x) for x in c]
    acc = np.float32(c[-1])
    for ck in reversed(c[:-1]):
        acc = np.float32(acc * f + ck)
    return np.float32(acc * f + np.float32(1.0))


if __name__ == "__main__":
    for deg in (2, 3, 4):
        c, e = fit(deg)
        f = np.linspace(0, 1, 1000001, endpoint=False)
        rel = np.max(np.abs(eval_f32(c, f).astype(np.float64) / np.exp2(f) - 1.0))
        print(f"degree {deg}: minimax rel err {e:.3e}, float32 Horner rel err {rel:.3e}")
        print("  coefficients:", ", ".join(f"{np.float32(x).item():.9e}f" for x in c))
