"""Fit the polynomial of the exponential-offload kernel variant.

2^x is computed as 2^n * p(f) with n = floor(x), f = x - n in [0, 1), and p
a polynomial of degree 3 chosen to minimise the largest RELATIVE error
max |p(f) / 2^f - 1| over [0, 1] (Remez exchange on the equioscillating
reference points). Prints the coefficients (lowest degree first) as fp32
literals and the error bound achieved after rounding them to fp32.

    python exact_attention_forward_05_amd/csrc/fit_exp2_poly.py
"""
import numpy as np

DEG = 3


def remez(deg=DEG, iters=30):
    n = deg + 2
    # initial reference: Chebyshev extrema mapped to [0, 1]
    x = 0.5 - 0.5 * np.cos(np.pi * np.arange(n) / (n - 1))
    grid = np.linspace(0.0, 1.0, 200001)
    for _ in range(iters):
        # p(x_i) - 2^x_i * (-1)^i * E = 2^x_i  (relative error equioscillates)
        A = np.zeros((n, n))
        for i in range(n):
            A[i, :deg + 1] = x[i] ** np.arange(deg + 1)
            A[i, deg + 1] = -((-1) ** i) * 2.0 ** x[i]
        sol = np.linalg.solve(A, 2.0 ** x)
        c = sol[:deg + 1]
        err = np.polyval(c[::-1], grid) / 2.0 ** grid - 1.0
        # new reference: the extremum of each sign-alternating segment
        idx = [0]
        sign = np.sign(err)
        cuts = np.where(np.diff(sign) != 0)[0]
        bounds = [0, *(cuts + 1), len(grid)]
        ext = [lo + int(np.argmax(np.abs(err[lo:hi]))) for lo, hi in zip(bounds[:-1], bounds[1:])]
        if len(ext) != n:
            break
        x = grid[ext]
    return c


def main():
    c = remez()
    c32 = c.astype(np.float32)
    f = np.linspace(0.0, 1.0, 1000001, dtype=np.float64)
    p = np.polyval(c32.astype(np.float64)[::-1], f)
    rel = np.abs(p / 2.0 ** f - 1.0).max()
    for i, v in enumerate(c32):
        print(f"c{i} = {float(v):.9e}f")
    print(f"max relative error over [0, 1] (fp32 coefficients, exact arithmetic): {rel:.3e}")


if __name__ == "__main__":
    main()
