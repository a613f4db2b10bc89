#!/usr/bin/env python3
"""Fit the cubic behind the forward's optional software exp2 and print its constants.

    python -m exact_attention_59_amd.fit_exp2_poly

The approximation (the FA4 softmax trick of computing part of the exponentials on the FMA
units instead of the transcendental unit; CUDA Kernel interview course, FlashAttention v4
card) reduces the argument exactly, x = n + f with n = floor(x) and f in [0, 1), and
evaluates 2^f with the cubic p(f) = 1 + f (c1 + c2 f + c3 f^2), then scales by 2^n with
ldexp.  p(0) = 1 is built in, so 2^x is exact at every integer x (the row maximum gives
p = 1 exactly).  c1..c3 minimise the largest relative error max |p(f) / 2^f - 1| over
[0, 1]: the Remez exchange algorithm on the linear system
    (p(f_i) - 2^f_i) / 2^f_i = (-1)^i E   at 4 reference points f_i,
moving the references to the error's alternating extrema until they stop moving.  The
coefficients are then rounded to fp32 (the kernel's constants) and the error of the rounded
cubic is measured on a dense grid; that figure is the bound the tests and the error
analysis use.

Prints the fp32 constants as C hex literals and the measured bound.  Deterministic: the
tests re-run it and compare with the constants compiled into the library.
"""
from __future__ import annotations

import numpy as np

DEGREE = 3
GRID = 1 << 20  # points of the dense error grid on (0, 1]


def _poly(c, f):
    acc = np.zeros_like(f)
    for cj in c[::-1]:
        acc = (acc + cj) * f
    return 1.0 + acc


def remez(degree: int = DEGREE, iters: int = 40):
    """Minimax relative-error coefficients c1..c_degree (fp64) and the levelled error E."""
    m = degree
    ref = 0.5 * (1.0 - np.cos(np.pi * (np.arange(m + 1) + 0.5) / (m + 1)))  # Chebyshev start
    grid = np.linspace(0.0, 1.0, 200001)[1:]
    c, E = None, None
    for _ in range(iters):
        t = 2.0 ** ref
        A = np.empty((m + 1, m + 1))
        for j in range(m):
            A[:, j] = ref ** (j + 1) / t
        A[:, m] = -((-1.0) ** np.arange(m + 1))
        sol = np.linalg.solve(A, (t - 1.0) / t)
        c, E = sol[:m], sol[m]
        e = _poly(c, grid) / 2.0 ** grid - 1.0
        # the error's extrema, one per run of equal sign
        idx, start = [], 0
        sgn = np.sign(e)
        for k in range(1, len(e) + 1):
            if k == len(e) or sgn[k] != sgn[start]:
                seg = np.arange(start, k)
                idx.append(seg[np.argmax(np.abs(e[seg]))])
                start = k
        if len(idx) > m + 1:  # keep the m + 1 consecutive extrema with the largest least |e|
            best = max(range(len(idx) - m), key=lambda s: np.min(np.abs(e[idx[s:s + m + 1]])))
            idx = idx[best:best + m + 1]
        if len(idx) != m + 1:
            break
        new = grid[np.array(idx)]
        if np.allclose(new, ref, rtol=0, atol=1e-12):
            break
        ref = new
    return c, abs(E)


def fp32_constants():
    """(c1, c2, c3) rounded to fp32, and the largest relative error of the rounded cubic on
    the dense grid (evaluated in fp64)."""
    c, _ = remez()
    c32 = np.asarray(c, dtype=np.float32)
    f = np.linspace(0.0, 1.0, GRID + 1)[1:]
    err = np.abs(_poly(c32.astype(np.float64), f) / 2.0 ** f - 1.0).max()
    return [float(x) for x in c32], float(err)


def main():
    c, err = fp32_constants()
    for i, x in enumerate(c, 1):
        print("c%d = %s  (%r)" % (i, float(np.float32(x)).hex(), x))
    print("max relative error of the fp32 cubic on [0, 1]: %.4g" % err)


if __name__ == "__main__":
    main()
