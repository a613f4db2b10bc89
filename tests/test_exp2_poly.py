"""The polynomial exp2 of fa_fwd_poly_exp2 (FA4's softmax trick; CUDA Kernel interview course,
FlashAttention v4 card): its constants come from the committed Remez fit, and the fit's
error bound holds.  CPU only; the GPU evaluation is checked in test_poly_exp2_gpu.py."""
import os
import re

import numpy as np

from exact_attention_59_amd import fit_exp2_poly

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "exact_attention_59_amd",
                      "csrc", "fa_common.hpp")
BOUND = 8.6e-5  # the relative error bound the library documents


def compiled_constants():
    text = open(HEADER).read()
    m = re.search(r"kExp2C1 = (\S+)f, kExp2C2 = (\S+)f, kExp2C3 = (\S+)f;", text)
    assert m, "exp2 constants not found in fa_common.hpp"
    return [float.fromhex(x) for x in m.groups()]


def test_constants_are_the_fitted_ones():
    c, _ = fit_exp2_poly.fp32_constants()
    assert compiled_constants() == c


def test_fit_bound_and_shape():
    c, err = fit_exp2_poly.fp32_constants()
    assert err <= BOUND
    # minimax: the error of the fp64 fit equioscillates, so it comes close to the bound at
    # several points, of both signs
    c64, E = fit_exp2_poly.remez()
    f = np.linspace(0.0, 1.0, 1 << 16)[1:]
    e = fit_exp2_poly._poly(c64, f) / 2.0 ** f - 1.0
    assert abs(e.max() - E) < 1e-3 * E and abs(-e.min() - E) < 1e-3 * E
    # p(0) = 1 exactly and p(1) = 2 within the bound: 2^x is continuous across integers
    p1 = fit_exp2_poly._poly(np.asarray(c, dtype=np.float64), np.array([1.0]))[0]
    assert abs(p1 / 2.0 - 1.0) <= BOUND


def test_cubic_against_taylor():
    # the minimax cubic stays close to the Taylor coefficients of 2^f = e^(f ln 2), as a
    # gross check of the fit (a transposed or mis-scaled coefficient fails this)
    c = compiled_constants()
    ln2 = np.log(2.0)
    assert abs(c[0] - ln2) < 0.01 and abs(c[1] - ln2 ** 2 / 2) < 0.02 and abs(c[2] - ln2 ** 3 / 6) < 0.03
