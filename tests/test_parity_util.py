"""The comparison the GPU parity tests use (tests/parity_util.py), on the host: it accepts
the oracle's own y rounded to fp32 and rejects one row wrong by 1%, a NaN, and a vector
off by 1e-3 overall."""

import numpy as np
import pytest

import synth
from oracle import gemv as ogemv
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y, row_bound


@pytest.mark.parametrize("fmt", [0, 1])
def test_check_y_accepts_rounding_rejects_errors(fmt):
    d_in, d_out = 1024, [512, 256]
    Ws = [synth.weights(3, d_in, r, m) for m, r in enumerate(d_out)]
    x16 = synth.activations(3, d_in, 1)
    nf, na = otiers.counts_from_fractions(d_in, 0.3, 0.3)
    _, f, a, _ = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nf, n_approx=na)
    O = opack.Layout(d_in, d_out, fmt, 128, 128)
    ref = ogemv.tiered_gemv(O, Ws, x16, f, a)
    bound = row_bound(O, Ws, x16, f, a)
    check_y(ref.astype(np.float32), ref, bound)
    for r in (0, 300, 767):
        bad = ref.copy()
        bad[r] *= 1.01
        with pytest.raises(AssertionError):
            check_y(bad, ref, bound)
    bad = ref.copy()
    bad[7] = np.nan
    with pytest.raises(AssertionError):
        check_y(bad, ref, bound)
    with pytest.raises(AssertionError):
        check_y(ref * (1 + 2e-3), ref, bound)
