"""The library as a user calls it: the usage shown in README.md, run as written (torch
tensors in, the library does the work) and checked against the oracle (masks and lists
bit-exact, y within rel-L2 1e-3); and a plain-C program that uses the C ABI directly."""

import math

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle

pytestmark = pytest.mark.gpu


def test_readme_usage():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax

    d_in, d_out = 4096, [4096, 4096, 4096]
    Ws = [synth.weights(31337, d_in, r, m) for m, r in enumerate(d_out)]
    W_q, W_k, W_v = [torch.from_numpy(w).to("cuda") for w in Ws]
    x16 = synth.activations(31337, d_in, 0)

    L = spax.spax_layout_init(d_in, d_out, spax.FMT_FP16, 128, 128)
    packed = torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda")
    spax.spax_pack_columns(L, [W_q, W_k, W_v], packed)
    x = torch.from_numpy(x16).to("cuda")
    lo, hi = spax.spax_guided_bounds(d_in, 0.5, 0.01)
    params = spax.guided_params(0.693147, lo, hi, 3, 10)
    f = torch.empty(d_in, dtype=torch.int32, device="cuda")
    a = torch.empty_like(f)
    c = torch.empty(3, dtype=torch.int32, device="cuda")
    spax.spax_build_tiers(x, d_in, params, None, f, a, c)
    y = torch.empty(L.d_out_total, dtype=torch.float32, device="cuda")
    spax.spax_tiered_gemv(L, packed, x, f, a, c, y, None)
    torch.cuda.synchronize()

    _, wf, wa, wc = otiers.build_tiers(x16, otiers.MODE_TOPK_GUIDED, tau=0.693147, n_lo=lo,
                                       n_hi=hi, num=3, den=10)
    cc = c.cpu().numpy()
    assert list(cc) == list(wc)
    assert np.array_equal(f.cpu().numpy()[:cc[0]], wf)
    assert np.array_equal(a.cpu().numpy()[:cc[1]], wa)
    check_y_oracle(y.cpu().numpy(), opack.Layout(d_in, d_out, 0, 128, 128), Ws, x16, wf, wa)


def test_c_abi_demo():
    """A plain-C program (tests/c/spax_abi_demo.c, no Python, no torch) packs, masks and
    multiplies through the C ABI and checks the dense product exactly, the TopK counts and
    lists, and the validation of a NULL pointer."""
    import os
    import subprocess
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__ as ge
    exe = ge.C_DEMO_BIN if os.path.exists(ge.C_DEMO_BIN) else ge.build_c_demo()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "spax C ABI demo: ok" in r.stdout
