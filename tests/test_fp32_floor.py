"""The float32 floor behind the GDN backward's tolerance bars (CPU).

tests/fp32_bwd_eval.py evaluates the chunked backward with every matrix
product in float32; the GPU backward computes in fp32, so its parity bars in
tests/test_parity_bwd.py are set above what that evaluation reaches.  On the
ragged cases below the float32 evaluation reaches (worst head):
  T=150 d=64:   dq 2.1e-6, dk 7.2e-6, dv 7.3e-6, dg 1.4e-6, dbeta 1.9e-6, dh0 7.2e-7
  T=200 d=128:  dq 3.4e-6, dk 3.4e-6, dv 9.7e-6, dg 3.2e-6, dbeta 1.6e-6, dh0 9.2e-7
  T=130 d=128:  dq 2.9e-6, dk 3.0e-6, dv 1.1e-5, dg 1.9e-6, dbeta 4.0e-5, dh0 1.3e-6
so the ragged-case bars (1e-4, dg 1e-3) sit 8x or more above it, except dbeta
on the last case (2.5x: dbeta sums dR (v - gamma K S) and dA . K K^T, which
cancel).  This test keeps the bars at least 2x above the floor there."""
import numpy as np
import pytest

import gdn_inputs as gi
from tests.fp32_bwd_eval import per_head_errors

TOL_BWD = (1e-4, 1e-4, 1e-4, 1e-3, 1e-4, 1e-4)   # dq, dk, dv, dg, dbeta, dh0 (tests/test_parity_bwd.py)


@pytest.mark.parametrize("T,D,seed", [(150, 64, 728), (200, 128, 820), (130, 128, 641)])
def test_fp32_evaluation_is_below_the_bars(T, D, seed):
    x = gi.gdn_inputs(1, T, 2, D, D, seed=seed, dtype="bf16", h0=True)
    rng = np.random.default_rng(seed + 7)
    do = rng.standard_normal((1, T, 2, D)).astype(np.float32).astype(np.float64)
    dht = rng.standard_normal((1, 2, D, D)).astype(np.float32).astype(np.float64)
    errs = per_head_errors(x, do, dht).max(axis=0)
    for name, e, bar in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), errs, TOL_BWD):
        assert e <= bar / 2, f"{name}: fp32 evaluation {e:.2e} > {bar / 2:.2e}"
