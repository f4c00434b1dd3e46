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
cancel).  This test keeps the bars at least 2x above the floor there, and
checks the same for the bf16 part plan of the per-chunk kernel's products
accumulated over the value columns."""
import numpy as np
import pytest

import gdn_inputs as gi
from tests import fp32_bwd2_eval
from tests.fp32_bwd_eval import BF16_ACCUM_PLAN, mm_parts, per_head_errors

TOL_BWD = (1e-4, 1e-4, 1e-4, 1e-3, 1e-4, 1e-4)   # dq, dk, dv, dg, dbeta, dh0 (tests/test_parity_bwd.py)


CASES = [(150, 64, 728), (200, 128, 820), (130, 128, 641)]


def _case(T, D, seed):
    x = gi.gdn_inputs(1, T, 2, D, D, seed=seed, dtype="bf16", h0=True)
    rng = np.random.default_rng(seed + 7)
    do = rng.standard_normal((1, T, 2, D)).astype(np.float32).astype(np.float64)
    dht = rng.standard_normal((1, 2, D, D)).astype(np.float32).astype(np.float64)
    return x, do, dht


@pytest.mark.parametrize("T,D,seed", CASES)
def test_fp32_evaluation_is_below_the_bars(T, D, seed):
    errs = per_head_errors(*_case(T, D, seed)).max(axis=0)
    for name, e, bar in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), errs, TOL_BWD):
        assert e <= bar / 2, f"{name}: fp32 evaluation {e:.2e} > {bar / 2:.2e}"


@pytest.mark.parametrize("T,D,seed", CASES)
def test_bf16_part_plan_is_below_the_bars(T, D, seed):
    """The per-chunk kernel forms dR Vn^T, dR S^T, (T - I) R and
    (T - I)^T dVn from two bf16 parts per operand and dO Vn^T, dO S^T,
    Vn dS'^T, P^T dO from three; evaluated with those roundings, every
    gradient stays under half its bar, and dq within twice the float32
    floor."""
    case = _case(T, D, seed)
    floor = per_head_errors(*case).max(axis=0)
    errs = per_head_errors(*case, prods=BF16_ACCUM_PLAN).max(axis=0)
    for name, e, bar in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), errs, TOL_BWD):
        assert e <= bar / 2, f"{name}: bf16 part plan {e:.2e} > {bar / 2:.2e}"
    assert errs[0] <= 2 * floor[0], f"dq: {errs[0]:.2e} against the floor {floor[0]:.2e}"


@pytest.mark.parametrize("T,D,seed", CASES)
def test_two_parts_for_dO_Vn_would_lose_dq(T, D, seed):
    """Why dO Vn^T takes three parts: with two, dq (through dP K) lands at
    more than 5x the float32 floor on every case."""
    case = _case(T, D, seed)
    floor = per_head_errors(*case).max(axis=0)
    errs = per_head_errors(*case, prods=dict(BF16_ACCUM_PLAN, dP=mm_parts(2))).max(axis=0)
    assert errs[0] >= 5 * floor[0], f"dq: {errs[0]:.2e} against the floor {floor[0]:.2e}"


# GDN-2 (tests/test_parity_bwd2.py): the same check for its ragged-case bars
TOL_BWD2 = (1e-4, 1e-4, 1e-4, 1e-3, 5e-4, 1e-4, 1e-4)   # dq, dk, dv, dlog_alpha, db, dw, dh0


@pytest.mark.parametrize("B,T,Dk,Dv,seed", [(2, 150, 64, 64, 1028), (2, 150, 128, 128, 1156), (2, 150, 64, 128, 1092),
                                            (1, 200, 128, 128, 1120), (1, 65, 128, 128, 985)])
def test_gdn2_fp32_evaluation_is_below_the_bars(B, T, Dk, Dv, seed):
    """tests/fp32_bwd2_eval.py on the GDN-2 backward's ragged cases (their
    shapes and seeds): every gradient of the float32 evaluation stays under
    half its bar."""
    x = gi.gdn2_inputs(B, T, 2, Dk, Dv, seed=seed, dtype="bf16", h0=True)
    rng = np.random.default_rng(seed + 7)
    do = rng.standard_normal((B, T, 2, Dv)).astype(np.float32).astype(np.float64)
    dht = rng.standard_normal((B, 2, Dk, Dv)).astype(np.float32).astype(np.float64)
    errs = fp32_bwd2_eval.per_head_errors(x, do, dht).max(axis=0)
    for name, e, bar in zip(fp32_bwd2_eval.GRADS, errs, TOL_BWD2):
        assert e <= bar / 2, f"{name}: fp32 evaluation {e:.2e} > {bar / 2:.2e}"
