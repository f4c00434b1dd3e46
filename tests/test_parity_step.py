"""GPU parity of the single-token decode step (gdn_recurrent_step) against the
fp64 oracle, and consistency of prefill + decode with the chunked forward."""
import numpy as np
import pytest

import gated_delta_rule_34_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import TOL, dev, gdn_dev_args, gdn_ref_args, host, rel_err

pytestmark = pytest.mark.gpu


def _step(x):
    S = dev(x["S"])
    o = gdn.gdn_recurrent_step(*[dev(x[n]) for n in ("q", "k", "v", "g", "beta")], S, scale=x["scale"])
    return host(o), host(S)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_step_small(dtype, Dk, Dv):
    x = gi.step_inputs(3, 5, Dk, Dv, seed=70 + Dk + Dv, dtype=dtype)
    o, S = _step(x)
    ro, rS = oracle.gdn_step(*[x[n + "_f64"] for n in ("q", "k", "v", "g", "beta", "S")], scale=x["scale"])
    # everything inside the step is fp32 arithmetic on exact inputs
    assert rel_err(o, ro) < 1e-5 and rel_err(S, rS) < 1e-5


def test_decode_workload_full_size():
    """B=256 H=16 d=128 bf16, fp32 state in place (the measured decode workload)."""
    x = gi.workload("decode_bf16")
    o, S = _step(x)
    ro, rS = oracle.gdn_step(*[x[n + "_f64"] for n in ("q", "k", "v", "g", "beta", "S")], scale=x["scale"])
    assert rel_err(o, ro) < 1e-5 <= TOL["bf16"]
    assert rel_err(S, rS) < 1e-5


def test_prefill_then_decode_matches_chunked():
    """Chunked prefill of T0 tokens, then one decode step per token, equals the
    chunked forward over all tokens (o and final state)."""
    import torch
    T0, T = 130, 140
    x = gi.gdn_inputs(2, T, 3, 128, 128, seed=71, dtype="bf16", h0=True)
    q, k, v, g, beta, h0 = gdn_dev_args(x)
    o_all, S_all = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0)
    o_pre, S = gdn.gdn_chunk_fwd(*[t[:, :T0].contiguous() for t in (q, k, v, g, beta)], h0)
    outs = [o_pre]
    for t in range(T0, T):
        o_t = gdn.gdn_recurrent_step(*[a[:, t].contiguous() for a in (q, k, v, g, beta)], S)
        outs.append(o_t[:, None])
    ref = oracle.gdn_fwd(*gdn_ref_args(x), scale=x["scale"])
    assert rel_err(host(torch.cat(outs, 1)), ref[0]) <= TOL["bf16"]
    assert rel_err(host(S), ref[1]) <= TOL["bf16"]
    assert rel_err(host(S), host(S_all)) <= TOL["bf16"]
