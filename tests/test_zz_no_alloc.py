"""gdn2_chunk_fwd_noalloc (the entry point that takes its workspace from the
library's fixed device array) against gdn2_chunk_fwd (caller-supplied
workspace), through the C ABI: the same kernels on the same inputs, so the
outputs must agree bit for bit; two calls in a row, the second smaller, so the
shared array's leftover contents from the first call cannot leak into the
second; both input types; the full-size GDN-2 workload; and the size limit."""
import numpy as np
import pytest
import torch

import gated_delta_rule_34_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "b", "w", "h0")


def _both(x):
    a = [dev(x[n]) for n in NAMES]
    B, T, H, _ = a[0].shape
    Dk, Dv = a[0].shape[-1], a[2].shape[-1]
    o_ref, s_ref = gdn.gdn2_chunk_fwd(*a, scale=x["scale"])
    torch.cuda.synchronize()
    o = torch.full((B, T, H, Dv), float("nan"), dtype=torch.float32, device=a[0].device)
    s = torch.full((B, H, Dk, Dv), float("nan"), dtype=torch.float32, device=a[0].device)
    gdn.gdn2_chunk_fwd_noalloc(*a, scale=x["scale"], out=o, final_state=s)
    torch.cuda.synchronize()
    return host(o), host(s), host(o_ref), host(s_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_equals_workspace_form_twice_second_smaller(dtype):
    big = gi.gdn2_inputs(2, 1000, 8, 128, 128, seed=501, dtype=dtype, h0=True)
    small = gi.gdn2_inputs(1, 130, 2, 128, 128, seed=502, dtype=dtype, h0=True)
    for x in (big, small):
        o, s, o_ref, s_ref = _both(x)
        np.testing.assert_array_equal(o, o_ref)
        np.testing.assert_array_equal(s, s_ref)
        ro, rs = oracle.gdn2_fwd(*[x[n + "_f64"] for n in NAMES], scale=x["scale"])
        assert rel_err(o, ro) <= TOL[dtype] and rel_err(s, rs) <= TOL[dtype]


def test_noalloc_full_size_workload():
    """B=4 H=8 T=4096 d=128 bf16 (2,048 chunk-heads, within the fixed array)."""
    x = gi.workload("gdn2_bf16")
    o, s, o_ref, s_ref = _both(x)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s, s_ref)


def test_noalloc_without_final_state():
    x = gi.gdn2_inputs(1, 200, 2, 64, 64, seed=503, dtype="bf16")
    a = [dev(x[n]) for n in NAMES]
    o_ref, _ = gdn.gdn2_chunk_fwd(*a, scale=x["scale"])
    o, ht = gdn.gdn2_chunk_fwd_noalloc(*a, scale=x["scale"])
    torch.cuda.synchronize()
    assert ht is None
    np.testing.assert_array_equal(host(o), host(o_ref))
