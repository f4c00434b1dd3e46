"""GPU parity of the chunked GDN backward (gdn_chunk_bwd through the C ABI)
against the fp64 oracle's backward (itself pinned to finite differences of
the forward), element by element.  The backward runs in fp32 on exact inputs
(bf16 inputs are exact in fp32), so both input types are held to the same bar
(max |diff| / rms of the oracle gradient): 1e-4 for dq, dk, dv, dbeta, dh0,
and 1e-3 for dg.  dg is a within-chunk reverse sum of differences of row and
column sums of much larger terms.

The bars stand on the float32 floor of the same chunk equations
(tests/fp32_bwd_eval.py, every product in float32; tests/test_fp32_floor.py).
At the full layer workload (T = 4096, the state gradient carried through 64
chunks, the maximum over 4096 x 128 entries of a head) that floor is, worst
head of 64: dq 7.9e-6, dk 9.9e-5, dv 7.3e-5, dg 5.3e-5, dbeta 4.7e-5, dh0
2.0e-6 (`python -m tests.fp32_bwd_eval`), so the full-size test holds each
head to about 8x that (TOL_FULL); the GPU measures dq 2.3e-5, dk 9.9e-5, dv
7.5e-5, dg 1.9e-4, dbeta 5.0e-5 and dh0 9.5e-6 there."""
import numpy as np
import pytest

import gated_delta_rule_34_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import dev, host, rel_err

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
TOL_BWD = {"dq": 1e-4, "dk": 1e-4, "dv": 1e-4, "dg": 1e-3, "dbeta": 1e-4, "dh0": 1e-4}
TOL_FULL = {"dq": 1e-4, "dk": 8e-4, "dv": 6e-4, "dg": 1e-3, "dbeta": 4e-4, "dh0": 1e-4}


def _case(B, T, H, Dk, Dv, seed, dtype, h0=True, dht=True):
    x = gi.gdn_inputs(B, T, H, Dk, Dv, seed=seed, dtype=dtype, h0=h0)
    rng = np.random.default_rng(seed + 7)
    x["do"] = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    x["dht"] = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32) if dht else None
    return x


def _gpu(x):
    r = gdn.gdn_chunk_bwd(*[dev(x[n]) for n in ("q", "k", "v", "g", "beta")],
                          dev(x["h0"]) if x["h0"] is not None else None, dev(x["do"]),
                          dev(x["dht"]) if x["dht"] is not None else None, scale=x["scale"])
    return [host(t) if t is not None else None for t in r]


def _ref(x):
    return oracle.gdn_bwd(*[x[n + "_f64"] for n in ("q", "k", "v", "g", "beta")], x["h0_f64"],
                          x["do"].astype(np.float64), None if x["dht"] is None else x["dht"].astype(np.float64),
                          scale=x["scale"])


def _check(got, ref):
    for name, a, b in zip(GRADS, got, ref):
        if b is None:
            assert a is None, name
            continue
        e = rel_err(a, b)
        assert e <= TOL_BWD[name], f"{name}: rel err {e:.3e} > {TOL_BWD[name]}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_bwd_head_sizes_ragged(dtype, Dk, Dv):
    x = _case(2, 150, 2, Dk, Dv, seed=600 + Dk + Dv, dtype=dtype)
    _check(_gpu(x), _ref(x))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_bwd_sequence_lengths(T):
    x = _case(1, T, 2, 128, 128, seed=620 + T, dtype="bf16")
    _check(_gpu(x), _ref(x))


def test_bwd_without_h0_and_final_state_gradient():
    x = _case(2, 130, 2, 64, 64, seed=640, dtype="fp32", h0=False, dht=False)
    _check(_gpu(x), _ref(x))


def test_bwd_weak_decay_long_carry():
    """Gates near zero: the state gradient is carried across many chunks."""
    x = _case(1, 512, 2, 128, 128, seed=641, dtype="bf16")
    x["g"] = (x["g"] * 0.01).astype(np.float32)
    x["g_f64"] = x["g"].astype(np.float64)
    _check(_gpu(x), _ref(x))


def test_bwd_deterministic():
    x = _case(2, 200, 2, 128, 128, seed=642, dtype="bf16")
    a, b = _gpu(x), _gpu(x)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_bwd_layer_workload_full_size_every_head():
    """B=8 H=8 T=4096 d=128 bf16 (the layer workload, with h0 and dht): every
    gradient of every head against the oracle, element by element, each head
    to the full-size bars (TOL_FULL)."""
    x = _case(8, 4096, 8, 128, 128, seed=643, dtype="bf16")
    got = _gpu(x)
    ref = _ref(x)
    B, H = x["h0"].shape[:2]
    for name, a, b in zip(GRADS, got, ref):
        heads = [(a[i, j], b[i, j]) if name == "dh0" else (a[i, :, j], b[i, :, j]) for i in range(B) for j in range(H)]
        worst = max(rel_err(u, w) for u, w in heads)
        print(f"{name}: worst head rel err {worst:.2e} (bar {TOL_FULL[name]:.0e})")
        assert worst <= TOL_FULL[name], f"{name}: worst head rel err {worst:.3e} > {TOL_FULL[name]}"
