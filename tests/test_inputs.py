import numpy as np
import pytest

import gdn_inputs as gi


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        [0.0, -0.0, 1.0, -1.0, 1.00390625, 1.0117188, 3.0e38]])
    bits = gi.bf16_bits_from_f64(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = gi.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_deterministic_and_shaped():
    a = gi.gdn_inputs(2, 70, 3, 16, 8, seed=5, dtype="bf16", h0=True)
    b = gi.gdn_inputs(2, 70, 3, 16, 8, seed=5, dtype="bf16", h0=True)
    for n in ("q", "k", "v", "g", "beta", "h0"):
        np.testing.assert_array_equal(a[n], b[n])
    assert a["q"].shape == (2, 70, 3, 16) and a["q"].dtype == np.uint16
    assert a["v"].shape == (2, 70, 3, 8)
    assert a["g"].shape == (2, 70, 3) and a["g"].dtype == np.float32
    assert a["h0"].shape == (2, 3, 16, 8)
    assert np.all(a["g"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))
    # q, k unit norm before quantisation; bf16 keeps the norm within ~2^-8
    n = np.linalg.norm(a["k_f64"], axis=-1)
    assert np.all(np.abs(n - 1) < 2e-2)


def test_generator_fp32_exact_view():
    a = gi.gdn_inputs(1, 10, 2, 8, 8, seed=3, dtype="fp32")
    np.testing.assert_array_equal(a["q"].astype(np.float64), a["q_f64"])


def test_gdn2_and_step_generators():
    x = gi.gdn2_inputs(1, 9, 2, 8, 4, seed=1)
    assert x["log_alpha"].shape == (1, 9, 2, 8) and np.all(x["log_alpha"] < 0)
    assert x["b"].shape == (1, 9, 2, 8) and x["w"].shape == (1, 9, 2, 4)
    s = gi.step_inputs(4, 2, 8, 8, seed=2)
    assert s["S"].shape == (4, 2, 8, 8) and s["q"].shape == (4, 2, 8)


def test_workload_table():
    assert gi.WORKLOADS["layer_bf16"]["T"] == 4096
    x = gi.workload("tiny_fp32")
    assert x["q"].shape == (1, 256, 2, 64) and x["q"].dtype == np.float32
