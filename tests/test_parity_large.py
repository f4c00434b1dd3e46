"""GPU parity at sizes whose element offsets pass 2^31: B = 8, T = 4096, H = 520,
d = 128, so every [B, T, H, 128] tensor holds 2.18e9 elements (bf16 inputs of
4.4 GB, fp32 outputs and gradients of 8.7 GB) and the decode steps carry an
fp32 state of 2.18e9 elements (B = 1040, H = 128).  Index arithmetic that
wraps at 32 bits would read or write the wrong rows of the high heads.

The inputs are 7 seeded head-sequences (generated as one small problem with
H = 7) laid out over the B * H heads by flat head index n = b H + h, variant
n mod 7, so that neighbouring heads and batch entries differ.  Two checks:
- every head equals, bit for bit, the first head of its variant (each kernel
  is deterministic and position-independent, so a wrongly indexed head would
  show up as a different value);
- the last head of each variant (the highest offsets) matches the fp64 oracle
  run on the small problem, to the bars of the full-size parity tests."""
import numpy as np
import pytest

import gated_delta_rule_34_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import TOL, host, rel_err

pytestmark = pytest.mark.gpu

NV = 7
B, T, H, D = 8, 4096, 520, 128
SB, SH = 1040, 128  # decode steps: B * H state heads of D x D


def _torch():
    import torch
    return torch


def _tile(a, nb, nh, time_axis=True):
    """Variant array [1, T, NV, ...] (time_axis) or [1, NV, ...] -> device
    tensor [nb, T, nh, ...] / [nb, nh, ...] with head n = b nh + h holding
    variant n mod NV."""
    torch = _torch()
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    t = t.to("cuda")[0]
    idx = torch.arange(nb * nh, device="cuda") % NV
    if time_axis:                                   # [T, NV, ...] -> [NV, T, ...]
        t = t.movedim(1, 0)
        big = t.index_select(0, idx)                # [nb nh, T, ...]
        big = big.view(nb, nh, *big.shape[1:]).movedim(1, 2).contiguous()
    else:                                           # [NV, ...]
        big = t.index_select(0, idx).view(nb, nh, *t.shape[1:]).contiguous()
    return big


def _heads(t, time_axis=True):
    """[nb, T, nh, ...] or [nb, nh, ...] -> [nb nh, -1] (a copy, head-major)."""
    if time_axis:
        t = t.movedim(2, 1)
    return t.reshape(t.shape[0] * t.shape[1], -1)


def _last_of_variant(nbh):
    return [max(n for n in range(j, nbh, NV)) for j in range(NV)]


def _check_variants(name, t, nh, time_axis=True):
    """Every head bitwise equal to the first head of its variant."""
    torch = _torch()
    hv = _heads(t, time_axis)
    idx = torch.arange(hv.shape[0], device="cuda") % NV
    ref = hv.index_select(0, idx)
    same = (hv == ref).all(dim=1)
    bad = (~same).nonzero().flatten().tolist()
    assert not bad, f"{name}: {len(bad)} heads differ from their variant's first head, e.g. {bad[:5]}"
    del hv, ref


def _head(t, n, nh, time_axis=True):
    b, h = divmod(n, nh)
    return host(t[b, :, h] if time_axis else t[b, h])


def _free():
    torch = _torch()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need_gib(gib):
    """Skip (not fail) when the device has less free memory than the case needs."""
    torch = _torch()
    _free()
    free, _ = torch.cuda.mem_get_info()
    if free < gib * 2 ** 30:
        pytest.skip(f"needs about {gib} GiB of free device memory, {free / 2 ** 30:.0f} GiB free")


def test_gdn_forward_past_2_31_elements():
    """gdn_chunk_fwd (bf16, the single fused kernel) over 4,160 heads."""
    torch = _torch()
    _need_gib(40)
    x = gi.gdn_inputs(1, T, NV, D, D, seed=4801, dtype="bf16", h0=True)
    q, k, v = (_tile(x[n], B, H) for n in ("q", "k", "v"))
    g, beta = (_tile(x[n], B, H) for n in ("g", "beta"))
    h0 = _tile(x["h0"], B, H, time_axis=False)
    assert q.numel() > 2 ** 31
    o, ht = gdn.gdn_chunk_fwd(q, k, v, g, beta, h0, scale=x["scale"])
    torch.cuda.synchronize()
    del q, k, v, g, beta, h0
    _check_variants("o", o, H)
    _check_variants("ht", ht, H, time_axis=False)
    ro, rS = oracle.gdn_fwd(*[x[n + "_f64"] for n in ("q", "k", "v", "g", "beta", "h0")], scale=x["scale"])
    for j, n in enumerate(_last_of_variant(B * H)):
        eo = rel_err(_head(o, n, H), ro[0, :, j])
        es = rel_err(_head(ht, n, H, False), rS[0, j])
        print(f"variant {j} at head {n}: o err {eo:.3e}, S err {es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    del o, ht
    _free()


def test_gdn2_forward_past_2_31_elements():
    """gdn2_chunk_fwd (bf16, prep and walk kernels) over 4,160 heads; the
    workspace holds 17.6 GB of per-chunk blocks."""
    torch = _torch()
    _need_gib(80)
    x = gi.gdn2_inputs(1, T, NV, D, D, seed=4802, dtype="bf16", h0=True)
    ins = [_tile(x[n], B, H) for n in ("q", "k", "v", "log_alpha", "b", "w")]
    h0 = _tile(x["h0"], B, H, time_axis=False)
    assert ins[0].numel() > 2 ** 31
    o, ht = gdn.gdn2_chunk_fwd(*ins, h0, scale=x["scale"])
    torch.cuda.synchronize()
    del ins, h0
    _free()
    _check_variants("o", o, H)
    _check_variants("ht", ht, H, time_axis=False)
    ro, rS = oracle.gdn2_fwd(*[x[n + "_f64"] for n in ("q", "k", "v", "log_alpha", "b", "w", "h0")],
                             scale=x["scale"])
    for j, n in enumerate(_last_of_variant(B * H)):
        eo = rel_err(_head(o, n, H), ro[0, :, j])
        es = rel_err(_head(ht, n, H, False), rS[0, j])
        print(f"variant {j} at head {n}: o err {eo:.3e}, S err {es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    del o, ht
    _free()


@pytest.mark.parametrize("kind", ["gdn", "gdn2"])
def test_decode_step_state_past_2_31_elements(kind):
    """gdn_recurrent_step / gdn2_recurrent_step on an fp32 state of 2.18e9
    elements (8.7 GB), updated in place."""
    torch = _torch()
    _need_gib(30)
    if kind == "gdn":
        x = gi.step_inputs(1, NV, D, D, seed=4803)
        names = ("q", "k", "v", "g", "beta")
        step, ref_step = gdn.gdn_recurrent_step, oracle.gdn_step
    else:
        x = gi.step2_inputs(1, NV, D, D, seed=4804)
        names = ("q", "k", "v", "log_alpha", "b", "w")
        step, ref_step = gdn.gdn2_recurrent_step, oracle.gdn2_step
    ins = [_tile(x[n], SB, SH, time_axis=False) for n in names]
    S = _tile(x["S"], SB, SH, time_axis=False)
    assert S.numel() > 2 ** 31
    o = step(*ins, S, scale=x["scale"])
    torch.cuda.synchronize()
    del ins
    _check_variants("o", o, SH, time_axis=False)
    _check_variants("S", S, SH, time_axis=False)
    ro, rS = ref_step(*[x[n + "_f64"] for n in names], x["S_f64"], scale=x["scale"])
    for j, n in enumerate(_last_of_variant(SB * SH)):
        eo = rel_err(_head(o, n, SH, False), ro[0, j])
        es = rel_err(_head(S, n, SH, False), rS[0, j])
        print(f"{kind} variant {j} at head {n}: o err {eo:.3e}, S err {es:.3e}")
        assert eo <= 1e-4 and es <= 1e-4
    del o, S
    _free()


def test_gdn_backward_past_2_31_elements():
    """gdn_chunk_bwd (bf16 inputs) over 4,160 heads, with h0 and a final-state
    gradient; every gradient to the full-size bars of the backward tests."""
    torch = _torch()
    _need_gib(130)
    from tests.test_parity_bwd import GRADS, TOL_FULL
    x = gi.gdn_inputs(1, T, NV, D, D, seed=4805, dtype="bf16", h0=True)
    rng = np.random.default_rng(4806)
    do_v = rng.standard_normal((1, T, NV, D)).astype(np.float32)
    dht_v = rng.standard_normal((1, NV, D, D)).astype(np.float32)
    ins = [_tile(x[n], B, H) for n in ("q", "k", "v", "g", "beta")]
    h0 = _tile(x["h0"], B, H, time_axis=False)
    do = _tile(do_v, B, H)
    dht = _tile(dht_v, B, H, time_axis=False)
    assert ins[0].numel() > 2 ** 31
    got = gdn.gdn_chunk_bwd(*ins, h0, do, dht, scale=x["scale"])
    torch.cuda.synchronize()
    del ins, h0, do, dht
    _free()
    ref = oracle.gdn_bwd(*[x[n + "_f64"] for n in ("q", "k", "v", "g", "beta")], x["h0_f64"],
                         do_v.astype(np.float64), dht_v.astype(np.float64), scale=x["scale"])
    last = _last_of_variant(B * H)
    for name, t, r in zip(GRADS, got, ref):
        ta = name != "dh0"
        _check_variants(name, t, H, time_axis=ta)
        for j, n in enumerate(last):
            e = rel_err(_head(t, n, H, ta), r[0, :, j] if ta else r[0, j])
            assert e <= TOL_FULL[name], f"{name} variant {j} at head {n}: rel err {e:.3e} > {TOL_FULL[name]}"
        print(f"{name}: all heads bitwise per variant, oracle parity at the last head of each variant")
    del got
    _free()


def test_gdn2_backward_past_2_31_elements():
    """gdn2_chunk_bwd (bf16 inputs) over 4,160 heads with a final-state
    gradient and no h0 (the GDN-2 workload's setting); each gradient to the
    full-size bars of the GDN-2 backward tests."""
    torch = _torch()
    _need_gib(200)
    from tests.test_parity_bwd2 import GRADS, NAMES, TOL_FULL
    x = gi.gdn2_inputs(1, T, NV, D, D, seed=4807, dtype="bf16")
    rng = np.random.default_rng(4808)
    do_v = rng.standard_normal((1, T, NV, D)).astype(np.float32)
    dht_v = rng.standard_normal((1, NV, D, D)).astype(np.float32)
    ins = [_tile(x[n], B, H) for n in NAMES]
    do = _tile(do_v, B, H)
    dht = _tile(dht_v, B, H, time_axis=False)
    assert ins[0].numel() > 2 ** 31
    got = gdn.gdn2_chunk_bwd(*ins, None, do, dht, scale=x["scale"])
    torch.cuda.synchronize()
    del ins, do, dht
    _free()
    assert got[6] is None
    ref = oracle.gdn2_bwd(*[x[n + "_f64"] for n in NAMES], None, do_v.astype(np.float64),
                          dht_v.astype(np.float64), scale=x["scale"])
    last = _last_of_variant(B * H)
    for name, t, r in zip(GRADS[:6], got[:6], ref[:6]):
        _check_variants(name, t, H)
        for j, n in enumerate(last):
            e = rel_err(_head(t, n, H), r[0, :, j])
            assert e <= TOL_FULL[name], f"{name} variant {j} at head {n}: rel err {e:.3e} > {TOL_FULL[name]}"
        print(f"{name}: all heads bitwise per variant, oracle parity at the last head of each variant")
    del got
    _free()
