"""Helpers for the GPU parity tests: move generator outputs onto the device and
measure the parity error the tolerances are stated in."""
import numpy as np


def dev(x, device="cuda"):
    """numpy generator output -> torch tensor on the GPU (uint16 = bf16 bits)."""
    import torch
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t):
    return t.detach().cpu().double().numpy()


def rel_err(x, ref):
    """max |x - ref| / rms(ref): the parity metric (per tensor)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.abs(x - ref).max())
    return float(np.abs(x - ref).max() / rms)


# Tolerances on max|diff| / rms(oracle), for o and for the final state.
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def gdn_dev_args(x):
    return [dev(x[n]) for n in ("q", "k", "v", "g", "beta", "h0")]


def gdn_ref_args(x):
    return [x[n + "_f64"] for n in ("q", "k", "v", "g", "beta", "h0")]
