"""Shared test helpers: device transfer of stored inputs and parity checks."""

import numpy as np

# Tolerances for bf16 inputs against the float64 CPU oracle.
BF16_MAX_ABS_O = 1e-2
BF16_MEAN_ABS_O = 1e-3
BF16_MAX_ABS_LSE = 1e-3
BF16_REL_L2_O = 1e-2      # stricter internal gate: flat softmaxes make |O| small
F32_MAX_ABS_O = 1e-5
F32_MAX_ABS_LSE = 1e-5


def to_dev(arr, dev):
    """Stored input array (uint16 bf16 bits, float32 or int32) -> torch tensor on dev."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def parity_stats(o, lse, ro, rl):
    """Max/mean |dO|, relative L2 of O, max |dLSE| (rows with -inf on both sides count as equal)."""
    do = np.abs(o - ro)
    both_inf = np.isneginf(lse) & np.isneginf(rl)
    with np.errstate(invalid="ignore"):
        dl = np.where(both_inf, 0.0, np.abs(lse - rl))
    denom = np.linalg.norm(ro)
    rel = np.linalg.norm(o - ro) / denom if denom > 0 else np.linalg.norm(o - ro)
    return {"max_o": float(do.max()) if do.size else 0.0, "mean_o": float(do.mean()) if do.size else 0.0,
            "rel_l2": float(rel), "max_lse": float(np.nan_to_num(dl, nan=np.inf).max()) if dl.size else 0.0}


def assert_bf16_parity(o, lse, ro, rl, what=""):
    st = parity_stats(o, lse, ro, rl)
    msg = f"{what}: {st}"
    assert st["max_o"] <= BF16_MAX_ABS_O, msg
    assert st["mean_o"] <= BF16_MEAN_ABS_O, msg
    assert st["max_lse"] <= BF16_MAX_ABS_LSE, msg
    assert st["rel_l2"] <= BF16_REL_L2_O, msg
    return st


def assert_f32_parity(o, lse, ro, rl, what=""):
    st = parity_stats(o, lse, ro, rl)
    msg = f"{what}: {st}"
    assert st["max_o"] <= F32_MAX_ABS_O, msg
    assert st["max_lse"] <= F32_MAX_ABS_LSE, msg
    return st
