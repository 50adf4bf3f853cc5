"""Shared helpers for the tests (no arithmetic of the method lives here)."""

import numpy as np
import torch


def relerr(x, ref):
    """max |x - ref| / max |ref| over the whole tensor (0 for an all-zero pair)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    return float(num / den) if den > 0 else float(num)


def dev(x, dtype=torch.float32, device="cuda"):
    """numpy float32 array -> contiguous device tensor of dtype (bf16 exact
    for arrays that synth already rounded)."""
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dtype).contiguous()


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def io_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32
