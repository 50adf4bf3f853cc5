"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module only draws numbers: it holds none of the gated delta rule's
arithmetic.  The distributions follow the sweep described on the page
"Adding VJP for gated delta net" (ml-explore/mlx pull request 4565,
"Performance": B in {1,4,8}, T = 8..4096, Hk=16, Hv=32, Dk=Dv=128):
q, k, v ~ N(0, 1); the decay pre-activation a and the write-strength
pre-activation b ~ N(0, 1) with g = log(alpha) = -softplus(a) and
beta = sigmoid(b); an optional initial state ~ N(0, std).

Draw order is fixed: q, k, v, a, b, h0, do.  Everything is drawn in float32
with numpy's PCG64; tensors declared bf16 are rounded to bf16 (round to
nearest even) here, so every consumer sees the identical bit patterns.
"""

import numpy as np


def round_bf16(x):
    """Round a float32 array to the nearest bf16 value (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    u = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32)


def make_inputs(seed, B, T, Hk, Hv, Dk, Dv, io_dtype="bf16",
                channelwise=False, h0_std=None, with_do=True, gate_preact=False):
    """Return a dict of float32 numpy arrays (bf16-exact where io is bf16).

    Keys: q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; g [B,T,Hv] or [B,T,Hv,Dk];
    beta [B,T,Hv]; h0 [B,Hv,Dk,Dv] or None; do [B,T,Hv,Dv] or None.
    With gate_preact, g and beta are the N(0, 1) draws themselves (the
    pre-activations of the fused-gate flag), from the same stream.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    rnd = lambda shape: rng.standard_normal(shape, dtype=np.float32)
    q = rnd((B, T, Hk, Dk))
    k = rnd((B, T, Hk, Dk))
    v = rnd((B, T, Hv, Dv))
    a = rnd((B, T, Hv, Dk) if channelwise else (B, T, Hv))
    b = rnd((B, T, Hv))
    h0 = None
    if h0_std is not None:
        h0 = (rnd((B, Hv, Dk, Dv)) * np.float32(h0_std)).astype(np.float32)
    do = rnd((B, T, Hv, Dv)) if with_do else None
    if gate_preact:
        g, beta = a, b
    else:
        g = (-np.logaddexp(0.0, a.astype(np.float64))).astype(np.float32)
        beta = (1.0 / (1.0 + np.exp(-b.astype(np.float64)))).astype(np.float32)
    if io_dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
        if do is not None:
            do = round_bf16(do)
    elif io_dtype != "f32":
        raise ValueError(io_dtype)
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, do=do)
