"""Plain fp64 CPU oracle for the gated delta rule: forward pass and its VJP.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may call it.  It shares no code, constants or helpers with the HIP
library; it receives plain numpy arrays and returns plain numpy arrays.

Sources (web pages; cited by title and section):
  [MLX]  "Adding VJP for gated delta net" (ml-explore/mlx pull request 4565):
         description (a VJP for the gated delta net, sequential and chunked
         kernels) and "Performance" (the backward sweep B in {1,4,8},
         T = 8..4096, Hk=16, Hv=32, Dk=Dv=128).
  [ET]   "Two-pass optimization for channelwise gated delta rule kernel"
         (pytorch/executorch pull request 21020): summary (a per-key-channel
         decay; pass one forms the prediction with the decay folded in, pass
         two applies decay plus the rank-one update and accumulates the
         output).
  [MEG]  "perf(gated_delta_net): fold q/k L2-norm into the gated_delta_rule
         kernel" (NVIDIA/Megatron-LM pull request 5396): "What" and "Why"
         (q/k are L2-normalised over the last dimension inside the kernel,
         eps 1e-6; with the flag off the inputs are used as given).

The pages name the gated delta rule but print no formula.  The recurrence
used here is the published gated delta rule (Yang, Kautz & Hatamizadeh,
"Gated Delta Networks", ICLR 2025), per head:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

with S of shape Dv x Dk.  This module carries H = S^T (Dk x Dv), the layout
the library stores, so with D_t = diag(alpha_t) H_{t-1}:

    p_t = D_t^T k_t,  u_t = beta_t (v_t - p_t),  H_t = D_t + k_t u_t^T,
    o_t = H_t^T q_t.

For a scalar alpha this is the line above transposed.  For the channelwise
gate of [ET] alpha_t is a Dk-vector; the decay is applied to the state before
the prediction is formed ("folding in decay" in [ET]), i.e.
S_t = S_{t-1} diag(alpha_t) (I - beta_t k k^T) + beta_t v k^T.

Readings where the pages are silent (each also listed in the design doc):
  * L2 norm: x * (sum x^2 + eps)^(-1/2) over the last dim, eps = 1e-6.
  * q has Hk heads like k (the pages split one joint query_key activation).
  * GQA: v-head hv reads k/q head hv // (Hv // Hk).
  * No output scale; beta is not clamped.
  * g = log(alpha) is passed in; alpha = exp(g).
  * Fused gate activation (the fold-the-caller's-prep-into-the-kernel idea of
    [MEG] applied to the gates; a reading, the pages name no activation):
    with fused_gates the g and beta arguments are pre-activations a, b and
    the recurrence uses g = -softplus(a) = -log(1 + e^a) (so alpha =
    1 / (1 + e^a) <= 1) and beta = sigmoid(b); the VJP then returns the
    gradients with respect to a and b.

Array shapes (all functions): q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv];
g [B,T,Hv] (scalar gate) or [B,T,Hv,Dk] (channelwise); beta [B,T,Hv];
h0 / ht / dh0 / dht [B,Hv,Dk,Dv].  Everything is computed in float64.
"""

import numpy as np

L2_EPS = 1e-6


def _f64(x):
    return np.array(x, dtype=np.float64, copy=True)


def _sigmoid(x):
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate_activation(a, b):
    """Fused gates: g = -softplus(a) = -(max(a, 0) + log1p(e^-|a|)) and
    beta = sigmoid(b), in float64."""
    a, b = _f64(a), _f64(b)
    return -(np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a)))), _sigmoid(b)


def gate_activation_vjp(a, b, dg, dbeta):
    """Chain rule through gate_activation: d/da = -sigmoid(a) dg,
    d/db = beta (1 - beta) dbeta."""
    sb = _sigmoid(_f64(b))
    return -_sigmoid(_f64(a)) * dg, sb * (1.0 - sb) * dbeta


def l2norm(x, eps=L2_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis ([MEG] "What"/"Why")."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def l2norm_vjp(x, dxhat, eps=L2_EPS):
    """Gradient of l2norm at x given the gradient of its output.

    With r = (sum x^2 + eps)^(-1/2) and xhat = r x:
    dx = r * (dxhat - xhat * <xhat, dxhat>)  (differentiate r x by hand).
    """
    x = _f64(x)
    dxhat = _f64(dxhat)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    xhat = x * r
    return r * (dxhat - xhat * np.sum(xhat * dxhat, axis=-1, keepdims=True))


def _prepare(q, k, use_qk_l2norm, Hv):
    """Normalised (or raw) q/k expanded from Hk to Hv heads (GQA reading)."""
    Hk = q.shape[2]
    if Hv % Hk != 0:
        raise ValueError("Hv must be a multiple of Hk")
    qh = l2norm(q) if use_qk_l2norm else _f64(q)
    kh = l2norm(k) if use_qk_l2norm else _f64(k)
    grp = Hv // Hk
    return np.repeat(qh, grp, axis=2), np.repeat(kh, grp, axis=2)


def _decay(g, t, channelwise):
    """alpha_t shaped to scale the rows of H [B,Hv,Dk,Dv]."""
    a = np.exp(_f64(g[:, t]))
    return a[..., :, None] if channelwise else a[..., None, None]


def forward(q, k, v, g, beta, h0=None, use_qk_l2norm=True, channelwise=False, fused_gates=False):
    """Token-by-token recurrence, returns (o [B,T,Hv,Dv], ht [B,Hv,Dk,Dv]).

    One step per token exactly as written in the module docstring: decay the
    state, predict, form the delta, rank-one update, read out.  With
    fused_gates, g and beta are the pre-activations of gate_activation.
    """
    if fused_gates:
        g, beta = gate_activation(g, beta)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    qh, kh = _prepare(q, k, use_qk_l2norm, Hv)
    vv, bb = _f64(v), _f64(beta)
    H = np.zeros((B, Hv, Dk, Dv)) if h0 is None else _f64(h0)
    o = np.zeros((B, T, Hv, Dv))
    for t in range(T):
        D = _decay(g, t, channelwise) * H
        kt, qt = kh[:, t], qh[:, t]
        p = np.einsum("bhij,bhi->bhj", D, kt)
        u = bb[:, t][..., None] * (vv[:, t] - p)
        H = D + kt[..., :, None] * u[..., None, :]
        o[:, t] = np.einsum("bhij,bhi->bhj", H, qt)
    return o, H


def backward(q, k, v, g, beta, h0, do, dht=None, use_qk_l2norm=True,
             channelwise=False, fused_gates=False):
    """Hand-derived VJP of ``forward``; returns dq, dk, dv, dg, dbeta, dh0.

    The forward is replayed once and every state H_0..H_T is kept (plain and
    memory hungry on purpose).  Then, per token in reverse, with dH the
    gradient arriving at H_t:
        dHt  = dH + q ⊗ do                 (o = H_t^T q)
        dq   = H_t do
        du   = dHt^T k,   dk = dHt u       (H_t = D + k u^T)
        dv   = beta du,   dbeta = <du, v - p>,   dp = -beta du
        dD   = dHt + k ⊗ dp,  dk += D dp   (p = D^T k)
        dg   = <dD, D>  (per row of D when channelwise),  dH = diag(alpha) dD
    After t = 0, dh0 = dH.  q/k gradients are summed over the v-heads that
    share a k-head (in v-head order) and then passed through ``l2norm_vjp``.
    With fused_gates, g and beta are pre-activations and dg, dbeta are
    returned with respect to them (``gate_activation_vjp``).
    """
    if fused_gates:
        a_pre, b_pre = g, beta
        g, beta = gate_activation(a_pre, b_pre)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    grp = Hv // Hk
    qh, kh = _prepare(q, k, use_qk_l2norm, Hv)
    vv, bb, dd = _f64(v), _f64(beta), _f64(do)
    states = np.zeros((T + 1, B, Hv, Dk, Dv))
    if h0 is not None:
        states[0] = _f64(h0)
    for t in range(T):
        D = _decay(g, t, channelwise) * states[t]
        p = np.einsum("bhij,bhi->bhj", D, kh[:, t])
        u = bb[:, t][..., None] * (vv[:, t] - p)
        states[t + 1] = D + kh[:, t][..., :, None] * u[..., None, :]

    dqh = np.zeros((B, T, Hv, Dk))
    dkh = np.zeros((B, T, Hv, Dk))
    dv = np.zeros((B, T, Hv, Dv))
    dg = np.zeros(g.shape)
    dbeta = np.zeros((B, T, Hv))
    dH = np.zeros((B, Hv, Dk, Dv)) if dht is None else _f64(dht)
    for t in range(T - 1, -1, -1):
        a = _decay(g, t, channelwise)
        D = a * states[t]
        kt, qt, dot = kh[:, t], qh[:, t], dd[:, t]
        bt = bb[:, t][..., None]
        p = np.einsum("bhij,bhi->bhj", D, kt)
        u = bt * (vv[:, t] - p)
        dHt = dH + qt[..., :, None] * dot[..., None, :]
        dqh[:, t] = np.einsum("bhij,bhj->bhi", states[t + 1], dot)
        du = np.einsum("bhij,bhi->bhj", dHt, kt)
        dk_t = np.einsum("bhij,bhj->bhi", dHt, u)
        dv[:, t] = bt * du
        dbeta[:, t] = np.sum(du * (vv[:, t] - p), axis=-1)
        dp = -bt * du
        dD = dHt + kt[..., :, None] * dp[..., None, :]
        dk_t += np.einsum("bhij,bhj->bhi", D, dp)
        dkh[:, t] = dk_t
        if channelwise:
            dg[:, t] = np.sum(dD * D, axis=-1)
        else:
            dg[:, t] = np.sum(dD * D, axis=(-2, -1))
        dH = a * dD
    dq_hat = dqh.reshape(B, T, Hk, grp, Dk).sum(axis=3)
    dk_hat = dkh.reshape(B, T, Hk, grp, Dk).sum(axis=3)
    if use_qk_l2norm:
        dq = l2norm_vjp(q, dq_hat)
        dk = l2norm_vjp(k, dk_hat)
    else:
        dq, dk = dq_hat, dk_hat
    if fused_gates:
        dg, dbeta = gate_activation_vjp(a_pre, b_pre, dg, dbeta)
    return dq, dk, dv, dg, dbeta, dH


def chunked_forward(q, k, v, g, beta, h0=None, chunk_size=64,
                    use_qk_l2norm=True, channelwise=False):
    """The same map as ``forward`` evaluated chunk by chunk in WY form.

    Within a chunk of L tokens starting from state H0, let G_r be the
    cumulative sum of g over the chunk up to row r (per channel when
    channelwise) and Gam_r = exp(G_r).  Unrolling the recurrence gives
        H_r = diag(Gam_r) H0 + sum_{s<=r} diag(exp(G_r - G_s)) k_s u_s^T,
    and the deltas solve the unit lower-triangular system
        u_r + sum_{s<r} A_rs u_s = beta_r (v_r - (Gam_r * k_r)^T H0),
        A_rs = beta_r * sum_i k_ri k_si exp(G_ri - G_si)       (s < r),
    solved here by forward substitution.  Then
        o_r = (Gam_r * q_r)^T H0 + sum_{s<=r} (sum_i q_ri k_si exp(G_ri - G_si)) u_s
    and the state passed to the next chunk is H_L.  Only exponents of
    differences G_r - G_s with r >= s (all <= 0 for g <= 0) are formed.
    This is the chunk-parallel form the [MLX] chunked kernel is built on.
    """
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    qh, kh = _prepare(q, k, use_qk_l2norm, Hv)
    vv, bb = _f64(v), _f64(beta)
    gg = _f64(g)
    if not channelwise:
        gg = np.repeat(gg[..., None], Dk, axis=-1)
    H = np.zeros((B, Hv, Dk, Dv)) if h0 is None else _f64(h0)
    o = np.zeros((B, T, Hv, Dv))
    for t0 in range(0, T, chunk_size):
        t1 = min(T, t0 + chunk_size)
        L = t1 - t0
        # [B,Hv,L,Dk] etc.: chunk rows first after the head axes
        Kc = np.moveaxis(kh[:, t0:t1], 1, 2)
        Qc = np.moveaxis(qh[:, t0:t1], 1, 2)
        Vc = np.moveaxis(vv[:, t0:t1], 1, 2)
        bc = np.moveaxis(bb[:, t0:t1], 1, 2)
        Gc = np.cumsum(np.moveaxis(gg[:, t0:t1], 1, 2), axis=2)
        lower = np.tril(np.ones((L, L), dtype=bool))          # s <= r
        diff = Gc[:, :, :, None, :] - Gc[:, :, None, :, :]     # G_r - G_s
        E = np.exp(np.where(lower[None, None, :, :, None], diff, -np.inf))
        KK = np.einsum("bhri,bhsi,bhrsi->bhrs", Kc, Kc, E)
        QK = np.einsum("bhri,bhsi,bhrsi->bhrs", Qc, Kc, E)
        A = bc[..., None] * np.tril(KK, -1)
        rhs = bc[..., None] * (Vc - np.einsum("bhri,bhij->bhrj", np.exp(Gc) * Kc, H))
        U = np.zeros_like(rhs)
        for r in range(L):
            U[:, :, r] = rhs[:, :, r] - np.einsum("bhs,bhsj->bhj", A[:, :, r, :r], U[:, :, :r])
        Oc = np.einsum("bhri,bhij->bhrj", np.exp(Gc) * Qc, H) + np.einsum("bhrs,bhsj->bhrj", QK, U)
        o[:, t0:t1] = np.moveaxis(Oc, 2, 1)
        last = Gc[:, :, L - 1, :]                               # [B,Hv,Dk]
        Kt = np.exp(last[:, :, None, :] - Gc) * Kc              # exp(G_L - G_s) k_s
        H = np.exp(last)[..., None] * H + np.einsum("bhsi,bhsj->bhij", Kt, U)
    return o, H
