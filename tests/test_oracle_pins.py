"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (closed forms, special cases that reduce to a library routine,
finite differences, autograd, exact identities).

Where a pin follows from a page it says which; otherwise it follows from the
gated delta rule recurrence (Yang, Kautz & Hatamizadeh, "Gated Delta
Networks", ICLR 2025) that all three pages are about.
"""

import numpy as np
import pytest
import torch

from oracle import gdr_oracle as orc

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def gates(B, T, Hv, Dk=None, channelwise=False):
    a = rand(B, T, Hv, Dk) if channelwise else rand(B, T, Hv)
    return -np.logaddexp(0.0, a), 1.0 / (1.0 + np.exp(-rand(B, T, Hv)))


def relerr(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


# ---------------------------------------------------------------- forward pins

def test_p1_unit_key_full_write_recovers_value():
    """alpha=1, beta=1, ||k||=1: the delta rule writes v exactly at key k,
    so reading the new state with q = k returns v (S_t k_t = v_t)."""
    B, T, H, D = 2, 7, 3, 8
    k = unit_rows(rand(B, T, H, D))
    v = rand(B, T, H, D)
    o, _ = orc.forward(k, k, v, np.zeros((B, T, H)), np.ones((B, T, H)),
                       h0=rand(B, H, D, D), use_qk_l2norm=False)
    assert relerr(o, v) < 1e-12


@pytest.mark.parametrize("channelwise", [False, True])
def test_p2_zero_beta_is_pure_decay(channelwise):
    """beta=0: the state only decays, H_T = diag(exp(sum_t g_t)) h0, and
    o_t = H_t^T q_t with H_t the decayed h0 (per channel for [ET]'s gate)."""
    B, T, Hk, Hv, D = 1, 9, 2, 4, 6
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, _ = gates(B, T, Hv, D, channelwise)
    h0 = rand(B, Hv, D, D)
    o, ht = orc.forward(q, k, v, g, np.zeros((B, T, Hv)), h0=h0,
                        channelwise=channelwise)
    cum = np.cumsum(g, axis=1)
    scale = np.exp(cum)[..., :, None] if channelwise else np.exp(cum)[..., None, None]
    ref_ht = scale[:, -1] * h0
    assert relerr(ht, ref_ht) < 1e-12
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    qn = np.repeat(qn, Hv // Hk, axis=2)
    for t in range(T):
        Ht = scale[:, t] * h0
        assert relerr(o[:, t], np.einsum("bhij,bhi->bhj", Ht, qn[:, t])) < 1e-12


def test_p3_orthonormal_keys_reduce_to_linear_attention():
    """alpha=1, beta=1, keys e_1..e_T orthonormal, h0=0: every delta is the
    value itself, so H_T = sum_t e_t v_t^T and o_t = sum_{s<=t} (q_t.e_s) v_s."""
    B, T, H, D = 1, 6, 1, 8
    k = np.zeros((B, T, H, D))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    q, v = rand(B, T, H, D), rand(B, T, H, D)
    o, ht = orc.forward(q, k, v, np.zeros((B, T, H)), np.ones((B, T, H)),
                        use_qk_l2norm=False)
    ref_ht = np.zeros((D, D))
    ref_ht[:T] = v[0, :, 0]
    assert relerr(ht[0, 0], ref_ht) < 1e-14
    scores = np.tril(q[0, :, 0] @ k[0, :, 0].T)          # (q_t . e_s), s<=t
    assert relerr(o[0, :, 0], scores @ v[0, :, 0]) < 1e-13


def test_p4_single_token_from_zero_state():
    """h0=0, T=1: H_1 = beta k v^T, so o = beta (k.q) v (normalised q, k)."""
    B, Hk, Hv, D = 3, 2, 4, 5
    q, k, v = rand(B, 1, Hk, D), rand(B, 1, Hk, D), rand(B, 1, Hv, D)
    g, beta = gates(B, 1, Hv)
    o, _ = orc.forward(q, k, v, g, beta)
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    kn = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6)
    dot = np.repeat(np.sum(qn * kn, -1), Hv // Hk, axis=2)
    assert relerr(o, beta[..., None] * dot[..., None] * v) < 1e-13


def test_p10_no_write_no_decay_is_a_plain_matmul():
    """alpha=1, beta=0: the state stays h0 and o_t = h0^T q_t."""
    B, T, H, D = 2, 5, 2, 6
    q, k, v = rand(B, T, H, D), rand(B, T, H, D), rand(B, T, H, D)
    h0 = rand(B, H, D, D)
    o, ht = orc.forward(q, k, v, np.zeros((B, T, H)), np.zeros((B, T, H)),
                        h0=h0, use_qk_l2norm=False)
    assert relerr(o, np.einsum("bthi,bhij->bthj", q, h0)) < 1e-13
    assert np.array_equal(ht, h0)


def test_p12_flag_off_uses_inputs_as_given():
    """use_qk_l2norm=False is a no-op on q/k ([MEG] "What": the False path
    stays as it was): T=1, h0=0 gives o = beta (k.q) v with the raw vectors."""
    B, H, D = 2, 3, 4
    q, k, v = rand(B, 1, H, D, scale=3.0), rand(B, 1, H, D, scale=3.0), rand(B, 1, H, D)
    g, beta = gates(B, 1, H)
    o, _ = orc.forward(q, k, v, g, beta, use_qk_l2norm=False)
    ref = beta[..., None] * np.sum(q * k, -1)[..., None] * v
    assert relerr(o, ref) < 1e-13


def test_p9_single_chunk_matches_library_triangular_solve():
    """alpha=1, one chunk: the deltas solve (I + A) U = diag(beta) (V - K H0)
    with A_rs = beta_r (k_r.k_s) for s < r; numpy.linalg.solve gives U and
    then o = Q H0 + tril(Q K^T) U must equal the token recurrence."""
    T, D = 11, 6
    q, k = unit_rows(rand(1, T, 1, D)), unit_rows(rand(1, T, 1, D))
    v = rand(1, T, 1, D)
    beta = 1.0 / (1.0 + np.exp(-rand(1, T, 1)))
    h0 = rand(1, 1, D, D)
    o, ht = orc.forward(q, k, v, np.zeros((1, T, 1)), beta, h0=h0,
                        use_qk_l2norm=False)
    K, Q, V, b, H0 = k[0, :, 0], q[0, :, 0], v[0, :, 0], beta[0, :, 0], h0[0, 0]
    A = b[:, None] * np.tril(K @ K.T, -1)
    U = np.linalg.solve(np.eye(T) + A, b[:, None] * (V - K @ H0))
    assert relerr(o[0, :, 0], Q @ H0 + np.tril(Q @ K.T) @ U) < 1e-12
    assert relerr(ht[0, 0], H0 + K.T @ U) < 1e-12


def test_p11_in_kernel_norm_equals_caller_norm_forward():
    """[MEG] "Why": normalising q/k inside the kernel (eps 1e-6, last dim)
    gives the same result as normalising them before the call."""
    B, T, Hk, Hv, D = 2, 6, 2, 4, 5
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv)
    h0 = rand(B, Hv, D, D)
    qt = torch.tensor(q)
    kt = torch.tensor(k)
    qn = (qt / torch.sqrt((qt * qt).sum(-1, keepdim=True) + 1e-6)).numpy()
    kn = (kt / torch.sqrt((kt * kt).sum(-1, keepdim=True) + 1e-6)).numpy()
    o1, h1 = orc.forward(q, k, v, g, beta, h0, use_qk_l2norm=True)
    o2, h2 = orc.forward(qn, kn, v, g, beta, h0, use_qk_l2norm=False)
    assert relerr(o1, o2) < 1e-14 and relerr(h1, h2) < 1e-14


@pytest.mark.parametrize("channelwise", [False, True])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_p13_chunked_form_equals_recurrence(C, channelwise):
    """The WY/chunk form is an exact rewrite of the recurrence: agreement to
    1e-12 for several chunk sizes, T not a multiple of C."""
    B, T, Hk, Hv, D = 2, 70, 1, 2, 8
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv, D, channelwise)
    h0 = rand(B, Hv, D, D, scale=0.5)
    o1, h1 = orc.forward(q, k, v, g, beta, h0, channelwise=channelwise)
    o2, h2 = orc.chunked_forward(q, k, v, g, beta, h0, chunk_size=C,
                                 channelwise=channelwise)
    assert relerr(o2, o1) < 1e-12
    assert relerr(h2, h1) < 1e-12


def test_p6_value_columns_are_independent():
    """Columns of H (value dims) never mix: a run on Dv equals two runs on
    the two halves of v and h0 (the reason the state can be split by Dv)."""
    B, T, Hk, Hv, D = 1, 8, 1, 2, 6
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv)
    h0 = rand(B, Hv, D, D)
    do = rand(B, T, Hv, D)
    o, ht = orc.forward(q, k, v, g, beta, h0)
    grads = orc.backward(q, k, v, g, beta, h0, do)
    parts = []
    for sl in (slice(0, 3), slice(3, 6)):
        oa, ha = orc.forward(q, k, v[..., sl], g, beta, h0[..., sl])
        assert relerr(oa, o[..., sl]) < 1e-13 and relerr(ha, ht[..., sl]) < 1e-13
        parts.append(orc.backward(q, k, v[..., sl], g, beta, h0[..., sl], do[..., sl]))
    for i in (0, 1, 3, 4):                      # dq, dk, dg, dbeta: summed over Dv
        assert relerr(parts[0][i] + parts[1][i], grads[i]) < 1e-12
    assert relerr(np.concatenate([parts[0][2], parts[1][2]], -1), grads[2]) < 1e-13
    assert relerr(np.concatenate([parts[0][5], parts[1][5]], -1), grads[5]) < 1e-13


def test_p7_gqa_equals_expanded_heads():
    """Hk < Hv equals Hk = Hv with q, k repeated per group; dq, dk are the
    group sums of the expanded run's gradients."""
    B, T, Hk, Hv, D = 2, 6, 2, 4, 5
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv)
    h0, do, dht = rand(B, Hv, D, D), rand(B, T, Hv, D), rand(B, Hv, D, D)
    qe, ke = np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2)
    o1, h1 = orc.forward(q, k, v, g, beta, h0)
    o2, h2 = orc.forward(qe, ke, v, g, beta, h0)
    assert relerr(o1, o2) < 1e-14 and relerr(h1, h2) < 1e-14
    g1 = orc.backward(q, k, v, g, beta, h0, do, dht)
    g2 = orc.backward(qe, ke, v, g, beta, h0, do, dht)
    assert relerr(g1[0], g2[0].reshape(B, T, Hk, 2, D).sum(3)) < 1e-13
    assert relerr(g1[1], g2[1].reshape(B, T, Hk, 2, D).sum(3)) < 1e-13
    for i in (2, 3, 4, 5):
        assert relerr(g1[i], g2[i]) < 1e-14


def test_p8_channelwise_with_equal_channels_is_scalar_gate():
    """[ET]'s per-channel decay with every channel equal is the scalar gate;
    the scalar dg is the sum of the per-channel dg."""
    B, T, Hk, Hv, D = 1, 7, 1, 2, 5
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv)
    gc = np.repeat(g[..., None], D, axis=-1)
    h0, do = rand(B, Hv, D, D), rand(B, T, Hv, D)
    o1, h1 = orc.forward(q, k, v, g, beta, h0)
    o2, h2 = orc.forward(q, k, v, gc, beta, h0, channelwise=True)
    assert relerr(o1, o2) < 1e-14 and relerr(h1, h2) < 1e-14
    g1 = orc.backward(q, k, v, g, beta, h0, do)
    g2 = orc.backward(q, k, v, gc, beta, h0, do, channelwise=True)
    assert relerr(g2[3].sum(-1), g1[3]) < 1e-12
    for i in (0, 1, 2, 4, 5):
        assert relerr(g1[i], g2[i]) < 1e-13


# --------------------------------------------------------------- backward pins

def _loss(q, k, v, g, beta, h0, do, dht, flag, cw):
    o, ht = orc.forward(q, k, v, g, beta, h0, use_qk_l2norm=flag, channelwise=cw)
    return np.sum(o * do) + np.sum(ht * dht)


@pytest.mark.parametrize("flag", [True, False])
@pytest.mark.parametrize("cw", [False, True])
@pytest.mark.parametrize("Hv", [1, 2])
def test_p14_finite_differences(flag, cw, Hv):
    """Central differences (step 1e-6) of <do, o> + <dht, ht> against every
    gradient the VJP returns, on tiny shapes, dht != 0."""
    rng = np.random.default_rng(7 + Hv + 2 * flag + 4 * cw)
    B, T, Hk, D = 1, 5, 1, 4
    r = lambda *s: rng.standard_normal(s)
    q, k, v = r(B, T, Hk, D), r(B, T, Hk, D), r(B, T, Hv, D)
    g = -np.logaddexp(0.0, r(B, T, Hv, D) if cw else r(B, T, Hv))
    beta = 1.0 / (1.0 + np.exp(-r(B, T, Hv)))
    h0, do, dht = r(B, Hv, D, D), r(B, T, Hv, D), r(B, Hv, D, D)
    grads = orc.backward(q, k, v, g, beta, h0, do, dht, use_qk_l2norm=flag,
                         channelwise=cw)
    args = [q, k, v, g, beta, h0]
    for gi, ai in zip((0, 1, 2, 3, 4, 5), (0, 1, 2, 3, 4, 5)):
        x = args[ai]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += 1e-6
            xm[idx] -= 1e-6
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            fd[idx] = (_loss(*ap, do, dht, flag, cw) - _loss(*am, do, dht, flag, cw)) / 2e-6
        assert relerr(grads[gi], fd) < 1e-6, ("grad", gi)


def _torch_forward(q, k, v, g, beta, h0, flag, cw, Hv):
    """Independent autograd reference: the recurrence in torch fp64 ops."""
    if flag:
        q = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
        k = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    grp = Hv // q.shape[2]
    q = q.repeat_interleave(grp, dim=2)
    k = k.repeat_interleave(grp, dim=2)
    S = h0.transpose(-1, -2)                       # S = H^T, Dv x Dk
    eye = torch.eye(k.shape[-1], dtype=torch.float64)
    outs = []
    for t in range(q.shape[1]):
        kt = k[:, t]
        a = torch.exp(g[:, t])
        decay = torch.diag_embed(a) if cw else a[..., None, None] * eye
        proj = eye - beta[:, t][..., None, None] * kt[..., :, None] * kt[..., None, :]
        S = S @ decay @ proj + beta[:, t][..., None, None] * v[:, t][..., :, None] * kt[..., None, :]
        outs.append((S @ q[:, t][..., None])[..., 0])
    return torch.stack(outs, 1), S.transpose(-1, -2)


@pytest.mark.parametrize("flag,cw", [(True, False), (False, True), (True, True)])
def test_p14b_autograd_of_the_textbook_form(flag, cw):
    """torch.autograd on the textbook form S_t = S_{t-1} diag(a)(I - b k k^T)
    + b v k^T (matrix products, not the oracle's per-step algebra) gives the
    same o, ht and all six gradients as the hand-derived VJP."""
    B, T, Hk, Hv, D = 2, 9, 2, 4, 6
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv, D, cw)
    h0, do, dht = rand(B, Hv, D, D), rand(B, T, Hv, D), rand(B, Hv, D, D)
    tens = [torch.tensor(x, requires_grad=True) for x in (q, k, v, g, beta, h0)]
    o_t, ht_t = _torch_forward(*tens, flag, cw, Hv)
    ((o_t * torch.tensor(do)).sum() + (ht_t * torch.tensor(dht)).sum()).backward()
    o, ht = orc.forward(q, k, v, g, beta, h0, use_qk_l2norm=flag, channelwise=cw)
    assert relerr(o, o_t.detach().numpy()) < 1e-12
    assert relerr(ht, ht_t.detach().numpy()) < 1e-12
    grads = orc.backward(q, k, v, g, beta, h0, do, dht, use_qk_l2norm=flag, channelwise=cw)
    for gi, tt in enumerate(tens):
        assert relerr(grads[gi], tt.grad.numpy()) < 1e-11, gi


def test_p11_l2norm_vjp_matches_autograd():
    """[MEG] "Validation" compares caller-side and in-kernel normalisation by
    their gradients too: the q/k gradient with the flag on is the caller-side
    normalisation's autograd VJP applied to the flag-off gradient."""
    B, T, Hk, Hv, D = 1, 6, 2, 4, 5
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv)
    h0, do = rand(B, Hv, D, D), rand(B, T, Hv, D)
    g_on = orc.backward(q, k, v, g, beta, h0, do, use_qk_l2norm=True)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    qn = qt / torch.sqrt((qt * qt).sum(-1, keepdim=True) + 1e-6)
    kn = kt / torch.sqrt((kt * kt).sum(-1, keepdim=True) + 1e-6)
    g_off = orc.backward(qn.detach().numpy(), kn.detach().numpy(), v, g, beta,
                         h0, do, use_qk_l2norm=False)
    (qn * torch.tensor(g_off[0])).sum().backward()
    (kn * torch.tensor(g_off[1])).sum().backward()
    assert relerr(g_on[0], qt.grad.numpy()) < 1e-12
    assert relerr(g_on[1], kt.grad.numpy()) < 1e-12
    for i in (2, 3, 4, 5):
        assert relerr(g_on[i], g_off[i]) < 1e-12


def test_p15_adjoint_identity_in_v_and_h0():
    """For fixed q, k, g, beta the map (v, h0) -> (o, ht) is linear, so
    <do, o> + <dht, ht> = <dv, v> + <dh0, h0> exactly (no FD error)."""
    B, T, Hk, Hv, D = 2, 12, 2, 4, 6
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv)
    h0, do, dht = rand(B, Hv, D, D), rand(B, T, Hv, D), rand(B, Hv, D, D)
    o, ht = orc.forward(q, k, v, g, beta, h0)
    _, _, dv, _, _, dh0 = orc.backward(q, k, v, g, beta, h0, do, dht)
    lhs = np.sum(do * o) + np.sum(dht * ht)
    rhs = np.sum(dv * v) + np.sum(dh0 * h0)
    assert abs(lhs - rhs) < 1e-12 * max(abs(lhs), 1.0)


@pytest.mark.parametrize("cw", [False, True])
def test_p5_split_sequence_forward_and_backward(cw):
    """Carrying ht into h0 splits a sequence: run(T1) then run(T2, h0=ht)
    equals run(T1+T2); the backward chains through dht/dh0 the same way."""
    B, T, T1, Hk, Hv, D = 1, 10, 4, 1, 2, 5
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    g, beta = gates(B, T, Hv, D, cw)
    h0, do, dht = rand(B, Hv, D, D), rand(B, T, Hv, D), rand(B, Hv, D, D)
    o, ht = orc.forward(q, k, v, g, beta, h0, channelwise=cw)
    a, b = slice(0, T1), slice(T1, T)
    oa, ha = orc.forward(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], h0, channelwise=cw)
    ob, hb = orc.forward(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], ha, channelwise=cw)
    assert relerr(np.concatenate([oa, ob], 1), o) < 1e-13 and relerr(hb, ht) < 1e-13
    full = orc.backward(q, k, v, g, beta, h0, do, dht, channelwise=cw)
    gb = orc.backward(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], ha, do[:, b], dht, channelwise=cw)
    ga = orc.backward(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], h0, do[:, a], gb[5], channelwise=cw)
    for i in range(5):
        assert relerr(np.concatenate([ga[i], gb[i]], 1), full[i]) < 1e-12
    assert relerr(ga[5], full[5]) < 1e-12


# --------------------------------------------------------- fused gate activation

def test_p16_gate_activation_closed_forms():
    """Fused gates at a = b = 0: g = -softplus(0) = -log 2 (alpha = 1/2) and
    beta = sigmoid(0) = 1/2; far out, softplus(a) -> a and sigmoid -> 0 / 1,
    with no overflow."""
    g, b = orc.gate_activation(np.array([0.0, 800.0, -800.0]), np.array([0.0, 800.0, -800.0]))
    assert np.allclose(g, [-np.log(2.0), -800.0, 0.0], rtol=0, atol=1e-15)
    assert np.allclose(b, [0.5, 1.0, 0.0], rtol=0, atol=1e-15)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(b))


def test_p16_saturated_gates_write_the_value():
    """Pre-activations a -> -inf (alpha -> 1) and b -> +inf (beta -> 1) turn
    the fused-gate recurrence into the plain full write of pin P1:
    S_t k_t = v_t for unit keys."""
    B, T, H, D = 2, 6, 3, 8
    k = unit_rows(rand(B, T, H, D))
    v = rand(B, T, H, D)
    o, _ = orc.forward(k, k, v, np.full((B, T, H), -80.0), np.full((B, T, H), 80.0),
                       h0=rand(B, H, D, D), use_qk_l2norm=False, fused_gates=True)
    assert relerr(o, v) < 1e-12


def _loss_fg(q, k, v, a, b, h0, do, dht, flag, cw):
    o, ht = orc.forward(q, k, v, a, b, h0, use_qk_l2norm=flag, channelwise=cw, fused_gates=True)
    return np.sum(o * do) + np.sum(ht * dht)


@pytest.mark.parametrize("flag,cw", [(True, False), (True, True), (False, False)])
def test_p16_fused_gate_finite_differences(flag, cw):
    """Central differences of <do, o> + <dht, ht> in the pre-activations a, b
    (and the other inputs) against the fused-gate VJP."""
    rng = np.random.default_rng(41 + 2 * flag + cw)
    B, T, Hk, Hv, D = 1, 5, 1, 2, 4
    r = lambda *s: rng.standard_normal(s)
    q, k, v = r(B, T, Hk, D), r(B, T, Hk, D), r(B, T, Hv, D)
    a = r(B, T, Hv, D) if cw else r(B, T, Hv)
    b = r(B, T, Hv)
    h0, do, dht = r(B, Hv, D, D), r(B, T, Hv, D), r(B, Hv, D, D)
    grads = orc.backward(q, k, v, a, b, h0, do, dht, use_qk_l2norm=flag, channelwise=cw, fused_gates=True)
    args = [q, k, v, a, b, h0]
    for ai in range(6):
        x = args[ai]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += 1e-6
            xm[idx] -= 1e-6
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            fd[idx] = (_loss_fg(*ap, do, dht, flag, cw) - _loss_fg(*am, do, dht, flag, cw)) / 2e-6
        assert relerr(grads[ai], fd) < 1e-6, ("grad", ai)


def test_p16_fused_gates_autograd_of_the_textbook_form():
    """torch autograd through -softplus / sigmoid followed by the textbook
    recurrence gives the fused-gate oracle's outputs and gradients."""
    B, T, Hk, Hv, D = 1, 7, 1, 2, 5
    q, k, v = rand(B, T, Hk, D), rand(B, T, Hk, D), rand(B, T, Hv, D)
    a, b = rand(B, T, Hv), rand(B, T, Hv)
    h0, do, dht = rand(B, Hv, D, D), rand(B, T, Hv, D), rand(B, Hv, D, D)
    tens = [torch.tensor(x, requires_grad=True) for x in (q, k, v, a, b, h0)]
    g_t = -torch.nn.functional.softplus(tens[3])
    beta_t = torch.sigmoid(tens[4])
    o_t, ht_t = _torch_forward(tens[0], tens[1], tens[2], g_t, beta_t, tens[5], True, False, Hv)
    ((o_t * torch.tensor(do)).sum() + (ht_t * torch.tensor(dht)).sum()).backward()
    o, ht = orc.forward(q, k, v, a, b, h0, fused_gates=True)
    assert relerr(o, o_t.detach().numpy()) < 1e-12
    assert relerr(ht, ht_t.detach().numpy()) < 1e-12
    grads = orc.backward(q, k, v, a, b, h0, do, dht, fused_gates=True)
    for gi, tt in enumerate(tens):
        assert relerr(grads[gi], tt.grad.numpy()) < 1e-11, gi


def test_p17_hand_worked_examples():
    """Three examples worked by hand on 2x2 states (tests/golden/
    hand_worked_2x2.yaml, derivations in the file): a two-token scalar-gate
    forward; a one-token channelwise forward with its full VJP, which fixes
    the key-channel side of the per-channel decay ([ET] summary) and every
    gradient's sign and index; and a two-token scalar-gate forward with its
    full VJP whose inputs are exact in bf16 (so the bf16 matrix-core path
    meets it too), which fixes the scalar dg and the carry of dH between
    tokens."""
    import os
    import yaml
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_2x2.yaml")
    with open(path) as fh:
        cases = yaml.safe_load(fh)
    assert set(cases) == {"scalar_two_tokens", "channelwise_one_token_with_vjp", "scalar_two_tokens_bf16_with_vjp"}
    for name, c in cases.items():
        cw = c["channelwise"]
        a = lambda key: np.asarray(c[key], dtype=np.float64)
        T = len(c["q"])
        q, k, v = (a(n).reshape(1, T, 1, 2) for n in ("q", "k", "v"))
        g = np.log(a("alpha")).reshape((1, T, 1, 2) if cw else (1, T, 1))
        beta = a("beta").reshape(1, T, 1)
        h0 = None if c["h0"] is None else a("h0").reshape(1, 1, 2, 2)
        o, ht = orc.forward(q, k, v, g, beta, h0, use_qk_l2norm=False, channelwise=cw)
        np.testing.assert_allclose(o.reshape(T, 2), a("o"), rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(ht.reshape(2, 2), a("ht"), rtol=0, atol=1e-12, err_msg=name)
        if "dout" not in c:
            continue
        do = a("dout").reshape(1, T, 1, 2)
        got = orc.backward(q, k, v, g, beta, h0, do, None, use_qk_l2norm=False, channelwise=cw)
        for key, x in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got):
            np.testing.assert_allclose(np.asarray(x).reshape(a(key).shape), a(key), rtol=0, atol=1e-12,
                                       err_msg=f"{name} {key}")
