"""Planted-mistake check for the oracle pins (CPU only).

Each mutant is the oracle's source with one plausible slip (a dropped term,
a wrong sign, a swapped operand, a wrong decay order, a wrong eps).  The
mutant is loaded as a separate module and a compact set of the independent
checks is run against it: at least one must fail, otherwise the pins would
not have caught that slip.
"""

import os
import types

import numpy as np
import pytest
import torch

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "gdr_oracle.py")

MUTANTS = {
    "backward drops dk += D dp":
        ('        dk_t += np.einsum("bhij,bhj->bhi", D, dp)\n', ""),
    "backward sign of dp":
        ("        dp = -bt * du\n", "        dp = bt * du\n"),
    "backward dH not decayed":
        ("        dH = a * dD\n", "        dH = dD\n"),
    "backward dq from the old state":
        ('        dqh[:, t] = np.einsum("bhij,bhj->bhi", states[t + 1], dot)\n',
         '        dqh[:, t] = np.einsum("bhij,bhj->bhi", states[t], dot)\n'),
    "backward dbeta uses v":
        ("        dbeta[:, t] = np.sum(du * (vv[:, t] - p), axis=-1)\n",
         "        dbeta[:, t] = np.sum(du * vv[:, t], axis=-1)\n"),
    "forward predicts before decay":
        ('        p = np.einsum("bhij,bhi->bhj", D, kt)\n        u = bb[:, t][..., None] * (vv[:, t] - p)\n        H = D + kt',
         '        p = np.einsum("bhij,bhi->bhj", H, kt)\n        u = bb[:, t][..., None] * (vv[:, t] - p)\n        H = D + kt'),
    "forward reads out the old state":
        ('        H = D + kt[..., :, None] * u[..., None, :]\n        o[:, t] = np.einsum("bhij,bhi->bhj", H, qt)\n',
         '        o[:, t] = np.einsum("bhij,bhi->bhj", H, qt)\n        H = D + kt[..., :, None] * u[..., None, :]\n'),
    "forward transposed readout":
        ('        o[:, t] = np.einsum("bhij,bhi->bhj", H, qt)\n',
         '        o[:, t] = np.einsum("bhji,bhi->bhj", H, qt)\n'),
    "l2norm eps outside the root":
        ("    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)\n",
         "    return x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)\n"),
    "l2norm vjp drops projection":
        ("    return r * (dxhat - xhat * np.sum(xhat * dxhat, axis=-1, keepdims=True))\n",
         "    return r * dxhat\n"),
    "gqa map interleaved":
        ("    return np.repeat(qh, grp, axis=2), np.repeat(kh, grp, axis=2)\n",
         "    return np.tile(qh, (1, 1, grp, 1)), np.tile(kh, (1, 1, grp, 1))\n"),
    "chunk mask drops the diagonal":
        ("        lower = np.tril(np.ones((L, L), dtype=bool))          # s <= r\n",
         "        lower = np.tril(np.ones((L, L), dtype=bool), -1)\n"),
    "chunk carry ignores in-chunk decay":
        ("        Kt = np.exp(last[:, :, None, :] - Gc) * Kc              # exp(G_L - G_s) k_s\n",
         "        Kt = Kc\n"),
    "channelwise decay on the value axis":
        ("    return a[..., :, None] if channelwise else a[..., None, None]\n",
         "    return a[..., None, :] if channelwise else a[..., None, None]\n"),
}


def load_mutant(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("gdr_oracle_mutant")
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def relerr(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


def _case(rng, B=1, T=5, Hk=1, Hv=2, D=4, cw=False):
    r = lambda *s: rng.standard_normal(s)
    q, k, v = r(B, T, Hk, D), r(B, T, Hk, D), r(B, T, Hv, D)
    g = -np.logaddexp(0.0, r(B, T, Hv, D) if cw else r(B, T, Hv))
    beta = 1.0 / (1.0 + np.exp(-r(B, T, Hv)))
    return q, k, v, g, beta, r(B, Hv, D, D), r(B, T, Hv, D), r(B, Hv, D, D)


def check_fd(orc):
    for cw in (False, True):
        q, k, v, g, beta, h0, do, dht = _case(np.random.default_rng(3), cw=cw)
        grads = orc.backward(q, k, v, g, beta, h0, do, dht, channelwise=cw)
        args = [q, k, v, g, beta, h0]
        for ai in range(6):
            x = args[ai]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += 1e-6
                xm[idx] -= 1e-6
                ap, am = list(args), list(args)
                ap[ai], am[ai] = xp, xm
                lp = sum(np.sum(a * b) for a, b in zip(orc.forward(*ap, channelwise=cw), (do, dht)))
                lm = sum(np.sum(a * b) for a, b in zip(orc.forward(*am, channelwise=cw), (do, dht)))
                fd[idx] = (lp - lm) / 2e-6
            if relerr(grads[ai], fd) > 1e-6:
                return False
    return True


def check_closed_forms(orc):
    rng = np.random.default_rng(5)
    B, T, H, D = 1, 6, 1, 8
    k = rng.standard_normal((B, T, H, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, D))
    o, _ = orc.forward(k, k, v, np.zeros((B, T, H)), np.ones((B, T, H)),
                       h0=rng.standard_normal((B, H, D, D)), use_qk_l2norm=False)
    if relerr(o, v) > 1e-12:
        return False
    q = rng.standard_normal((B, 1, H, D))
    k1 = rng.standard_normal((B, 1, H, D))
    v1 = rng.standard_normal((B, 1, H, D))
    o, _ = orc.forward(q, k1, v1, np.zeros((B, 1, H)), np.full((B, 1, H), 0.7))
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    kn = k1 / np.sqrt(np.sum(k1 * k1, -1, keepdims=True) + 1e-6)
    return relerr(o, 0.7 * np.sum(qn * kn, -1)[..., None] * v1) < 1e-13


def check_chunked(orc):
    q, k, v, g, beta, h0, _, _ = _case(np.random.default_rng(9), T=13, D=6)
    o1, h1 = orc.forward(q, k, v, g, beta, h0)
    o2, h2 = orc.chunked_forward(q, k, v, g, beta, h0, chunk_size=4)
    return relerr(o2, o1) < 1e-12 and relerr(h2, h1) < 1e-12


def check_caller_norm(orc):
    q, k, v, g, beta, h0, do, _ = _case(np.random.default_rng(11), Hk=2, Hv=4)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    qn = qt / torch.sqrt((qt * qt).sum(-1, keepdim=True) + 1e-6)
    kn = kt / torch.sqrt((kt * kt).sum(-1, keepdim=True) + 1e-6)
    o1, _ = orc.forward(q, k, v, g, beta, h0)
    o2, _ = orc.forward(qn.detach().numpy(), kn.detach().numpy(), v, g, beta, h0,
                        use_qk_l2norm=False)
    if relerr(o1, o2) > 1e-13:
        return False
    g_on = orc.backward(q, k, v, g, beta, h0, do)
    g_off = orc.backward(qn.detach().numpy(), kn.detach().numpy(), v, g, beta, h0,
                         do, use_qk_l2norm=False)
    (qn * torch.tensor(g_off[0])).sum().backward()
    return relerr(g_on[0], qt.grad.numpy()) < 1e-12


def check_gqa_block_map(orc):
    """v-heads 2j, 2j+1 read k-head j: zeroing k-head 1 must leave v-heads
    0 and 1 untouched."""
    q, k, v, g, beta, h0, _, _ = _case(np.random.default_rng(13), Hk=2, Hv=4)
    o1, _ = orc.forward(q, k, v, g, beta, h0)
    k2, q2 = k.copy(), q.copy()
    k2[:, :, 1] *= 3.0
    q2[:, :, 1] *= -1.0
    o2, _ = orc.forward(q2, k2, v, g, beta, h0)
    return relerr(o2[:, :, :2], o1[:, :, :2]) < 1e-14


def check_hand_examples(orc):
    """The 2x2 examples worked by hand in tests/golden/hand_worked_2x2.yaml."""
    import yaml
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked_2x2.yaml")
    with open(path) as fh:
        cases = yaml.safe_load(fh)
    for c in cases.values():
        cw = c["channelwise"]
        a = lambda key: np.asarray(c[key], dtype=np.float64)
        T = len(c["q"])
        q, k, v = (a(n).reshape(1, T, 1, 2) for n in ("q", "k", "v"))
        g = np.log(a("alpha")).reshape((1, T, 1, 2) if cw else (1, T, 1))
        beta = a("beta").reshape(1, T, 1)
        h0 = None if c["h0"] is None else a("h0").reshape(1, 1, 2, 2)
        o, ht = orc.forward(q, k, v, g, beta, h0, use_qk_l2norm=False, channelwise=cw)
        if np.max(np.abs(o.reshape(T, 2) - a("o"))) > 1e-12 or np.max(np.abs(ht.reshape(2, 2) - a("ht"))) > 1e-12:
            return False
        if "dout" in c:
            got = orc.backward(q, k, v, g, beta, h0, a("dout").reshape(1, T, 1, 2), None, use_qk_l2norm=False,
                               channelwise=cw)
            for key, x in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got):
                if np.max(np.abs(np.asarray(x).reshape(a(key).shape) - a(key))) > 1e-12:
                    return False
    return True


CHECKS = [check_fd, check_closed_forms, check_chunked, check_caller_norm,
          check_gqa_block_map, check_hand_examples]


def test_unmutated_oracle_passes_every_check():
    from oracle import gdr_oracle
    for chk in CHECKS:
        assert chk(gdr_oracle), chk.__name__


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_planted_mistake_is_caught(name):
    orc = load_mutant(name)
    failed = [c.__name__ for c in CHECKS if not c(orc)]
    assert failed, f"no pin catches mutant: {name}"
