"""GPU parity of ragged (packed) batches, through gdr_forward_varlen /
gdr_backward_varlen: sequences of unequal length laid end to end, one state
per sequence.  Every sequence is checked against the fp64 oracle run on that
sequence alone (the definition of the interface: a ragged call equals
separate calls).  Tolerances as elsewhere: 1e-4 fp32 io, 2e-3 bf16 io."""

import numpy as np
import pytest
import torch

import gated_delta_rule_54_amd as gdr
from gated_delta_rule_54_amd.synth import make_inputs
from oracle import gdr_oracle as orc
from tests._util import dev, host, io_dtype, relerr

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-3}
GRAD_NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def ragged_inputs(lengths, Hk, Hv, D, io, cw=False, seed=0, dht=True):
    """Per-sequence inputs (b = 0 of make_inputs with its own seed) and the
    packed tensors: token-axis concatenation with a leading 1, states [N]."""
    seqs = [make_inputs(seed + 31 * i, 1, n, Hk, Hv, D, D, io_dtype=io, channelwise=cw,
                        h0_std=0.02 if D == 128 else 0.5) for i, n in enumerate(lengths)]
    rng = np.random.default_rng(seed)
    for x in seqs:
        x["dht"] = (0.1 * rng.standard_normal((1, Hv, D, D))).astype(np.float32) if dht else None
    packed = {n: np.concatenate([x[n] for x in seqs], axis=1) for n in ("q", "k", "v", "g", "beta", "do")}
    packed["h0"] = np.concatenate([x["h0"] for x in seqs], axis=0)
    packed["dht"] = np.concatenate([x["dht"] for x in seqs], axis=0) if dht else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return seqs, packed, cu


def to_dev(p, io):
    dt = io_dtype(io)
    return {n: (None if a is None else dev(a, dt if n in ("q", "k", "v", "do") else torch.float32))
            for n, a in p.items()}


def run_and_check(lengths, io, algo, C=0, cw=False, bwd=True, save=False, max_seqlen=None, seed=0,
                  Hk=2, Hv=4, D=128):
    seqs, packed, cu = ragged_inputs(lengths, Hk, Hv, D, io, cw, seed)
    t = to_dev(packed, io)
    cud = torch.from_numpy(cu).cuda()
    kw = dict(algo=algo, chunk_size=C, channelwise=cw, cu_seqlens=cud, max_seqlen=max_seqlen)
    res = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=save, **kw)
    o, ht = res[0], res[1]
    grads = None
    if bwd:
        grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], t["dht"],
                                 saved=res[2] if save else None, **kw)
    torch.cuda.synchronize()
    o, ht = host(o), host(ht)
    grads = None if grads is None else [host(a) for a in grads]
    for i, x in enumerate(seqs):
        r0, r1 = cu[i], cu[i + 1]
        ro, rht = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], channelwise=cw)
        eo, eh = relerr(o[:, r0:r1], ro), relerr(ht[i:i + 1], rht)
        print(f"  seq {i} (T={r1 - r0}): o {eo:.2e} ht {eh:.2e}")
        assert eo < TOL[io] and eh < TOL[io], (i, eo, eh)
        if bwd:
            ref = orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["do"], x["dht"],
                               channelwise=cw)
            for name, a, r in zip(GRAD_NAMES + ("dh0",), grads, ref):
                got = a[i:i + 1] if name == "dh0" else a[:, r0:r1]
                e = relerr(got, r)
                assert e < TOL[io], (i, name, e)


@pytest.mark.parametrize("C", [64, 32])
def test_ragged_chunked_forward_and_vjp(C):
    """Lengths 0 (state passes through), 1, C - 1, C, a ragged 130 and 200,
    GQA 2:4, bf16, D=128, h0 and dht per sequence."""
    run_and_check([0, 1, C - 1, C, 130, 200], "bf16", "chunked", C)


def test_ragged_chunked_saved_chunks():
    run_and_check([70, 5, 190, 64], "bf16", "chunked", 64, save=True, seed=5)


def test_ragged_chunked_vjp_group_launches():
    """A ragged batch whose (chunk, k-head, sequence) grid fills the GPU, so
    one gradient workgroup walks the v-heads of its k-head group (Hk=32,
    Hv=64): empty, 1-token and ragged-chunk sequences."""
    run_and_check([0, 1, 130, 200], "bf16", "chunked", 64, seed=7, Hk=32, Hv=64)


@pytest.mark.parametrize("n,cw", [(64, False), (65, False), (64, True)])
def test_ragged_chunked_many_sequences(n, cw):
    """64 sequences, the most for which the kernels rank the chain
    workgroups by length and number the gradient workgroups by the batch's
    chunk list, and 65, which keep the plain block order: lengths 0 to 150
    (empty, one-token, whole- and part-chunk sequences) on Hk=2, Hv=4."""
    rng = np.random.default_rng(n)
    lens = [int(x) for x in rng.integers(0, 151, size=n)]
    lens[:4] = [0, 1, 64, 150]
    run_and_check(lens, "bf16", "chunked", 64, cw=cw, seed=n)


def test_ragged_bf16_outputs_benchmark_heads():
    """The ragged prefill leg's launch configuration: Hk=16, Hv=32, D=128,
    C=64, bf16 io and outputs, the forward saving its chunks for the VJP, on
    sequences of 1 to 1,911 tokens; sampled (sequence, k-head) groups against
    the oracle run on that sequence alone (bf16-rounded o / dq / dk / dv get
    2^-8 more)."""
    lengths, Hk, Hv, D = [128, 1911, 1, 700, 1300], 16, 32, 128
    seqs, packed, cu = ragged_inputs(lengths, Hk, Hv, D, "bf16", seed=41, dht=False)
    t = to_dev(packed, "bf16")
    cud = torch.from_numpy(cu).cuda()
    kw = dict(algo="chunked", chunk_size=64, cu_seqlens=cud, out_dtype=torch.bfloat16)
    o, ht, saved = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=True, **kw)
    grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], None, saved=saved, **kw)
    torch.cuda.synchronize()
    o, ht = host(o), host(ht)
    grads = [host(a) for a in grads]
    grp = Hv // Hk
    for i, kh in ((1, 3), (2, 0), (4, 15)):
        x, r0, r1, vs = seqs[i], cu[i], cu[i + 1], slice(kh * grp, (kh + 1) * grp)
        xs = {n: x[n][:, :, kh:kh + 1] if n in ("q", "k") else x[n][:, :, vs] for n in ("q", "k", "v", "g", "beta", "do")}
        xs["h0"] = x["h0"][:, vs]
        ro, rht = orc.forward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"])
        ref = orc.backward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"], xs["do"], None)
        got = {"o": o[:, r0:r1, vs], "ht": ht[i:i + 1, vs]}
        exp = {"o": ro, "ht": rht}
        for name, a, r in zip(GRAD_NAMES + ("dh0",), grads, ref):
            got[name] = (a[i:i + 1, vs] if name == "dh0" else a[:, r0:r1, kh:kh + 1] if name in ("dq", "dk")
                         else a[:, r0:r1, vs])
            exp[name] = r
        for name in got:
            e = relerr(got[name], exp[name])
            print(f"  seq {i} kh {kh} {name}: {e:.2e}")
            assert e < TOL["bf16"] + (2 ** -8 if name in ("o", "dq", "dk", "dv") else 0.0), (i, name, e)


def test_ragged_length_bound_above_every_length():
    """max_seqlen larger than every length (more workspace chunks than any
    sequence uses)."""
    run_and_check([33, 100, 17], "bf16", "chunked", 64, max_seqlen=512, seed=9)


def test_ragged_channelwise_chunked_forward():
    run_and_check([0, 90, 1, 150], "bf16", "chunked", 64, cw=True, bwd=False, seed=13)


@pytest.mark.parametrize("io,D", [("f32", 16), ("bf16", 128)])
def test_ragged_sequential_forward(io, D):
    run_and_check([0, 3, 40, 1, 17], io, "sequential", cw=False, bwd=False, seed=17, D=D)


def test_ragged_sequential_channelwise_forward():
    run_and_check([5, 0, 29], "f32", "sequential", cw=True, bwd=False, seed=19, D=16)


def test_ragged_equal_lengths_match_uniform_batch():
    """Equal lengths: the ragged call gives bit for bit the uniform batch."""
    B, T, Hk, Hv, D = 3, 150, 2, 4, 128
    x = make_inputs(21, B, T, Hk, Hv, D, D, io_dtype="bf16", h0_std=0.02)
    t = {n: (None if a is None else dev(a, torch.bfloat16 if n in ("q", "k", "v", "do") else torch.float32))
         for n, a in x.items()}
    flat = lambda a: a.reshape(1, B * T, *a.shape[2:]).contiguous()
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int64, device="cuda")
    kw = dict(algo="chunked", chunk_size=64)
    o0, h0 = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], **kw)
    g0 = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], None, **kw)
    o1, h1 = gdr.gdr_forward(flat(t["q"]), flat(t["k"]), flat(t["v"]), flat(t["g"]), flat(t["beta"]),
                             t["h0"], cu_seqlens=cu, **kw)
    g1 = gdr.gdr_backward(flat(t["q"]), flat(t["k"]), flat(t["v"]), flat(t["g"]), flat(t["beta"]),
                          t["h0"], flat(t["do"]), None, cu_seqlens=cu, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host(o0).reshape(1, B * T, Hv, D), host(o1))
    assert np.array_equal(host(h0), host(h1))
    for a, b_ in zip(g0, g1):
        assert np.array_equal(host(a).reshape(host(b_).shape), host(b_))


@pytest.mark.parametrize("io,D,cw", [("f32", 16, False), ("f32", 16, True), ("bf16", 128, False),
                                     ("bf16", 128, True)])
def test_ragged_sequential_vjp(io, D, cw):
    """The sequential VJP (and its epilogue) on a ragged batch: lengths 0,
    20, 1, 37 (segments of 16 tokens, ragged), both gate modes."""
    run_and_check([0, 20, 1, 37], io, "sequential", cw=cw, seed=23 + D + cw, D=D)


def test_ragged_channelwise_chunked_vjp():
    run_and_check([0, 90, 1, 150], "bf16", "chunked", 64, cw=True, seed=29)


def test_ragged_offsets_and_shapes_checked_before_launch():
    """Offsets past the packed rows, before row 0 or falling, and operands
    whose shape disagrees with the problem, raise ValueError in the binding
    before anything is launched (offsets are read back when max_seqlen is not
    given)."""
    seqs, packed, cu = ragged_inputs([10, 20], 2, 4, 128, "bf16", dht=False)
    t = to_dev(packed, "bf16")
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"])
    for bad in ([0, 10, 31], [0, 20, 10], [-1, 10, 30]):
        with pytest.raises(ValueError, match="cu_seqlens"):
            gdr.gdr_forward(*args, algo="chunked", chunk_size=64,
                            cu_seqlens=torch.tensor(bad, dtype=torch.int64, device="cuda"))
    cud = torch.from_numpy(cu).cuda()
    with pytest.raises(ValueError, match="h0"):
        gdr.gdr_forward(*args[:5], t["h0"][:1].contiguous(), algo="chunked", chunk_size=64, cu_seqlens=cud)
    with pytest.raises(ValueError, match="v"):
        gdr.gdr_forward(t["q"], t["k"], t["v"][:, :29].contiguous(), *args[3:], algo="chunked", chunk_size=64,
                        cu_seqlens=cud)
    with pytest.raises(ValueError, match="dout"):
        gdr.gdr_backward(*args, t["do"][..., :64].contiguous(), None, algo="chunked", chunk_size=64, cu_seqlens=cud)
    torch.cuda.synchronize()
