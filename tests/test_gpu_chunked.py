"""GPU parity of the chunked (matrix-core) kernels against the fp64 oracle,
through the C ABI.  Tolerances: 1e-4 for fp32 io, 2e-3 for bf16 io (max
|x - ref| / max |ref| per tensor, fp32 outputs)."""

import numpy as np
import pytest

from gated_delta_rule_54_amd.synth import make_inputs, round_bf16
from tests.test_gpu_sequential import check_bwd, check_fwd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("C", [16, 32, 64])
def test_tiny_oracle_case_chunked_forward(C):
    """B=1, T=64, Hk=Hv=2, D=16, fp32, zero h0: one chunk at C=64, several
    at C=16/32 (fp32 matrix-core operands)."""
    x = make_inputs(0, 1, 64, 2, 2, 16, 16, io_dtype="f32")
    check_fwd(x, "f32", h0=False, algo=("chunked", C))


@pytest.mark.parametrize("T,C", [(1, 16), (17, 16), (100, 64), (100, 32), (129, 64)])
@pytest.mark.parametrize("l2", [True, False])
def test_fp32_d16_ragged(T, C, l2):
    x = make_inputs(200 + T, 2, T, 1, 4, 16, 16, io_dtype="f32", h0_std=0.5)
    check_fwd(x, "f32", l2=l2, algo=("chunked", C))


@pytest.mark.parametrize("T,C", [(1, 64), (50, 64), (64, 64), (200, 64), (200, 32), (77, 16)])
def test_bf16_d128_chunked_forward(T, C):
    """bf16 io, Dk=Dv=128: fp16 matrix-core operands for C >= 32, fp32 for C=16."""
    x = make_inputs(300 + T + C, 2, T, 2, 4, 128, 128, io_dtype="bf16", h0_std=0.02)
    check_fwd(x, "bf16", algo=("chunked", C))


def test_fp32_d128_chunked_forward():
    x = make_inputs(77, 1, 150, 2, 4, 128, 128, io_dtype="f32", h0_std=0.02)
    check_fwd(x, "f32", algo=("chunked", 64))


def test_prefill_b4_t4096():
    """Chunked prefill forward: B=4, T=4096, Hk=16, Hv=32, D=128, bf16,
    zero h0, C=64.  The GPU runs the whole problem; the oracle checks three
    sampled (b, k-head) groups (both v-heads each)."""
    x = make_inputs(2, 4, 4096, 16, 32, 128, 128, io_dtype="bf16", with_do=False)
    check_fwd(x, "bf16", h0=False, heads=[(0, 0), (2, 7), (3, 15)], algo=("chunked", 64))


# ------------------------------------------------------------------ VJP

from tests.test_gpu_sequential import SWEEP, check_bwd  # noqa: E402


@pytest.mark.parametrize("C", [16, 32, 64])
def test_tiny_oracle_case_chunked_vjp(C):
    """B=1, T=64, Hk=Hv=2, D=16, fp32, do ~ N(0,1), zero h0."""
    x = make_inputs(0, 1, 64, 2, 2, 16, 16, io_dtype="f32")
    check_bwd(x, "f32", h0=False, algo=("chunked", C))


@pytest.mark.parametrize("T,C", [(1, 16), (17, 16), (100, 64), (100, 32), (129, 64)])
@pytest.mark.parametrize("l2", [True, False])
def test_fp32_d16_ragged_vjp(T, C, l2):
    """Ragged T, GQA 1:4, nonzero h0 and dht, flag on/off."""
    x = make_inputs(500 + T, 2, T, 1, 4, 16, 16, io_dtype="f32", h0_std=0.5)
    dht = np.random.default_rng(T).standard_normal((2, 4, 16, 16)).astype(np.float32)
    check_bwd(x, "f32", l2=l2, dht=dht, algo=("chunked", C))


@pytest.mark.parametrize("T,C", [(1, 64), (50, 64), (64, 64), (200, 64), (200, 32), (77, 16)])
def test_bf16_d128_chunked_vjp(T, C):
    x = make_inputs(600 + T + C, 2, T, 2, 4, 128, 128, io_dtype="bf16", h0_std=0.02)
    dht = (0.1 * np.random.default_rng(T).standard_normal((2, 4, 128, 128))).astype(np.float32)
    check_bwd(x, "bf16", dht=dht, algo=("chunked", C))


def test_fp32_d128_chunked_vjp():
    x = make_inputs(78, 1, 150, 2, 4, 128, 128, io_dtype="f32", h0_std=0.02)
    check_bwd(x, "f32", algo=("chunked", 64))


@pytest.mark.parametrize("B,T", SWEEP)
def test_chunked_vjp_sweep(B, T):
    """The backward sweep of the MLX page's benchmark (B in {1,4,8}, T in
    {8,64,512,4096}, Hk=16, Hv=32, D=128, bf16, C=64), h0 ~ N(0, 0.02);
    oracle on every head for short T, on sampled groups for long T."""
    Hk, Hv, D = 16, 32, 128
    x = make_inputs(3000 + 10 * B + [8, 64, 512, 4096].index(T), B, T, Hk, Hv, D, D,
                    io_dtype="bf16", h0_std=0.02)
    heads = None if T <= 64 else ([(B - 1, Hk - 1)] if T == 4096 else [(0, 0), (B - 1, 5)])
    check_bwd(x, "bf16", heads=heads, algo=("chunked", 64))


@pytest.mark.parametrize("B,T,Hk,Hv,C", [(2, 500, 16, 64, 64), (1, 1000, 16, 48, 32)])
def test_chunked_vjp_group_launches(B, T, Hk, Hv, C):
    """The gradient work of a k-head group in one workgroup per (chunk,
    k-head, b) (that grid fills the GPU): GQA 1:4 and 1:3, so the workgroup
    walks four or three v-heads and the middle ones add to the group sums it
    holds, ragged last chunk, h0 and dht nonzero; sampled groups against the
    oracle."""
    x = make_inputs(3100 + T + Hv, B, T, Hk, Hv, 128, 128, io_dtype="bf16", h0_std=0.02)
    dht = (0.1 * np.random.default_rng(T + Hv).standard_normal((B, Hv, 128, 128))).astype(np.float32)
    check_bwd(x, "bf16", dht=dht, heads=[(0, 0), (B - 1, Hk - 1)], algo=("chunked", C))


@pytest.mark.parametrize("cw", [False, True])
@pytest.mark.parametrize("B", [1, 2, 4])
def test_chain_slice_widths(B, cw):
    """The chain kernels' value slice follows the grid: on a 256-CU GPU,
    Hv=32 takes one compute wave per workgroup (16 columns, 8 workgroups
    per v-head) at B=1, two at B=2 and four at B=4.  Forward and VJP (scalar
    and channelwise gates, ragged last chunk, h0 and dht nonzero) on sampled
    (b, k-head) groups against the oracle."""
    Hk, Hv, T = 16, 32, 200
    x = make_inputs(3200 + B + 10 * cw, B, T, Hk, Hv, 128, 128, io_dtype="bf16", h0_std=0.02, channelwise=cw)
    dht = (0.1 * np.random.default_rng(B + 10 * cw).standard_normal((B, Hv, 128, 128))).astype(np.float32)
    heads = [(0, 0), (B - 1, Hk - 1)]
    check_fwd(x, "bf16", h0=True, heads=heads, algo=("chunked", 64), cw=cw)
    check_bwd(x, "bf16", cw=cw, dht=dht, heads=heads, algo=("chunked", 64))


@pytest.mark.parametrize("Hk,Hv", [(2, 8), (1, 3)])
def test_chunked_vjp_split_group(Hk, Hv):
    """The gradient work of every v-head in one launch with the epilogue
    summing each group (grid smaller than the GPU): GQA 1:4 and 1:3, ragged
    last chunk, h0 and dht nonzero; every head against the oracle."""
    x = make_inputs(3200 + Hv, 2, 130, Hk, Hv, 128, 128, io_dtype="bf16", h0_std=0.02)
    dht = (0.1 * np.random.default_rng(Hv).standard_normal((2, Hv, 128, 128))).astype(np.float32)
    check_bwd(x, "bf16", dht=dht, algo=("chunked", 64))


BF16_OUT = ("o", "dq", "dk", "dv")  # rounded to bf16 by out_dtype; ht, dg, dbeta, dh0 stay fp32


def check_bf16_out(x, heads, C, save, dht=None, cw=False, fg=False):
    """Chunked forward + VJP with bf16 outputs (the benchmark's launch
    configuration), optionally through GDR_SAVE_CHUNKS, against the oracle on
    the (b, k-head) groups in heads; bf16-rounded outputs get 2^-8 more."""
    import torch
    import gated_delta_rule_54_amd as gdr
    from oracle import gdr_oracle as orc
    from tests._util import dev, host, relerr
    from tests.test_gpu_sequential import group_slice, to_dev
    t = to_dev(x, "bf16")
    kw = dict(algo="chunked", chunk_size=C, out_dtype=torch.bfloat16, channelwise=cw, fused_gates=fg)
    res = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=save, **kw)
    grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], dev(dht),
                             saved=res[2] if save else None, **kw)
    torch.cuda.synchronize()
    assert res[0].dtype == torch.bfloat16 and grads[0].dtype == torch.bfloat16
    o, ht = host(res[0]), host(res[1])
    grads = [host(a) for a in grads]
    grp = x["v"].shape[2] // x["q"].shape[2]
    for (b, kh) in heads:
        xs = group_slice(x, b, kh, grp)
        vs = slice(kh * grp, (kh + 1) * grp)
        dh = None if dht is None else dht[b:b + 1, vs]
        ro, rht = orc.forward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"], channelwise=cw,
                              fused_gates=fg)
        ref = orc.backward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"], xs["do"], dh, channelwise=cw,
                           fused_gates=fg)
        got = {"o": o[b:b + 1, :, vs], "ht": ht[b:b + 1, vs]}
        exp = {"o": ro, "ht": rht}
        for name, a, r in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), grads, ref):
            got[name] = (a[b:b + 1, :, kh:kh + 1] if name in ("dq", "dk")
                         else a[b:b + 1, vs] if name == "dh0" else a[b:b + 1, :, vs])
            exp[name] = r
        for name in got:
            e = relerr(got[name], exp[name])
            print(f"  b={b} kh={kh} {name}: {e:.2e}")
            assert e < 2e-3 + (2 ** -8 if name in BF16_OUT else 0.0), (name, e)


@pytest.mark.parametrize("save", [False, True])
def test_bf16_outputs_small(save):
    """bf16 o / dq / dk / dv on a small GQA 2:4 problem with a ragged last
    chunk (grid smaller than the GPU: one gradient launch plus the epilogue),
    h0 and dht nonzero."""
    x = make_inputs(3300 + save, 2, 150, 2, 4, 128, 128, io_dtype="bf16", h0_std=0.02)
    dht = (0.1 * np.random.default_rng(33).standard_normal((2, 4, 128, 128))).astype(np.float32)
    check_bf16_out(x, [(0, 0), (0, 1), (1, 0), (1, 1)], 64, save, dht)


def test_bf16_outputs_benchmark_shape():
    """The benchmark's step: B=4, T=4096, Hk=16, Hv=32, D=128, C=64, bf16 io
    and outputs, the forward saving its chunks for the VJP (one gradient
    workgroup per k-head group, writing bf16 dq / dk through LDS); six
    sampled (b, k-head) groups, every sequence of the batch, against the
    oracle."""
    x = make_inputs(3400, 4, 4096, 16, 32, 128, 128, io_dtype="bf16")  # zero h0, as benchmarked
    assert x["h0"] is None
    check_bf16_out(x, [(0, 0), (1, 5), (1, 12), (2, 3), (2, 10), (3, 15)], 64, True)


def test_benchmark_shape_every_head_matches_sequential():
    """Every head of the benchmark shape (B=4, T=4096, Hk=16, Hv=32, D=128),
    forward and VJP: the chunked path (C=64, chunks saved for the VJP)
    against the token-by-token kernels, both with fp32 outputs.  Each is
    within 2e-3 of the oracle where the oracle is run, so they must agree to
    4e-3 on every head, including the ones no oracle call samples."""
    import torch
    import gated_delta_rule_54_amd as gdr
    from tests._util import host, relerr
    from tests.test_gpu_sequential import to_dev
    x = make_inputs(3410, 4, 4096, 16, 32, 128, 128, io_dtype="bf16", h0_std=0.02)
    t = to_dev(x, "bf16")
    out = {}
    for algo in ("sequential", "chunked"):
        kw = dict(algo=algo, out_dtype=torch.float32)
        if algo == "chunked":
            kw["chunk_size"] = 64
            o, ht, sv = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=True,
                                        **kw)
            grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], saved=sv, **kw)
        else:
            o, ht = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], **kw)
            grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], **kw)
        torch.cuda.synchronize()
        out[algo] = [host(a) for a in (o, ht, *grads)]
    names = ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0")
    for name, a, r in zip(names, out["chunked"], out["sequential"]):
        # per (b, head) slice, so no head hides behind another's scale
        heads = a.shape[2] if a.ndim >= 3 and name not in ("ht", "dh0") else a.shape[1]
        for b in range(a.shape[0]):
            for h in range(heads):
                sl = (b, slice(None), h) if name not in ("ht", "dh0") else (b, h)
                err = relerr(a[sl], r[sl])
                assert err < 4e-3, (name, b, h, err)


def test_bf16_outputs_fused_gates_benchmark_shape():
    """The fused-gate leg of the benchmark: B=4, T=4096, g and beta passed as
    pre-activations, bf16 outputs, saved chunks; one sampled group."""
    x = make_inputs(3450, 4, 4096, 16, 32, 128, 128, io_dtype="bf16", gate_preact=True)
    check_bf16_out(x, [(2, 9)], 64, True, fg=True)


def test_bf16_outputs_channelwise_prefill_shape():
    """The channelwise prefill leg of the benchmark: B=1, T=2048, Hk=16,
    Hv=32, D=128, channelwise gate, bf16 io and outputs, zero h0, forward and
    chunked VJP; one sampled (b, k-head) group against the oracle."""
    x = make_inputs(3500, 1, 2048, 16, 32, 128, 128, io_dtype="bf16", channelwise=True)
    check_bf16_out(x, [(0, 7)], 64, False, cw=True)


@pytest.mark.parametrize("io,D,T,C", [("f32", 16, 70, 32), ("bf16", 128, 150, 64), ("bf16", 128, 77, 32)])
def test_fused_gates_chunked(io, D, T, C):
    """GDR_FUSED_GATES on the chunked path (fp32 operands at D=16, fp16
    operands at D=128; ragged last chunk; GQA 2:4): pre-activation gates,
    forward and VJP against the fused-gate oracle."""
    x = make_inputs(1200 + T + C, 2, T, 2, 4, D, D, io_dtype=io, h0_std=0.02 if D == 128 else 0.5,
                    gate_preact=True)
    dht = (0.1 * np.random.default_rng(T).standard_normal((2, 4, D, D))).astype(np.float32)
    check_fwd(x, io, algo=("chunked", C), fg=True)
    check_bwd(x, io, dht=dht, algo=("chunked", C), fg=True)


# ------------------------------------------------- channelwise chunked forward

@pytest.mark.parametrize("T,C", [(1, 64), (50, 64), (64, 64), (200, 64), (200, 32), (97, 32)])
@pytest.mark.parametrize("l2", [True, False])
def test_channelwise_chunked_forward(T, C, l2):
    """Per-channel gate on the chunked forward (bf16 io, D=128, fp16 operands):
    ragged last chunk, GQA 2:4, nonzero h0, flag on/off.  With the flag off
    the rows of q and k are unit vectors already (rounded to bf16), as raw
    N(0, 1) keys of norm ~11 make the recurrence itself diverge."""
    x = make_inputs(1400 + T + C + l2, 2, T, 2, 4, 128, 128, io_dtype="bf16", channelwise=True,
                    h0_std=0.02, with_do=False)
    if not l2:
        for n in ("q", "k"):
            u = x[n] / np.linalg.norm(x[n].astype(np.float64), axis=-1, keepdims=True)
            x[n] = round_bf16(u.astype(np.float32))
    check_fwd(x, "bf16", l2=l2, cw=True, algo=("chunked", C))


def test_channelwise_chunked_forward_fused_gates():
    x = make_inputs(1500, 2, 150, 2, 4, 128, 128, io_dtype="bf16", channelwise=True,
                    h0_std=0.02, with_do=False, gate_preact=True)
    check_fwd(x, "bf16", cw=True, algo=("chunked", 64), fg=True)


@pytest.mark.parametrize("T", [128, 512, 2048])
def test_channelwise_chunked_prefill(T):
    """Channelwise prefill B=1, Hk=16, Hv=32, D=128, bf16, zero h0, C=64:
    the GPU runs every head; the oracle checks two sampled k-head groups."""
    x = make_inputs(1600 + T, 1, T, 16, 32, 128, 128, io_dtype="bf16", channelwise=True,
                    with_do=False)
    check_fwd(x, "bf16", cw=True, h0=False, heads=[(0, 0), (0, 11)], algo=("chunked", 64))


@pytest.mark.parametrize("scale,C", [(4.0, 64), (4.0, 32), (30.0, 64), (30.0, 32)])
def test_channelwise_chunked_strong_decay(scale, C):
    """Per-channel gates g = -scale * U(0.9, 1.0): at scale 4 a 16-row block
    decays by up to e^-64 per channel (diagonal blocks still factored, the
    factors near 2^92); at scale 30 the diagonal blocks take the exact
    per-pair sums."""
    x = make_inputs(1700 + int(scale) + C, 2, 150, 2, 4, 128, 128, io_dtype="bf16",
                    channelwise=True, h0_std=0.02, with_do=False)
    u = np.random.default_rng(C).uniform(0.9, 1.0, x["g"].shape)
    x["g"] = (-scale * u).astype(np.float32)
    check_fwd(x, "bf16", cw=True, algo=("chunked", C))


def test_channelwise_chunked_mixed_decay():
    """Strong decay (g = -30) on a few channels of the second chunk only:
    that chunk takes the exact diagonal sums, the others the factored ones."""
    x = make_inputs(1750, 2, 200, 2, 4, 128, 128, io_dtype="bf16", channelwise=True,
                    h0_std=0.02, with_do=False)
    x["g"][:, 64:128, :, 5:9] = -30.0
    check_fwd(x, "bf16", cw=True, algo=("chunked", 64))


# ------------------------------------------------ forward saves for the VJP

@pytest.mark.parametrize("T,C", [(200, 64), (97, 32), (64, 64)])
def test_saved_chunks_match_stateless(T, C):
    """GDR_SAVE_CHUNKS: the forward that keeps its images and chunk states
    gives the same o / ht, and the VJP that reads them the same gradients,
    bit for bit, as the stateless calls (GQA 2:4, h0 and dht nonzero);
    the stateless results are checked against the oracle."""
    import torch
    import gated_delta_rule_54_amd as gdr
    from tests._util import host
    x = make_inputs(1800 + T + C, 2, T, 2, 4, 128, 128, io_dtype="bf16", h0_std=0.02)
    dht = (0.1 * np.random.default_rng(T).standard_normal((2, 4, 128, 128))).astype(np.float32)
    check_fwd(x, "bf16", algo=("chunked", C))
    check_bwd(x, "bf16", dht=dht, algo=("chunked", C))
    from tests.test_gpu_sequential import to_dev
    from tests._util import dev
    t = to_dev(x, "bf16")
    kw = dict(algo="chunked", chunk_size=C)
    o0, ht0 = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], **kw)
    o1, ht1, saved = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"],
                                     save_for_backward=True, **kw)
    g0 = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], dev(dht), **kw)
    g1 = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], dev(dht),
                          saved=saved, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host(o0), host(o1)) and np.array_equal(host(ht0), host(ht1))
    for a0, a1 in zip(g0, g1):
        assert np.array_equal(host(a0), host(a1))


# ------------------------------------------------ channelwise chunked VJP

@pytest.mark.parametrize("T,C", [(1, 64), (50, 64), (64, 64), (200, 64), (97, 32), (130, 32)])
def test_channelwise_chunked_vjp(T, C):
    """Channelwise gates on the chunked VJP (chunk states from the chains,
    then every chunk's gradients with the per-channel decay inside the
    chunk-local sums): ragged last chunk, GQA 2:4, h0 and dht nonzero, bf16
    io, D=128."""
    x = make_inputs(1900 + T + C, 2, T, 2, 4, 128, 128, io_dtype="bf16", channelwise=True, h0_std=0.02)
    dht = (0.1 * np.random.default_rng(T + C).standard_normal((2, 4, 128, 128))).astype(np.float32)
    check_bwd(x, "bf16", cw=True, dht=dht, algo=("chunked", C))


def test_channelwise_chunked_vjp_fused_gates_and_strong_decay():
    x = make_inputs(1950, 2, 150, 2, 4, 128, 128, io_dtype="bf16", channelwise=True, h0_std=0.02,
                    gate_preact=True)
    check_bwd(x, "bf16", cw=True, algo=("chunked", 64), fg=True)
    y = make_inputs(1951, 2, 150, 2, 4, 128, 128, io_dtype="bf16", channelwise=True, h0_std=0.02)
    y["g"][:, 64:128, :, 5:9] = -30.0   # the exact diagonal sums in the second chunk
    check_bwd(y, "bf16", cw=True, algo=("chunked", 64))


@pytest.mark.parametrize("Hk,Hv,C,l2", [(1, 3, 64, True), (2, 8, 32, True), (1, 4, 64, False)])
def test_channelwise_chunked_vjp_group_walk(Hk, Hv, C, l2):
    """The channelwise gradient workgroup walks a k-head's v-heads in order
    (GQA 1:3 and 1:4, both chunk sizes), summing dq_hat / dk_hat before the
    L2-norm VJP, or with the norm flag off (then the rows of q and k are unit
    vectors already, as in the forward tests); ragged last chunk, h0 and dht
    nonzero."""
    x = make_inputs(1970 + Hv + C, 2, 150, Hk, Hv, 128, 128, io_dtype="bf16", channelwise=True, h0_std=0.02)
    if not l2:
        for n in ("q", "k"):
            u = x[n] / np.linalg.norm(x[n].astype(np.float64), axis=-1, keepdims=True)
            x[n] = round_bf16(u.astype(np.float32))
    dht = (0.1 * np.random.default_rng(Hv + C).standard_normal((2, Hv, 128, 128))).astype(np.float32)
    check_bwd(x, "bf16", l2=l2, cw=True, dht=dht, algo=("chunked", C))


def test_channelwise_chunked_vjp_prefill_t2048():
    """B=1, Hk=16, Hv=32, T=2048 (the channelwise prefill shape), sampled
    k-head groups against the oracle."""
    x = make_inputs(1960, 1, 2048, 16, 32, 128, 128, io_dtype="bf16", channelwise=True)
    check_bwd(x, "bf16", cw=True, h0=False, heads=[(0, 3)], algo=("chunked", 64))


# ------------------------------------------------ long sequence

def test_long_sequence_saved_chunks():
    """One sequence of 65,535 tokens (1,024 chunks of 64, the last one 63
    rows): the chunk grids' longest axis and a workspace of a thousand chunk
    states per head.  GQA 2:4, D=128, bf16 io, fp32 outputs, h0 and dht
    nonzero, the forward saving its chunks for the VJP; k-head group 1
    (v-heads 2, 3) against the oracle over the whole sequence."""
    import torch
    import gated_delta_rule_54_amd as gdr
    from oracle import gdr_oracle as orc
    from tests._util import dev, host, relerr
    from tests.test_gpu_sequential import group_slice, to_dev
    T = 65535
    x = make_inputs(6553, 1, T, 2, 4, 128, 128, io_dtype="bf16", h0_std=0.02)
    dht = (0.1 * np.random.default_rng(6553).standard_normal((1, 4, 128, 128))).astype(np.float32)
    t = to_dev(x, "bf16")
    kw = dict(algo="chunked", chunk_size=64)
    o, ht, saved = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=True, **kw)
    grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], dev(dht), saved=saved,
                             **kw)
    torch.cuda.synchronize()
    o, ht = host(o), host(ht)
    grads = [host(a) for a in grads]
    del t, saved
    xs, vs = group_slice(x, 0, 1, 2), slice(2, 4)
    ro, rht = orc.forward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"])
    ref = orc.backward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"], xs["do"], dht[:, vs])
    got = {"o": o[:, :, vs], "ht": ht[:, vs]}
    exp = {"o": ro, "ht": rht}
    for name, a, r in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), grads, ref):
        got[name] = a[:, :, 1:2] if name in ("dq", "dk") else a[:, vs] if name == "dh0" else a[:, :, vs]
        exp[name] = r
    for name in got:
        e = relerr(got[name], exp[name])
        print(f"  T={T} kh=1 {name}: {e:.2e}")
        assert e < 2e-3, (name, e)
