"""GPU checks of what include/gdr.h promises beyond parity: results are
bitwise reproducible from run to run, NaN inputs propagate (to the outputs
that depend on them and no further), the kernels write nothing outside the
buffers the problem names, the fp16 chunked path turns out-of-range operands
into non-finite outputs rather than finite wrong ones, and GDR_SAVE_CHUNKS is
harmless where the library ignores it.  Every case exits normally: nothing
here makes a kernel fault or trap."""

import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_54_amd as gdr
from gated_delta_rule_54_amd import binding as B
from gated_delta_rule_54_amd.synth import make_inputs
from oracle import gdr_oracle as orc
from tests._util import dev, host, relerr

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def to_dev(x, io="bf16"):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    return {n: (None if a is None else dev(a, dt if n in ("q", "k", "v", "do") else torch.float32))
            for n, a in x.items()}


def step(t, **kw):
    """Forward (saving chunks where kept) + VJP; every output, on the host."""
    o, ht, sv = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=True, **kw)
    grads = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], saved=sv, **kw)
    torch.cuda.synchronize()
    out = {"o": o, "ht": ht}
    out.update(zip(GRADS, grads))
    return {n: a.detach().cpu() for n, a in out.items()}


def bits(a):
    return a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32).numpy()


# ---------------------------------------------------------------- bitwise

def test_step_bitwise_reproducible():
    """The headline step (B=4, T=4096, Hk=16, Hv=32, D=128, bf16, chunks
    saved for the VJP) twice on the same inputs: every output bit-identical."""
    x = make_inputs(2, 4, 4096, 16, 32, 128, 128, io_dtype="bf16")
    t = to_dev(x)
    kw = dict(algo="chunked", chunk_size=64, out_dtype=torch.bfloat16)
    r1 = step(t, **kw)
    r2 = step(t, **kw)
    for n in r1:
        assert np.array_equal(bits(r1[n]), bits(r2[n])), n


def test_decode_bitwise_reproducible():
    """256 single-token steps at B=8, Hv=32 carrying the state in place, run
    twice from the same initial state: outputs and final state identical."""
    g = torch.Generator(device="cuda").manual_seed(3)
    rn = lambda *s: torch.randn(*s, device="cuda", generator=g)
    n = 256
    q, k, v = (rn(n, 8, 1, h, 128).bfloat16() for h in (16, 16, 32))
    gg = -torch.nn.functional.softplus(rn(n, 8, 1, 32))
    bb = torch.sigmoid(rn(n, 8, 1, 32))
    h0 = rn(8, 32, 128, 128) * 0.02
    runs = []
    for _ in range(2):
        s = h0.clone()
        outs = [gdr.gdr_forward(q[i], k[i], v[i], gg[i], bb[i], s, ht=s, algo="sequential",
                                out_dtype=torch.bfloat16)[0] for i in range(n)]
        torch.cuda.synchronize()
        runs.append((torch.stack(outs).cpu(), s.cpu()))
    assert np.array_equal(bits(runs[0][0]), bits(runs[1][0]))
    assert np.array_equal(bits(runs[0][1]), bits(runs[1][1]))


# ---------------------------------------------------------------- NaN

@pytest.mark.parametrize("algo", ["chunked", "sequential"])
def test_nan_propagates_to_its_head_only(algo):
    """A NaN in one element of v (sequence 1, token 150, v-head 3, column
    7): o, ht, dg, dbeta of that (sequence, v-head) and dq, dk of its k-head
    become non-finite (dv and dh0 do not depend on v mathematically and may
    stay finite); every element outside that set is bit-identical to the
    clean run."""
    Bn, T, Hk, Hv, D = 2, 200, 2, 4, 128
    x = make_inputs(5, Bn, T, Hk, Hv, D, D, io_dtype="bf16", h0_std=0.02)
    kw = dict(algo=algo, out_dtype=torch.float32)
    clean = step(to_dev(x), **kw)
    xp = {n: (None if a is None else a.copy()) for n, a in x.items()}
    b, t, hv = 1, 150, 3
    kh = hv // (Hv // Hk)
    xp["v"][b, t, hv, 7] = np.nan
    bad = step(to_dev(xp), **kw)
    head = {"o": (b, slice(None), hv), "ht": (b, hv), "dq": (b, slice(None), kh), "dk": (b, slice(None), kh),
            "dv": (b, slice(None), hv), "dg": (b, slice(None), hv), "dbeta": (b, slice(None), hv),
            "dh0": (b, hv)}
    must = ("o", "ht", "dq", "dk", "dg", "dbeta")
    for n, idx in head.items():
        c, p = clean[n].numpy().copy(), bad[n].numpy().copy()
        if n in must:
            assert not np.all(np.isfinite(p[idx])), n
        if n == "o":
            assert np.isnan(p[b, t, hv, 7])
            if algo == "sequential":  # tokens before the NaN are untouched
                assert np.array_equal(c[b, :t, hv].view(np.int32), p[b, :t, hv].view(np.int32))
        c[idx] = 0
        p[idx] = 0
        assert np.array_equal(c.view(np.int32), p.view(np.int32)), n


# ---------------------------------------------------------------- canaries

GUARD_HEAD, GUARD_TAIL = 256, 4096
PATTERN = 0xA5


class Guarded:
    """A device buffer of `nbytes` with guard bytes before and after, filled
    with PATTERN; .ptr is the 256-byte aligned start of the usable part."""

    def __init__(self, nbytes, fill=None):
        self.n = nbytes
        self.buf = torch.full((GUARD_HEAD + nbytes + GUARD_TAIL,), PATTERN, dtype=torch.uint8, device="cuda")
        if fill is not None:
            self.buf[GUARD_HEAD:GUARD_HEAD + nbytes].copy_(fill.contiguous().view(torch.uint8).reshape(-1))
        self.ptr = self.buf.data_ptr() + GUARD_HEAD

    def guards_intact(self):
        h = self.buf.cpu().numpy()
        return bool(np.all(h[:GUARD_HEAD] == PATTERN) and np.all(h[GUARD_HEAD + self.n:] == PATTERN))

    def view(self, dtype, shape):
        return self.buf[GUARD_HEAD:GUARD_HEAD + self.n].view(dtype).reshape(shape)


def raw_pair(x, T, lengths=None, algo=2, C=64, io=1, out=1):
    """gdr_forward(_varlen) + gdr_backward(_varlen) straight through the C
    ABI on guarded buffers (inputs, outputs and workspaces); returns the
    guarded outputs."""
    Bn = len(lengths) if lengths is not None else x["q"].shape[0]
    Hk, Hv, D = x["q"].shape[2], x["v"].shape[2], x["q"].shape[3]
    td = torch.bfloat16 if io == 1 else torch.float32
    od = torch.bfloat16 if out == 1 else torch.float32
    t = {n: (None if a is None else dev(a, td if n in ("q", "k", "v", "do") else torch.float32))
         for n, a in x.items()}
    ins = {n: Guarded(a.numel() * a.element_size(), a) for n, a in t.items() if a is not None}
    esz = 2 if out == 1 else 4
    rows = x["q"].shape[0] * x["q"].shape[1]
    outs = {"o": Guarded(rows * Hv * D * esz), "ht": Guarded(Bn * Hv * D * D * 4),
            "dq": Guarded(rows * Hk * D * esz), "dk": Guarded(rows * Hk * D * esz),
            "dv": Guarded(rows * Hv * D * esz), "dg": Guarded(rows * Hv * 4), "dbeta": Guarded(rows * Hv * 4),
            "dh0": Guarded(Bn * Hv * D * D * 4)}
    p = B.GdrProblem(Bn, T, Hk, Hv, D, D, io, out, 1, algo, C)
    L = B.lib()
    wf, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.gdr_forward_workspace(ctypes.byref(p), ctypes.byref(wf)) == 0
    assert L.gdr_backward_workspace(ctypes.byref(p), ctypes.byref(wb)) == 0
    wsf, wsb = Guarded(max(wf.value, 256)), Guarded(max(wb.value, 256))
    st = torch.cuda.current_stream().cuda_stream
    I = lambda n: ins[n].ptr if n in ins else None
    if lengths is not None:
        cu = Guarded(8 * (Bn + 1), torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64))
        r = L.gdr_forward_varlen(ctypes.byref(p), cu.ptr, I("q"), I("k"), I("v"), I("g"), I("beta"), I("h0"),
                                 outs["o"].ptr, outs["ht"].ptr, wsf.ptr, wf.value, st)
        assert r == 0
        r = L.gdr_backward_varlen(ctypes.byref(p), cu.ptr, I("q"), I("k"), I("v"), I("g"), I("beta"), I("h0"),
                                  I("do"), None, outs["dq"].ptr, outs["dk"].ptr, outs["dv"].ptr, outs["dg"].ptr,
                                  outs["dbeta"].ptr, outs["dh0"].ptr, wsb.ptr, wb.value, st)
        assert r == 0
        ins["cu"] = cu
    else:
        r = L.gdr_forward(ctypes.byref(p), I("q"), I("k"), I("v"), I("g"), I("beta"), I("h0"), outs["o"].ptr,
                          outs["ht"].ptr, wsf.ptr, wf.value, st)
        assert r == 0
        r = L.gdr_backward(ctypes.byref(p), I("q"), I("k"), I("v"), I("g"), I("beta"), I("h0"), I("do"), None,
                           outs["dq"].ptr, outs["dk"].ptr, outs["dv"].ptr, outs["dg"].ptr, outs["dbeta"].ptr,
                           outs["dh0"].ptr, wsb.ptr, wb.value, st)
        assert r == 0
    torch.cuda.synchronize()
    for name, gb in list(ins.items()) + list(outs.items()) + [("ws_fwd", wsf), ("ws_bwd", wsb)]:
        assert gb.guards_intact(), name
    return outs


@pytest.mark.parametrize("algo,C,T", [(2, 64, 200), (2, 32, 77), (1, 64, 70)])
def test_canary_guards_uniform_batch(algo, C, T):
    """Chunked (ragged last chunk) and sequential forward + VJP on guarded
    buffers: no byte outside any buffer changes, and the results still match
    the oracle."""
    x = make_inputs(9, 2, T, 2, 4, 128, 128, io_dtype="bf16", h0_std=0.02)
    outs = raw_pair(x, T, algo=algo, C=C, out=0)
    ro, rht = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    assert relerr(outs["o"].view(torch.float32, ro.shape).cpu().numpy(), ro) < 2e-3
    ref = orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["do"])
    for n, r in zip(GRADS, ref):
        assert relerr(outs[n].view(torch.float32, r.shape).cpu().numpy(), r) < 2e-3, n


@pytest.mark.parametrize("algo", [2, 1])
def test_canary_guards_ragged_batch(algo):
    """A ragged batch (lengths 0, 1, 63, 64, 130 and 200 tokens; bound 256)
    through the varlen entry points on guarded buffers: the kernels touch
    only the rows the offsets name."""
    lengths = [130, 0, 1, 63, 64, 200]
    rows = sum(lengths)
    x = make_inputs(12, 1, rows, 2, 4, 128, 128, io_dtype="bf16")
    x["h0"] = (0.02 * np.random.default_rng(1).standard_normal((len(lengths), 4, 128, 128))).astype(np.float32)
    raw_pair(x, 256, lengths=lengths, algo=algo)


# ---------------------------------------------------------------- fp16 range

def test_fp16_range_of_the_chunked_path():
    """A bf16 v element of 1e6 (beyond fp16's +-65504 after the write
    strength 0.5) in one (sequence, v-head): the chunked path gives that
    head non-finite outputs from the token on and leaves every other head
    bit-identical; the sequential path (fp32 throughout) still matches the
    oracle.  A value of 1e5 (in range once scaled) gives either a finite
    result within the bar or a non-finite one, never a finite wrong one."""
    Bn, T, Hk, Hv, D = 1, 160, 2, 4, 128
    x = make_inputs(21, Bn, T, Hk, Hv, D, D, io_dtype="bf16")
    b, t, hv = 0, 70, 1
    x["beta"][b, t, hv] = 0.5
    kw = dict(algo="chunked", chunk_size=64)
    clean = gdr.gdr_forward(*(dev(x[n], torch.bfloat16) for n in ("q", "k", "v")), dev(x["g"]), dev(x["beta"]),
                            None, **kw)[0].cpu().numpy()
    for big, must_overflow in ((1e6, True), (1e5, False)):
        xp = {n: (None if a is None else a.copy()) for n, a in x.items()}
        xp["v"][b, t, hv, 5] = big
        tv = {n: dev(xp[n], torch.bfloat16) for n in ("q", "k", "v")}
        o = gdr.gdr_forward(tv["q"], tv["k"], tv["v"], dev(xp["g"]), dev(xp["beta"]), None, **kw)[0]
        o = o.cpu().numpy()
        vbf = tv["v"].float().cpu().numpy()
        ro, _ = orc.forward(xp["q"], xp["k"], vbf, xp["g"], xp["beta"])
        head = o[b, t:, hv]
        if must_overflow:
            assert not np.all(np.isfinite(head))
        elif np.all(np.isfinite(head)):
            assert relerr(head, ro[b, t:, hv]) < 2e-3
        keep = np.ones(o.shape, bool)
        keep[b, :, hv] = False
        assert np.array_equal(o[keep].view(np.int32), clean[keep].view(np.int32))
        if big == 1e6:
            os_ = gdr.gdr_forward(tv["q"], tv["k"], tv["v"], dev(xp["g"]), dev(xp["beta"]), None,
                                  algo="sequential")[0].cpu().numpy()
            assert np.all(np.isfinite(os_))
            assert relerr(os_, ro) < 2e-3


# ---------------------------------------------------------------- saved chunks

@pytest.mark.parametrize("case", ["auto_T8", "sequential", "fp32_chunked", "channelwise"])
def test_save_for_backward_where_ignored(case):
    """save_for_backward=True on problems where the library keeps no chunks
    (AUTO's forward at T=8 picks the sequential kernels, its backward the
    chunked ones; the sequential algorithm; fp32 io; the channelwise gate):
    the backward runs the stateless VJP and gives exactly what it gives
    without the flag."""
    T = 8 if case == "auto_T8" else 130
    io = "f32" if case == "fp32_chunked" else "bf16"
    cw = case == "channelwise"
    x = make_inputs(31, 1, T, 2, 4, 128, 128, io_dtype=io, channelwise=cw, h0_std=0.02)
    t = to_dev(x, io)
    kw = dict(algo={"auto_T8": "auto", "sequential": "sequential"}.get(case, "chunked"), channelwise=cw)
    o, ht, sv = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], save_for_backward=True, **kw)
    assert not sv.kept
    g1 = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], saved=sv, **kw)
    g0 = gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], **kw)
    torch.cuda.synchronize()
    for a, b_ in zip(g1, g0):
        assert torch.equal(a, b_)
    ref = orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["do"], channelwise=cw)
    for n, a, r in zip(GRADS, g1, ref):
        assert relerr(host(a), r) < 2e-3, n
