"""gdr_forward_noalloc (the allocation-free forward for callers that cannot
allocate device memory) through the C ABI, against gdr_forward on the same
inputs: two calls in a row, the second on a smaller problem, so that the
second reuses the scratch the first left behind; both bit-identical to
gdr_forward (the same kernels run, only the workspace differs).  Also the
size limit and the rejected flag, which return before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_54_amd as gdr
from gated_delta_rule_54_amd import binding as B
from gated_delta_rule_54_amd.synth import make_inputs
from oracle import gdr_oracle as orc
from tests._util import dev, relerr

pytestmark = pytest.mark.gpu


def tensors(seed, b, t, hk, hv, d, io="bf16", h0=True):
    x = make_inputs(seed, b, t, hk, hv, d, d, io_dtype=io, h0_std=0.02 if h0 else None, with_do=False)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    return x, {n: (None if a is None else dev(a, dt if n in ("q", "k", "v") else torch.float32))
               for n, a in x.items()}


def raw_noalloc(t, algo, C, out_dtype=torch.float32):
    """One gdr_forward_noalloc call straight through ctypes into outputs
    allocated here (the call itself allocates nothing)."""
    Bn, T, Hk, D = t["q"].shape
    Hv = t["v"].shape[2]
    o = torch.full((Bn, T, Hv, D), float("nan"), dtype=out_dtype, device="cuda")
    ht = torch.full((Bn, Hv, D, D), float("nan"), dtype=torch.float32, device="cuda")
    io = 1 if t["q"].dtype == torch.bfloat16 else 0
    p = B.GdrProblem(Bn, T, Hk, Hv, D, D, io, 1 if out_dtype == torch.bfloat16 else 0, 1, algo, C)
    ptr = lambda a: None if a is None else a.data_ptr()
    st = B.lib().gdr_forward_noalloc(ctypes.byref(p), ptr(t["q"]), ptr(t["k"]), ptr(t["v"]), ptr(t["g"]),
                                     ptr(t["beta"]), ptr(t["h0"]), o.data_ptr(), ht.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().gdr_status_str(st)
    return o, ht


def bitwise_equal(a, b):
    return np.array_equal(a.cpu().contiguous().view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                          b.cpu().contiguous().view(torch.int32 if b.dtype == torch.float32 else torch.int16))


@pytest.mark.parametrize("algo,C", [(2, 64), (2, 32), (1, 64)])
def test_noalloc_matches_forward_two_calls(algo, C):
    """A larger call, then a smaller one reusing the same scratch; each equals
    gdr_forward bit for bit and the oracle within the bf16 bar."""
    for seed, (b, t, hk, hv) in ((1, (2, 700, 16, 32)), (2, (1, 130, 4, 8))):
        x, tt = tensors(seed, b, t, hk, hv, 128)
        o, ht = raw_noalloc(tt, algo, C)
        kw = dict(algo={1: "sequential", 2: "chunked"}[algo], chunk_size=C)
        ro, rht = gdr.gdr_forward(tt["q"], tt["k"], tt["v"], tt["g"], tt["beta"], tt["h0"], **kw)
        torch.cuda.synchronize()
        assert bitwise_equal(o, ro) and bitwise_equal(ht, rht), (b, t)
        if seed == 2:  # the small problem against the oracle as well
            wo, wht = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
            assert relerr(o.cpu().double().numpy(), wo) < 2e-3
            assert relerr(ht.cpu().double().numpy(), wht) < 2e-3


def test_noalloc_binding_and_in_place_decode():
    """The binding's gdr_forward_noalloc with caller-given outputs, and
    decode steps that update the state in place (ht = h0, no workspace)."""
    _, tt = tensors(3, 8, 1, 16, 32, 128)
    s = tt["h0"].clone()
    ref = tt["h0"].clone()
    o = torch.empty((8, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    for _ in range(4):
        gdr.gdr_forward_noalloc(tt["q"], tt["k"], tt["v"], tt["g"], tt["beta"], s, o=o, ht=s, algo="sequential",
                                out_dtype=torch.bfloat16)
        ro, _ = gdr.gdr_forward(tt["q"], tt["k"], tt["v"], tt["g"], tt["beta"], ref, ht=ref, algo="sequential",
                                out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert bitwise_equal(o, ro)
    assert bitwise_equal(s, ref)


def test_noalloc_limits():
    """Problems beyond the fixed scratch, and GDR_SAVE_CHUNKS, are refused
    before anything is launched."""
    lib = B.lib()
    need = ctypes.c_size_t(0)
    big = B.GdrProblem(8, 4096, 16, 32, 128, 128, 1, 1, 1, 2, 64)
    assert lib.gdr_forward_workspace(ctypes.byref(big), ctypes.byref(need)) == 0
    assert need.value > (64 << 20)
    fake = 0x10000  # never dereferenced: the call fails validation first
    args = [fake] * 8 + [None]
    assert lib.gdr_forward_noalloc(ctypes.byref(big), *args) == 5
    saved = B.GdrProblem(1, 512, 16, 32, 128, 128, 1, 1, 1 | 8, 2, 64)
    assert lib.gdr_forward_noalloc(ctypes.byref(saved), *args) == 3
