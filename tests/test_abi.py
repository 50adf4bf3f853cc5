"""CPU checks of the C ABI: the library loads, exports every symbol in
include/gdr.h, and rejects bad arguments before touching the GPU (every call
below fails validation, so no HIP call is made)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_54_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions(name="gdr.h"):
    txt = open(os.path.join(ROOT, "include", name)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", txt))


def test_every_declared_symbol_is_exported():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["gdr.h", "gdr_calib.h"]
    assert header_functions("gdr.h") == set(B.SYMBOLS)
    assert header_functions("gdr_calib.h") == set(B.CALIB_SYMBOLS)
    lib = B.lib()
    for name in B.SYMBOLS + B.CALIB_SYMBOLS:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = B.lib()
    assert lib.gdr_abi_version() == 4
    for s in range(7):
        assert len(lib.gdr_status_str(s)) > 0
    assert lib.gdr_status_str(99) == b"unknown gdr_status"
    assert lib.gdr_last_hip_error() == b""


def prob(**kw):
    base = dict(B=2, T=8, Hk=2, Hv=4, Dk=16, Dv=16, io_dtype=0, out_dtype=0, flags=1,
                algo=0, chunk_size=0)
    base.update(kw)
    return B.GdrProblem(**base)


def fwd_ws(p):
    n = ctypes.c_size_t(12345)
    return B.lib().gdr_forward_workspace(ctypes.byref(p), ctypes.byref(n)), n.value


def bwd_ws(p):
    n = ctypes.c_size_t(12345)
    return B.lib().gdr_backward_workspace(ctypes.byref(p), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(Hv=3), 2), (dict(T=-1), 2), (dict(B=-2), 2), (dict(Hk=0), 2), (dict(Dk=0), 2),
    (dict(Dk=64, Dv=64), 3), (dict(Dk=16, Dv=128), 3), (dict(io_dtype=2), 3),
    (dict(out_dtype=-1), 3), (dict(flags=16), 3), (dict(algo=3), 3), (dict(chunk_size=48), 3),
])
def test_workspace_query_rejects_bad_problems(kw, status):
    assert fwd_ws(prob(**kw))[0] == status
    assert bwd_ws(prob(**kw))[0] == status


def test_workspace_query_null_args():
    assert B.lib().gdr_forward_workspace(None, None) == 1
    p = prob()
    assert B.lib().gdr_backward_workspace(ctypes.byref(p), None) == 1


def test_workspace_sizes_scale_with_problem():
    st, n0 = bwd_ws(prob(T=0))
    assert st == 0 and n0 == 0
    st, n1 = bwd_ws(prob(T=64, algo=1))
    st2, n2 = bwd_ws(prob(T=128, algo=1))
    assert st == 0 and st2 == 0 and 0 < n1 < n2 and n1 % 256 == 0


FAKE = 0x10000  # an aligned address that is never dereferenced


def call_fwd(p, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, o=FAKE, ht=None,
             ws=None, nws=0):
    return B.lib().gdr_forward(ctypes.byref(p), q, k, v, g, beta, h0, o, ht, ws, nws, None)


def call_bwd(p, ws=None, nws=0, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, dout=FAKE, dht=None,
                dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dh0=None)
    args.update(over)
    return B.lib().gdr_backward(ctypes.byref(p), *args.values(), ws, nws, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "o"])
def test_forward_null_inputs(name):
    assert call_fwd(prob(), **{name: None}) == 1


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "dout", "dq", "dk", "dv",
                                  "dg", "dbeta"])
def test_backward_null_inputs(name):
    assert call_bwd(prob(), **{name: None}) == 1


@pytest.mark.parametrize("name", ["q", "v", "h0", "o", "ht"])
def test_forward_misaligned(name):
    assert call_fwd(prob(), **{name: FAKE + 8}) == 4


def test_backward_misaligned_and_workspace():
    assert call_bwd(prob(), dq=FAKE + 4) == 4
    assert call_bwd(prob(), ws=FAKE + 16, nws=1 << 30) == 4      # workspace needs 256 B
    st, need = bwd_ws(prob())
    assert st == 0 and need > 0
    assert call_bwd(prob()) == 1                                   # missing workspace
    assert call_bwd(prob(), ws=FAKE, nws=need - 1) == 5            # too small


def test_bad_problem_beats_everything():
    assert call_fwd(prob(Hv=3), q=None) == 2
    assert call_bwd(prob(Dk=32, Dv=32), dq=None) == 3
    assert B.lib().gdr_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == 1


def test_channelwise_chunked_support():
    """Channelwise gates: chunked forward and VJP only with bf16 io, D = 128
    and C in {32, 64}; AUTO falls back to the sequential kernels (forward:
    no workspace) where the chunked ones are absent."""
    cw = dict(flags=3, io_dtype=1, Dk=128, Dv=128, T=256)
    for C in (0, 32, 64):
        st, n = fwd_ws(prob(algo=2, chunk_size=C, **cw))
        assert st == 0 and n > 0
        st, n2 = bwd_ws(prob(algo=2, chunk_size=C, **cw))
        assert st == 0 and n2 > n
    assert fwd_ws(prob(algo=2, chunk_size=16, **cw))[0] == 3
    assert bwd_ws(prob(algo=2, chunk_size=16, **cw))[0] == 3
    assert fwd_ws(prob(algo=2, flags=3, T=256))[0] == 3          # fp32 io, D = 16
    assert bwd_ws(prob(algo=2, flags=3, T=256))[0] == 3
    st, n = fwd_ws(prob(algo=0, **cw))
    assert st == 0 and n > 0                                      # AUTO -> chunked
    assert bwd_ws(prob(algo=0, **cw)) == bwd_ws(prob(algo=2, **cw))
    assert fwd_ws(prob(algo=0, **dict(cw, T=11))) == (0, 0)       # short: sequential
    assert fwd_ws(prob(algo=0, **dict(cw, T=12)))[1] > 0          # AUTO's shortest chunked forward
    assert fwd_ws(prob(algo=0, flags=3, T=256)) == (0, 0)         # fp32: sequential


def test_save_chunks_workspace():
    """GDR_SAVE_CHUNKS: on the fp16 chunked path the forward asks for the
    backward's workspace (it leaves images and chunk states there); where the
    flag changes nothing the sizes are those without it."""
    base = dict(io_dtype=1, Dk=128, Dv=128, T=256, algo=2)
    for C in (32, 64):
        st, nf = fwd_ws(prob(flags=1 | 8, chunk_size=C, **base))
        st2, nb = bwd_ws(prob(flags=1 | 8, chunk_size=C, **base))
        assert st == 0 and st2 == 0 and nf == nb
        assert bwd_ws(prob(flags=1, chunk_size=C, **base)) == (0, nb)
        assert fwd_ws(prob(flags=1, chunk_size=C, **base))[1] < nf
    assert fwd_ws(prob(flags=1 | 8, **dict(base, algo=1))) == (0, 0)            # sequential
    for f in (1, 1 | 8):                                                         # fp32 io, D = 16
        assert fwd_ws(prob(flags=f, algo=2, T=256)) == fwd_ws(prob(flags=1, algo=2, T=256))
    cw = dict(base, chunk_size=64)
    assert fwd_ws(prob(flags=3 | 8, **cw)) == fwd_ws(prob(flags=3, **cw))       # channelwise


def call_fwd_varlen(p, cu, ws=None, nws=0):
    return B.lib().gdr_forward_varlen(ctypes.byref(p), cu, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                      ws, nws, None)


def call_bwd_varlen(p, cu, ws=None, nws=0):
    return B.lib().gdr_backward_varlen(ctypes.byref(p), cu, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                       FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, nws, None)


def test_varlen_validation():
    """Ragged batches: offsets required and 8-byte aligned; the fp32 chunked
    path refuses them (all before any launch)."""
    bf = dict(io_dtype=1, Dk=128, Dv=128, T=256)
    assert call_fwd_varlen(prob(**bf), None) == 1
    assert call_bwd_varlen(prob(**bf), None) == 1
    assert call_fwd_varlen(prob(**bf), FAKE + 4) == 4
    assert call_bwd_varlen(prob(algo=2, T=256), FAKE) == 3          # fp32 io, D = 16 chunked
    assert call_bwd_varlen(prob(algo=2, flags=3, **bf), FAKE) == 1  # channelwise chunked VJP: no workspace
    assert call_fwd_varlen(prob(algo=2, T=256), FAKE) == 3          # fp32 chunked forward
    assert call_bwd_varlen(prob(algo=2, **bf), FAKE) == 1           # chunked: workspace missing
    assert call_bwd_varlen(prob(algo=1, **bf), FAKE) == 1           # sequential: workspace missing
    assert call_bwd_varlen(prob(algo=0, T=256), FAKE) == 1          # AUTO -> sequential


def test_binding_shape_checks():
    """The binding compares every operand's shape with the problem before it
    calls the library (which takes pointers and sizes only): a wrong head
    count, token count, gate shape or state shape raises ValueError."""
    import torch
    Bb, T, Hk, Hv, D = 2, 5, 2, 4, 16
    ok = dict(q=torch.zeros(Bb, T, Hk, D), k=torch.zeros(Bb, T, Hk, D), v=torch.zeros(Bb, T, Hv, D),
              g=torch.zeros(Bb, T, Hv), beta=torch.zeros(Bb, T, Hv), h0=torch.zeros(Bb, Hv, D, D),
              dout=torch.zeros(Bb, T, Hv, D), dht=None)
    B._check_shapes(Bb, T, Hk, Hv, D, D, Bb, False, ok)
    B._check_shapes(Bb, T, Hk, Hv, D, D, Bb, True, dict(ok, g=torch.zeros(Bb, T, Hv, D)))
    bad = [("k", torch.zeros(Bb, T, Hv, D)), ("v", torch.zeros(Bb, T - 1, Hv, D)),
           ("g", torch.zeros(Bb, T, Hv, D)), ("beta", torch.zeros(Bb, T, Hk)),
           ("h0", torch.zeros(Bb, Hk, D, D)), ("dout", torch.zeros(Bb, T, Hv, 2 * D)),
           ("dht", torch.zeros(1, Hv, D, D))]
    for name, t in bad:
        with pytest.raises(ValueError, match=name):
            B._check_shapes(Bb, T, Hk, Hv, D, D, Bb, False, dict(ok, **{name: t}))
    # ragged: tensors [1, rows, ...], N states
    rag = dict(ok, q=torch.zeros(1, 9, Hk, D), k=torch.zeros(1, 9, Hk, D), v=torch.zeros(1, 9, Hv, D),
               g=torch.zeros(1, 9, Hv), beta=torch.zeros(1, 9, Hv), dout=torch.zeros(1, 9, Hv, D),
               h0=torch.zeros(3, Hv, D, D))
    B._check_shapes(1, 9, Hk, Hv, D, D, 3, False, rag)
    with pytest.raises(ValueError, match="h0"):
        B._check_shapes(1, 9, Hk, Hv, D, D, 2, False, rag)


def keeps(p):
    n = ctypes.c_int(-1)
    st = B.lib().gdr_keeps_chunks(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,kept", [
    (dict(B=4, T=4096, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=0), 1),        # AUTO: chunked fp16
    (dict(B=4, T=4096, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=2, chunk_size=32), 1),
    (dict(B=1, T=64, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=0), 1),
    (dict(B=1, T=12, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=0), 1),          # AUTO's shortest chunked forward
    (dict(B=1, T=11, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=0), 0),          # AUTO picks sequential
    (dict(B=1, T=8, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=0), 0),
    (dict(B=1, T=512, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=1), 0),         # sequential
    (dict(B=1, T=512, Hk=2, Hv=4, Dk=128, Dv=128, io_dtype=0, algo=2), 0),           # fp32 io
    (dict(B=1, T=512, Hk=2, Hv=4, Dk=16, Dv=16, io_dtype=1, algo=2), 0),             # Dk = 16
    (dict(B=1, T=512, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=2, chunk_size=16), 0),
    (dict(B=1, T=512, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=2, flags=3), 0),  # channelwise
])
def test_keeps_chunks_query(kw, kept):
    for flags in (kw.get("flags", 1), kw.get("flags", 1) | 8):
        st, n = keeps(prob(**dict(kw, flags=flags)))
        assert st == 0 and n == kept


def test_keeps_chunks_query_validates():
    assert keeps(prob(Hv=3))[0] == 2
    assert B.lib().gdr_keeps_chunks(None, None) == 1
    p = prob()
    assert B.lib().gdr_keeps_chunks(ctypes.byref(p), None) == 1


def test_saved_chunks_only_where_kept():
    """Where the library ignores GDR_SAVE_CHUNKS, the forward with and without
    the flag needs the same workspace and the binding keeps nothing; where it
    honours it, the forward needs the backward's workspace."""
    # AUTO at T = 8 and 10: the forward runs the sequential kernels, the backward the chunked ones
    for kw in (dict(T=8, algo=0), dict(T=10, algo=0), dict(T=512, algo=1), dict(T=200, algo=2, io_dtype=0, Dk=128, Dv=128),
               dict(T=200, algo=2, flags=3, Dk=128, Dv=128, io_dtype=1)):
        base = dict(B=1, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, flags=1)
        base.update(kw)
        p0, p1 = prob(**base), prob(**dict(base, flags=base["flags"] | 8))
        assert keeps(p1) == (0, 0)
        assert fwd_ws(p0) == fwd_ws(p1)
        assert bwd_ws(p0) == bwd_ws(p1)
    p1 = prob(B=1, T=200, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, flags=9, algo=2)
    assert keeps(p1) == (0, 1)
    assert fwd_ws(p1) == bwd_ws(p1)
    assert fwd_ws(p1)[1] > fwd_ws(prob(B=1, T=200, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, flags=1, algo=2))[1]


def test_calib_entry_points_validate():
    lib = B.lib()
    fl = ctypes.c_double(0)
    assert lib.gdr_calib_copy(None, FAKE, 16, None) == 1
    assert lib.gdr_calib_copy(FAKE, FAKE + 16, 0, None) == 2
    assert lib.gdr_calib_copy(FAKE, FAKE + 16, 24, None) == 2
    assert lib.gdr_calib_copy(FAKE + 8, FAKE, 16, None) == 4
    assert lib.gdr_calib_mfma(None, 1, 1, ctypes.byref(fl), None) == 1
    assert lib.gdr_calib_mfma(FAKE, 0, 1, ctypes.byref(fl), None) == 2
    assert lib.gdr_calib_mfma(FAKE, 1, -1, ctypes.byref(fl), None) == 2
    assert lib.gdr_calib_mfma(FAKE + 4, 1, 1, ctypes.byref(fl), None) == 4


def test_noalloc_forward_validates_before_touching_the_device():
    """gdr_forward_noalloc refuses a problem beyond its fixed scratch and the
    GDR_SAVE_CHUNKS flag during validation (no device call is made)."""
    lib = B.lib()
    args = [FAKE] * 8 + [None]
    big = prob(B=8, T=4096, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype=1, algo=2)
    assert fwd_ws(big)[1] > (64 << 20)
    assert lib.gdr_forward_noalloc(ctypes.byref(big), *args) == 5
    assert lib.gdr_forward_noalloc(ctypes.byref(prob(flags=9)), *args) == 3
    assert lib.gdr_forward_noalloc(ctypes.byref(prob(Hv=3)), *args) == 2
    assert lib.gdr_forward_noalloc(None, *args) == 1
