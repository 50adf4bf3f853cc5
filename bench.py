"""Benchmark of the gated delta rule hot path on one MI355X.

One step = chunked forward + VJP (gdr_forward then gdr_backward, C = 64) over
a batch of B=4 sequences of T=4096 tokens, Hk=16, Hv=32, Dk=Dv=128, bf16
inputs, the backward sweep shape of the page "Adding VJP for gated delta
net" (ml-explore/mlx pull request 4565, "Performance").  Inputs are seeded
synthetic data resident in HBM before timing starts.  The decode path
(B=8, 256 single-token steps over 32 rotated state buffers) is measured in
the same run and reported under "decode".

Prints one JSON line.  `value` is fwd+bwd tokens/s; `roofline` is for the
kernel that takes the most time in the timed region (per-kernel durations
come from HIP events the library records around each launch);
`cpu_baseline` is the fp64 oracle timed on a bounded sample on the host.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0   # MI355X dense fp16/bf16 matrix cores, TFLOP/s
VALU_F32_PEAK_TFS = 157.3    # MI355X fp32 vector ALUs, TFLOP/s

B, T, HK, HV, D, C = 4, 4096, 16, 32, 128, 64
DEC_B, DEC_STEPS, DEC_BUFFERS = 8, 256, 32


# ---- algorithmic counts of the method (per (token, v-head)) ---------------
# FLOPs: every matrix product once at 2mnk, products used on one triangle of
# a C x C block at half.  Canonical step count (forward + VJP with one
# recompute of the chunk states and chunk operands, as a stateless VJP
# needs): F_fwd = 6d^2 + 5Cd + C^2/3, F_bwd = 16d^2 + 14Cd + C^2.
# Bytes: the method's own tensors (q, k, v, g, beta, o; dout, dq, dk, dv,
# dg, dbeta; bf16 rows, fp32 gates), each moved once, q/k rows shared by the
# grp v-heads of a k-head; intermediates a design chooses to materialise are
# never counted.  Per step that is 24,832 B/token for the forward and
# 41,472 B/token for the VJP at Hk=16, Hv=32, d=128, plus ht / dh0.


def canonical_flops_per_token_head(d=D, c=C):
    """F_fwd + F_bwd per (token, v-head)."""
    return (6 * d * d + 5 * c * d + c * c / 3) + (16 * d * d + 14 * c * d + c * c)


def algorithmic_bytes_per_token(d=D, hk=HK, hv=HV):
    """Minimum HBM bytes of one forward + VJP step per token (without the
    B * Hv * d^2 * 4 bytes of ht and of dh0)."""
    row_k, row_v, gates = hk * d * 2, hv * d * 2, hv * 4
    fwd = 2 * row_k + row_v + 2 * gates + row_v                       # q, k, v, g, beta -> o
    bwd = 2 * row_k + 2 * row_v + 2 * gates + 2 * row_k + row_v + 2 * gates  # q,k,v,do,g,beta -> dq,dk,dv,dg,dbeta
    return fwd + bwd


def kernel_share_per_token_head(name, d=D, c=C, grp=HV // HK):
    """(FLOPs, bytes) of the method that a kernel carries, per (token,
    v-head), summed over its launches in one step.  The canonical FLOPs are
    split by the step of the chunk algebra each kernel performs: prep forms
    A, P (2Cd) and T = (I + A)^-1 (C^2/3); a forward chain the inter-chunk
    products (6d^2 + 3Cd); the reverse chain dU, dRHS and the dH update
    (6d^2 + 3Cd); the gradient kernel the rest of F_bwd less the recompute
    (6d^2 + 8Cd + 2C^2/3).  Bytes are the method's tensors the kernel must
    read or write (q/k rows counted once per k-head group)."""
    kq = 2 * d * 2 / grp     # q and k rows (bf16), shared by the group
    row = d * 2              # one bf16 row of v / o / dout / dv
    gates = 8                # g and beta (fp32)
    prep_f = 2 * c * d + c * c / 3
    chain_f = 6 * d * d + 3 * c * d
    grad_f = 6 * d * d + 8 * c * d + 2 * c * c / 3
    return {
        "chunk_prep": (prep_f, kq + gates),
        "chunk_fwd": (chain_f, 2 * row),
        "chunk_fwd_save": (chain_f, 2 * row),
        "chunk_states": (4 * d * d + c * d, row),
        "chunk_dh": (chain_f, 2 * row),
        "chunk_grad": (grad_f, kq + 2 * row + gates + kq + gates),
    }.get(name)


def image_bytes(d=D, c=C):
    """Byte sizes of the per-chunk operand images the prep kernel writes (fp16
    tiles padded by 8 halves per row, fp32 gate vectors): key image (Kn | Qn)
    per (b, k-head, chunk) and chunk image (gates | T | P) per (b, v-head,
    chunk); forward and VJP read the same format."""
    kn, tm, gt = c * (d + 8) * 2, c * (c + 8) * 2, 4 * c * 4
    return {"KEY": 2 * kn, "CHK": gt + 2 * tm, "KN": kn, "TM": tm, "GT": gt}


def design_bytes_per_token_head(name, d=D, c=C, grp=HV // HK, saved=True):
    """HBM bytes each kernel of this design moves in one step, per (token,
    v-head), summed over its launches: what the kernel reads and writes once,
    including the intermediates the design materialises (operand images,
    fp16 chunk states, chunk-end gradients); k/q rows and key images shared
    by the `grp` v-heads of a k-head.  This is the design's own traffic, not
    the method's minimum (kernel_share_per_token_head).  chunk_prep runs once
    for the forward and, unless the forward saved its chunks for the VJP,
    once more for the VJP; chunk_grad covers a whole k-head group per
    workgroup (the key image once, both v-heads' chunk images, states, v and
    dout rows, dv rows; dq, dk written once); chunk_dh reads dout and writes
    the chunk-end gradients."""
    im = image_bytes(d, c)
    kq = 2 * d * 2 / grp     # k and q rows, bf16
    vec = d * 2              # one bf16 row of v / o / do
    gates = 8                # g and beta, fp32
    st = 2 * d * d / c       # one fp16 d x d state per chunk
    prep = kq + gates + im["KEY"] / (c * grp) + im["CHK"] / c
    return {
        "chunk_prep": (1 if saved else 2) * prep,
        "chunk_fwd": im["KEY"] / (c * grp) + im["CHK"] / c + 2 * vec,
        "chunk_fwd_save": im["KEY"] / (c * grp) + im["CHK"] / c + 2 * vec + st,
        "chunk_states": im["KN"] / (c * grp) + (im["GT"] + im["TM"]) / c + vec + st,
        "chunk_dh": im["KEY"] / (c * grp) + im["CHK"] / c + vec + st,
        "chunk_grad": im["KEY"] / (c * grp) + im["CHK"] / c + 2 * st + 3 * vec + gates + 2 * d * 2 / grp,
    }.get(name)


def stored_traffic(kernel):
    """HBM bytes per launch from the committed counter profile of this kernel,
    or None when there is none or the sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from gated_delta_rule_54_amd.profiling import src_digest
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or rec.get("src_digest") != src_digest():
        return None
    return ent["bytes_per_launch"]


def make_device_inputs(torch, seed, b, t, with_do=True, gate_preact=False):
    from gated_delta_rule_54_amd.synth import make_inputs
    x = make_inputs(seed, b, t, HK, HV, D, D, io_dtype="bf16", with_do=with_do, gate_preact=gate_preact)
    dev = torch.device("cuda")
    out = {}
    for n, a in x.items():
        if a is None:
            out[n] = None
            continue
        tt = torch.from_numpy(a).to(dev)
        out[n] = tt.to(torch.bfloat16) if n in ("q", "k", "v", "do") else tt
    return x, out


def bench_chunked(torch, gdr, steps, warmup, fused_gates=False, saved=True):
    """One step = chunked forward + VJP of the whole workload.  With saved
    the forward keeps its chunk images and chunk entry states for the VJP
    (GDR_SAVE_CHUNKS), else the VJP recomputes them.  With fused_gates the
    gates are passed as pre-activations (same draws) and activated inside
    the kernels."""
    _, t = make_device_inputs(torch, 2, B, T, gate_preact=fused_gates)
    kw = dict(algo="chunked", chunk_size=C, out_dtype=torch.bfloat16, fused_gates=fused_gates)

    def step():
        if saved:
            _, _, sv = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], None,
                                       save_for_backward=True, **kw)
            gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["do"], saved=sv, **kw)
        else:
            gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, **kw)
            gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["do"], **kw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    gdr.gdr_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kernels = gdr.gdr_profile_read()
    gdr.gdr_profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    return ms, wall, kernels


def bench_decode(torch, gdr, graph=True, legs=("rotated", "single_buffer_cache_warm")):
    """B=8 single-token steps, state updated in place, rotating over
    DEC_BUFFERS independent states so a step's 16 MiB state is not served
    from the 256 MB last-level cache.  Per step: the kernel time from the
    library's events around each launch (which include the launch's own
    dispatch), the host wall time, and the time per step of a HIP graph of
    all steps replayed once."""
    g = torch.Generator(device="cuda").manual_seed(1)
    sh = lambda *s: torch.randn(*s, device="cuda", generator=g)
    q = sh(DEC_STEPS, DEC_B, 1, HK, D).bfloat16()
    k = sh(DEC_STEPS, DEC_B, 1, HK, D).bfloat16()
    v = sh(DEC_STEPS, DEC_B, 1, HV, D).bfloat16()
    gg = -torch.nn.functional.softplus(sh(DEC_STEPS, DEC_B, 1, HV))
    bb = torch.sigmoid(sh(DEC_STEPS, DEC_B, 1, HV))
    states = [sh(DEC_B, HV, D, D) * 0.02 for _ in range(DEC_BUFFERS)]

    def run(n, buffers):
        for i in range(n):
            s = states[i % buffers]
            gdr.gdr_forward(q[i % DEC_STEPS], k[i % DEC_STEPS], v[i % DEC_STEPS], gg[i % DEC_STEPS],
                            bb[i % DEC_STEPS], s, ht=s, algo="sequential", out_dtype=torch.bfloat16)

    out = {}
    for label, buffers in (("rotated", DEC_BUFFERS), ("single_buffer_cache_warm", 1)):
        if label not in legs:
            continue
        run(32, buffers)
        torch.cuda.synchronize()
        gdr.gdr_profile_enable(True)
        w0 = time.perf_counter()
        run(DEC_STEPS, buffers)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        kt = gdr.gdr_profile_read()
        gdr.gdr_profile_enable(False)
        ms, n = kt["seq_fwd"]
        us = 1000.0 * ms / n
        state_bytes = 2 * DEC_B * HV * D * D * 4
        out[label] = {"launch_event_us_per_step": round(us, 3), "wall_us_per_step": round(1e6 * wall / DEC_STEPS, 2),
                      "launch_event_state_GBps": round(state_bytes / (us * 1e-6) / 1e9, 1),
                      "launch_event_frac_hbm_peak": round(state_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if not graph:
            continue
        # the same steps captured once into a HIP graph and replayed: no host
        # launch gaps and no per-kernel events
        graph_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_):
            run(DEC_STEPS, buffers)
        graph_.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph_.replay()
        e1.record()
        torch.cuda.synchronize()
        gus = 1000.0 * e0.elapsed_time(e1) / DEC_STEPS
        del graph_
        out[label].update({"graph_us_per_step": round(gus, 3),
                           "graph_state_GBps": round(state_bytes / (gus * 1e-6) / 1e9, 1),
                           "graph_frac_hbm_peak": round(state_bytes / (gus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    out["state_bytes_per_step"] = 2 * DEC_B * HV * D * D * 4
    out["note"] = ("launch_event_*: library HIP events around each launch, which include its dispatch; graph_*: "
                   "one replayed HIP graph of all steps, the closest to the kernel's own duration "
                   "(rocprofv3 kernel trace in profiles/)")
    out["config"] = f"B={DEC_B} Hk={HK} Hv={HV} Dk=Dv={D}, {DEC_STEPS} single-token steps, bf16 io, fp32 state"
    return out


def bench_channelwise(torch, gdr, reps=20):
    """Channelwise-gate prefill forward (per-channel g of shape [B, T, Hv, Dk])
    at B=1, Hk=16, Hv=32, D=128, bf16 io, zero h0, for T in {128, 512, 2048}:
    the chunked path (C=64) against the sequential one; time per call from
    events around `reps` back-to-back calls, plus the chunked kernels' own
    times; then the VJP of the same call, chunked against sequential."""
    from gated_delta_rule_54_amd.synth import make_inputs
    dev = torch.device("cuda")
    out = {}
    for t_len in (128, 512, 2048):
        x = make_inputs(7000 + t_len, 1, t_len, HK, HV, D, D, io_dtype="bf16", channelwise=True, with_do=False)
        t = {n: (None if a is None else torch.from_numpy(a).to(dev)) for n, a in x.items()}
        for n in ("q", "k", "v"):
            t[n] = t[n].to(torch.bfloat16)
        ent = {}
        for algo in ("sequential", "chunked"):
            kw = dict(algo=algo, channelwise=True, out_dtype=torch.bfloat16)
            if algo == "chunked":
                kw["chunk_size"] = C

            def call():
                gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, **kw)

            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = 1000.0 * e0.elapsed_time(e1) / reps
            ent[f"{algo}_us"] = round(us, 2)
            if algo == "chunked":  # a separate pass with the library's per-kernel events
                gdr.gdr_profile_enable(True)
                for _ in range(reps):
                    call()
                kt = gdr.gdr_profile_read()
                gdr.gdr_profile_enable(False)
                ent["chunked_kernels_us"] = {k: round(1000.0 * v[0] / v[1], 2) for k, v in kt.items()}
        ent["speedup"] = round(ent["sequential_us"] / ent["chunked_us"], 2)
        ent["chunked_tokens_per_s"] = round(t_len / (ent["chunked_us"] * 1e-6), 1)
        # the VJP of the same call (do ~ N(0, 1)), chunked against sequential
        do = torch.randn(t["v"].shape, device=dev, generator=torch.Generator(device=dev).manual_seed(t_len))
        do = do.to(torch.bfloat16)
        for algo in ("sequential", "chunked"):
            kw = dict(algo=algo, channelwise=True, out_dtype=torch.bfloat16)
            if algo == "chunked":
                kw["chunk_size"] = C

            def vjp():
                gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, do, **kw)

            vjp()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(2, reps // 4)
            e0.record()
            for _ in range(n):
                vjp()
            e1.record()
            torch.cuda.synchronize()
            ent[f"vjp_{algo}_us"] = round(1000.0 * e0.elapsed_time(e1) / n, 2)
        ent["vjp_speedup"] = round(ent["vjp_sequential_us"] / ent["vjp_chunked_us"], 2)
        out[f"T={t_len}"] = ent
    out["config"] = f"B=1 Hk={HK} Hv={HV} Dk=Dv={D}, channelwise gate, bf16 io, zero h0, chunk {C}"
    return out


def bench_vjp_sweep(torch, gdr):
    """The backward sweep of the page "Adding VJP for gated delta net"
    (ml-explore/mlx pull request 4565, "Performance"): B in {1, 4, 8} x T in
    {8, 64, 512, 4096}, Hk=16, Hv=32, D=128, bf16 io, h0 ~ N(0, 0.02),
    do ~ N(0, 1).
    The stateless VJP (gdr_backward alone, which recomputes what it needs),
    chunked (C=64) against sequential; time per call from events around
    back-to-back calls.  Inputs drawn on the device with the same
    distributions as the other legs."""
    gen = torch.Generator(device="cuda").manual_seed(5)
    bmax, tmax = 8, 4096
    rn = lambda *s: torch.randn(*s, device="cuda", generator=gen)
    full = {"q": rn(bmax, tmax, HK, D).bfloat16(), "k": rn(bmax, tmax, HK, D).bfloat16(),
            "v": rn(bmax, tmax, HV, D).bfloat16(), "do": rn(bmax, tmax, HV, D).bfloat16(),
            "g": -torch.nn.functional.softplus(rn(bmax, tmax, HV)), "beta": torch.sigmoid(rn(bmax, tmax, HV)),
            "h0": rn(bmax, HV, D, D) * 0.02}
    out = {}
    for b in (1, 4, 8):
        for t_len in (8, 64, 512, 4096):
            t = {n: (a[:b] if n == "h0" else a[:b, :t_len]).contiguous() for n, a in full.items()}
            ent = {}
            for algo in ("sequential", "chunked"):
                kw = dict(algo=algo, out_dtype=torch.bfloat16)
                if algo == "chunked":
                    kw["chunk_size"] = C

                def vjp():
                    gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], t["do"], **kw)

                vjp()
                torch.cuda.synchronize()
                reps = 2 if (algo == "sequential" and t_len >= 512) else 10
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    vjp()
                e1.record()
                torch.cuda.synchronize()
                ent[f"{algo}_us"] = round(1000.0 * e0.elapsed_time(e1) / reps, 2)
            ent["chunked_tokens_per_s"] = round(b * t_len / (ent["chunked_us"] * 1e-6), 1)
            ent["speedup"] = round(ent["sequential_us"] / ent["chunked_us"], 2)
            # the chunked VJP against both roofs: the canonical VJP count
            # (16d^2 + 14Cd + C^2 per token-head, one recompute of the chunk
            # states included) and the algorithmic bytes of its kernels
            th = b * t_len * HV
            sec = ent["chunked_us"] * 1e-6
            cc = min(C, t_len)
            ent["chunked_TFLOPs"] = round((16 * D * D + 14 * cc * D + cc * cc) * th / sec / 1e12, 2)
            ent["chunked_frac_mfma"] = round(ent["chunked_TFLOPs"] / MFMA_F16_PEAK_TFS, 4)
            # the VJP's minimum I/O: q, k, v, dout, g, beta in; dq, dk, dv,
            # dg, dbeta out (41,472 B per token here), plus h0 and dh0
            vjp_bytes = (4 * HK * D * 2 + 2 * HV * D * 2 + 4 * HV * 4 + HV * D * 2) * b * t_len \
                + 2 * b * HV * D * D * 4
            ent["chunked_frac_hbm"] = round(vjp_bytes / sec / 1e9 / HBM_PEAK_GBS, 4)
            # the sequential VJP on the fp32 vector ALUs: about 22 d^2 FLOPs per
            # token-head (forward replay, reverse step, checkpoint pass)
            ent["sequential_TFLOPs"] = round(22 * D * D * th / (ent["sequential_us"] * 1e-6) / 1e12, 3)
            ent["sequential_frac_valu"] = round(ent["sequential_TFLOPs"] / VALU_F32_PEAK_TFS, 4)
            out[f"B={b},T={t_len}"] = ent
            del t
    out["config"] = (f"Hk={HK} Hv={HV} Dk=Dv={D}, bf16 io, scalar gate, h0 ~ N(0, 0.02), chunk {C}; "
                     "stateless VJP, sequential against chunked; chunked_frac_* against the fp16 MFMA and "
                     "HBM peaks, sequential_frac_valu against the fp32 vector-ALU peak")
    return out


def bench_channelwise_decode(torch, gdr, t_prefill=2048, steps=128):
    """Channelwise gate: a B=1 prefill of t_prefill tokens (chunked), then
    `steps` single-token steps carrying the state in place (Hk=16, Hv=32,
    D=128, bf16 io).  The 2 MiB state stays in the last-level cache between
    steps, so the per-step figure is cache-warm."""
    from gated_delta_rule_54_amd.synth import make_inputs
    dev = torch.device("cuda")
    x = make_inputs(9000 + t_prefill, 1, t_prefill + steps, HK, HV, D, D, io_dtype="bf16", channelwise=True,
                    with_do=False)
    t = {n: (None if a is None else torch.from_numpy(a).to(dev)) for n, a in x.items()}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    sl = lambda a, i, j: a[:, i:j].contiguous()
    _, state = gdr.gdr_forward(sl(t["q"], 0, t_prefill), sl(t["k"], 0, t_prefill), sl(t["v"], 0, t_prefill),
                               sl(t["g"], 0, t_prefill), sl(t["beta"], 0, t_prefill), None, algo="chunked",
                               chunk_size=C, channelwise=True, out_dtype=torch.bfloat16)
    toks = [{n: sl(t[n], t_prefill + i, t_prefill + i + 1) for n in ("q", "k", "v", "g", "beta")}
            for i in range(steps)]

    def run():
        for z in toks:
            gdr.gdr_forward(z["q"], z["k"], z["v"], z["g"], z["beta"], state, ht=state, algo="sequential",
                            channelwise=True, out_dtype=torch.bfloat16)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / steps
    graph = torch.cuda.CUDAGraph()  # the same steps as one replayed HIP graph (no host launch gaps)
    with torch.cuda.graph(graph):
        run()
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    gus = 1000.0 * e0.elapsed_time(e1) / steps
    del graph
    state_bytes = 2 * HV * D * D * 4
    return {"us_per_step": round(us, 3), "graph_us_per_step": round(gus, 3),
            "graph_state_GBps_cache_warm": round(state_bytes / (gus * 1e-6) / 1e9, 1),
            "config": f"B=1 Hk={HK} Hv={HV} Dk=Dv={D}, channelwise gate, chunked prefill of {t_prefill} tokens "
                      f"then {steps} single-token steps in place (events around back-to-back calls, and one "
                      "replayed HIP graph of the steps)"}


def ragged_lengths(seed=11, total=B * T, lo=128, hi=2048):
    """A prefill batch of prompts of unequal length: lengths uniform in
    [lo, hi] (seeded) until their sum reaches `total` tokens (the last one
    trimmed)."""
    rng = np.random.default_rng(seed)
    out, s = [], 0
    while s < total:
        n = int(min(rng.integers(lo, hi + 1), total - s))
        out.append(n)
        s += n
    return out


def bench_ragged(torch, gdr, reps=10):
    """Fwd + VJP (forward saving its chunks) of a ragged batch with the same
    16,384 tokens as the headline workload (Hk=16, Hv=32, D=128, bf16,
    C=64, zero h0), against the same sequences zero-padded to the longest
    one as a uniform batch (gdr_forward / gdr_backward)."""
    from gated_delta_rule_54_amd.synth import make_inputs
    lens = ragged_lengths()
    n, rows, tmax = len(lens), sum(lens), max(lens)
    x = make_inputs(8, 1, rows, HK, HV, D, D, io_dtype="bf16")
    dev = torch.device("cuda")
    t = {k: (None if a is None else torch.from_numpy(a).to(dev)) for k, a in x.items()}
    for k in ("q", "k", "v", "do"):
        t[k] = t[k].to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev)
    kw = dict(algo="chunked", chunk_size=C, out_dtype=torch.bfloat16)

    def ragged():
        _, _, sv = gdr.gdr_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, save_for_backward=True,
                                   cu_seqlens=cu, max_seqlen=tmax, **kw)
        gdr.gdr_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["do"], saved=sv, cu_seqlens=cu,
                         max_seqlen=tmax, **kw)

    pad = {}
    for k, a in t.items():
        if a is None:
            continue
        z = torch.zeros((n, tmax) + tuple(a.shape[2:]), dtype=a.dtype, device=dev)
        for i in range(n):
            z[i, :lens[i]] = a[0, int(cu[i]):int(cu[i + 1])]
        pad[k] = z

    def padded():
        _, _, sv = gdr.gdr_forward(pad["q"], pad["k"], pad["v"], pad["g"], pad["beta"], None,
                                   save_for_backward=True, **kw)
        gdr.gdr_backward(pad["q"], pad["k"], pad["v"], pad["g"], pad["beta"], None, pad["do"], saved=sv, **kw)

    out = {}
    for name, fn in (("ragged", ragged), ("padded", padded)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(rows / (ms * 1e-3), 1)}
    out["config"] = (f"{n} sequences, lengths U[128, 2048] (seed 11), {rows} tokens, longest {tmax}; "
                     f"Hk={HK} Hv={HV} D={D} bf16, C={C}, fwd saving chunks + VJP; padded = the same "
                     f"sequences zero-padded to {tmax} as a uniform batch")
    return out


_GROUP_INPUTS = None  # the workload's host inputs, shared with forked workers


def _oracle_group(i):
    """fp64 oracle forward + VJP of (b, k-head) group i of the workload (its
    Hv/Hk v-heads over the full length) on one thread; returns seconds."""
    from threadpoolctl import threadpool_limits
    from oracle import gdr_oracle as orc
    x, grp = _GROUP_INPUTS, HV // HK
    b, kh = divmod(i, HK)
    sl = lambda a, h0, h1: np.ascontiguousarray(a[b:b + 1, :, h0:h1])
    q, k = sl(x["q"], kh, kh + 1), sl(x["k"], kh, kh + 1)
    v, do = sl(x["v"], grp * kh, grp * kh + grp), sl(x["do"], grp * kh, grp * kh + grp)
    g, beta = sl(x["g"], grp * kh, grp * kh + grp), sl(x["beta"], grp * kh, grp * kh + grp)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        orc.forward(q, k, v, g, beta)
        orc.backward(q, k, v, g, beta, None, do)
        return time.perf_counter() - t0


def host_cpu_share():
    """Worker processes for the oracle: the CPUs this process may run on,
    at most 16 (the host share that goes with one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_pool():
    """The oracle's worker processes, one per host CPU of this GPU's share,
    forked before anything touches the GPU (they inherit the workload's
    inputs).  They wait idle until cpu_baseline hands them work after the
    GPU legs: the workers hold about 1 GB of fp64 states each, and freeing
    that much memory stalls the host for seconds, which would starve the
    GPU of launches if any timing followed."""
    import multiprocessing as mp
    from gated_delta_rule_54_amd.synth import make_inputs
    global _GROUP_INPUTS
    _GROUP_INPUTS = make_inputs(2, B, T, HK, HV, D, D, io_dtype="bf16")
    cores = host_cpu_share()
    return mp.get_context("fork").Pool(cores), cores


def cpu_baseline(pool, cores):
    """The fp64 oracle (forward + VJP, numpy, one BLAS thread per process)
    timed on the host: a sample of the headline workload's (b, k-head)
    groups (each = the Hv/Hk v-heads of one k-head over all T tokens), one
    group per worker process of oracle_pool, all workers at once;
    whole-workload tokens/s from the sample's wall time.  Also the oracle's
    single-thread seconds on the tiny case (B=1, T=64, Hk=Hv=2, D=16, fp32,
    fwd + VJP) and on the decode case (B=8, Hk=16, Hv=32, D=128, 256 tokens,
    forward)."""
    from threadpoolctl import threadpool_limits
    from gated_delta_rule_54_amd.synth import make_inputs
    from oracle import gdr_oracle as orc
    global _GROUP_INPUTS
    n_groups = B * HK
    sample = min(n_groups, cores)
    try:
        w0 = time.perf_counter()
        secs = pool.map(_oracle_group, range(sample), chunksize=1)
        wall = time.perf_counter() - w0
    finally:
        pool.terminate()
        pool.join()
    _GROUP_INPUTS = None
    whole = wall * n_groups / sample  # the sample is one round of the pool
    single = {}
    with threadpool_limits(limits=1):
        x = make_inputs(0, 1, 64, 2, 2, 16, 16, io_dtype="f32")
        t0 = time.perf_counter()
        orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
        orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, x["do"])
        single["tiny_fwd_vjp_B1_T64_D16_s"] = round(time.perf_counter() - t0, 4)
        x = make_inputs(1, 8, 256, HK, HV, D, D, io_dtype="bf16", h0_std=0.02, with_do=False)
        t0 = time.perf_counter()
        orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
        single["decode_B8_256_steps_fwd_s"] = round(time.perf_counter() - t0, 3)
    return {"value": round(B * T / whole, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample} of the {n_groups} (b, k-head) groups of B={B}, T={T}, Hk={HK}, Hv={HV}, D={D} "
                      f"(each {HV // HK} v-heads x {T} tokens, fwd + VJP in fp64 numpy), one per worker process, "
                      f"all at once: {wall:.1f} s wall, {sum(secs):.1f} CPU-s; whole workload = wall x "
                      f"{n_groups}/{sample}",
            "cpu_model": _cpu_model(), "host_threads": os.cpu_count(), "single_thread": single}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def variants(torch, gdr, args, tokens):
    """The other measured legs: the same step with fused gates and with the
    stateless VJP, the channelwise prefill and decode, the ragged prefill and
    the backward sweep."""
    fms, _, _ = bench_chunked(torch, gdr, args.steps, args.warmup, fused_gates=True)
    sms, _, skern = bench_chunked(torch, gdr, args.steps, args.warmup, saved=False)
    return {
        "fused_gates": {"ms_per_step": round(fms, 4), "tokens_per_s": round(tokens / (fms * 1e-3), 1),
                        "note": "same step with g, beta passed as pre-activations"},
        "stateless_vjp": {"ms_per_step": round(sms, 4), "tokens_per_s": round(tokens / (sms * 1e-3), 1),
                          "kernels_avg_us": {k: round(1000 * v[0] / v[1], 2) for k, v in skern.items()},
                          "note": "same step without GDR_SAVE_CHUNKS: the VJP recomputes the chunk "
                                  "images and chunk states"},
        "channelwise_prefill": bench_channelwise(torch, gdr),
        "channelwise_decode": bench_channelwise_decode(torch, gdr),
        "ragged_prefill": bench_ragged(torch, gdr),
        "vjp_sweep": bench_vjp_sweep(torch, gdr),
    }


def calibration(torch, gdr):
    """Measured ceilings of this GPU (include/gdr_calib.h): a streaming copy
    of 16 MiB (the same buffers every call: partly served by the last-level
    cache), of 16 MiB rotating over 32 buffer pairs (the decode step's
    traffic shape, from HBM) and of 512 MiB (HBM), read + write bytes per
    second from the library's events around each launch; and a loop of
    independent fp16 16x16x32 matrix-core products on register operands
    (enough waves to fill every SIMD)."""
    out = {}
    for mib, reps in ((16, 50), (512, 10)):
        n = mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            gdr.gdr_calib_copy(src, dst)
        torch.cuda.synchronize()
        gdr.gdr_profile_enable(True)
        for _ in range(reps):
            gdr.gdr_calib_copy(src, dst)
        ms, cnt = gdr.gdr_profile_read()["calib_copy"]
        gdr.gdr_profile_enable(False)
        us = 1000.0 * ms / cnt
        out[f"copy_{mib}MiB"] = {"us": round(us, 2), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1),
                                 "frac_hbm_peak": round(2 * n / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del src, dst
    # the decode step's traffic shape: 16 MiB read + 16 MiB written per
    # launch, rotating over 32 buffer pairs (1 GiB, beyond the last-level
    # cache) as the decode leg rotates its states
    n = 16 << 20
    bufs = [(torch.ones(n // 4, dtype=torch.float32, device="cuda"),
             torch.empty(n // 4, dtype=torch.float32, device="cuda")) for _ in range(DEC_BUFFERS)]
    for sb, db in bufs:
        gdr.gdr_calib_copy(sb, db)
    torch.cuda.synchronize()
    gdr.gdr_profile_enable(True)
    for i in range(DEC_STEPS):
        gdr.gdr_calib_copy(*bufs[i % DEC_BUFFERS])
    ms, cnt = gdr.gdr_profile_read()["calib_copy"]
    gdr.gdr_profile_enable(False)
    us = 1000.0 * ms / cnt
    out["copy_16MiB_rotated_32"] = {"us": round(us, 2), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1),
                                    "frac_hbm_peak": round(2 * n / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del bufs
    wgs, iters = 4096, 4096
    buf = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    gdr.gdr_calib_mfma(buf, wgs, 64)
    torch.cuda.synchronize()
    gdr.gdr_profile_enable(True)
    flops = gdr.gdr_calib_mfma(buf, wgs, iters)
    ms, _ = gdr.gdr_profile_read()["calib_mfma"]
    gdr.gdr_profile_enable(False)
    tfs = flops / (ms * 1e-3) / 1e12
    out["mfma_f16_16x16x32"] = {"us": round(1000 * ms, 1), "TFLOPs": round(tfs, 1),
                                "frac_mfma_peak": round(tfs / MFMA_F16_PEAK_TFS, 4),
                                "launch": f"{wgs} workgroups x 256 threads, {iters} rounds of 8 products"}
    out["note"] = ("library events around each launch; the rocprofv3 kernel trace of the same kernels is in "
                   "profiles/")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="time only the headline step (no fused-gate, stateless, channelwise or ragged legs)")
    ap.add_argument("--only-decode", action="store_true",
                    help="run only the decode leg (for counter runs of the decode kernel)")
    ap.add_argument("--only-calibration", action="store_true",
                    help="run only the calibration leg (copy and matrix-core ceilings)")
    ap.add_argument("--no-graph", action="store_true", help="decode leg without the replayed HIP graph")
    ap.add_argument("--decode-rotated-only", action="store_true",
                    help="decode leg: only the rotated (HBM) steps, so that a kernel trace holds those alone")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy this many MiB once with a plain elementwise kernel "
                         "(reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    # the oracle's worker pool is forked before anything touches the GPU and
    # given its work after the last GPU leg
    pool = None
    if not (args.no_cpu_baseline or args.only_decode or args.only_calibration):
        pool = oracle_pool()

    import torch
    import gated_delta_rule_54_amd as gdr
    gdr.lib()  # fail loudly if the library was not built

    if args.only_decode:
        legs = ("rotated",) if args.decode_rotated_only else ("rotated", "single_buffer_cache_warm")
        print(json.dumps({"decode": bench_decode(torch, gdr, graph=not args.no_graph, legs=legs)}), flush=True)
        copy_calibration(torch, args.copy_calibration_mib)
        return
    if args.only_calibration:
        print(json.dumps({"calibration": calibration(torch, gdr)}), flush=True)
        return
    ms, wall, kernels = bench_chunked(torch, gdr, args.steps, args.warmup)
    tokens = B * T
    th = B * T * HV
    per_kernel = {}
    for name, (tot, n) in kernels.items():
        avg_ms = tot / n
        ent = {"avg_us": round(1000 * avg_ms, 2), "launches_per_step": n / args.steps,
               "share_of_step": round(tot / args.steps / ms, 4)}
        units = th / (n / args.steps)  # (token, v-head) units one launch processes
        share = kernel_share_per_token_head(name)
        if share is not None:
            ent["alg_TFLOPs"] = round(share[0] * units / (avg_ms * 1e-3) / 1e12, 2)
            ent["alg_GBps"] = round(share[1] * units / (avg_ms * 1e-3) / 1e9, 1)
        db = design_bytes_per_token_head(name)
        if db is not None:
            ent["design_GBps"] = round(db * units / (avg_ms * 1e-3) / 1e9, 1)
        per_kernel[name] = ent
    # roofline of the kernel with the largest share of the step, on the
    # method's algorithmic FLOPs and bytes that kernel carries
    dom = max(kernels, key=lambda n: kernels[n][0])
    avg_s = kernels[dom][0] / kernels[dom][1] * 1e-3
    units = th / (kernels[dom][1] / args.steps)
    fl, by = kernel_share_per_token_head(dom)
    f_launch, b_launch = fl * units, by * units
    cands = [{"bound": "mfma", "achieved": round(f_launch / avg_s / 1e12, 2), "peak": MFMA_F16_PEAK_TFS,
              "unit": "TFLOP/s", "frac": round(f_launch / avg_s / 1e12 / MFMA_F16_PEAK_TFS, 4)},
             {"bound": "hbm", "achieved": round(b_launch / avg_s / 1e9, 1), "peak": HBM_PEAK_GBS,
              "unit": "GB/s", "frac": round(b_launch / avg_s / 1e9 / HBM_PEAK_GBS, 4)}]
    roof = max(cands, key=lambda r: r["frac"])  # the roof the kernel is closest to
    roof["kernel"] = dom
    roof["avg_us"] = round(avg_s * 1e6, 2)
    roof["units_per_launch"] = int(units)
    roof["alg_flops_per_launch"] = int(f_launch)
    roof["alg_bytes_per_launch"] = int(b_launch)
    roof["other_roof"] = [c for c in cands if c is not roof][0]
    grids = {"chunk_prep": ((T // C, HV, B), 512), "chunk_fwd_save": ((2 * HV * B, 1, 1), 320),
             "chunk_fwd": ((2 * HV * B, 1, 1), 320), "chunk_states": ((2 * HV * B, 1, 1), 320),
             "chunk_dh": ((2 * HV * B, 1, 1), 320), "chunk_grad": ((T // C, HK, B), 512)}
    if dom in grids:  # to find the same launches in a rocprofv3 kernel trace
        (gx, gy, gz), th_ = grids[dom]
        roof["launch"] = f"{gx} x {gy} x {gz} workgroups x {th_} threads"
    roof["traffic"] = stored_traffic(dom)
    roof["traffic_over_algorithmic"] = (None if roof["traffic"] is None
                                        else round(roof["traffic"] / b_launch, 3))
    canon = canonical_flops_per_token_head() * th
    alg_bytes = algorithmic_bytes_per_token() * tokens + 2 * B * HV * D * D * 4  # + ht, dh0
    sec = ms * 1e-3
    line = {
        "metric": "fwd+bwd tokens/s at B=4,T=4096,Hv=32,D=128; decode state GB/s vs HBM peak",
        "value": round(tokens / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded numpy PCG64; q,k,v,do ~ N(0,1) in bf16, g=-softplus(N(0,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "chunked gated delta rule forward + VJP", "B": B, "T": T, "Hk": HK, "Hv": HV,
                   "Dk": D, "Dv": D, "chunk": C, "io": "bf16", "matrix_core_operands": "f16",
                   "accumulate_and_state": "f32", "use_qk_l2norm": True, "gate": "scalar",
                   "vjp_inputs": "forward saves chunk images and chunk states (GDR_SAVE_CHUNKS)",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "path": {"canonical_flops_per_step": int(canon),
                 "canonical_TFLOPs": round(canon / sec / 1e12, 2),
                 "canonical_frac_mfma": round(canon / sec / 1e12 / MFMA_F16_PEAK_TFS, 4),
                 "alg_bytes_per_step": int(alg_bytes),
                 "alg_GBps": round(alg_bytes / sec / 1e9, 1),
                 "alg_frac_hbm": round(alg_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                 "combined_roofline_frac": round(max(canon / (MFMA_F16_PEAK_TFS * 1e12),
                                                     alg_bytes / (HBM_PEAK_GBS * 1e9)) / sec, 4),
                 "wall_ms_per_step": round(1000 * wall / args.steps, 3)},
        "kernels": per_kernel,
    }
    if args.no_variants:
        line["variants"] = None
    else:
        line["variants"] = variants(torch, gdr, args, tokens)
    if not args.no_decode:
        line["decode"] = bench_decode(torch, gdr, graph=not args.no_graph)
    if not args.no_calibration:
        line["calibration"] = calibration(torch, gdr)
    line["cpu_baseline"] = cpu_baseline(*pool) if pool is not None else None
    print(json.dumps(line), flush=True)
    copy_calibration(torch, args.copy_calibration_mib)


def copy_calibration(torch, mib):
    """One copy of `mib` MiB with the library's streaming copy kernel
    (gdr_calib_copy: each byte read once and written once), the reference
    the HBM byte counters of a profiled run are scaled by."""
    if not mib:
        return
    import gated_delta_rule_54_amd as gdr
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    gdr.gdr_calib_copy(src, dst)
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
