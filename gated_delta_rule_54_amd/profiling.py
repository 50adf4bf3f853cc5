"""Per-kernel HBM traffic of a bench.py run, from rocprofv3 counter databases.

Two profiled runs of the same command,

    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o f -- python3 bench.py --steps 1 --warmup 1 \\
        --no-decode --no-cpu-baseline --copy-calibration-mib 256
    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o w -- python3 bench.py ... (same flags)

give, per dispatch, the KiB the L2 read from and wrote to memory.  The last
kernels of that command are a plain elementwise copy of a known size
(``--copy-calibration-mib``), which moves exactly that many bytes each way;
the ratio of its counters to its size is the calibration factor the kernel
figures are divided by.  Then

    python -m gated_delta_rule_54_amd.profiling traffic DIR_F/f_results.db DIR_W/w_results.db \\
        --copy-mib 256 --json profiles/traffic.json --md profiles/<name>.md

writes the per-launch bytes of each library kernel (keyed by the names the
library's own event timing uses) together with a digest of the kernel
sources; bench.py reports the dominant kernel's figure only while that
digest matches.

    python -m gated_delta_rule_54_amd.profiling trace KT_results.db --md profiles/<name>.md

summarises a ``rocprofv3 --kernel-trace --stats`` database (per-kernel calls,
total and average duration), and

    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_F32 \
        SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -d DIR_M -o m -- python3 bench.py ...
    python -m gated_delta_rule_54_amd.profiling mfma DIR_M/m_results.db --md profiles/<name>.md

the matrix-core busy fraction and executed matrix-core FLOPs per launch.

and two runs of the same command with the wave-state counters (at most
eight SQ counters a run)

    rocprofv3 --pmc SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU \
        SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_SCA -d DIR_S1 -o s -- python3 bench.py ...
    rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_MFMA SQ_INSTS_SALU SQ_LDS_BANK_CONFLICT \
        SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -d DIR_S2 -o s -- python3 bench.py ...
    python -m gated_delta_rule_54_amd.profiling sq DIR_S1/s_results.db DIR_S2/s_results.db --md profiles/<name>.md

give each kernel's wave time split by what its waves were doing.
"""

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3

_HERE = os.path.dirname(os.path.abspath(__file__))

# demangled kernel name pattern -> library timing name
KERNELS = [
    (r"cwprep16_kernel", "chunk_prep_cw"),
    (r"cwchain16_kernel<\d+, [^,]+, true, false(?:, \d+)?>", "chunk_fwd_cw"),
    (r"cwchain16_kernel<\d+, [^,]+, false, true(?:, \d+)?>", "chunk_states_cw"),
    (r"cwdh16_kernel", "chunk_dh_cw"),
    (r"cwgrad16_kernel", "chunk_grad_cw"),
    (r"prep16_kernel", "chunk_prep"),
    (r"chain16_kernel<\d+, [^,]+, true, false(?:, \d+)?>", "chunk_fwd"),
    (r"chain16_kernel<\d+, [^,]+, true, true(?:, \d+)?>", "chunk_fwd_save"),
    (r"chain16_kernel<\d+, [^,]+, false, true(?:, \d+)?>", "chunk_states"),
    (r"dh16_kernel", "chunk_dh"),
    (r"grad16_kernel", "chunk_grad"),
    (r"epilogue128_kernel", "bwd_epilogue"),
    (r"seq_bwd_kernel", "seq_bwd"),
    (r"seq_fwd_kernel", "seq_fwd"),
    (r"decode_kernel", "decode"),
    (r"calib_copy_kernel", "calib_copy"),
    (r"calib_mfma_kernel", "calib_mfma"),
]
COPY_PATTERN = r"calib_copy_kernel"


def src_digest():
    """Digest of the kernel sources (same definition as bench.py's)."""
    h = hashlib.sha256()
    csrc = os.path.join(_HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def per_dispatch(db, counter):
    """{dispatch_id: (kernel name, summed counter value)} for one counter."""
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, name, counter_value from pmc_events where counter_name = ?",
                       (counter,)).fetchall()
    out = {}
    for did, name, v in rows:
        n, s = out.get(did, (name, 0.0))
        out[did] = (n, s + float(v))
    return out


def label(name):
    if re.search(COPY_PATTERN, name):
        return "copy"
    for pat, lab in KERNELS:
        if re.search(pat, name):
            return lab
    return None


def per_kernel(db, counter):
    """{label: (mean KiB per launch, launches)} over the dispatches of each
    kernel; for the calibration copy, its largest dispatch (the command may
    run small elementwise kernels of the same name for its inputs)."""
    acc = collections.defaultdict(list)
    for name, v in per_dispatch(db, counter).values():
        lab = label(name)
        if lab is not None:
            acc[lab].append(v)
    return {k: ((max(v), 1) if k == "copy" else (sum(v) / len(v), len(v))) for k, v in acc.items()}


def traffic(args):
    fetch = per_kernel(args.fetch_db, "FETCH_SIZE")
    write = per_kernel(args.write_db, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the calibration copy kernel was not found in the databases")
    size_kib = args.copy_mib * 1024.0
    f_scale = fetch["copy"][0] / size_kib
    w_scale = write["copy"][0] / size_kib
    kernels = {}
    for lab in sorted(set(fetch) | set(write)):
        if lab == "copy" or lab not in fetch or lab not in write:
            continue
        fb = fetch[lab][0] * 1024.0 / f_scale
        wb = write[lab][0] * 1024.0 / w_scale
        kernels[lab] = {"fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
                        "bytes_per_launch": int(fb + wb), "launches": fetch[lab][1]}
    rec = {"src_digest": src_digest(),
           "calibration": {"copy_mib": args.copy_mib, "fetch_factor": round(f_scale, 4),
                           "write_factor": round(w_scale, 4)},
           "kernels": kernels}
    with open(args.json, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    if args.md:
        lines = ["# HBM traffic per kernel launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", ""]
        if args.command:
            lines += ["Commands (from the repository root on one MI355X, library built):", "", "```", args.command,
                      "```", ""]
        lines += [f"Calibration: a {args.copy_mib:g} MiB elementwise copy read {f_scale:.4f}x and wrote "
                  f"{w_scale:.4f}x its size by these counters; the figures below are divided by those "
                  "factors.", "",
                  "| kernel | launches | fetch MB/launch | write MB/launch | total MB/launch |",
                  "|---|---:|---:|---:|---:|"]
        for lab, k in kernels.items():
            lines.append(f"| {lab} | {k['launches']} | {k['fetch_bytes_per_launch'] / 1e6:.1f} | "
                         f"{k['write_bytes_per_launch'] / 1e6:.1f} | {k['bytes_per_launch'] / 1e6:.1f} |")
        lines += ["", f"Kernel sources digest: `{rec['src_digest']}`", ""]
        with open(args.md, "w") as fh:
            fh.write("\n".join(lines))
    print(json.dumps(rec))


def mfma(args):
    """Matrix-core use per kernel launch from one counter run with
    SQ_INSTS_VALU_MFMA_MOPS_F16, SQ_INSTS_VALU_MFMA_MOPS_F32 (units of 512
    FLOPs, summed over shader engines), SQ_VALU_MFMA_BUSY_CYCLES (summed over
    SIMDs) and GRBM_GUI_ACTIVE (GPU busy cycles, the same on every XCD: the
    largest is taken).  Busy fraction = MFMA busy cycles / (GPU busy cycles x
    SIMDs), the definition of rocprofv3's derived MfmaUtil counter."""
    con = sqlite3.connect(args.db)
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    names, durs = {}, {}
    for did, name, cn, cv, dur in con.execute(
            "select dispatch_id, name, counter_name, counter_value, duration from pmc_events"):
        per[did][cn].append(float(cv))
        names[did], durs[did] = name, float(dur)
    acc = collections.defaultdict(list)
    for did, x in per.items():
        lab = label(names[did])
        if lab is None or lab == "copy" or not x.get("GRBM_GUI_ACTIVE"):
            continue
        gui = max(x["GRBM_GUI_ACTIVE"])
        busy = sum(x.get("SQ_VALU_MFMA_BUSY_CYCLES", [0.0]))
        f16 = 512.0 * sum(x.get("SQ_INSTS_VALU_MFMA_MOPS_F16", [0.0]))
        f32 = 512.0 * sum(x.get("SQ_INSTS_VALU_MFMA_MOPS_F32", [0.0]))
        acc[lab].append((busy / (gui * args.simds), f16, f32, durs[did]))
    lines = ["# Matrix-core use per kernel launch (rocprofv3 counters)", ""]
    if args.command:
        lines += ["Command (from the repository root on one MI355X, library built):", "", "```", args.command, "```",
                  ""]
    lines += [f"Busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x {args.simds} SIMDs).  FLOPs = executed "
              "matrix-core FLOPs (MOPS counters x 512), including the zero padding of partial tiles.  "
              "Rate = FLOPs / counter-run duration (the counter run serialises launches).", "",
              "| kernel | launches | MFMA busy | fp16 GFLOP/launch | fp32 GFLOP/launch | duration us | "
              "fp16+fp32 TFLOP/s |", "|---|---:|---:|---:|---:|---:|---:|"]
    for lab in sorted(acc):
        v = acc[lab]
        n = len(v)
        busy, f16, f32, dur = (sum(e[i] for e in v) / n for i in range(4))
        lines.append(f"| {lab} | {n} | {100 * busy:.1f}% | {f16 / 1e9:.2f} | {f32 / 1e9:.2f} | "
                     f"{dur / 1000.0:.1f} | {(f16 + f32) / dur / 1e3:.1f} |")
    lines += ["", f"Kernel sources digest: `{src_digest()}`", ""]
    text = "\n".join(lines)
    if args.md:
        with open(args.md, "w") as fh:
            fh.write(text)
    print(text)


def sq(args):
    """Wave-state shares per kernel from SQ counter runs: each counter is
    summed over the dispatch's counter instances and averaged over the
    kernel's launches; the cycle counters share one unit (quad-cycles), so
    ACTIVE_INST_* and WAIT_* over SQ_WAVE_CYCLES are the fractions of the
    waves' resident time spent issuing that kind of instruction or waiting
    (on memory, LDS or a barrier: WAIT_ANY; for an issue slot:
    WAIT_INST_ANY).  The instruction counts are per launch."""
    vals = collections.defaultdict(dict)
    for db in args.dbs:
        con = sqlite3.connect(db)
        for (cn,) in con.execute("select distinct counter_name from pmc_events"):
            for lab, (v, n) in per_kernel(db, cn).items():
                if lab != "copy":
                    vals[lab][cn] = (v, n)
    cols = [("issuing", "SQ_ACTIVE_INST_ANY"), ("VALU", "SQ_ACTIVE_INST_VALU"), ("LDS", "SQ_ACTIVE_INST_LDS"),
            ("VMEM", "SQ_ACTIVE_INST_VMEM"), ("scalar", "SQ_ACTIVE_INST_SCA"), ("waiting", "SQ_WAIT_ANY"),
            ("waiting for issue", "SQ_WAIT_INST_ANY")]
    lines = ["# Wave states per kernel launch (rocprofv3 SQ counters)", ""]
    if args.command:
        lines += ["Commands (from the repository root on one MI355X, library built):", "", "```", args.command,
                  "```", ""]
    lines += ["Shares of SQ_WAVE_CYCLES (the waves' resident time): issuing any instruction, issuing each "
              "kind, waiting (memory, LDS, barriers), waiting for an issue slot.  Bank conflicts: "
              "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (share of the LDS's active cycles lost to "
              "conflicts).  Instructions: millions per launch over all waves.", "",
              "| kernel | launches | " + " | ".join(c for c, _ in cols) +
              " | LDS bank conflicts | VALU / LDS / MFMA / SALU instructions (M) |",
              "|---|---:|" + "---:|" * (len(cols) + 2)]
    for lab in sorted(vals):
        d = vals[lab]
        if "SQ_WAVE_CYCLES" not in d:
            continue
        wc = d["SQ_WAVE_CYCLES"][0]
        row = [lab, str(d["SQ_WAVE_CYCLES"][1])]
        for _, cn in cols:
            row.append(f"{100.0 * d[cn][0] / wc:.0f}%" if cn in d and wc else "")
        bc, la = d.get("SQ_LDS_BANK_CONFLICT"), d.get("SQ_LDS_IDX_ACTIVE")
        row.append(f"{100.0 * bc[0] / la[0]:.0f}%" if bc and la and la[0] else "")
        ins = [d.get(k) for k in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_SALU")]
        row.append(" / ".join(f"{x[0] / 1e6:.1f}" if x else "-" for x in ins))
        lines.append("| " + " | ".join(row) + " |")
    lines += ["", f"Kernel sources digest: `{src_digest()}`", ""]
    text = "\n".join(lines)
    if args.md:
        with open(args.md, "w") as fh:
            fh.write(text)
    print(text)


def trace(args):
    con = sqlite3.connect(args.db)
    rows = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels "
                       "order by total_duration desc").fetchall()  # durations in microseconds
    lines = ["# Kernel trace (rocprofv3 --kernel-trace --stats)", ""]
    if args.command:
        lines += ["Command (from the repository root on one MI355X, library built):", "", "```", args.command, "```",
                  ""]
    lines += ["| kernel | library name | calls | total us | avg us | % of GPU time |", "|---|---|---:|---:|---:|---:|"]
    for name, calls, tot, avg, pct in rows[:args.top]:
        short = re.sub(r"gdr::\(anonymous namespace\)::", "", name)
        short = re.sub(r"\(gdr::[^)]*\)$", "", short)
        if len(short) > 90:
            short = short[:87] + "..."
        lines.append(f"| `{short}` | {label(name) or ''} | {calls} | {tot:.1f} | {avg:.2f} | "
                     f"{pct:.1f} |")
    # the same launches split by grid (workgroups), so a workload's launches
    # can be told apart from other shapes of the same kernel in the command
    acc = collections.defaultdict(lambda: [0, 0.0])
    for name, gx, gy, gz, wx, n, tot in con.execute(
            "select name, grid_x / workgroup_x, grid_y, grid_z, workgroup_x, count(*), sum(duration) "
            "from kernels group by name, grid_x, grid_y, grid_z, workgroup_x"):
        lab = label(name)
        if lab is not None:
            a = acc[(lab, int(gx), gy, gz, wx)]
            a[0] += n
            a[1] += tot
    lines += ["", "Library kernels by launch grid (all template instances of a kernel together):", "",
              "| library name | grid (workgroups) | threads | calls | avg us |", "|---|---|---:|---:|---:|"]
    for (lab, gx, gy, gz, wx), (n, tot) in sorted(acc.items(), key=lambda kv: (kv[0][0], -kv[1][0])):
        lines.append(f"| {lab} | {gx} x {gy} x {gz} | {wx} | {n} | {tot / n / 1000.0:.2f} |")
    lines += ["", f"Kernel sources digest: `{src_digest()}`", ""]
    text = "\n".join(lines)
    if args.md:
        with open(args.md, "w") as fh:
            fh.write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_db")
    t.add_argument("write_db")
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--json", required=True)
    t.add_argument("--md", default=None)
    t.add_argument("--command", default="")
    k = sub.add_parser("trace")
    k.add_argument("db")
    k.add_argument("--md", default=None)
    k.add_argument("--command", default="")
    k.add_argument("--top", type=int, default=16)
    m = sub.add_parser("mfma")
    m.add_argument("db")
    m.add_argument("--md", default=None)
    m.add_argument("--command", default="")
    m.add_argument("--simds", type=int, default=1024, help="SIMDs on the GPU (MI355X: 256 CUs x 4)")
    q = sub.add_parser("sq")
    q.add_argument("dbs", nargs="+")
    q.add_argument("--md", default=None)
    q.add_argument("--command", default="")
    args = ap.parse_args()
    {"traffic": traffic, "trace": trace, "mfma": mfma, "sq": sq}[args.cmd](args)


if __name__ == "__main__":
    main()
