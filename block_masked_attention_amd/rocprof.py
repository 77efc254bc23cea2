"""rocprofv3 harness for the bdattn kernels: duration, shader clock, matrix-core
(MFMA) utilisation, LDS utilisation and HBM traffic per kernel, for one
workload of ``bench.py``.

Each measurement is its own rocprofv3 run of ``bench.py`` (one warm-up step
and one timed step, so that every pass averages the same two launches of each
kernel), started as a child process with a time limit:

  trace   --kernel-trace --stats                     kernel durations
  fetch   --pmc FETCH_SIZE, with a 1 GiB plain copy  HBM reads
  write   --pmc WRITE_SIZE, with a 1 GiB plain copy  HBM writes
  sq1     --pmc SQ wave/instruction counters         issue and waits
  sq2     --pmc SQ MFMA/LDS counters                 MFMA busy, LDS busy

rocprofv3 does not split counters over passes, so every counter set stays
within the per-block limits of one pass. The copy is read and written once,
so it calibrates FETCH_SIZE and WRITE_SIZE (KiB per dispatch) to bytes. The
shader clock of a kernel is GRBM_GUI_ACTIVE / XCDs / duration. MFMA busy is
SQ_VALU_MFMA_BUSY_CYCLES over (SIMDs x cycles), and LDS busy is
SQ_LDS_IDX_ACTIVE over (CUs x cycles); the counts of XCDs, SIMDs and CUs are
read from the profiler's agent description.

Usage (repository root, on the GPU machine):

    python -m block_masked_attention_amd.rocprof --workload 256k --out DIR

It prints one JSON line and writes DIR/summary.json and DIR/summary.md; the
raw rocprofv3 output stays in DIR/<pass>/. With ``--profiles P`` it also
writes the four summaries kept in the repository under P:
bdattn_<workload>_{rocprof_summary,kernel_trace,hbm_traffic,sq_counters}.md.
The HBM traffic file ends with machine-readable lines (dominant kernel,
workload, kernel source hash, HBM bytes per launch, shader clock) that
bench.py reports in its roofline while the kernel sources are unchanged.

``--bwd fused10`` profiles the one-kernel backward (BDATTN_BWD=fused10, the
measured alternative in kernels_bwd_fused.hip) instead of the split one; its
write pass also counts TCC_EA0_ATOMIC (the float-atomic requests the L2
passes on to memory), and its summaries are named <workload>_bwd_fused10.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the kernels, their shared device code and tile constants (plan.h), and the
# host code that orders their work and picks their launch shapes (plan.cpp,
# api.cpp)
KERNEL_SOURCES = ("kernels.hip", "kernels_dq_docs.hip", "kernels_dkdv.hip", "device.h", "bdattn_mask.h",
                  "launch.h", "plan.h", "plan.cpp", "api.cpp")
# bench.py times the one-kernel backward in the dK/dV slot
BENCH_NAME = {"fwd_kernel": "fwd", "bwd_dq_kernel": "bwd_dq", "bwd_dkdv_kernel": "bwd_dkdv",
              "bwd_fused_kernel": "bwd_dkdv"}
MAIN_KERNELS = ("fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_prep_kernel",
                "merge_kernel", "bwd_fused_kernel", "fill_zero_f32", "store_dq")
ATOMIC = "TCC_EA0_ATOMIC_sum"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30  # the calibration copy reads and writes 1 GiB
MIN_CLOCK_MS = 0.1  # shorter kernels get no clock-derived figures
WARMUP = 1  # bench.py warm-up steps in every pass (durations and counters average all launches)
SQ1 = ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
       "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
       "GRBM_GUI_ACTIVE"]
SQ2 = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_IDX_ACTIVE",
       "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
       "GRBM_GUI_ACTIVE"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_lines(text: str):
    """The lines of a C++ source without // comments, trailing blanks and empty
    lines (a "//" inside a string literal is kept)."""
    out = []
    for line in text.splitlines():
        cut, quoted = len(line), False
        for i, ch in enumerate(line):
            if ch == '"' and (i == 0 or line[i - 1] != "\\"):
                quoted = not quoted
            elif not quoted and line.startswith("//", i):
                cut = i
                break
        line = line[:cut].rstrip()
        if line:
            out.append(line)
    return out


def kernel_source_hash(csrc: str = None) -> str:
    """Hash of the code of the kernel sources whose counters a profile
    describes (comments do not count) and of their compiler options."""
    import hashlib
    csrc = csrc or os.path.join(ROOT, "block_masked_attention_amd", "csrc")
    from block_masked_attention_amd import build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f)) as fh:
            h.update("\n".join(code_lines(fh.read())).encode() + b"\n")
    # and the compiler options they are built with
    h.update(repr((build.HIP_FLAGS, sorted(build.FILE_FLAGS.items()))).encode())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """'void bdattn::(anonymous namespace)::bwd_dq_kernel<true, 128>(...)' ->
    'bwd_dq_kernel<true, 128>'; 'void bdattn::(anonymous namespace)::store_dq(...)'
    -> 'store_dq'; other kernels keep their name up to '('."""
    m = re.search(r"::(\w+<[^>]*>)\(", kernel)
    if m:
        return m.group(1)
    # a library kernel that is not a template (rocprofv3 drops the "void ")
    m = re.match(r"(?:void )?bdattn::(?:\(anonymous namespace\)::)?(\w+)\(", kernel)
    if m:
        return m.group(1)
    return kernel.split("(")[0].replace("void ", "").strip()


def run_pass(name, flags, bench_args, out_dir, limit):
    """One rocprofv3 run of bench.py; returns its output directory. The
    program follows '--' directly (no launcher in between)."""
    d = os.path.join(out_dir, name)
    shutil.rmtree(d, ignore_errors=True)
    cmd = (["rocprofv3"] + flags + ["-f", "csv", "-d", d, "-o", "run", "--", sys.executable,
                                    os.path.join(ROOT, "bench.py")] + bench_args)
    log(f"[rocprof] pass {name}: {' '.join(cmd)}")
    with open(os.path.join(out_dir, f"{name}.log"), "w") as fh:
        try:
            res = subprocess.run(cmd, cwd=ROOT, stdout=fh, stderr=subprocess.STDOUT,
                                 timeout=limit)
            rc = res.returncode
        except subprocess.TimeoutExpired:  # the child is killed (SIGKILL)
            raise RuntimeError(f"rocprofv3 pass {name} exceeded {limit} s")
    # rocprofv3 may end with a signal after the program finished and wrote its
    # results; the results decide
    if not any(f.endswith(".csv") for f in os.listdir(d) if os.path.isfile(os.path.join(d, f))):
        raise RuntimeError(f"rocprofv3 pass {name} wrote no results (exit status {rc})")
    log(f"[rocprof] pass {name} done (exit status {rc})")
    return d


def read_csv(d, suffix):
    path = os.path.join(d, f"run_{suffix}.csv")
    with open(path) as fh:
        return list(csv.DictReader(fh))


def durations(d):
    """Average ms per call and call count of every kernel of a trace pass."""
    out = {}
    for r in read_csv(d, "kernel_stats"):
        out[short_name(r["Name"])] = dict(ms=float(r["AverageNs"]) / 1e6, calls=int(r["Calls"]))
    return out


def counter_rows(d):
    """The counter rows of a pass. Of the runtime's copy kernel only the
    calibration copy is kept: the dispatch with the largest grid (the runtime
    also runs small copies of the same kernel, e.g. for host uploads, which
    would otherwise dilute the per-dispatch average)."""
    rows = read_csv(d, "counter_collection")
    copies = [r for r in rows if short_name(r["Kernel_Name"]) == COPY_KERNEL]
    keep = max(copies, key=lambda r: int(r["Grid_Size"]))["Dispatch_Id"] if copies else None
    return [r for r in rows
            if short_name(r["Kernel_Name"]) != COPY_KERNEL or r["Dispatch_Id"] == keep]


def counters(d):
    """Counter totals per kernel, divided by the kernel's dispatch count."""
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in counter_rows(d):
        k = short_name(r["Kernel_Name"])
        tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    return {k: dict({c: v / len(disp[k]) for c, v in cs.items()}, _dispatches=len(disp[k]))
            for k, cs in tot.items()}


def agent(d):
    for r in read_csv(d, "agent_info"):
        if r.get("Name", "").startswith("gfx"):
            return dict(simds=int(r["Simd_Count"]), cus=int(r["Cu_Count"]),
                        xcds=int(r.get("Num_Xcc") or 1), name=r["Name"])
    raise RuntimeError("no GPU agent in the profiler's agent description")


def summarise(dur, fetch, write, sq1, sq2, dev):
    copy_fetch = fetch.get(COPY_KERNEL, {}).get("FETCH_SIZE")
    copy_write = write.get(COPY_KERNEL, {}).get("WRITE_SIZE")
    f_scale = COPY_BYTES / (copy_fetch * 1024) if copy_fetch else None
    w_scale = COPY_BYTES / (copy_write * 1024) if copy_write else None
    rows = {}
    for k, t in dur.items():
        if not k.startswith(MAIN_KERNELS):
            continue
        s = t["ms"] * 1e-3
        r = dict(ms=round(t["ms"], 3), calls=t["calls"])
        if k in fetch and f_scale:
            r["hbm_read_gb"] = round(fetch[k]["FETCH_SIZE"] * 1024 * f_scale / 1e9, 2)
        if k in write and w_scale:
            r["hbm_write_gb"] = round(write[k]["WRITE_SIZE"] * 1024 * w_scale / 1e9, 3)
        if "hbm_read_gb" in r and "hbm_write_gb" in r:
            r["hbm_gbps"] = round((r["hbm_read_gb"] + r["hbm_write_gb"]) / s, 1)
        if k in write and ATOMIC in write[k]:  # atomic requests beyond the L2, per launch
            r["atomic_requests"] = write[k][ATOMIC]
        # (GRBM_GUI_ACTIVE also counts the launch around a kernel, so the
        # clock and the figures per cycle mean nothing for very short ones)
        clocks = [c["GRBM_GUI_ACTIVE"] / dev["xcds"] / s / 1e9
                  for c in (sq1.get(k), sq2.get(k)) if c and "GRBM_GUI_ACTIVE" in c
                  and t["ms"] >= MIN_CLOCK_MS]
        if clocks:
            ghz = sum(clocks) / len(clocks)
            cycles = ghz * 1e9 * s
            r["clock_ghz"] = round(ghz, 3)
            c2 = sq2.get(k, {})
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c2:
                r["mfma_busy"] = round(c2["SQ_VALU_MFMA_BUSY_CYCLES"] / (dev["simds"] * cycles), 4)
            if "SQ_LDS_IDX_ACTIVE" in c2:
                r["lds_busy"] = round(c2["SQ_LDS_IDX_ACTIVE"] / (dev["cus"] * cycles), 4)
            if c2.get("SQ_INSTS_MFMA"):
                m = c2["SQ_INSTS_MFMA"]
                r["valu_per_mfma"] = round(c2["SQ_INSTS_VALU"] / m, 2)
                r["lds_per_mfma"] = round(c2["SQ_INSTS_LDS"] / m, 2)
                r["salu_per_mfma"] = round(c2["SQ_INSTS_SALU"] / m, 2)
            if "SQ_LDS_BANK_CONFLICT" in c2:
                r["lds_bank_conflicts"] = c2["SQ_LDS_BANK_CONFLICT"]
        rows[k] = r
    return dict(device=dev, fetch_scale=f_scale, write_scale=w_scale, kernels=rows)


def markdown(summary, workload, cmd):
    cols = [("ms", "ms"), ("clock_ghz", "clock GHz"), ("mfma_busy", "MFMA busy"),
            ("lds_busy", "LDS busy"), ("valu_per_mfma", "VALU/MFMA"),
            ("hbm_read_gb", "HBM read GB"), ("hbm_write_gb", "HBM write GB"),
            ("hbm_gbps", "HBM GB/s")]
    if any("atomic_requests" in r for r in summary["kernels"].values()):
        cols.append(("atomic_requests", "atomic requests"))
    out = [f"# bdattn kernels, {workload} workload: rocprofv3 summary", "",
           "Command (run from the repository root on one GPU):", "", "```", cmd, "```", "",
           f"Device {summary['device']['name']}: {summary['device']['cus']} CUs, "
           f"{summary['device']['simds']} SIMDs, {summary['device']['xcds']} XCDs. HBM counters "
           f"scaled by a 1 GiB plain copy (factors {summary['fetch_scale']:.3f} fetch, "
           f"{summary['write_scale']:.3f} write).", "",
           "| kernel | " + " | ".join(c[1] for c in cols) + " |",
           "|---|" + "---|" * len(cols)]
    for k, r in summary["kernels"].items():
        cells = []
        for key, _ in cols:
            v = r.get(key)
            if v is None:
                cells.append("")
            elif key in ("mfma_busy", "lds_busy"):
                cells.append(f"{100 * v:.0f}%")
            else:
                cells.append(f"{v:g}")
        out.append(f"| `{k}` | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def _base(k):
    return k.split("<")[0]


def _main_rows(d_trace):
    return [r for r in read_csv(d_trace, "kernel_stats") if short_name(r["Name"]).startswith(MAIN_KERNELS)]


def profile_key(workload, docs=1, bwd="split"):
    """Name of a profiled configuration: the workload, with the number of
    packed documents when there are several and the backward when it is not
    the split one."""
    return workload + (f"_docs{docs}" if docs > 1 else "") + ("" if bwd == "split" else f"_bwd_{bwd}")


def write_profiles(dest, workload, cmd, d_trace, fetch, write, sq1, sq2, dev, summary, docs=1,
                   bwd="split"):
    """The four repository summaries of one harness run (tables only)."""
    sys.path.insert(0, ROOT)
    from workloads import config
    spec = config(workload)
    desc = (f"clean {spec.n_clean_q} + corrupted {spec.n_corr} tokens, B={spec.B}, GQA "
            f"{spec.H}/{spec.Hkv}, d={spec.d}, {spec.dtype}; one forward and one backward")
    if docs > 1:
        desc += f"; {docs} packed documents (bench.py --docs {docs})"
    bench_extra = f" --docs {docs}" if docs > 1 else ""
    if bwd != "split":
        desc += (f"; the one-kernel backward (environment BDATTN_BWD={bwd}, "
                 "block_masked_attention_amd/csrc/kernels_bwd_fused.hip)")
    workload = profile_key(workload, docs, bwd)
    head = ["Command (run from the repository root on one MI355X):", "", "```", cmd, "```", "",
            f"Workload {workload}: {desc}. Kernel source hash {kernel_source_hash()}.", ""]
    os.makedirs(dest, exist_ok=True)
    name = lambda kind: os.path.join(dest, f"bdattn_{workload}_{kind}.md")
    # 1. the harness summary
    with open(name("rocprof_summary"), "w") as fh:
        fh.write(markdown(summary, workload, cmd))
        fh.write("\nClock = GRBM_GUI_ACTIVE / XCDs / duration (the mean of the two SQ passes); "
                 "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles); LDS busy = "
                 "SQ_LDS_IDX_ACTIVE / (CUs x cycles); HBM bytes per launch from FETCH_SIZE and "
                 "WRITE_SIZE, scaled by the plain copy. Each figure comes from its own rocprofv3 "
                 "run of one warm-up and one timed bench step, averaged per launch "
                 "(block_masked_attention_amd/rocprof.py lists the "
                 "passes); durations come from the kernel-trace pass.\n")
    # 2. kernel trace
    rows = _main_rows(d_trace)
    out = [f"# bdattn kernels, {workload} workload: rocprofv3 kernel trace", ""] + head + [
        "The `trace` pass: `rocprofv3 --kernel-trace --stats` over `bench.py --workload "
        f"{spec.name}{bench_extra} --no-cpu-baseline --steps 1 --warmup {WARMUP}`.", "",
        "| kernel | calls | avg ms | min ms | max ms | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                   f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {r['Percentage']} |")
    out += ["", "The rest of the GPU time is torch's input generation (random fill and scaling)."]
    with open(name("kernel_trace"), "w") as fh:
        fh.write("\n".join(out) + "\n")
    # 3. HBM traffic, with the machine-readable lines
    cf, cw = fetch.get(COPY_KERNEL, {}), write.get(COPY_KERNEL, {})
    out = [f"# bdattn kernels, {workload} workload: HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE)",
           ""] + head + [
        "The `fetch` and `write` passes: `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE"
        + (f" {ATOMIC}" if bwd != "split" else "") + "` over "
        f"`bench.py --workload {spec.name}{bench_extra} --no-cpu-baseline --steps 1 --warmup {WARMUP} "
        "--copy-calibration`. The calibration copy (`__amd_rocclr_copyBuffer`) reads and writes "
        f"exactly {COPY_BYTES // 1024} KiB; the counters read FETCH_SIZE = "
        f"{cf.get('FETCH_SIZE', 0):.0f} KiB and WRITE_SIZE = {cw.get('WRITE_SIZE', 0):.0f} KiB for "
        f"it, so the scale factors are {summary['fetch_scale']:.3f} (fetch) and "
        f"{summary['write_scale']:.3f} (write). Counts are per launch.", "",
        "| kernel | launches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (GB, scaled) | write (GB, scaled) |"
        + (f" {ATOMIC} |" if bwd != "split" else ""),
        "|---|---|---|---|---|---|" + ("---|" if bwd != "split" else "")]
    for k, r in summary["kernels"].items():
        f, w = fetch.get(k, {}), write.get(k, {})
        out.append(f"| `{k}` | {f.get('_dispatches', '')} | {f.get('FETCH_SIZE', 0):.0f} | "
                   f"{w.get('WRITE_SIZE', 0):.0f} | {r.get('hbm_read_gb', '')} | {r.get('hbm_write_gb', '')} |"
                   + (f" {w.get(ATOMIC, 0):.4g} |" if bwd != "split" else ""))
    main = {k: r for k, r in summary["kernels"].items() if _base(k) in BENCH_NAME}
    dom = max(main, key=lambda k: main[k]["ms"])
    r = main[dom]
    nbytes = (fetch[dom]["FETCH_SIZE"] * summary["fetch_scale"]
              + write[dom]["WRITE_SIZE"] * summary["write_scale"]) * 1024
    out += ["", f"Dominant kernel (longest): `{dom}`, {nbytes / 1e9:.1f} GB per launch beyond the "
            f"L2 over {r['ms']:.0f} ms ({nbytes / 1e9 / (r['ms'] * 1e-3):.0f} GB/s).", "",
            "Machine-readable lines for bench.py (valid only for the kernel source hash below):", "",
            f"kernel: {BENCH_NAME[_base(dom)]}", f"workload: {workload}",
            f"kernel_source: {kernel_source_hash()}",
            f"hbm_bytes_per_launch: {nbytes:.6e}"]
    if "clock_ghz" in r:  # the kernel's mean shader clock over the two SQ passes
        out.append(f"clock_ghz: {r['clock_ghz']}")
    with open(name("hbm_traffic"), "w") as fh:
        fh.write("\n".join(out) + "\n")
    # 4. SQ counters
    ks = [k for k in summary["kernels"] if _base(k) in BENCH_NAME]
    out = [f"# bdattn kernels, {workload} workload: SQ counters (rocprofv3 --pmc)", ""] + head + [
        "The `sq1` and `sq2` passes run `rocprofv3 --pmc` with these counter sets over "
        f"`bench.py --workload {spec.name}{bench_extra} --no-cpu-baseline --steps 1 --warmup {WARMUP}`: sq1 = "
        f"{' '.join(SQ1)}; sq2 = {' '.join(SQ2)}. Clock = GRBM_GUI_ACTIVE / {dev['xcds']} XCDs / "
        f"duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({dev['simds']} SIMDs x cycles); LDS "
        f"busy = SQ_LDS_IDX_ACTIVE / ({dev['cus']} CUs x cycles).", "",
        "| counter | " + " | ".join(f"`{k}`" for k in ks) + " |", "|---|" + "---|" * len(ks),
        "| duration (ms, kernel trace) | " + " | ".join(f"{summary['kernels'][k]['ms']:.4g}" for k in ks) + " |"]
    for c in dict.fromkeys(SQ1 + SQ2):
        vals = []
        for k in ks:
            v = [x[k][c] for x in (sq1, sq2) if k in x and c in x[k]]
            vals.append(" / ".join(f"{y:.4g}" for y in v))
        out.append(f"| {c} | " + " | ".join(vals) + " |")
    for key, label, fmt in (("clock_ghz", "derived: shader clock (GHz)", "{:.2f}"),
                            ("mfma_busy", "derived: MFMA busy", "{:.0%}"),
                            ("lds_busy", "derived: LDS busy", "{:.0%}"),
                            ("valu_per_mfma", "derived: VALU instructions per MFMA", "{:.2f}"),
                            ("lds_per_mfma", "derived: LDS instructions per MFMA", "{:.2f}"),
                            ("salu_per_mfma", "derived: SALU instructions per MFMA", "{:.2f}")):
        out.append(f"| {label} | " + " | ".join(fmt.format(summary['kernels'][k][key])
                                              if key in summary['kernels'][k] else "" for k in ks) + " |")
    out.append("")
    out.append("GRBM_GUI_ACTIVE is read in both passes (sq1 / sq2).")
    with open(name("sq_counters"), "w") as fh:
        fh.write("\n".join(out) + "\n")
    log(f"[rocprof] wrote the four summaries under {dest}")


# ------------------------------------------------ linear cross-entropy
LCE_SOURCES = ("lce.hip",)
# the three products of a chunk, told apart by the transposes in the library
# kernels' names (Tensile naming: A "lik" = A transposed, B "jlk" = B transposed)
LCE_GEMMS = (("lce_logits", "_Alik_Bljk"), ("lce_dh", "_Ailk_Bljk"), ("lce_dw", "_Ailk_Bjlk"))


def lce_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in LCE_SOURCES:
        with open(os.path.join(ROOT, "block_masked_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def lce_role(name: str):
    """lce_logits / lce_dh / lce_dw for the library products, lce_rows for the
    fused row kernels, None for anything else."""
    if "lce_fused_kernel" in name or "lce_loss_kernel" in name or "lce_grad_kernel" in name:
        return "lce_rows"
    for role, tag in LCE_GEMMS:
        if name.startswith("Cijk") and tag in name:
            return role
    return None


def lce_profile(args):
    """Kernel trace and calibrated HBM traffic of one linear cross-entropy
    step (bench.py --workload lce_*), per role."""
    b = ["--workload", args.workload, "--no-cpu-baseline", "--steps", "1"]
    d_trace = run_pass("trace", ["--kernel-trace", "--stats"], b + ["--warmup", str(WARMUP)], args.out,
                       args.limit)
    cal = b + ["--warmup", str(WARMUP), "--copy-calibration"]
    d_fetch = run_pass("fetch", ["--pmc", "FETCH_SIZE"], cal, args.out, args.limit)
    d_write = run_pass("write", ["--pmc", "WRITE_SIZE"], cal, args.out, args.limit)
    fetch_raw, write_raw = lce_counters(d_fetch), lce_counters(d_write)
    cf = fetch_raw.pop(COPY_KERNEL, {}).get("FETCH_SIZE")
    cw = write_raw.pop(COPY_KERNEL, {}).get("WRITE_SIZE")
    fs = COPY_BYTES / (cf * 1024) if cf else None
    ws = COPY_BYTES / (cw * 1024) if cw else None
    rows = {}
    for r in read_csv(d_trace, "kernel_stats"):
        role = lce_role(r["Name"])
        if role is None:
            continue
        x = rows.setdefault(role, dict(calls=0, ns=0.0, names=set()))
        x["calls"] += int(r["Calls"])
        x["ns"] += float(r["TotalDurationNs"])
        x["names"].add(short_name(r["Name"])[:60])
    for role, x in rows.items():
        x["ms"] = x["ns"] / x["calls"] / 1e6
        f, w = fetch_raw.get(role), write_raw.get(role)
        if f and fs:
            x["read_gb"] = f["FETCH_SIZE"] * 1024 * fs / 1e9
        if w and ws:
            x["write_gb"] = w["WRITE_SIZE"] * 1024 * ws / 1e9
    sys.path.insert(0, ROOT)
    from workloads import LCE_CONFIGS
    spec = next(c for c in LCE_CONFIGS if c.name == args.workload)
    cmd = f"python -m block_masked_attention_amd.rocprof --workload {args.workload} --out {args.out}"
    if args.profiles:
        cmd += f" --profiles {args.profiles}"
    per_gemm = 2.0 * spec.chunk * spec.V * spec.D
    out = [f"# linear cross-entropy, {args.workload} workload: rocprofv3 kernel trace and HBM traffic",
           "", "Command (run from the repository root on one MI355X):", "", "```", cmd, "```", "",
           f"Workload {args.workload}: {spec.description}; one forward + backward step "
           f"(`bench.py --workload {args.workload} --no-cpu-baseline --steps 1`). Source hash of "
           f"lce.hip {lce_source_hash()}. Per chunk: the logits product, the fused row kernel, the "
           "dH product and the dW product; the products are rocBLAS kernels, told apart by the "
           "transposes in their names. HBM bytes from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), "
           f"scaled by a 1 GiB plain copy (factors {fs or 0:.3f} fetch, {ws or 0:.3f} write).", "",
           "| role | kernel | launches | avg ms | TFLOP/s | HBM read GB | HBM write GB | HBM GB/s |",
           "|---|---|---|---|---|---|---|---|"]
    for role in ("lce_logits", "lce_rows", "lce_dh", "lce_dw"):
        if role not in rows:
            continue
        x = rows[role]
        tf = f"{per_gemm / (x['ms'] * 1e-3) / 1e12:.0f}" if role != "lce_rows" else ""
        rd, wr = x.get("read_gb"), x.get("write_gb")
        bw = f"{(rd + wr) / (x['ms'] * 1e-3):.0f}" if rd is not None and wr is not None else ""
        out.append(f"| {role} | `{sorted(x['names'])[0]}` | {x['calls']} | {x['ms']:.3f} | {tf} | "
                   f"{'' if rd is None else f'{rd:.2f}'} | {'' if wr is None else f'{wr:.2f}'} | {bw} |")
    dom = max((k for k in rows if k != "lce_rows"), key=lambda k: rows[k]["ms"])
    d = rows[dom]
    nbytes = (d.get("read_gb", 0) + d.get("write_gb", 0)) * 1e9
    out += ["", f"Dominant kernel (longest): {dom}.", "",
            "Machine-readable lines for bench.py (valid only for the source hash below):", "",
            f"kernel: {dom}", f"workload: {args.workload}", f"kernel_source: {lce_source_hash()}",
            f"hbm_bytes_per_launch: {nbytes:.6e}"]
    text = "\n".join(out) + "\n"
    with open(os.path.join(args.out, "summary.md"), "w") as fh:
        fh.write(text)
    if args.profiles:
        os.makedirs(args.profiles, exist_ok=True)
        with open(os.path.join(args.profiles, f"{args.workload}_kernel_trace_hbm.md"), "w") as fh:
            fh.write(text)
    print(json.dumps({k: {kk: vv for kk, vv in v.items() if kk != "names"} for k, v in rows.items()}),
          flush=True)


def lce_counters(d):
    """Counter totals per role (and the calibration copy), per dispatch."""
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in counter_rows(d):
        name = r["Kernel_Name"]
        k = COPY_KERNEL if short_name(name) == COPY_KERNEL else lce_role(name)
        if k is None:
            continue
        tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    return {k: dict({c: v / len(disp[k]) for c, v in cs.items()}) for k, cs in tot.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="256k")
    ap.add_argument("--out", required=True, help="directory for the raw output and summaries")
    ap.add_argument("--limit", type=int, default=300, help="seconds allowed per pass")
    ap.add_argument("--docs", type=int, default=1, help="packed documents (bench.py --docs)")
    ap.add_argument("--profiles", default=None,
                    help="also write the repository summaries of this run into this directory")
    ap.add_argument("--bwd", choices=("split", "fused10"), default="split",
                    help="backward to profile (fused10: the one-kernel backward)")
    args = ap.parse_args()
    if shutil.which("rocprofv3") is None:
        sys.exit("rocprofv3 not found")
    os.makedirs(args.out, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")
    if args.workload.startswith("lce"):
        lce_profile(args)
        return
    b = ["--workload", args.workload, "--no-cpu-baseline", "--steps", "1"]
    if args.docs > 1:
        b += ["--docs", str(args.docs)]
    if args.bwd != "split":  # read by the library at every backward call
        os.environ["BDATTN_BWD"] = args.bwd
    d_trace = run_pass("trace", ["--kernel-trace", "--stats"], b + ["--warmup", str(WARMUP)], args.out,
                       args.limit)
    cal = b + ["--warmup", str(WARMUP), "--copy-calibration"]
    d_fetch = run_pass("fetch", ["--pmc", "FETCH_SIZE"], cal, args.out, args.limit)
    d_write = run_pass("write", ["--pmc", "WRITE_SIZE"] + ([ATOMIC] if args.bwd != "split" else []),
                       cal, args.out, args.limit)
    d_sq1 = run_pass("sq1", ["--pmc"] + SQ1, b + ["--warmup", str(WARMUP)], args.out, args.limit)
    d_sq2 = run_pass("sq2", ["--pmc"] + SQ2, b + ["--warmup", str(WARMUP)], args.out, args.limit)
    summary = summarise(durations(d_trace), counters(d_fetch), counters(d_write),
                        counters(d_sq1), counters(d_sq2), agent(d_trace))
    summary["workload"] = profile_key(args.workload, args.docs, args.bwd)
    cmd = f"python -m block_masked_attention_amd.rocprof --workload {args.workload} --out {args.out}"
    if args.docs > 1:
        cmd += f" --docs {args.docs}"
    if args.bwd != "split":
        cmd += f" --bwd {args.bwd}"
    if args.profiles:
        cmd += f" --profiles {args.profiles}"
    with open(os.path.join(args.out, "summary.json"), "w") as fh:
        json.dump(summary, fh, indent=1)
    with open(os.path.join(args.out, "summary.md"), "w") as fh:
        fh.write(markdown(summary, profile_key(args.workload, args.docs, args.bwd), cmd))
    if args.profiles:
        write_profiles(args.profiles, args.workload, cmd, d_trace, counters(d_fetch),
                       counters(d_write), counters(d_sq1), counters(d_sq2), agent(d_trace), summary,
                       docs=args.docs, bwd=args.bwd)
    print(json.dumps(summary), flush=True)


if __name__ == "__main__":
    main()
