#!/usr/bin/env python3
"""Benchmark of bdattn: block-diffusion attention forward + backward on one GPU.

One step = bdattn_fwd then bdattn_bwd over the whole workload (every row of
both streams, every head), inputs resident in device memory. Prints one JSON
line: whole-step useful TFLOP/s (12*d*H*pairs flops per step: QK^T and PV in
the forward, dV, dP, dQ and dK in the backward; masked pairs and the
backward's QK^T recompute are not counted), the roofline position of the
dominant kernel (timed live with HIP events on its launch stream), and the
float64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 256k]
"""
import argparse
import bisect
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "bdattn fwd+bwd useful TFLOP/s at 256K ctx; % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_CLOCK_GHZ = 2.4  # the shader clock both peaks assume
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bdattn_{}_hbm_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_profile(workload: str, kernel: str):
    """(HBM bytes per launch, shader clock in GHz or None) of `kernel` from
    the committed rocprofv3 counter summary, if it was taken on the current
    kernel source and this workload; else (None, None)."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None, None
    txt = open(path).read()
    m = {k: v for k, v in re.findall(r"^(\w+):\s*(\S+)\s*$", txt, re.M)}
    from block_masked_attention_amd.rocprof import kernel_source_hash
    if (m.get("kernel_source") != kernel_source_hash() or m.get("workload") != workload
            or m.get("kernel") != kernel):
        return None, None
    try:
        clock = float(m["clock_ghz"]) if "clock_ghz" in m else None
        return float(m["hbm_bytes_per_launch"]), clock
    except (KeyError, ValueError):
        return None, None


def cpu_baseline(spec, t, seconds: float):
    """The float64 oracle, as it stands, on whole query blocks of the
    workload (one KV head group each, blocks spread over both streams and
    the whole sequence) until about `seconds` of work; returns useful
    TFLOP/s over the sample."""
    import numpy as np

    from oracle import Oracle, layout

    f64 = lambda x: x.float().cpu().numpy().astype(np.float64)
    B, G, d = spec.B, spec.H // spec.Hkv, spec.d
    ids = list(spec.corr_block_ids) if spec.corr_block_ids is not None else \
        list(range(spec.n_corr_blocks))
    cb0 = spec.clean_q_start // B
    ncb = spec.n_clean_q // B
    docs = list(spec.doc_starts or [0])
    doc_start = lambda pos: docs[bisect.bisect_right(docs, pos) - 1]  # of the document at pos
    sub_docs = lambda end: [x for x in docs if x < end]  # document starts before `end`
    order = []
    for i in range(max(ncb, len(ids))):  # spread: stride through both streams
        frac = ((i * 0.6180339887) % 1.0)
        if ncb:
            order.append(("c", cb0 + int(frac * ncb)))
        if ids:
            order.append(("x", int(frac * len(ids))))
    flops = 0.0
    spent = 0.0
    n_blocks = 0
    rows = 0
    for k, (stream, b) in enumerate(order):
        g = k % spec.Hkv
        hq, hk = slice(g * G, (g + 1) * G), slice(g, g + 1)
        if stream == "c":
            r0 = b * B - spec.clean_q_start
            lay = layout(B, G, 1, d, B, b * B, (b + 1) * B, 0, corr_block_ids=[],
                         clean_mask=spec.clean_mask, doc_starts=sub_docs((b + 1) * B))
            e, ek = np.zeros((0, G, d)), np.zeros((0, 1, d))
            args = (f64(t["q_c"][r0:r0 + B, hq]), f64(t["k_c"][:(b + 1) * B, hk]),
                    f64(t["v_c"][:(b + 1) * B, hk]), e, ek, ek,
                    f64(t["do_c"][r0:r0 + B, hq]), e)
            # a block-causal clean row sees (b+1)B - s keys (s: its document's
            # start); a token-causal one at position bB + r sees bB + r + 1 - s
            s0 = doc_start(b * B)
            pairs = (B * ((b + 1) * B - s0) if spec.clean_mask == 0
                     else B * (b * B - s0) + B * (B + 1) // 2)
        else:
            bid = ids[b]
            rr = slice(b * B, (b + 1) * B)
            lay = layout(B, G, 1, d, 0, 0, bid * B, 0, corr_block_ids=[bid],
                         doc_starts=sub_docs(bid * B + 1))
            e = np.zeros((0, G, d))
            args = (e, f64(t["k_c"][:bid * B, hk]), f64(t["v_c"][:bid * B, hk]),
                    f64(t["q_x"][rr, hq]), f64(t["k_x"][rr, hk]), f64(t["v_x"][rr, hk]),
                    e, f64(t["do_x"][rr, hq]))
            pairs = B * (bid * B - doc_start(bid * B) + B)
        t0 = time.perf_counter()
        orc = Oracle(lay, *args)
        orc.forward()
        orc.backward()
        spent += time.perf_counter() - t0
        flops += 12.0 * d * G * pairs
        n_blocks += 1
        rows += B * G
        if spent >= seconds:
            break
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    if not threads:
        threads = len(os.sched_getaffinity(0))
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_blocks} whole query blocks x {G} q heads ({rows} query rows, "
                      f"full visible prefixes), float64 numpy fwd+bwd, {spent:.1f} s",
            "seconds": round(spent, 2), "cpu": platform.processor() or platform.machine(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def time_split_forward(bd, spec, t, shards, reps):
    """The forward as the appendix's Implementation 1 runs it: one partial
    launch for the block-diagonal corrupted part, one per clean K/V shard (at
    original positions), and a merge after each shard. Returns the mean ms
    per forward over `reps` after one untimed pass."""
    import torch

    from workloads import INPUT_NAMES

    B, nkv = spec.B, spec.n_clean_kv
    if spec.kv_chunk_len:  # a gathered buffer: one clean launch over all of it
        shards = 1
    cuts = [B * (i * (nkv // B) // shards) for i in range(shards + 1)]
    parts = [(0, 0, True)] + [(a, b, False) for a, b in zip(cuts, cuts[1:]) if b > a]
    probs, ins = [], []
    for lo, hi, ck in parts:
        gathered = spec.kv_chunk_len if hi > lo else 0
        probs.append(bd.problem(spec.B, spec.H, spec.Hkv, spec.d, spec.dtype, spec.n_clean_q,
                                spec.clean_q_start, hi - lo, lo, spec.n_corr_blocks,
                                spec.corr_block_ids, clean_mask=spec.clean_mask, partial=True,
                                doc_starts=spec.doc_starts,
                                omit_corr_keys=not ck, kv_chunk_len=gathered,
                                kv_chunk_pos=spec.kv_chunk_pos if gathered else None))
        u = dict(t)
        u["k_c"], u["v_c"] = t["k_c"][lo:hi], t["v_c"][lo:hi]  # row ranges stay contiguous
        ins.append([u[k] for k in INPUT_NAMES])
    wss = [torch.empty(bd.workspace_size(p, 0), dtype=torch.uint8, device=t["q_c"].device)
           for p in probs]
    acc = bd.fwd(probs[0], *ins[0], workspace=wss[0])
    part = [torch.empty_like(x) for x in acc]

    def once():
        bd.fwd(probs[0], *ins[0], workspace=wss[0], out=acc)
        for p, a, w in zip(probs[1:], ins[1:], wss[1:]):
            bd.fwd(p, *a, workspace=w, out=part)
            bd.merge(acc[0], acc[2], part[0], part[2], out=(acc[0], acc[2]))
            bd.merge(acc[1], acc[3], part[1], part[3], out=(acc[1], acc[3]))

    once()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    return {"shards": shards, "launches": len(parts), "ms": round((time.perf_counter() - t0) * 1e3 / reps, 3)}


LCE_METRIC = "token-chunked linear CE fwd+bwd useful TFLOP/s (6*N*V*D); % of MI355X bf16 MFMA peak"


def lce_cpu_baseline(spec, t, seconds: float):
    """The float64 linear cross-entropy oracle, as it stands, on the first
    tokens of the workload (full vocabulary), forward and backward, growing
    the sample until about `seconds` of work; useful TFLOP/s over it."""
    import numpy as np

    from oracle import LinearCE

    f64 = lambda x: x.float().cpu().numpy().astype(np.float64)
    w = f64(t["w"])

    def run(n):
        h = f64(t["h"][:n])
        tg = t["targets"][:n].cpu().numpy()
        g = t["dloss"][:n].cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        o = LinearCE(h, w, tg)
        _, lse = o.forward()
        o.backward(g, lse)
        return time.perf_counter() - t0

    # grow the sample until it takes a tenth of the budget, then size the
    # timed sample to the whole budget from that rate
    n = 8
    spent = run(n)
    while spent < seconds / 10 and n < spec.N:
        n = min(spec.N, 2 * n)
        spent = run(n)
    for _ in range(3):  # (the work has a fixed part: the dW product over the vocabulary)
        if spent >= seconds / 2 or n >= spec.N:
            break
        n = min(spec.N, max(n + 1, int(n * seconds / max(spent, 1e-3))))
        spent = run(n)
    flops = 6.0 * n * spec.V * spec.D
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or threads
    except Exception:
        pass
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the first {n} tokens, full vocabulary, float64 numpy forward + backward "
                      f"(dW included), {spent:.1f} s", "seconds": round(spent, 2),
            "cpu": platform.processor() or platform.machine(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def read_lce_profile(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 summary of
    the linear cross-entropy workload, if it was taken on the current lce.hip
    source; else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_trace_hbm.md")
    if not os.path.exists(path):
        return None
    m = {k: v for k, v in re.findall(r"^(\w+):\s*(\S+)\s*$", open(path).read(), re.M)}
    from block_masked_attention_amd.rocprof import lce_source_hash
    if m.get("kernel_source") != lce_source_hash() or m.get("kernel") != kernel:
        return None
    try:
        return float(m["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def lce_main(args):
    """The linear cross-entropy leg: one step = bdattn_lce_fwd_bwd over the
    whole workload (every chunk: logits product, fused row kernel, dH and dW
    products), inputs resident in device memory."""
    import torch

    import block_masked_attention_amd as bd
    from workloads import LCE_CONFIGS, make_lce_inputs

    spec = next((c for c in LCE_CONFIGS if c.name == args.workload), None)
    if spec is None:
        sys.exit(f"unknown workload {args.workload}")
    if args.lce_chunk:
        from dataclasses import replace
        spec = replace(spec, chunk=args.lce_chunk)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = make_lce_inputs(spec, device=dev)
    p = bd.lce_problem(spec.N, spec.D, spec.V, chunk=spec.chunk)
    N, D, V = spec.N, spec.D, spec.V
    useful = 6.0 * N * V * D
    log(f"[bench] workload {spec.name}: {spec.description}; useful flops/step {useful:.4e}")
    out = (torch.empty(N, device=dev), torch.empty(N, device=dev),
           torch.empty(N, D, dtype=torch.bfloat16, device=dev),
           torch.empty(V, D, dtype=torch.float32, device=dev))
    ws = torch.empty(bd.lce_workspace_size(p, 1), dtype=torch.uint8, device=dev)

    def step():
        bd.lce_fwd_bwd(p, t["h"], t["w"], t["targets"], t["dloss"], workspace=ws, out=out)

    if args.copy_calibration:
        src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] ran one plain device copy of 1 GiB (counter calibration)")

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    bd.profile_read_all()
    bd.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        log(f"[bench] step {i + 1}/{args.steps} enqueued")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    bd.profile_enable(False)
    prof = bd.profile_read_all()
    ms_step = (t1 - t0) * 1e3 / max(1, args.steps)
    value = useful / (ms_step * 1e-3) / 1e12
    n_chunks = -(-N // spec.chunk)
    kern = {}
    for k in bd.LCE_PROFILED:
        r = prof[k]
        ms = r["ms"] / max(1, r["launches"])
        kern[k] = dict(ms=round(ms, 4), launches_per_step=r["launches"] // max(1, args.steps))
    # per launch (one chunk): each product 2*chunk*V*D flops; the row kernel's
    # algorithmic bytes are one read of the chunk's fp32 logits and one write
    # of its bf16 gradient (the kernel reads the logits a second time)
    per_gemm = 2.0 * spec.chunk * V * D
    for k in ("lce_logits", "lce_dh", "lce_dw"):
        kern[k]["tflops"] = round(per_gemm / (kern[k]["ms"] * 1e-3) / 1e12, 1)
    row_bytes = spec.chunk * V * (4 + 2)
    kern["lce_rows"]["gb_per_s"] = round(row_bytes / (kern["lce_rows"]["ms"] * 1e-3) / 1e9, 1)
    dom = max(("lce_logits", "lce_dh", "lce_dw"), key=lambda k: kern[k]["ms"])
    traffic = read_lce_profile(spec.name, dom)
    log(f"[bench] {ms_step:.2f} ms/step, {value:.1f} useful TFLOP/s "
        f"({100 * value / PEAK_BF16_TFLOPS:.1f}% of peak); " +
        ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in kern.items()))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = lce_cpu_baseline(spec, t, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")
    res = {
        "metric": LCE_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "description": spec.description, "tokens": N,
                   "hidden": D, "vocab": V, "chunk": spec.chunk, "chunks": n_chunks,
                   "useful_flops_per_step": useful, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernels": kern,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": kern[dom]["tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern[dom]["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": per_gemm},
        "row_kernel_roofline": {"bound": "hbm", "achieved": kern["lce_rows"]["gb_per_s"],
                                "peak": 8000.0, "unit": "GB/s",
                                "frac": round(kern["lce_rows"]["gb_per_s"] / 8000.0, 4),
                                "bytes_per_launch": row_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="256k",
                    help="workload name (tiny, 8k, 64k, 256k, 512k_rank15; lce_8k, lce_256k "
                         "for the token-chunked linear cross-entropy)")
    ap.add_argument("--precision", choices=("default", "f32-out", "split"), default="default",
                    help="bf16 workloads: float32 outputs (f32-out), or float32 outputs with P "
                         "and dS as two bf16 terms in their products (split); the useful-flop "
                         "count stays 12d per pair and q head")
    ap.add_argument("--clean-mask", choices=("block", "token"), default="block",
                    help="what a clean query sees of its own block: all of it (block-causal, "
                         "the workloads' definition) or the keys up to its own position")
    ap.add_argument("--split-forward", type=int, default=0, metavar="N",
                    help="also time the forward in the split form: the block-diagonal corrupted "
                         "launch plus N clean K/V shards at original positions, merged "
                         "(reported under 'split_forward', after the main timing)")
    ap.add_argument("--docs", type=int, default=1, metavar="N",
                    help="pack N documents into the workload's sequence: N-1 distinct seeded "
                         "random block boundaries cut it (attention stays inside each)")
    ap.add_argument("--gathered", type=int, default=0, metavar="P",
                    help="hold the clean K/V buffer in the zigzag all-gather order of P ranks "
                         "(2P chunks; rank r brings position chunks r and 2P-1-r), each key "
                         "masked by its original position; with --split-forward the clean part "
                         "is one launch over the whole gathered buffer")
    ap.add_argument("--lce-chunk", type=int, default=0, metavar="C",
                    help="linear cross-entropy workloads: tokens per chunk (default: the "
                         "workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("lce"):
        lce_main(args)
        return

    import torch

    import block_masked_attention_amd as bd
    from workloads import GRAD_NAMES, INPUT_NAMES, config, make_inputs

    spec = config(args.workload)
    if args.clean_mask == "token":
        spec = spec.with_(clean_mask=1)
    mask_name = "token-causal" if spec.clean_mask else "block-causal"
    if args.docs > 1:
        import numpy as np
        nb = (spec.clean_q_start + spec.n_clean_q) // spec.B  # blocks of the sequence
        if args.docs > nb:
            sys.exit(f"--docs {args.docs}: the sequence has only {nb} blocks")
        cuts = np.sort(np.random.default_rng(1234).choice(np.arange(1, nb), args.docs - 1,
                                                          replace=False))
        spec = spec.with_(doc_starts=(0,) + tuple(int(c) * spec.B for c in cuts))
    if args.gathered > 0:
        P = args.gathered
        C = spec.n_clean_kv // (2 * P)
        if spec.n_clean_kv % (2 * P) or C % 128 or C % spec.B or spec.clean_kv_start:
            sys.exit(f"--gathered {P}: the clean buffer does not split into 2P chunks of a "
                     "multiple of 128 and of B keys")
        spec = spec.with_(kv_chunk_len=C, kv_chunk_pos=tuple(
            c * C for r in range(P) for c in (r, 2 * P - 1 - r)))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prec = {"default": bd.PRECISION_DEFAULT, "f32-out": bd.PRECISION_F32_OUT,
            "split": bd.PRECISION_SPLIT}[args.precision]
    if prec and (spec.dtype != "bf16" or args.split_forward):
        sys.exit("--precision other than default: bf16 workloads, fused forward only")
    p = bd.from_spec(spec, precision=prec)
    pairs = bd.visible_pairs(p)
    useful_step = 12.0 * spec.d * spec.H * pairs
    log(f"[bench] workload {spec.name}: {spec.description}; visible pairs/head {pairs}; "
        f"useful flops/step {useful_step:.4e}")
    t = make_inputs(spec, device=dev)
    tin = [t[k] for k in INPUT_NAMES]
    dt = t["q_c"].dtype
    H, Hkv, d = spec.H, spec.Hkv, spec.d
    nc, nkv, nx = spec.n_clean_q, spec.n_clean_kv, spec.n_corr
    e = lambda *s, dtype=dt: torch.empty(s, dtype=dtype, device=dev)
    ot = torch.float32 if prec else dt  # O, dQ, dK, dV
    fout = [e(nc, H, d, dtype=ot), e(nx, H, d, dtype=ot), e(H, nc, dtype=torch.float32),
            e(H, nx, dtype=torch.float32)]
    bout = [e(nc, H, d, dtype=ot), e(nx, H, d, dtype=ot), e(nkv, Hkv, d, dtype=ot),
            e(nkv, Hkv, d, dtype=ot), e(nx, Hkv, d, dtype=ot), e(nx, Hkv, d, dtype=ot)]
    ws_f = e(bd.workspace_size(p, 0), dtype=torch.uint8)
    ws_b = e(bd.workspace_size(p, 1), dtype=torch.uint8)

    def step():
        bd.fwd(p, *tin, workspace=ws_f, out=fout)
        bd.bwd(p, *tin, *fout, t["do_c"], t["do_x"], workspace=ws_b, out=bout)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
        log("[bench] ran one plain device copy of 1 GiB (counter calibration)")

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    bd.profile_read()  # drop anything recorded before
    bd.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        log(f"[bench] step {i + 1}/{args.steps} enqueued")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    bd.profile_enable(False)
    prof = bd.profile_read()
    ms_step = (t1 - t0) * 1e3 / max(1, args.steps)
    value = useful_step / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if spec.dtype == "bf16" else PEAK_F32_TFLOPS
    # useful flops per visible pair and q head of each kernel (12d in total:
    # QK^T, PV forward; dP, dV, dK in the dK/dV kernel; dQ in the dQ kernel)
    # and the MFMA flops it executes (recomputed QK^T and dP included)
    useful_d = {"fwd": 4, "bwd_dq": 2, "bwd_dkdv": 6}
    executed_d = {"fwd": 4, "bwd_dq": 6, "bwd_dkdv": 8}
    if prec == bd.PRECISION_SPLIT:  # the products with a split operand run twice
        executed_d = {"fwd": 6, "bwd_dq": 8, "bwd_dkdv": 12}
    kern = {}
    for k, r in prof.items():
        ms = r["ms"] / max(1, r["launches"])
        kern[k] = dict(ms=round(ms, 3),
                       useful_tflops=round(useful_d[k] * d * H * pairs / (ms * 1e-3) / 1e12, 1),
                       executed_tflops=round(executed_d[k] * d * H * pairs / (ms * 1e-3) / 1e12, 1))
    dom = max(kern, key=lambda k: kern[k]["ms"])
    achieved = kern[dom]["useful_tflops"]
    from block_masked_attention_amd.rocprof import profile_key
    traffic, clock = read_profile(profile_key(spec.name, args.docs)
                                  + ("_token_causal" if spec.clean_mask else ""), dom)
    if args.gathered or prec:  # the committed profiles are of the default kernels over
        traffic, clock = None, None  # the position-ordered buffer
    log(f"[bench] {ms_step:.2f} ms/step, {value:.1f} useful TFLOP/s "
        f"({100 * value / peak:.1f}% of {peak} peak); " +
        ", ".join(f"{k} {v['ms']:.2f} ms ({v['useful_tflops']} useful, {v['executed_tflops']} "
                  f"executed TFLOP/s)" for k, v in kern.items()))

    split = None
    if args.split_forward > 0:
        split = time_split_forward(bd, spec, t, args.split_forward, max(1, args.steps))
        log(f"[bench] split forward ({split['shards']} clean launch(es) + block-diagonal part, "
            f"merged): {split['ms']:.2f} ms against {kern['fwd']['ms']:.2f} ms fused")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the float64 oracle on a sample (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(spec, t, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "description": spec.description,
                   "clean_q": nc, "clean_kv": nkv, "corrupted": nx, "B": spec.B, "H": H,
                   "Hkv": Hkv, "d": d, "clean_mask": mask_name, "documents": args.docs,
                   "precision": args.precision,
                   "clean_kv_order": (f"zigzag all-gather of {args.gathered} ranks"
                                      if args.gathered else "positions"),
                   "visible_pairs_per_head": pairs,
                   "useful_flops_per_step": useful_step, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / peak, 2),
        # the same step under the FlashAttention convention (14d per pair and q
        # head: the backward's QK^T recompute counted as work)
        "fa_convention_tflops": round(14.0 * d * H * pairs / (ms_step * 1e-3) / 1e12, 2),
        "fwd_ms": kern["fwd"]["ms"],
        "bwd_ms": round(kern["bwd_dq"]["ms"] + kern["bwd_dkdv"]["ms"], 3),
        "kernels": dict(kern, other_ms=round(ms_step - sum(v["ms"] for v in kern.values()), 3)),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "flops_per_pair_head": f"{useful_d[dom]}*d useful "
                                            f"({executed_d[dom]}*d executed)",
                     # the peak scaled to the kernel's shader clock measured by rocprofv3
                     # (the 2.5 PFLOP/s peak assumes 2.4 GHz), from the same profile
                     "clock_ghz": clock,
                     "frac_at_clock": (round(achieved / (peak * clock / PEAK_CLOCK_GHZ), 4)
                                       if clock else None)},
        "cpu_baseline": cpu,
    }
    if split is not None:
        out["split_forward"] = split
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
