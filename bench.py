"""Benchmark of the block-sparse paged attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C2]

A step is one call of the hot path over one batch: for the decode workloads
msa_sparse_decode (row positions, top-k compaction, paged gather with
in-register dequant, split attention and merge), for the prefill workload
msa_sparse_prefill.  Inputs are resident in HBM before timing.  Each step
reads a different layer's cache (--layers independent copies, rotated), as a
model's consecutive attention layers do, so no step finds the previous step's
pages in the 256 MB last-level cache.

Prints one JSON line.  value = algorithmic work of a step / wall time per step
over the K timed steps; roofline.achieved = the same work / the average kernel
time of a step from HIP events on the launch stream (one pair around the
timed steps); config.call_ms_median / call_ms_min = the median and the
fastest of the same number of single calls timed one by one after the timed
region (an event pair around each); cpu_baseline = the fp64
CPU oracle timed on a bounded sample of the same workload.

The default run (C2) also times C3 (fp8 multi-token decode), C4 (bf16
prefill) and C5 (NVFP4 decode) in the same process, the same way, and lists
them under config.also, each with its own value, unit and roofline
(--also picks other workloads, e.g. C4/fp8 for the C4 shapes on fp8 pages;
--also "" times the main workload only).
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode gathered-KV GB/s (% HBM peak); prefill sparse-attn TFLOP/s (% MFMA)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix, published
BYTES_PER_TOKEN_HEAD = {"bf16": lambda d: 2 * d * 2, "fp8": lambda d: 2 * d,
                        "nvfp4": lambda d: 2 * (d // 2 + d // 16)}
DESCR = {
    "C1": "tiny decode bf16: 2 requests (seq 1000, 700), dql 1, 4 q / 1 kv heads, head_dim 64, top-k 4",
    "C2": "decode bf16: batch 64, dql 1, 64 q / 8 kv heads, head_dim 128, top-k 16, seq U[4096, 32768]",
    "C3": "multi-token decode fp8 e4m3: batch 32, dql 4, 64 q / 8 kv heads, head_dim 128, top-k 32, "
          "seq U[8192, 65536]",
    "C4": "ragged causal prefill bf16: 2048/4096/8192/8192 new tokens + 64 padded rows, 64 q / 8 kv heads, "
          "head_dim 128, top-k 16",
    "C5": "decode NVFP4: batch 128, dql 1, 64 q / 8 kv heads, head_dim 128, top-k 32, seq U[32768, 131072]",
}


def workload_key(args):
    """Config name, with the page format when --kv-dtype overrides it."""
    return (args.config + (f"/{args.kv_dtype}" if args.kv_dtype else "")
            + (f"/heads{args.heads.replace('/', '-')}" if getattr(args, "heads", None) else "")
            + ("/rows128" if args.layout == "rows128" else "")
            + ("/per-block-selection" if args.selection == "per_block" else ""))


def describe(args):
    d = DESCR[args.config]
    if args.kv_dtype:
        d = d.replace("bf16", args.kv_dtype).replace("fp8 e4m3", args.kv_dtype).replace("NVFP4", args.kv_dtype)
    if getattr(args, "heads", None):
        hq, hkv = args.heads.split("/")
        d = re.sub(r"\d+ q / \d+ kv heads", f"{hq} q / {hkv} kv heads", d)
    if args.layout == "rows128":
        d += ", 128-token pages with K|V-interleaved rows"
    if args.selection == "per_block":
        d += ", rows sharing a 128-token block share one top-k draw (variant, not the named workload)"
    return d


def _cpu_baseline(wl, cache, q, ctx, seconds):
    """Time the CPU oracle on the workload's non-empty rows, eight at a time in
    a fixed random order, until `seconds` of oracle time pass; a workload whose
    rows all finish sooner is walked again (passes counted in the sample)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from tests.helpers import compact_oracle_inputs, oracle_positions

    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    order = rng.permutation(np.flatnonzero(ctx > 0))
    req, pos = oracle_positions(wl)
    done, work, elapsed, passes = 0, 0.0, 0.0, 0
    with threadpool_limits(cores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        while elapsed < seconds and len(order):
            passes += 1
            for start in range(0, len(order), 8):
                rows = order[start:start + 8]
                oc, bt, _, _ = compact_oracle_inputs(wl, cache, rows)
                qf = np.zeros((wl.total_q, wl.num_q_heads, wl.head_dim))
                qf[rows] = q[rows].float().cpu().numpy()
                t0 = time.perf_counter()
                oracle.sparse_attention(qf, oc, wl.topk, bt, req, pos, wl.softmax_scale, rows=rows)
                elapsed += time.perf_counter() - t0
                done += len(rows)
                work += float(ctx[rows].sum())
                if elapsed >= seconds:
                    break
    if wl.mode == "decode":
        value = work * wl.num_kv_heads * BYTES_PER_TOKEN_HEAD[wl.kv_dtype](wl.head_dim) / elapsed / 1e9
        unit = "GB/s"
    else:
        value = work * 4 * wl.head_dim * wl.num_q_heads / elapsed / 1e12
        unit = "TFLOP/s"
    if passes > 1:
        what = f"{passes} passes over the {len(order)} non-empty rows ({done} row evaluations)"
    else:
        what = f"{done} of {wl.total_q} rows (random, non-empty)"
    return {"value": value, "unit": unit, "cores": min(cores, threads), "kind": "oracle",
            "sample": f"{what}, {elapsed:.1f} s of fp64 numpy"}


KERNEL_SOURCES = {
    "decode": ["attend_rows.hip", "msa_device.h", "msa_internal.h"],
    "prefill": ["prefill.hip", "msa_device.h", "msa_internal.h"],
}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(mode):
    """Hash of the code (comments and whitespace dropped) of a mode's kernel sources."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_paged_query_amd", "csrc")
    for f in KERNEL_SOURCES[mode]:
        p = os.path.join(csrc, f)
        if os.path.exists(p):
            text = open(p).read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(config, mode):
    """HBM bytes per launch from a committed counter summary of this config,
    if it was taken on the current kernel sources; else None."""
    if not os.path.isdir(PROFILES):
        return None
    want = kernel_source_hash(mode)
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        for ln in open(os.path.join(PROFILES, name)):
            if ln.startswith("<!-- traffic-json: "):
                d = json.loads(ln[len("<!-- traffic-json: "):].rsplit("-->", 1)[0])
                if d.get("config") == config and d.get("source_hash") == want:
                    return d.get("traffic_bytes")
    return None


def _read_csv(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def _counter_section(args, key):
    """Per-dispatch medians of the SQ counters in --counter-dirs, with the
    matrix-core busy fraction they imply."""
    import numpy as np
    vals = {}
    for d in args.counter_dirs.split(","):
        per = {}
        for r in _read_csv(d):
            if key in r.get("Kernel_Name", "") and "Counter_Name" in r:
                per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for name, by_dispatch in per.items():
            vals[name] = float(np.median(list(by_dispatch.values())))
    out = ["", "Counters (median per dispatch; SQ wave counters count 4-cycle units):", "",
           "| counter | value |", "|---|---|"]
    out += [f"| {k} | {v:.4g} |" for k, v in sorted(vals.items())]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
        # GRBM_GUI_ACTIVE sums the 8 XCDs; the MFMA busy count sums the 4 SIMDs of all 256 CUs
        cycles = vals["GRBM_GUI_ACTIVE"] / 8
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 256 * 4)
        out += ["", f"* matrix cores busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs x 4 SIMDs) "
                f"= {100 * busy:.1f} %"]
    if "SQ_INSTS_MFMA" in vals:
        out += [f"* MFMA instructions: {vals['SQ_INSTS_MFMA']:.4g} x 16384 flop (16x16x32) = "
                f"{vals['SQ_INSTS_MFMA'] * 16384 / 1e12:.3f} Tflop executed per dispatch"]
        if "SQ_INSTS_LDS" in vals:
            out += [f"* LDS instructions per MFMA: {vals['SQ_INSTS_LDS'] / vals['SQ_INSTS_MFMA']:.2f}"]
        if "SQ_INSTS_VALU" in vals:
            out += [f"* other VALU instructions per MFMA: "
                    f"{(vals['SQ_INSTS_VALU'] - vals['SQ_INSTS_MFMA']) / vals['SQ_INSTS_MFMA']:.2f}"]
    if "SQ_WAIT_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
        out += [f"* waves waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES): {100 * vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES']:.1f} %"]
    return out


def summarize(args):
    """Write profiles/<name>.md from rocprofv3 outputs (kernel trace + two counter runs + copy calibration)."""
    import numpy as np
    mode = "prefill" if args.config == "C4" else "decode"
    cfg_key = workload_key(args)
    key = args.kernel
    stats = [r for r in _read_csv(args.trace_dir) if "Calls" in r and key in r["Name"]]
    trace = [r for r in _read_csv(args.trace_dir) if "Start_Timestamp" in r and key in r.get("Kernel_Name", "")]
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace]

    def counter(d, name, kern):
        return [float(r["Counter_Value"]) for r in _read_csv(d)
                if r.get("Counter_Name") == name and kern in r.get("Kernel_Name", "")]
    fetch = counter(args.fetch_dir, "FETCH_SIZE", key)
    write = counter(args.write_dir, "WRITE_SIZE", key)
    cfetch = counter(args.copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cwrite = counter(args.copy_write_dir, "WRITE_SIZE", "copyBuffer")
    copy_kib = args.copy_mib * 1024.0
    fscale = copy_kib / float(np.median(cfetch))
    wscale = copy_kib / float(np.median(cwrite))
    fetch_b = float(np.median(fetch)) * 1024 * fscale
    write_b = float(np.median(write)) * 1024 * wscale
    info = {"config": cfg_key, "kernel": key, "source_hash": kernel_source_hash(mode),
            "avg_ns": float(np.mean(durs)), "dispatches": len(durs),
            "fetch_kib_raw": float(np.median(fetch)), "write_kib_raw": float(np.median(write)),
            "fetch_scale": fscale, "write_scale": wscale,
            "traffic_bytes": fetch_b + write_b}
    lines = [f"# {key}: {cfg_key} ({describe(args)})", "",
             "Commands (run from the repository root on one MI355X; rocprofv3 writes CSVs):", "",
             "```", *args.commands.split(" ;; "), "```", "",
             f"* kernel dispatches traced: {len(durs)}; average duration {np.mean(durs) / 1e3:.2f} us "
             f"(min {min(durs) / 1e3:.2f}, max {max(durs) / 1e3:.2f})",
             f"* FETCH_SIZE per dispatch (median): {info['fetch_kib_raw']:.1f} KiB raw x {fscale:.4f} "
             f"= {fetch_b / 1e6:.2f} MB",
             f"* WRITE_SIZE per dispatch (median): {info['write_kib_raw']:.1f} KiB raw x {wscale:.4f} "
             f"= {write_b / 1e6:.2f} MB",
             f"* copy calibration: a {args.copy_mib} MiB device copy reads {np.median(cfetch):.1f} KiB "
             f"(FETCH_SIZE) and writes {np.median(cwrite):.1f} KiB (WRITE_SIZE)",
             "", "Kernel statistics (rocprofv3 --stats), top entries:", "", "| kernel | calls | avg us | % |",
             "|---|---|---|---|"]
    allstats = sorted([r for r in _read_csv(args.trace_dir) if "Calls" in r and r["Name"] != "KERNEL_DISPATCH"],
                      key=lambda r: -float(r["TotalDurationNs"]))[:8]
    for r in allstats:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {r['Percentage']} |")
    if args.counter_dirs:
        lines += _counter_section(args, key)
    lines += ["", f"<!-- traffic-json: {json.dumps(info)} -->", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(info))


def _ceilings(torch, dev):
    """Measured context for the datasheet fractions: what a plain device copy,
    a plain read (a torch reduction) and a large bf16 GEMM reach on this GPU."""
    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / 1e3 / reps
    n = 4 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    t_read = timed(lambda: src.sum(dtype=torch.float32))
    del dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    b = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    t_mm = timed(lambda: a @ b)
    return {"ceilings": {"copy_GBs": 2 * n / t_copy / 1e9, "read_GBs": n / t_read / 1e9,
                         "bf16_gemm_TFLOPs": 2 * m ** 3 / t_mm / 1e12,
                         "what": "4 GiB device copy (read + write bytes), 4 GiB bf16 sum (read bytes), "
                                 "8192^3 bf16 torch matmul"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C2", choices=sorted(DESCR))
    ap.add_argument("--kv-dtype", choices=["bf16", "fp8", "nvfp4"], default=None,
                    help="page format instead of the workload's own (fp8 / NVFP4 prefill)")
    ap.add_argument("--selection", choices=["independent", "per_block"], default="independent",
                    help="top-k draws: one per row (the named workloads) or one per request and 128-token block")
    ap.add_argument("--layout", choices=["page16", "rows128"], default="page16",
                    help="cache layout (rows128: bf16 / fp8 only)")
    ap.add_argument("--heads", default=None, metavar="Q/KV",
                    help="query / kv head counts instead of the workload's own (e.g. 32/8)")
    ap.add_argument("--layers", type=int, default=4, help="independent caches rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default=None,
                    help="other workloads timed after the main one, comma-separated (e.g. C3,C4,C5,C4/fp8); "
                         "default: C3,C4,C5 when the main one is the default C2, else none")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--ceilings", action="store_true", help="measure copy / read / bf16 GEMM ceilings and exit")
    ap.add_argument("--summarize", action="store_true", help="write a profiles/ summary from rocprofv3 CSVs")
    ap.add_argument("--kernel", default="attend_rows_kernel")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--counter-dirs", default="", help="comma-separated rocprofv3 --pmc outputs of SQ counters")
    ap.add_argument("--commands", default="")
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.also is None:
        default_main = args.config == "C2" and not args.kv_dtype and args.layout == "page16" \
            and args.selection == "independent" and not args.heads
        args.also = "C3,C4,C5" if default_main else ""
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_paged_query_amd as msa

    dev = "cuda"
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    if args.ceilings:
        print(json.dumps(_ceilings(torch, dev)), flush=True)
        return
    primary = measure(args, torch, msa, dev, keep_inputs=not args.no_cpu_baseline)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        wl, cache, q, ctx = primary.pop("_inputs")
        cpu = _cpu_baseline(wl, cache, q, ctx, args.cpu_seconds)
        del wl, cache, q
    primary.pop("_inputs", None)
    torch.cuda.empty_cache()
    # the other named workloads, timed the same way in the same process
    also = []
    for name in [c for c in args.also.split(",") if c]:
        cfg, _, kvd = name.partition("/")
        sub = argparse.Namespace(**vars(args))
        sub.config, sub.kv_dtype, sub.layout, sub.selection = cfg, (kvd or None), "page16", "independent"
        sub.heads = None
        res = measure(sub, torch, msa, dev, keep_inputs=False)
        res.pop("_inputs", None)
        also.append({"workload": res["config"]["workload"], "value": res["value"], "unit": res["unit"],
                     "ms_per_step": res["ms_per_step"], "kernel_ms": res["config"]["kernel_ms"],
                     "call_ms_median": res["config"]["call_ms_median"], "call_ms_min": res["config"]["call_ms_min"],
                     "sum_ctx": res["config"]["sum_ctx"], "tokens_per_s": res["config"]["tokens_per_s"],
                     "dtype": res["dtype"], "roofline": res["roofline"]})
        torch.cuda.empty_cache()
    line = {
        "metric": METRIC, "value": primary["value"], "unit": primary["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": primary["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": primary["dtype"], "data": "synthetic",
        "config": dict(primary["config"], also=also),
        "roofline": primary["roofline"], "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def measure(args, torch, msa, dev, keep_inputs):
    """Build one workload's inputs on the GPU, time K steps after W warm-up
    steps, and return the bench fields of that workload."""
    import numpy as np
    from synth import make_kv_cache, make_query, make_workload, rows128_cache

    over = {"kv_dtype": args.kv_dtype} if args.kv_dtype else {}
    if getattr(args, "heads", None):
        hq, hkv = (int(x) for x in args.heads.split("/"))
        over.update(Hq=hq, Hkv=hkv)
    wl = make_workload(args.config, selection=args.selection, **over)
    print(f"[bench] {workload_key(args)}: building inputs", file=sys.stderr, flush=True)
    cache = make_kv_cache(wl, dev)
    if args.layout == "rows128":
        cache = rows128_cache(cache, wl)
    q = make_query(wl, dev)
    topk = torch.from_numpy(wl.topk).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    seq = torch.from_numpy(wl.seq_lens).to(dev)
    cu = None if wl.cu_seqlens_q is None else torch.from_numpy(wl.cu_seqlens_q).to(dev)
    ks = vs = None
    if wl.kv_dtype != "bf16":
        ks = torch.tensor([cache["k_scale"]], dtype=torch.float32, device=dev)
        vs = torch.tensor([cache["v_scale"]], dtype=torch.float32, device=dev)
    layers = []
    for i in range(max(args.layers, 1)):
        kp = cache["k_pages"] if i == 0 else cache["k_pages"].clone()
        vp = cache["v_pages"]
        if vp is not None and i > 0:
            vp = vp.clone()
        layers.append(msa.KVCache(wl.kv_dtype, kp, vp, wl.num_kv_heads, wl.head_dim, wl.block_page_stride, ks, vs,
                                  layout=cache["layout"]))
    out = torch.empty_like(q)

    # work of one step, from the library's own context lengths
    if wl.mode == "decode":
        _, ctx = msa.msa_build_sparse_block_table(topk, bt, seq_lens=seq, decode_query_len=wl.decode_query_len)
    else:
        qlen = np.diff(wl.cu_seqlens_q)
        req_id, abs_pos = msa.msa_query_token_positions(cu, seq - torch.from_numpy(qlen).to(dev, torch.int32),
                                                         wl.total_q)
        _, ctx = msa.msa_build_sparse_block_table(topk, bt, query_req_id=req_id, query_abs_pos=abs_pos)
    ctx = ctx.cpu().numpy().astype(np.int64)
    sum_ctx = int(ctx.sum())
    if wl.mode == "decode":
        work = sum_ctx * wl.num_kv_heads * BYTES_PER_TOKEN_HEAD[wl.kv_dtype](wl.head_dim)   # bytes
        ws = torch.empty(max(msa.msa_decode_workspace_size(wl.total_q, wl.num_q_heads, wl.head_dim, wl.topk_k), 1),
                         dtype=torch.uint8, device=dev)

        def step(i):
            msa.msa_sparse_decode(q, layers[i % len(layers)], topk, bt, seq, wl.softmax_scale,
                                  decode_query_len=wl.decode_query_len, out=out, workspace=ws)
    else:
        work = 4.0 * wl.head_dim * wl.num_q_heads * sum_ctx                                   # flops
        ws = torch.empty(max(msa.msa_prefill_workspace_size(wl.total_q, wl.num_q_heads, wl.head_dim, wl.topk_k), 1),
                         dtype=torch.uint8, device=dev)

        def step(i):
            msa.msa_sparse_prefill(q, layers[i % len(layers)], topk, bt, cu, seq, wl.softmax_scale, out=out,
                                   workspace=ws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # HIP events on the stream the library launches on (torch's current one),
    # one pair around the whole timed region: back-to-back launches, no
    # per-step event overhead
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    # spread of single calls: the same steps again, an event pair around each
    # (after the timed region, so its figures are not affected)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(pairs):
        e0.record()
        step(i)
        e1.record()
    torch.cuda.synchronize()
    call_ms = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
    if wl.mode == "decode":
        value, unit = work / (ms_per_step * 1e-3) / 1e9, "GB/s"
        achieved = work / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(workload_key(args), "decode")}
        dtype = "f16" if wl.kv_dtype == "nvfp4" else "bf16"
    else:
        value, unit = work / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
        achieved = work / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": profiled_traffic(workload_key(args), "prefill")}
        dtype = "f16" if wl.kv_dtype == "nvfp4" else "bf16"
    res = {"value": value, "unit": unit, "ms_per_step": ms_per_step, "dtype": dtype, "roofline": roof,
           "config": {"workload": f"{workload_key(args)} {describe(args)}", "rows": wl.total_q,
                      "sum_ctx": sum_ctx, "kernel_ms": kernel_ms, "call_ms_median": call_ms[len(call_ms) // 2],
                      "call_ms_min": call_ms[0], "layers": len(layers),
                      "tokens_per_s": wl.total_q / (ms_per_step * 1e-3)}}
    if keep_inputs:
        res["_inputs"] = (wl, cache, q, ctx)
    return res


if __name__ == "__main__":
    main()
