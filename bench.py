"""Benchmark of the paged MLA decode hot path on one MI355X.

A step is one pass of the whole path over one batch: host split plan (C++),
plan upload (pinned host -> device, async), decode kernel, merge kernel (when a
row is split). Inputs are resident in HBM before the timed region. Successive
steps rotate over three disjoint index lists of the same pool, so a step does
not find the previous step's KV rows in the 256 MB Infinity Cache.

Prints one JSON line. `value` is the effective KV bandwidth of the whole step
(KV bytes gathered / step time); MFMA TFLOP/s (visible pairs only) and the
decode kernel's roofline entry are reported beside it; `cpu_baseline` times
the float64 CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode effective KV GB/s + MFMA TFLOP/s (128 heads, q_len 8, fp8 KV)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
# The sources of the kernels one mla_decode_fwd call launches (decode, merge).
KERNEL_SRCS = [os.path.join(ROOT, "paged_mla_decode_02_amd", "csrc", f) for f in ("decode.hip", "kernels.hip")]
# The source of the latent cache write (mla_cache_write).
CACHE_WRITE_SRCS = [os.path.join(ROOT, "paged_mla_decode_02_amd", "csrc", "cache_write.hip")]


def traffic_srcs(workload):
    """The sources whose kernels a traffic record's workload launches."""
    return CACHE_WRITE_SRCS if workload.startswith("cache_write") else KERNEL_SRCS


def kernel_sha(srcs=None):
    """Hash of the kernel code: the sources with // comments and blank lines
    dropped, so a comment edit does not invalidate a traffic record."""
    h = hashlib.sha256()
    for path in srcs or KERNEL_SRCS:
        for line in open(path, encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def visible_pairs(kv_lens, q_lens, causal):
    total = 0
    for L, q in zip(kv_lens, q_lens):
        L, q = int(L), int(q)
        if causal:
            total += sum(min(max(L - q + i + 1, 0), L) for i in range(q))
        else:
            total += L * q
    return total


def measured_traffic(workload):
    """HBM bytes per launch (decode + merge, or one cache write) from
    committed rocprofv3 counter runs, if they were taken on the current
    kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_sha") != kernel_sha(traffic_srcs(workload)):
        return None
    return d.get("bytes_per_launch")


def traffic_from_counters(workload, fetch_csv, write_csv, copy_mib):
    """HBM bytes per mla_decode_fwd call (or, for a cache_write_* workload,
    per mla_cache_write call) from two rocprofv3 --pmc passes (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch) of `bench.py --copy-mib N`.
    Each counter is divided by what it reads for the known-size device copy
    (the largest __amd_rocclr_copyBuffer dispatch: copy_mib MiB read and
    written). Writes profiles/traffic_<workload>.json and returns it."""
    import csv

    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    out = {"workload": workload, "kernel_sha": kernel_sha(traffic_srcs(workload)), "copy_mib": copy_mib}
    main_kernel, extra = (("cache_write", ()) if workload.startswith("cache_write")
                          else ("decode_kernel", ("merge_kernel", "merge_wide_kernel")))
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_dispatch(path, name)
        copy_kib = max(v for (d, k), v in vals.items() if "copyBuffer" in k)
        factor = copy_kib / (copy_mib * 1024.0)
        decode = [v for (d, k), v in vals.items() if main_kernel in k]
        # (the W-way shard merge of a dcp run is timed on its own, not part of a decode call)
        merge = [v for (d, k), v in vals.items() if any(e in k for e in extra) and "shard_merge" not in k]
        launches = len(decode)
        kib = (sum(decode) + sum(merge)) / launches
        out[name] = {"raw_kib_per_launch": round(kib, 3), "copy_raw_kib": round(copy_kib, 3),
                     "scale": round(factor, 5), "bytes_per_launch": round(kib * 1024.0 / factor),
                     "launches": launches, "merge_dispatches": len(merge)}
        total += kib * 1024.0 / factor
    out["bytes_per_launch"] = round(total)
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_build():
    """numpy's BLAS build (name, version, configuration)."""
    try:
        b = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        return " ".join(str(b.get(k, "")) for k in ("name", "version", "openblas configuration")).strip()
    except Exception:
        return "unknown"


def cpu_baseline(case, budget_s):
    """Time the float64 oracle on whole rows of the workload until about
    budget_s seconds of CPU work (at least one row)."""
    from oracle.attention import attend_case
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    order = list(range(case.rows))
    attend_case(case, rows=order[:1])          # warm-up
    rows_done, keys_done, t_used, passes = 0, 0, 0.0, 0
    elem = 2 if case.kv_dtype == "bf16" else 1
    # Whole rows, in order, wrapping around for further passes, until the
    # budget is used (at least one row).
    while t_used < budget_s:
        for b in order:
            t0 = time.perf_counter()
            attend_case(case, rows=[b])
            t_used += time.perf_counter() - t0
            rows_done += 1
            keys_done += int(case.kv_lens[b])
            if t_used >= budget_s:
                break
        else:
            passes += 1
    return {"value": keys_done * 576 * elem / t_used / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu": host_cpu_model(), "blas": blas_build(),
            "sample": f"{rows_done} row evaluations ({passes} full passes) over the {case.rows} rows of "
                      f"{case.name}, {keys_done} keys, float64 numpy, {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="verify_causal")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work; 0 skips")
    ap.add_argument("--rotate", type=int, default=3, help="disjoint index lists cycled over steps")
    ap.add_argument("--plan", default="auto", choices=["auto", "uniform", "length_aware"],
                    help="split plan mode (the library's default, AUTO, unless asked; the mode it did "
                         "not use is also timed beside it)")
    ap.add_argument("--no-uniform", "--no-other-plan", dest="no_uniform", action="store_true",
                    help="skip the comparison run with the other plan mode (counter passes use this)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before warm-up, one plain device copy of this many MiB: the known-size "
                         "reference for scaling hardware byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="only turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-mib run into profiles/traffic_<workload>.json (with --op cache_write: "
                         "profiles/traffic_cache_write_<kv-dtype>.json)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up steps, run untimed decode calls until the GPU has been busy "
                         "this long and two consecutive batches of 10 calls agree within 2%% (clocks settle "
                         "under sustained load); 0 skips")
    ap.add_argument("--fp8-pv", action="store_true",
                    help="fp8 PV products (plan flag PLAN_FP8_PV; fp8-KV workloads only)")
    ap.add_argument("--merge-in-kernel", action="store_true",
                    help="plan flag PLAN_MERGE_IN_KERNEL (rows with at most 16 splits merged by the decode kernel)")
    ap.add_argument("--graph-replay", type=int, default=0, metavar="N",
                    help="also capture one decode call (plan uploaded, workspace allocated beforehand) "
                         "in a HIP graph and time N back-to-back replays: the launch-amortized call time")
    ap.add_argument("--op", default="decode", choices=["decode", "cache_write", "dcp"],
                    help="decode: the hot path (default); cache_write: the latent cache writer; "
                         "dcp: one decode-context-parallel rank and the shard merge")
    ap.add_argument("--dcp-world", type=int, default=8, help="dcp: ranks")
    ap.add_argument("--heads", type=int, default=64, help="dcp: gathered query heads per rank")
    ap.add_argument("--tokens", type=int, default=65536, help="cache_write: tokens per call")
    ap.add_argument("--kv-dtype", default="fp8", choices=["fp8", "bf16"], help="cache_write: pool dtype")
    args = ap.parse_args()
    if args.traffic_from:
        wl = (f"cache_write_{args.kv_dtype}" if args.op == "cache_write"
              else dcp_workload(args) if args.op == "dcp" else args.workload)
        print(json.dumps(traffic_from_counters(wl, *args.traffic_from, args.copy_mib or 256)))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode has no "
                                   "multi-GPU path in this build (see the design notes on sharding)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    if args.op == "cache_write":
        bench_cache_write(args)
        return
    if args.op == "dcp":
        bench_dcp(args)
        return

    import torch
    import paged_mla_decode_02_amd as mla
    from workloads import make_config

    torch.cuda.set_device(0)
    mla.load_library()
    from workloads import index_set_capacity
    rotate = max(1, min(args.rotate, index_set_capacity(args.workload)))
    case = make_config(args.workload, extra_index_sets=rotate - 1)
    index_sets = [case.kv_indices] + list(case.alt_kv_indices)
    dev = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                            case.qo_indptr, case.kv_indptr, case.kv_indices)
    idx_dev = [dev["kv_indices"]] + [torch.from_numpy(i).cuda() for i in index_sets[1:]]
    inputs = [dict(dev, kv_indices=t) for t in idx_dev]
    plan_modes = {"auto": mla.PLAN_AUTO, "uniform": mla.PLAN_UNIFORM,
                  "length_aware": mla.PLAN_LENGTH_AWARE}
    if args.fp8_pv and case.kv_dtype != "fp8":
        raise SystemExit("--fp8-pv needs a workload with fp8 KV")
    if args.fp8_pv and args.merge_in_kernel:
        raise SystemExit("--fp8-pv does not combine with --merge-in-kernel")
    pv_flag = (mla.PLAN_FP8_PV if args.fp8_pv else 0) | (mla.PLAN_MERGE_IN_KERNEL if args.merge_in_kernel else 0)
    dec = mla.MlaDecoder(case.heads, case.q_len, case.q_dtype, case.kv_dtype, case.causal,
                         float(case.sm_scale), mode=plan_modes[args.plan] | pv_flag)
    T = case.num_tokens
    o = torch.empty((T, case.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, case.heads), dtype=torch.float32, device="cuda")
    kv_lens = case.kv_lens
    stream = torch.cuda.current_stream()
    # Without disjoint index lists to rotate over, each step first overwrites
    # 512 MB (twice the Infinity Cache) so the decode does not find its KV
    # rows cached; the fill is outside the decode's events but inside the step.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if len(inputs) < 2 else None

    def step(k, ev=None, dec=dec):
        words = dec.make_plan(kv_lens)                 # A1: host plan
        plan_dev = dec.upload_plan(words)              # A2: upload
        ws = dec.workspace(words)
        if flush is not None:
            flush.fill_(k & 255)
        if ev is not None:
            ev[0].record(stream)
        mla.decode_fwd(inputs[k % len(inputs)]["q"], dec.q_dtype, dev["q_scale"], dev["kv_pool"],
                       dec.kv_dtype, dev["kv_scale"], dev["qo_indptr"], dev["kv_indptr"],
                       inputs[k % len(inputs)]["kv_indices"], words, plan_dev, case.rows,
                       case.heads, case.q_len, case.causal, float(case.sm_scale), o, lse, ws,
                       stream)
        if ev is not None:
            ev[1].record(stream)
        return words

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    settle = settle_device(step, args.settle_ms) if args.settle_ms > 0 else None
    for k in range(args.warmup):
        words = step(k)
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for k in range(args.steps):
        words = step(k, evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = max(wall * 1e3, gpu_ms) / args.steps
    fwd_ms = [a.elapsed_time(b) for a, b in evs]
    fwd_avg = float(np.mean(fwd_ms))
    fwd_p = [float(x) for x in np.percentile(fwd_ms, [10, 50, 90])]

    plan_info = mla_plan_info(words)
    # The plan mode this run did not use, timed the same way, for comparison.
    other = None
    if not args.no_uniform:
        other_mode = mla.PLAN_LENGTH_AWARE if plan_info["mode"] == "uniform" else mla.PLAN_UNIFORM
        dec_u = mla.MlaDecoder(case.heads, case.q_len, case.q_dtype, case.kv_dtype, case.causal,
                               float(case.sm_scale), mode=other_mode | pv_flag)
        for k in range(args.warmup):
            words_u = step(k, dec=dec_u)
        evs_u = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for k in range(args.steps):
            words_u = step(k, evs_u[k], dec=dec_u)
        torch.cuda.synchronize()
        info_u = mla_plan_info(words_u)
        other = {"plan_mode": info_u["mode"],
                 "launch_ms": round(float(np.mean([a.elapsed_time(b) for a, b in evs_u])), 4),
                 "splits": info_u["S"], "workgroups": info_u["G"]}
    elem = 2 if case.kv_dtype == "bf16" else 1
    keys = int(kv_lens.sum())
    kv_bytes = keys * 576 * elem
    pairs = visible_pairs(kv_lens, case.q_lens, case.causal)
    flops = 2.0 * (576 + 512) * case.heads * pairs
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    tflops_step = flops / (ms_per_step * 1e-3) / 1e12

    # Dominant kernel: the decode kernel (plus the merge, when the plan splits
    # rows, since one mla_decode_fwd call launches both).
    q_elem = 2 if case.q_dtype == "bf16" else 1
    alg_bytes = (kv_bytes + keys * 4 + T * case.heads * 576 * q_elem + T * case.heads * (512 * 2 + 4))
    # QK (576 of every 1088 flops) runs at the fp8 rate with fp8 Q and KV and
    # at the bf16 rate otherwise (bf16 Q against fp8 KV takes two fp8
    # products, hi and lo, per bf16 one); PV at the fp8 rate with the fp8 PV
    # products and at the bf16 rate otherwise. The peak is the rate at which
    # both parts would finish at their own dtype's peak.
    qk_dt = "fp8" if (case.q_dtype == "fp8" and case.kv_dtype == "fp8") else "bf16"
    pv_dt = "fp8" if args.fp8_pv else "bf16"
    compute_dtype = qk_dt if qk_dt == pv_dt else f"{qk_dt}+{pv_dt}"
    peak_tflops = (576 + 512) / (576 / MFMA_PEAK_TFLOPS[qk_dt] + 512 / MFMA_PEAK_TFLOPS[pv_dt])
    achieved_tflops = flops / (fwd_avg * 1e-3) / 1e12
    achieved_gbs = alg_bytes / (fwd_avg * 1e-3) / 1e9
    ridge = peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if flops / alg_bytes > ridge else "hbm"
    traffic = measured_traffic(args.workload)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 2),
                "peak": round(peak_tflops, 1), "unit": "TFLOP/s",
                "frac": round(achieved_tflops / peak_tflops, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic
    roof["kernel"] = "decode_kernel" + (("+merge_wide_kernel" if plan_info["max_splits"] > 16 else "+merge_kernel")
                                        if plan_info["P"] > 0 else "")
    roof["launch_ms"] = round(fwd_avg, 4)
    roof["launch_ms_p10_p50_p90"] = [round(x, 4) for x in fwd_p]
    roof["algorithmic_bytes"] = alg_bytes
    roof["algorithmic_flops"] = flops

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": compute_dtype, "data": "synthetic",
        "config": {"workload": args.workload, "rows": case.rows, "q_len": case.q_len,
                   "heads": case.heads, "q_dtype": case.q_dtype, "kv_dtype": case.kv_dtype,
                   "causal": case.causal, "kv_keys": keys, "pv_dtype": pv_dt, "plan_mode": plan_info["mode"],
                   "merge_in_kernel": bool(args.merge_in_kernel),
                   "splits": plan_info["S"], "workgroups": plan_info["G"],
                   "index_rotation": len(inputs), "cache_flush": flush is not None},
        "mfma_tflops": round(tflops_step, 2),
        "roofline": roof,
    }
    if other is not None:
        ach = flops / (other["launch_ms"] * 1e-3) / 1e12
        other["mfma_frac"] = round(ach / peak_tflops, 4)
        out["other_plan"] = other
    if settle is not None:
        out["settle"] = settle
    if args.graph_replay > 0:
        out["graph_replay"] = graph_replay(args.graph_replay, dec, mla, inputs[0], dev, case, o, lse, flops)
    if args.cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(out), flush=True)


def settle_device(step, settle_ms, batch=10, cap_ms=3000.0):
    """Untimed decode calls until the device has run them for settle_ms and two
    consecutive batches of `batch` calls agree within 2% (or cap_ms of GPU
    time has passed). Under sustained load the GPU's clocks take tens of
    milliseconds to settle; the timed steps should see the settled device,
    as a serving loop does. Returns the calls made and the GPU time spent."""
    import torch
    total, calls, prev = 0.0, 0, None
    while True:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for k in range(batch):
            step(calls + k)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        total += ms
        calls += batch
        if (total >= settle_ms and prev is not None and abs(ms - prev) <= 0.02 * prev) or total >= cap_ms:
            break
        prev = ms
    return {"calls": calls, "gpu_ms": round(total, 2), "last_batch_ms_per_call": round(ms / batch, 4)}


def graph_replay(n, dec, mla, inp, dev, case, o, lse, flops):
    """One mla_decode_fwd call captured in a HIP graph (the plan built and
    uploaded and the workspace allocated before capture), replayed n times
    back to back between two events: the call time with the launch cost
    amortized. The replays recompute the same outputs; the last one is
    compared bit for bit with an eager call."""
    import torch
    words = dec.make_plan(case.kv_lens)
    plan_dev = dec.upload_plan(words)
    ws = dec.workspace(words)
    torch.cuda.synchronize()

    def call():
        mla.decode_fwd(inp["q"], dec.q_dtype, dev["q_scale"], dev["kv_pool"], dec.kv_dtype, dev["kv_scale"],
                       dev["qo_indptr"], dev["kv_indptr"], inp["kv_indices"], words, plan_dev, case.rows,
                       case.heads, case.q_len, case.causal, float(case.sm_scale), o, lse, ws)

    call()
    torch.cuda.synchronize()
    eager = (o.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    for _ in range(10):
        g.replay()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(n):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / n
    same = torch.equal(o.view(torch.int16), eager[0].view(torch.int16)) and torch.equal(lse, eager[1])
    return {"calls": n, "us_per_call": round(us, 3), "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 2),
            "matches_eager": bool(same)}


def bench_cache_write(args):
    """Latent cache write (mla_cache_write): `tokens` rows of bf16 kv_c [512]
    and k_pe [64] into random distinct slots of a fp8 (or bf16) pool. HBM-bound:
    algorithmic bytes = tokens * (576 * 2 read + 576 * elem written + 8 slot)."""
    import torch
    import paged_mla_decode_02_amd as mla
    torch.cuda.set_device(0)
    mla.load_library()
    rng = np.random.default_rng(9)
    T, slots_n = args.tokens, max(4 * args.tokens, 1 << 20)
    kv_dtype = args.kv_dtype
    elem = 1 if kv_dtype == "fp8" else 2
    pool = torch.zeros((slots_n, 576), dtype=torch.uint8 if elem == 1 else torch.int16, device="cuda")
    kv_c = torch.randn((T, 512), device="cuda").to(torch.bfloat16)
    k_pe = torch.randn((T, 64), device="cuda").to(torch.bfloat16)
    slot_sets = [torch.from_numpy(rng.permutation(slots_n)[:T].astype(np.int64)).cuda() for _ in range(3)]
    scale = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if args.copy_mib > 0:   # the known-size reference for the byte counters
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for k in range(args.warmup):
        mla.cache_write(kv_c, k_pe, slot_sets[k % 3], pool, kv_dtype, scale)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record(stream)
        mla.cache_write(kv_c, k_pe, slot_sets[k % 3], pool, kv_dtype, scale)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    alg = T * (576 * 2 + 576 * elem + 8)
    gbs = alg / (launch_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "latent cache write GB/s", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": kv_dtype,
        "data": "synthetic",
        "config": {"workload": "cache_write", "tokens": T, "src": "bf16", "kv_dtype": kv_dtype,
                   "pool_slots": slots_n},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(f"cache_write_{kv_dtype}"),
                     "kernel": "cache_write_fp8x16_kernel" if kv_dtype == "fp8" else "cache_write_bf16_vec_kernel",
                     "launch_ms": round(launch_ms, 4), "algorithmic_bytes": alg}}), flush=True)


def dcp_workload(args):
    return f"dcp_verify_rank0_w{args.dcp_world}_h{args.heads}"


def bench_dcp(args):
    """One decode-context-parallel rank at the verify shape: 32 rows, q_len 8,
    `heads` gathered query heads, bf16, causal; the rows' lengths of the verify
    workload dealt round-robin over `world` ranks (rank 0 measured: its keys
    sit at global positions 0, W, 2W, ...). Also times the W-way shard merge
    (mla_merge_shards) of W bf16 shard results of that shape."""
    import torch
    import paged_mla_decode_02_amd as mla
    from workloads import config_lengths, make_case
    torch.cuda.set_device(0)
    mla.load_library()
    W, H = args.dcp_world, args.heads
    lens = config_lengths("verify_causal")
    case = make_case(2, lens, heads=H, q_len=8, q_dtype="bf16", kv_dtype="bf16", causal=True,
                     pool_slots=524288, name="dcp_verify")
    idx, loc = [], []
    for b in range(case.rows):
        lo, hi = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        part = np.asarray(case.kv_indices[lo:hi])[0::W]
        idx.append(part)
        loc.append(len(part))
    loc = np.array(loc, np.int32)
    indptr = torch.from_numpy(np.concatenate([[0], np.cumsum(loc)]).astype(np.int32)).cuda()
    flat = torch.from_numpy(np.concatenate(idx).astype(np.int32)).cuda()
    dev = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                            case.qo_indptr, case.kv_indptr, case.kv_indices)
    glob = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    words = mla.plan(loc, H, 8, "bf16")
    plan_dev = torch.from_numpy(words).cuda()
    ws = mla.alloc_workspace(words)
    T = case.num_tokens
    o = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    o_parts = torch.randn((W, T, H, 512), device="cuda").to(torch.bfloat16)
    lse_parts = torch.randn((W, T, H), device="cuda")
    om = torch.empty_like(o)
    lm = torch.empty_like(lse)
    stream = torch.cuda.current_stream()
    if args.copy_mib > 0:   # the known-size reference for the byte counters
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def fwd():
        mla.decode_fwd_dcp(dev["q"], "bf16", None, dev["kv_pool"], "bf16", None, dev["qo_indptr"], indptr,
                           flat, words, plan_dev, case.rows, H, 8, True, float(case.sm_scale), o, lse,
                           W, 0, glob, ws)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    settle = settle_device(lambda k: fwd(), args.settle_ms) if args.settle_ms > 0 else None
    t_dec = timed(fwd)
    t_mrg = timed(lambda: mla.merge_shards(o_parts, lse_parts, om, lm))
    keys = int(loc.sum())
    qpos = [(int(L) - 8 + i) for L in lens for i in range(8)]
    pairs = sum(len(range(0, qp + 1, W)) for qp in qpos if qp >= 0)
    flops = 2.0 * (576 + 512) * H * pairs
    tf = flops / (t_dec * 1e-3) / 1e12
    mbytes = W * T * H * (1024 + 4) + T * H * (1024 + 4)
    gbs = mbytes / (t_mrg * 1e-3) / 1e9
    print(json.dumps({
        "metric": "DCP shard decode MFMA TFLOP/s (one rank) + shard merge GB/s", "value": round(tf, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_dec + t_mrg, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dcp_verify_rank0", "dcp_world": W, "heads": H, "rows": case.rows,
                   "q_len": 8, "local_keys": keys, "splits": int(words[14])},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4),
                     "traffic": measured_traffic(dcp_workload(args)),
                     "kernel": "decode_kernel (+merge_kernel if split)", "launch_ms": round(t_dec, 4),
                     "algorithmic_flops": flops},
        "merge": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "shard_merge_kernel",
                  "launch_ms": round(t_mrg, 4), "algorithmic_bytes": mbytes},
        "settle": settle}), flush=True)


def mla_plan_info(words):
    names = ["magic", "version", "R", "H", "q_len_max", "kv_dtype", "C", "mode", "M_UNIT", "u",
             "N_MAX", "MIN_SPLIT_KEYS", "ITEM_OVERHEAD", "OCC", "S", "W", "G", "P"]
    d = dict(zip(names, [int(x) for x in words[:18]]))
    d["mode"] = {1: "uniform", 2: "length_aware"}.get(d["mode"] & 0xFF, d["mode"])
    indptr = np.asarray(words[20:20 + d["R"] + 1], dtype=np.int64)   # split_indptr follows the 20-word header
    d["max_splits"] = int(np.diff(indptr).max()) if d["R"] > 0 else 0
    return d


if __name__ == "__main__":
    main()
