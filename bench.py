"""Benchmark of the DSA decode hot path on one MI355X: dsa_indexer_topk followed by dsa_sparse_attn.

One step = one batch of the workload through both calls (all query rows of the batch).  Inputs are
synthetic (workloads/), resident in HBM before timing, and rotated across copies totalling >= 2 GiB
of touched bytes so the 256 MiB Infinity Cache cannot serve a step from the previous one.

Prints ONE JSON line on stdout.  Progress goes to stderr.

  value       queries/s over exactly --steps steps (barrier + synchronize on both sides)
  roofline    the dominant kernel (the longer of li_score and sfa_main): algorithmic bytes per
              launch / its mean duration, from HIP events the library records around each launch
              during a second, profiled pass over the same steps; peak = 8 TB/s HBM.  `traffic` is
              the kernel's measured HBM bytes per launch (FETCH_SIZE and WRITE_SIZE counters,
              calibrated against a copy of known size) from profiles/traffic.json, used only when
              the recorded source hash and workload match the kernel being timed, else null
  path        whole-step algorithmic bytes / step time, against the same peak and (frac_of_ceiling)
              against the measured streaming-read ceiling
  step_us     median / p10 / p90 of single steps, from a separate pass with an event between steps
  ceiling_gbs HBM streaming-read ceiling measured here: a read-only kernel (libdsa_ceiling.so) over
              256 MiB buffers rotated across 2 GiB, best of several launch shapes
  workloads   with the default workload 2: the same figures for workload 4 (B=8 x 131072, fp8
              indexer) and workload 5 (B=16 x T=4 verify at 65536)
  cpu_baseline  the float64 CPU oracle timed on this host on the first rows of the same batch
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "indexer+SFA decode queries/sec at 32k ctx, K=2048; achieved HBM GB/s % of peak"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def visible(spec, seq_lens):
    """Per row (b, t): number of visible keys n."""
    return [(b, t, int(seq_lens[b]) - spec.T + t + 1) for b in range(spec.B) for t in range(spec.T)]


def algorithmic_bytes(spec, seq_lens):
    """Bytes the method must move per step (no over-fetch, no scratch)."""
    fp8, mx = spec.idx_dtype == "fp8", spec.idx_dtype == "mxfp8"
    elt = 1 if (fp8 or mx) else 2
    mxs = spec.DI // 32 if mx else 0      # MXFP8: one E8M0 byte per 32 elements
    rows = visible(spec, seq_lens)
    k_bytes = 0
    for b in range(spec.B):
        n = int(seq_lens[b])              # keys read once per sequence, shared by its T queries
        pages = (n + 63) // 64
        k_bytes += n * (spec.DI * elt + mxs) + pages * 4 + (pages * 4 if fp8 else 0)
    q_idx = spec.B * spec.T * spec.HI * (spec.DI * elt + mxs + 4 + (4 if fp8 else 0))
    li_score = k_bytes + q_idx
    idx_rw = 2 * spec.B * spec.T * spec.K * 4
    kp = sum(min(spec.K, n) for _, _, n in rows)
    # attention: q rows, bf16 output + lse, the index rows, and the selected latent rows; a causal
    # prefill chunk gathers the same cache-resident rows many times, so each is counted once there
    gathered = sum(int(n) for n in seq_lens) if prefill(spec) else kp
    row_bytes = 576 + 32 if spec.kv_dtype == "fp8" else 1152   # fp8 cache: codes + 8 fp32 tile scales
    sfa = spec.B * spec.T * spec.H * (576 * 2 + 512 * 2 + 4) + gathered * row_bytes
    sfa_main = sfa + spec.B * spec.T * spec.K * 4
    # contraction work: the score over every visible key of the rows that select (n > K), and the
    # two attention products over the K' selected rows
    fl_score = sum(2 * spec.HI * spec.DI * n for _, _, n in rows if n > spec.K)
    fl_sfa = sum(2 * spec.H * (576 + 512) * min(spec.K, n) for _, _, n in rows)
    return dict(li_score=li_score, sfa_main=sfa_main, step=li_score + idx_rw + sfa, sfa=sfa, kp=kp,
                flops=dict(li_score=fl_score, sfa_main=fl_sfa))


def prefill(spec):
    """Causal prefill chunks (more query rows per sequence than the verify kernel takes) are
    MFMA-bound: they report MFMA utilisation rather than HBM bandwidth."""
    return spec.T > 4


# dense MFMA peaks of MI355X by operand type (TFLOP/s)
MFMA_PEAK = {"bf16": 2500.0, "fp8": 5000.0}


KERNEL_SOURCE = {"li_score": "indexer.hip", "sfa_main": "sfa.hip", "fp8_page_append": "quant.hip",
                 "mx_quant_rows (paged)": "quant.hip"}


def recorded_traffic(kernel, workload):
    """Measured HBM bytes per launch of `kernel` on `workload` from profiles/traffic.json, or None
    when absent or taken on a different source of the kernel."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[kernel]
        src = os.path.join(ROOT, "sparse_attention_15_amd", "csrc", KERNEL_SOURCE[kernel])
        if rec["workload"] != workload or rec["source_sha256"] != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
        return int(rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"] +
                   rec["write_kib_per_dispatch"] * 1024 * rec["write_scale"])
    except (OSError, KeyError, ValueError):
        return None


def describe(spec):
    lens = np.asarray(spec.lens)
    kind = {1: "decode", 2: "decode", 3: "causal prefill", 4: "decode, fp8 indexer",
            5: "speculative verify", 6: "decode, MXFP8 indexer",
            7: "causal prefill, MXFP8 indexer", 8: "speculative verify, MXFP8 indexer",
            9: "decode, FP8 latent cache"}.get(spec.cfg_id, "custom")
    return (f"{kind}: B={spec.B} T={spec.T} ctx " +
            (f"{lens.min()}..{lens.max()} (mean {lens.mean():.0f})" if lens.min() != lens.max() else f"{lens[0]}")
            + f", K={spec.K}, indexer {spec.HI}x{spec.DI} {spec.idx_dtype}, attention {spec.H} heads 576/512 "
            + ("bf16 products over an fp8 E4M3 latent cache (fp32 scale per token and 128 columns)"
               if spec.kv_dtype == "fp8" else "bf16") + ", page 64")


def cpu_baseline(case, max_rows: int, budget_s: float, min_s: float = 10.0):
    """Times the float64 oracle on the first rows of the batch (a bounded sample)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    spec = case.spec
    rows = [(b, t) for b in range(spec.B) for t in range(spec.T)]
    dt = spec.idx_dtype
    # passes over the first rows of the batch until about min_s of CPU time (at most budget_s)
    sample = rows[:max_rows]
    done, passes, t0 = 0, 0, time.perf_counter()
    while True:
        for sel in sample:
            idx = oracle.indexer_topk_ref(case.q_idx, case.q_scale, case.w, case.k_cache, case.k_scale,
                                          case.block_table, case.seq_lens, spec.T, spec.K, dt, rows=[sel])
            if spec.kv_dtype == "fp8":
                oracle.sparse_attn_fp8kv_ref(case.q_attn, case.kv_codes, case.kv_scale, case.block_table,
                                             case.seq_lens, idx, spec.sm_scale, rows=[sel])
            else:
                oracle.sparse_attn_ref(case.q_attn, case.kv_cache, case.block_table, case.seq_lens, idx,
                                       spec.sm_scale, rows=[sel])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
        if time.perf_counter() - t0 > min(min_s, budget_s):
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "queries/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} query rows: {passes} pass(es) over the first {len(sample)} of "
                      f"{len(rows)} rows of one step (indexer + attention, float64 NumPy), "
                      f"{el:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2,
                    help="named workload 1..5 (default 2); 6 / 7 / 8 = workload 4 / 3 / 5 with an MXFP8 "
                         "indexer; 9 = workload 2 with an FP8 latent cache")
    ap.add_argument("--rotate-gib", type=float, default=2.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32)
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    ap.add_argument("--no-extra", action="store_true",
                    help="with workload 2, skip the additional workload 4 and 5 entries")
    ap.add_argument("--append-kv8", action="store_true",
                    help="time dsa_latent_cache_append_fp8 instead: 8 sequences x 16384 new latent "
                         "rows (576 bf16) into the FP8 latent cache")
    ap.add_argument("--append", action="store_true",
                    help="time dsa_indexer_cache_append instead: a prefill chunk of MXFP8 keys "
                         "(8 sequences x 65536 tokens x 128 dims) into the paged cache")
    ap.add_argument("--append-fp8", action="store_true",
                    help="time dsa_indexer_cache_append_fp8 instead: a prefill chunk of keys "
                         "(8 sequences x 65536 tokens x 128 dims) into the per-page fp8 cache, "
                         "and a decode step (32 sequences x 1 key into partly filled pages)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_15_amd as dsa
    import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calib_mib} MiB x5")
        return

    if args.append:
        return bench_append(args, dev, dsa)
    if args.append_kv8:
        return bench_append_kv8(args, dev, dsa)
    if args.append_fp8:
        return bench_append_fp8(args, dev, dsa)

    r = run_workload(args.workload, args, dev, torch, dsa, W, None, cpu=not args.no_cpu_baseline)
    res = r["line"]
    extra = {}
    if args.workload == 2 and not args.no_extra:
        for w in (4, 5):
            extra[w] = run_workload(w, args, dev, torch, dsa, W, None, cpu=False)["line"]
    # the ceiling's two-gigabyte streams run after the timed workloads, never just before them
    ceiling = measure_ceiling(dev, torch) if not args.no_ceiling else None
    if ceiling:
        log(f"streaming-read ceiling: {ceiling['gbs']:.1f} GB/s ({ceiling['config']})")
        for line in [res] + list(extra.values()):
            for key in ("path", "roofline"):
                o = line.get(key)
                if o and o.get("unit") == "GB/s":
                    o["frac_of_ceiling"] = round(o["achieved"] / ceiling["gbs"], 4)
    res["ceiling_gbs"] = None if ceiling is None else ceiling["gbs"]
    res["ceiling"] = ceiling
    if extra:
        res["workloads"] = {}
        for w, e in extra.items():
            res["workloads"][str(w)] = {
                "workload": e["config"]["workload"], "ms_per_step": e["ms_per_step"],
                "queries_per_s": e["value"], "step_us": e["step_us"], "path": e["path"],
                "roofline": e["roofline"], "kernels": e["kernels"]}
    print(json.dumps(res), flush=True)


def measure_ceiling(dev, torch, total_gib: float = 2.0, chunk_mib: int = 256, launches: int = 24):
    """HBM streaming-read ceiling: the read-only kernel of libdsa_ceiling.so over chunk_mib-MiB
    buffers, rotated across total_gib GiB so the 256 MiB last-level cache holds none of the next
    chunk, timed with HIP events for several launch shapes; the best shape is the ceiling."""
    import ctypes
    from sparse_attention_15_amd.build import CEILING_LIB
    if not os.path.exists(CEILING_LIB):
        raise ImportError(f"{CEILING_LIB} not found: build it first")
    L = ctypes.CDLL(CEILING_LIB)
    L.dsa_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    L.dsa_stream_read.restype = ctypes.c_int
    nbuf = max(2, int(total_gib * 1024 // chunk_mib))
    nbytes = chunk_mib << 20
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(nbuf)]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for blocks in (512, 1024, 2048, 4096, 8192):
        for unroll in (2, 4, 8, -4, -8):
            def run(k):
                st = L.dsa_stream_read(ctypes.c_void_p(bufs[k % nbuf].data_ptr()), nbytes, blocks, unroll,
                                       ctypes.c_void_p(sink.data_ptr()), stream)
                if st:
                    raise RuntimeError(f"dsa_stream_read returned {st}")
            for k in range(3):
                run(k)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(launches):
                run(k + 3)
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes * launches / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, unroll)
    del bufs
    torch.cuda.empty_cache()
    gbs, blocks, unroll = best
    return {"gbs": round(gbs, 1), "kernel": "stream_read_kernel (libdsa_ceiling.so)",
            "config": f"{blocks} workgroups x 256 threads, {abs(unroll)} 16-B loads in flight per thread"
                      + (", nontemporal" if unroll < 0 else "") + f", {chunk_mib} MiB per launch rotated over "
                      f"{nbuf * chunk_mib / 1024:.0f} GiB, best of 25 launch shapes"}


def percentiles(xs):
    a = np.sort(np.asarray(xs, dtype=np.float64))
    return {"median": round(float(np.percentile(a, 50)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def run_workload(wid, args, dev, torch, dsa, W, ceiling, cpu: bool):
    """One named workload: upload rotated copies, warm up, time exactly args.steps steps, then a
    per-step pass and a profiled pass.  Returns {"line": the JSON fields for this workload}."""
    spec = W.config(wid)
    log("workload", describe(spec))
    t0 = time.perf_counter()
    case = W.make_case(spec)
    log(f"generated inputs in {time.perf_counter() - t0:.1f}s")
    ab = algorithmic_bytes(spec, case.seq_lens)
    R = max(1, math.ceil(args.rotate_gib * 2 ** 30 / ab["step"]))

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    fp8 = spec.idx_dtype == "fp8"
    mx = spec.idx_dtype == "mxfp8"
    kv8 = spec.kv_dtype == "fp8"
    base = dict(q=up(case.q_idx), w=up(case.w), k=up(case.k_cache),
                qs=None if case.q_scale is None else up(case.q_scale),
                ks=None if case.k_scale is None else up(case.k_scale),
                qa=up(case.q_attn), kv=up(case.kv_codes if kv8 else case.kv_cache),
                kvs=up(case.kv_scale) if kv8 else None)
    copies = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(R - 1)]
    bt, sl = up(case.block_table), up(case.seq_lens)
    log(f"uploaded {R} rotation copies ({ab['step'] * R / 2 ** 30:.2f} GiB of touched bytes)")

    layout = dsa.make_layout(bt, sl, case.num_pages, spec.max_len)
    ishape = dsa.IndexerShape(spec.T, spec.HI, spec.DI, spec.K,
                              dsa.DSA_MXFP8_E4M3 if mx else (dsa.DSA_FP8_E4M3 if fp8 else dsa.DSA_BF16))
    ashape = dsa.AttnShape(spec.T, spec.H, 576, 512, spec.K, spec.sm_scale)
    iws = torch.empty(max(256, dsa.dsa_indexer_workspace_size(layout, ishape)), dtype=torch.uint8, device=dev)
    aws_n = dsa.dsa_sparse_attn_workspace_size(layout, ashape)
    aws = torch.empty(max(256, aws_n), dtype=torch.uint8, device=dev)
    idx = torch.empty((spec.B, spec.T, spec.K), dtype=torch.int32, device=dev)
    out = torch.empty((spec.B, spec.T, spec.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((spec.B, spec.T, spec.H), dtype=torch.float32, device=dev)

    import ctypes
    L = dsa.lib()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lref, iref, aref = ctypes.byref(layout), ctypes.byref(ishape), ctypes.byref(ashape)
    calls = []
    for c in copies:   # pre-marshalled arguments: the timed loop only issues the two C calls
        calls.append(((P(c["q"]), P(c["qs"]), P(c["w"]), P(c["k"]), P(c["ks"]), lref, iref, P(idx),
                       P(iws), iws.numel(), stream),
                      ((P(c["qa"]), P(c["kv"]), P(c["kvs"])) if kv8 else (P(c["qa"]), P(c["kv"])))
                      + (P(idx), lref, aref, P(out), P(lse), P(aws), aws.numel(), stream)))
    attn_call = L.dsa_sparse_attn_fp8kv if kv8 else L.dsa_sparse_attn

    def step(i):
        a, b = calls[i % R]
        s1 = L.dsa_indexer_topk(*a)
        s2 = attn_call(*b)
        if s1 or s2:
            raise RuntimeError(L.dsa_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    qps = spec.B * spec.T / (ms * 1e-3)
    log(f"timed {args.steps} steps: {ms * 1e3:.1f} us/step, {qps:,.0f} queries/s")

    # per-step distribution: a separate pass with an event between consecutive steps
    n_ps = max(100, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ps + 1)]
    evs[0].record()
    for i in range(n_ps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_us = percentiles([1e3 * evs[i].elapsed_time(evs[i + 1]) for i in range(n_ps)])
    log(f"per-step us over {n_ps} steps: {step_us}")

    kernels = {}
    roof = None
    if not args.no_profile:
        dsa.dsa_profile_start()
        for i in range(args.steps):
            step(i)
        prof = dsa.dsa_profile_stop()
        kernels = {k: {"launches": n, "mean_us": round(1e3 * t / max(n, 1), 2)} for k, (n, t) in prof.items()}
        log("per-kernel:", json.dumps(kernels))
        cands = [k for k in ("li_score", "sfa_main") if k in prof]
        if cands:
            kern = max(cands, key=lambda k: prof[k][1] / prof[k][0])
            n, t = prof[kern]
            mean_s = t / n * 1e-3
            if prefill(spec):
                # the indexer's E4M3 formats multiply on the fp8 MFMA; attention is bf16
                pk = MFMA_PEAK["fp8" if kern == "li_score" and spec.idx_dtype != "bf16" else "bf16"]
                ach = ab["flops"][kern] / mean_s / 1e12
                roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": pk, "unit": "TFLOP/s",
                        "frac": round(ach / pk, 4), "traffic": None, "kernel": kern,
                        "kernel_mean_us": round(mean_s * 1e6, 2),
                        "algorithmic_flops_per_launch": int(ab["flops"][kern])}
            else:
                ach = ab[kern] / mean_s / 1e9
                roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4),
                        "frac_of_ceiling": None if ceiling is None else round(ach / ceiling["gbs"], 4),
                        "traffic": recorded_traffic(kern, wid), "kernel": kern,
                        "kernel_mean_us": round(mean_s * 1e6, 2),
                        "algorithmic_bytes_per_launch": int(ab[kern])}

    path_gbs = ab["step"] / (ms * 1e-3) / 1e9
    cpu_res = None
    if cpu:
        log("timing the CPU oracle ...")
        cpu_res = cpu_baseline(case, args.cpu_rows, args.cpu_budget)
        log("cpu baseline:", cpu_res)

    lens = np.asarray(spec.lens)
    res = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8+bf16" if mx else ("fp8+bf16" if fp8 else "bf16"),
        "data": "synthetic",
        "config": {"workload": describe(spec), "batch": spec.B, "query_tokens": spec.T,
                   "ctx_min": int(lens.min()), "ctx_max": int(lens.max()), "ctx_mean": float(lens.mean()),
                   "top_k": spec.K, "indexer_heads": spec.HI, "indexer_dim": spec.DI,
                   "attn_heads": spec.H, "page": 64, "rotation_copies": R},
        "roofline": roof,
        "step_us": step_us,
        "path": {"algorithmic_bytes_per_step": int(ab["step"]), "achieved": round(path_gbs, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                 "frac_of_ceiling": None if ceiling is None else round(path_gbs / ceiling["gbs"], 4)},
        "kernels": kernels,
        "cpu_baseline": cpu_res,
    }
    return {"line": res}


def bench_append_kv8(args, dev, dsa):
    """dsa_latent_cache_append_fp8 of a prefill chunk: B sequences x T new latent rows (576 bf16),
    written as E4M3 codes plus 8 fp32 tile scales per token at each token's page and slot.
    Algorithmic bytes per call: 1152 B read + 576 + 32 B written per row (plus the tables)."""
    import torch
    import oracle.quant as oq
    B, T, D = 8, 16384, 576
    P = B * T // 64 + 1
    gen = torch.Generator(device=dev).manual_seed(16)
    perm = torch.randperm(P, device=dev, generator=gen).to(torch.int32)
    bt = perm[:B * T // 64].view(B, T // 64).contiguous()
    sl = torch.full((B,), T, dtype=torch.int32, device=dev)
    nbytes = B * T * (D * 2 + D + 32) + bt.numel() * 4
    R = max(1, math.ceil(args.rotate_gib * 2 ** 30 / nbytes))
    srcs = [(torch.randn(B, T, D, device=dev, generator=gen) / 24).to(torch.bfloat16) for _ in range(R)]
    kcs = [torch.empty(P, 64, D, dtype=torch.uint8, device=dev) for _ in range(R)]
    kss = [torch.empty(P, 64, 8, dtype=torch.float32, device=dev) for _ in range(R)]
    log(f"latent fp8 append: B={B} T={T}, {nbytes / 1e6:.1f} MB per call, {R} rotation copies")

    def step(i):
        j = i % R
        dsa.dsa_latent_cache_append_fp8(srcs[j], kcs[j], kss[j], bt, sl, max_seq_len=T, num_pages=P)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"timed {args.steps} calls: {ms * 1e3:.1f} us/call, {gbs:.1f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's quantiser on the first rows of one call (NumPy float32 / float64)
        x = srcs[0].float().cpu().numpy().reshape(-1, D)
        rows, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oq.latent_fp8_quantize_rows(x[rows % (B * T):rows % (B * T) + 1024])
            rows += 1024
        el = time.perf_counter() - t0
        cpu = {"value": round(rows / el * D * 2 / 1e9, 4), "unit": "GB/s (bf16 read)", "cores": 1,
               "kind": "oracle", "sample": f"{rows} rows of one call in {el:.1f} s"}
    print(json.dumps({
        "metric": "FP8 latent-cache append throughput", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->e4m3",
        "data": "synthetic",
        "config": {"workload": f"latent cache append B={B} T={T} dim={D}, page 64, permuted pages",
                   "rotation_copies": R},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "kv8_append_rows", "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": cpu}), flush=True)


def bench_append(args, dev, dsa):
    """dsa_indexer_cache_append of a prefill chunk: B sequences x T new keys x 128 dims, bf16 in,
    MXFP8 out (E4M3 codes + one E8M0 byte per 32 elements) at each token's page and slot.
    Algorithmic bytes per call: 2 B read + 1 + 1/32 B written per element (plus the tables)."""
    import torch
    import oracle.quant as oq
    B, T, D = 8, 65536, 128
    P = B * T // 64 + 1
    gen = torch.Generator(device=dev).manual_seed(15)
    perm = torch.randperm(P, device=dev, generator=gen).to(torch.int32)
    bt = perm[:B * T // 64].view(B, T // 64).contiguous()
    sl = torch.full((B,), T, dtype=torch.int32, device=dev)
    nbytes = B * T * D * 2 + B * T * D + B * T * D // 32 + bt.numel() * 4
    R = max(1, math.ceil(args.rotate_gib * 2 ** 30 / nbytes))
    srcs = [torch.randn(B, T, D, device=dev, generator=gen).to(torch.bfloat16) for _ in range(R)]
    kcs = [torch.empty(P, 64, D, dtype=torch.uint8, device=dev) for _ in range(R)]
    kss = [torch.empty(P, 64, D // 32, dtype=torch.uint8, device=dev) for _ in range(R)]
    log(f"append: B={B} T={T} D={D}, {nbytes / 1e6:.1f} MB per call, {R} rotation copies")

    def step(i):
        j = i % R
        dsa.dsa_indexer_cache_append(srcs[j], kcs[j], kss[j], bt, sl, max_seq_len=T, num_pages=P)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's quantiser on the first rows of one call (float64 NumPy)
        x = srcs[0].float().cpu().numpy().reshape(-1, D)
        rows, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oq.mxfp8_quantize_rows(x[rows % (B * T):rows % (B * T) + 4096].astype(np.float64))
            rows += 4096
        el = time.perf_counter() - t0
        cpu = {"value": round(rows / el * D * 2 / 1e9, 4), "unit": "GB/s (bf16 read)", "cores": 1,
               "kind": "oracle", "sample": f"{rows} rows of one call in {el:.1f} s"}
    print(json.dumps({
        "metric": "MXFP8 indexer-K cache append throughput", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->mxfp8",
        "data": "synthetic",
        "config": {"workload": f"cache append B={B} T={T} dim={D}, page 64, permuted pages",
                   "rotation_copies": R},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("mx_quant_rows (paged)", "append"),
                     "kernel": "mx_quant_rows (paged)", "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": cpu}), flush=True)


def bench_append_fp8(args, dev, dsa):
    """dsa_indexer_cache_append_fp8 of a prefill chunk: B sequences x T new keys x 128 dims, bf16
    in, E4M3 codes out with one fp32 scale per 64-key page, into fresh permuted pages.
    Algorithmic bytes per call: 2 B read + 1 B written per element, plus 4 B of scale written and
    4 B of table read per page.  Also times a decode step: 32 sequences appending one key each to
    pages that already hold keys (launch-bound; reported as us per call)."""
    import torch
    import oracle.quant as oq
    B, T, D = 8, 65536, 128
    P = B * T // 64 + 1
    gen = torch.Generator(device=dev).manual_seed(17)
    perm = torch.randperm(P, device=dev, generator=gen).to(torch.int32)
    bt = perm[:B * T // 64].view(B, T // 64).contiguous()
    sl = torch.full((B,), T, dtype=torch.int32, device=dev)
    nbytes = B * T * D * 2 + B * T * D + bt.numel() * (4 + 4)
    R = max(1, math.ceil(args.rotate_gib * 2 ** 30 / nbytes))
    srcs = [(torch.randn(B, T, D, device=dev, generator=gen) / math.sqrt(D)).to(torch.bfloat16) for _ in range(R)]
    kcs = [torch.empty(P, 64, D, dtype=torch.uint8, device=dev) for _ in range(R)]
    kss = [torch.empty(P, dtype=torch.float32, device=dev) for _ in range(R)]
    log(f"fp8 page append: B={B} T={T} D={D}, {nbytes / 1e6:.1f} MB per call, {R} rotation copies")

    def step(i):
        j = i % R
        dsa.dsa_indexer_cache_append_fp8(srcs[j], kcs[j], kss[j], bt, sl, max_seq_len=T, num_pages=P)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms = timed(step, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"timed {args.steps} calls: {ms * 1e3:.1f} us/call, {gbs:.1f} GB/s")

    # decode step: sequence b of 32 holds lens[b] - 1 keys (in pages the prefill chunk filled) and
    # appends one; lengths are spread over the slot offsets of a page.  After the first call the
    # key fits the page's scale, so the timed calls re-encode nothing
    Bd = 32
    lens_d = torch.tensor([1000 + 197 * b for b in range(Bd)], dtype=torch.int32, device=dev)
    bt_d = perm[:Bd * 112].view(Bd, 112).contiguous()      # 112 pages = 7168 positions per sequence
    new_d = (torch.randn(Bd, 1, D, device=dev, generator=gen) / math.sqrt(D)).to(torch.bfloat16)

    def dstep(i):
        dsa.dsa_indexer_cache_append_fp8(new_d, kcs[0], kss[0], bt_d, lens_d, max_seq_len=112 * 64,
                                         num_pages=P)

    for i in range(args.warmup):
        dstep(i)
    torch.cuda.synchronize()
    ms_d = timed(dstep, args.steps)
    log(f"decode step B={Bd}: {ms_d * 1e3:.2f} us/call")
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's append over the first sequences of one call (NumPy float32 / float64)
        x = srcs[0].float().cpu().numpy()
        btn, ksn = bt.cpu().numpy(), np.zeros(P, np.float32)
        kcn = np.zeros((P, 64, D), np.uint8)
        keys, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            n = 4096
            oq.indexer_cache_append_fp8_ref(x[:1, :n], kcn, ksn, btn[:1], np.array([n]), n)
            keys += n
        el = time.perf_counter() - t0
        cpu = {"value": round(keys / el * D * 2 / 1e9, 4), "unit": "GB/s (bf16 read)", "cores": 1,
               "kind": "oracle", "sample": f"{keys} keys of one call in {el:.1f} s"}
    print(json.dumps({
        "metric": "fp8 per-page indexer-K cache append throughput", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->e4m3",
        "data": "synthetic",
        "config": {"workload": f"cache append B={B} T={T} dim={D}, page 64, permuted fresh pages",
                   "rotation_copies": R},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("fp8_page_append", "append-fp8"),
                     "kernel": "fp8_page_append", "algorithmic_bytes_per_launch": nbytes},
        "decode_step": {"batch": Bd, "T": 1, "us_per_call": round(ms_d * 1e3, 2)},
        "cpu_baseline": cpu}), flush=True)


if __name__ == "__main__":
    main()
