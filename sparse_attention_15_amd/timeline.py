"""Per-workgroup timeline of one decode step: when each workgroup of the decode score kernel
(li_score_decode) and of the attention kernel (sfa_pipe: split and
combine workgroups) starts, finishes its set-up, finishes streaming, and ends.

Runs the timeline variant of the library (libdsa_timeline.so, built with -DDSA_TIMELINE by
sparse_attention_15_amd.build.build_timeline_library): thread 0 of every workgroup records the
GPU's 100 MHz real-time counter at numbered points.  A measurement tool, not part of the library's
path: the stamps cost a few stores per workgroup.

    python -m sparse_attention_15_amd.timeline --workload 2 [--build]

prints a markdown summary: microseconds from the kernel's first workgroup start, as percentiles
over workgroups, plus the per-XCD mean end time (workgroup i runs on XCD i mod 8).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TICK_US = 0.01   # s_memrealtime runs at 100 MHz

DECODE_POINTS = ["start", "set-up done", "streaming done (histogram flushed)"]
SPLIT_POINTS = ["start", "indices resolved + q loaded", "tile loop done", "partial published / output written"]
COMBINE_POINTS = ["start", "all split flags seen", "end"]


def _pcts(x):
    x = np.asarray(x, dtype=np.float64)
    return [np.percentile(x, p) for p in (0, 10, 50, 90, 100)]


def _table(title, names, raw, t0):
    """raw: [workgroups, points] counter stamps (0 = the workgroup did not reach that point)."""
    n = raw.shape[0]
    out = [f"**{title}** ({n} workgroups), us from the first workgroup start:", "",
           "| point | workgroups | min | p10 | p50 | p90 | max |", "|---|---|---|---|---|---|---|"]
    for name, c in zip(names, range(raw.shape[1])):
        hit = raw[:, c] != 0
        if not hit.any():
            out.append(f"| {name} | 0 | - | - | - | - | - |")
            continue
        us = (raw[hit, c].astype(np.int64) - int(t0)) * TICK_US
        out.append(f"| {name} | {int(hit.sum())} | " + " | ".join(f"{v:.1f}" for v in _pcts(us)) + " |")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--build", action="store_true", help="build libdsa_timeline.so first")
    ap.add_argument("--warmup", type=int, default=5)
    args = ap.parse_args()

    from sparse_attention_15_amd import build as B
    if args.build:
        B.build_timeline_library()
    if not os.path.exists(B.TIMELINE_LIB):
        raise ImportError(f"{B.TIMELINE_LIB} not found: run with --build")
    from sparse_attention_15_amd import _lib
    _lib.LIB_PATH = B.TIMELINE_LIB
    import torch
    import sparse_attention_15_amd as dsa
    import workloads as W

    L = _lib.lib()
    for fn in ("dsa_timeline_fetch_indexer", "dsa_timeline_fetch_attn"):
        getattr(L, fn).argtypes = [ctypes.c_void_p, ctypes.c_int]
        getattr(L, fn).restype = ctypes.c_int
    for fn in ("dsa_timeline_reset_indexer", "dsa_timeline_reset_attn"):
        getattr(L, fn).argtypes = []
        getattr(L, fn).restype = ctypes.c_int

    spec = W.config(args.workload)
    c = W.make_case(spec)
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    fp8, mx, kv8 = spec.idx_dtype == "fp8", spec.idx_dtype == "mxfp8", spec.kv_dtype == "fp8"
    if spec.T != 1:
        raise SystemExit("the timeline covers the decode kernels (T = 1)")
    q, w, k = up(c.q_idx), up(c.w), up(c.k_cache)
    qs = None if c.q_scale is None else up(c.q_scale)
    ks = None if c.k_scale is None else up(c.k_scale)
    qa, kv = up(c.q_attn), up(c.kv_codes if kv8 else c.kv_cache)
    kvs = up(c.kv_scale) if kv8 else None
    bt, sl = up(c.block_table), up(c.seq_lens)

    def step():
        idx = dsa.dsa_indexer_topk(q, qs, w, k, ks, bt, sl, T=1, top_k=spec.K, max_seq_len=spec.max_len,
                                   fp8=fp8, mx=mx, num_pages=c.num_pages)
        if kv8:
            dsa.dsa_sparse_attn_fp8kv(qa, kv, kvs, idx, bt, sl, sm_scale=spec.sm_scale, max_seq_len=spec.max_len,
                                      num_pages=c.num_pages)
        else:
            dsa.dsa_sparse_attn(qa, kv, idx, bt, sl, sm_scale=spec.sm_scale, max_seq_len=spec.max_len,
                                num_pages=c.num_pages)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert L.dsa_timeline_reset_indexer() == 0 and L.dsa_timeline_reset_attn() == 0
    step()
    torch.cuda.synchronize()
    n = 8192
    ti = np.zeros((n, 8), dtype=np.uint64)
    ta = np.zeros((n, 8), dtype=np.uint64)
    assert L.dsa_timeline_fetch_indexer(ti.ctypes.data, n) == 0
    assert L.dsa_timeline_fetch_attn(ta.ctypes.data, n) == 0

    lines = [f"# Per-workgroup timeline: {spec.name} (B={spec.B}, ctx {min(spec.lens)}..{max(spec.lens)}, "
             f"K={spec.K}, indexer {spec.idx_dtype}, latent cache {spec.kv_dtype})", "",
             "Command (repo root, GPU box, after `python -c 'import __graft_entry__ as g; g.build()'` here): "
             "`python -m sparse_attention_15_amd.timeline " + " ".join(sys.argv[1:]) + "`", ""]
    wi = np.nonzero(ti[:, 0])[0]
    if wi.size:
        t0 = ti[wi, 0].min()
        lines += _table("li_score_decode", DECODE_POINTS, ti[wi, :3], t0)
        r = (ti[wi, :3].astype(np.int64) - int(t0)) * TICK_US
        xcd = [f"{r[wi % 8 == x, 2].mean():.1f}" for x in range(8)]
        lines += ["", "Streaming done, mean per XCD 0..7: " + ", ".join(xcd) + " us", ""]
        rows = spec.B * spec.T
        sel = ti[:rows]
        if (sel[:, 3] != 0).all():
            lines += _table("li_select (one row per line of stamps)",
                            ["start (first segment)", "digit-0 bin found (first segment)",
                             "candidates collected (segment finishing the row)",
                             "threshold resolved", "indices written"], sel[:, 3:8], t0)
            lines += [""]
    ws = np.nonzero(ta[:, 0])[0]
    wc = np.nonzero(ta[:, 4])[0]
    if ws.size:
        t0 = min(ta[ws, 0].min(), ta[wc, 4].min() if wc.size else ta[ws, 0].min())
        lines += _table("sfa_pipe split workgroups", SPLIT_POINTS, ta[ws, :4], t0)
        if wc.size:
            lines += [""] + _table("sfa_pipe combine workgroups", COMBINE_POINTS, ta[wc, 4:7], t0)
        lines += [""]
    print("\n".join(lines))


if __name__ == "__main__":
    main()
