"""Benchmark: one Ulysses rank's attention hot path on one MI355X.

A step is one pass of the whole hot path for one attention layer on one rank
of a P-way Ulysses job (all-to-all exchange excluded: there is one GPU):
    pack Q, K, V of this rank's sequence slice (send buffers)
    attention forward over the full sequence on this rank's heads
    unpack O back to the rank's slice
    pack dO, attention backward, unpack dQ, dK, dV
Inputs are seeded synthetic tensors resident in HBM before the timed region.

Printed (one JSON line): value = attention FLOPs (algorithmic: causal pairs,
4 d h_q per pair forward, 10 d h_q backward) of one step / step time. The
line also carries forward-only and forward+backward attention rates, the
permute bandwidth of the composite pack (all P ranks' Q, K and V), the
roofline of the dominant kernel (live HIP-event timing through the library's
kernel trace) and the CPU oracle timed on a bounded sample.

--path selects other layouts of the same attention (one JSON line each, no
pack/unpack, no CPU baseline):
  ring   one GPU's share of USP with Ulysses degree U = P / R and ring degree
         R on the same P GPUs: the heads of one Ulysses group (H/U query,
         H_kv/U key/value heads) and the LAST ring rank's block of S/R query
         rows against all R key blocks in ring order (its own block first),
         fp32 partials merged in place, the backward accumulated in fp32
  cp     the heaviest rank of a C-way contiguous context-parallel split: its
         query rows (global offset) against every key up to its last row
  bidir  bidirectional (non-causal) attention over the whole share
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn TFLOP/s fwd & fwd+bwd at S=120K (4Q/1KV heads, d=128); permute GB/s"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0       # HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="s120k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (reported beside the eager time)")
    ap.add_argument("--cpu-sample-rows", type=int, default=24000)
    ap.add_argument("--path", choices=("ulysses", "ring", "cp", "bidir"), default="ulysses")
    ap.add_argument("--ring", type=int, default=4, help="ring degree R for --path ring")
    ap.add_argument("--cp", type=int, default=8, help="context-parallel degree for --path cp")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc runs: one warm-up step, one step, then a plain "
                         "1 GiB device copy that calibrates the byte counters; no JSON line")
    return ap.parse_args()


def causal_pairs(s: int) -> int:
    return s * (s + 1) // 2


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "ulysses_sequence_parallelism_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# kernel -> (source files, algorithmic FLOP per causal pair per query head / d)
KERNELS = {
    "attn_fwd_bf16": (("attn_fwd_bf16.hip", "usp_common.h"), 4),
    # the key-stationary kernel does 4 of the 5 backward products: QK^T, dO V^T,
    # P^T dO, dS^T Q
    "attn_bwd_dkdv_bf16": (("attn_bwd_bf16.hip", "usp_common.h"), 8),
    # the query-stationary kernel does dS K (2d); its QK^T and dO V^T are
    # recomputations beyond the algorithmic count
    "attn_bwd_dq_bf16": (("attn_bwd_bf16.hip", "usp_common.h"), 2),
}


def counter_summary(kernel: str, workload: str) -> dict:
    """Key/value pairs of the committed rocprofv3 counter summary
    (profiles/traffic_<kernel>_<workload>.txt), or {} when absent or taken on
    a different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path) or kernel not in KERNELS:
        return {}
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != src_hash(*KERNELS[kernel][0]):
        return {}
    return kv


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the counter summary, or None."""
    try:
        return float(counter_summary(kernel, workload)["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, rows: int):
    """The fp64 oracle on the causal prefix [0, rows) of the rank's share:
    rows < R only see keys < R, so this is exactly a bounded part of the
    workload. Forward + full backward, all query heads."""
    import numpy as np
    import torch

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    p, r = w.p, min(rows, w.s_pad)
    share = []
    for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
        heads = w.hq_full if t in (workloads.Q, workloads.DO) else w.hkv_full
        x = workloads.tensor(w, t, s=r)   # same draw prefix as the full tensor
        share.append(x[:, : heads // p].to(torch.float64).numpy())
    q, k, v, do = share
    # packed documents: the ones that start inside the prefix, the last cut at r
    cu = None
    if w.thd:
        cu = [c for c in workloads.cu_seqlens(workloads.doc_lengths(w.s)).tolist() if c < r] + [r]
    # the generator draws row-major, so the first r rows equal the full tensor's
    t0 = time.perf_counter()
    o, lse = oracle.attn_fwd(q, k, v, w.scale, r, cu, True)
    oracle.attn_bwd(q, k, v, o, lse, do, w.scale, r, cu, True)
    dt = time.perf_counter() - t0
    pairs = causal_pairs(r) if cu is None else sum(causal_pairs(b - a) for a, b in zip(cu, cu[1:]))
    flops = (4 + 10) * w.d * w.hq * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"causal prefix rows 0..{r - 1} of the {w.name} rank share "
                      f"({w.hq} Q / {w.hkv} KV heads, d={w.d}): fp64 forward + full backward, "
                      f"{dt:.1f} s, {flops / 1e12:.3f} TFLOP algorithmic",
            "seconds": dt, "cpu": platform.processor() or platform.machine()}


def rows_pairs(a: int, b: int, s_valid: int) -> int:
    """Allowed (row, key) pairs of causal rows [a, b) with keys < s_valid."""
    c = min(max(s_valid, a), b)  # rows [a, c) see i + 1 keys, rows [c, b) see s_valid
    return causal_pairs(c) - causal_pairs(a) + (b - c) * s_valid


def interval_path(args, w, dev, share, full):
    """Timed fwd+bwd of the ring, cp or bidir layout; prints one JSON line."""
    import torch

    import ulysses_sequence_parallelism_amd as usp
    import workloads

    q, k, v, do = (share[t] for t in (workloads.Q, workloads.K, workloads.V, workloads.DO))
    s_pad, hq, hkv, d = q.shape[0], w.hq, w.hkv, w.d
    f32 = dict(dtype=torch.float32, device=dev)
    if args.path == "ring":
        r = args.ring
        if r < 1 or w.p % r or w.hkv_full % (w.p // r) or s_pad % r:
            print(f"--ring {r}: needs R | P={w.p}, (P/R) | H_kv and R | s_pad", file=sys.stderr)
            sys.exit(2)
        u = w.p // r
        hq, hkv = w.hq_full // u, w.hkv_full // u
        group = {}
        for t, x in full.items():  # Ulysses head group 0, every row, zero padding rows
            y = torch.zeros((s_pad, x.shape[1] // u, d), dtype=x.dtype, device=dev)
            y[: w.s] = x[:, : x.shape[1] // u]
            group[t] = y
        q, k, v, do = (group[t] for t in (workloads.Q, workloads.K, workloads.V, workloads.DO))
    full.clear()
    torch.cuda.synchronize()
    ws_f = torch.empty(usp.usp_attn_fwd_workspace_bytes(s_pad, hq, hkv, d, 0), dtype=torch.uint8,
                       device=dev)
    # backward scratch for the largest call this layout makes (a short
    # interval can need more than the whole share: dK/dV row-chunk partials)
    if args.path == "ring":
        nb = usp.usp_attn_bwd_interval_workspace_bytes(s_pad // args.ring, s_pad // args.ring, hq,
                                                       hkv, d, 0)
    elif args.path == "cp":
        a_cp = s_pad * (args.cp - 1) // args.cp
        nb = usp.usp_attn_bwd_interval_workspace_bytes(s_pad - a_cp, s_pad, hq, hkv, d, 0)
    else:
        nb = 0
    nb = max(nb, usp.usp_attn_bwd_workspace_bytes(s_pad, hq, hkv, d, 0))
    ws_b = torch.empty(nb, dtype=torch.uint8, device=dev)
    if args.path == "ring":
        blk = s_pad // r
        qa, qb = (r - 1) * blk, s_pad                      # the last ring rank's query rows
        order = [r - 1] + list(range(r - 2, -1, -1))      # own block, then the ring's others
        pairs_alg = rows_pairs(qa, qb, w.s)
        qs, dos = q[qa:qb], do[qa:qb]
        o_fin = torch.empty_like(qs)
        acc_o, acc_l = torch.empty((blk, hq, d), **f32), torch.empty((hq, blk), **f32)
        part_o, part_l = torch.empty((blk, hq, d), **f32), torch.empty((hq, blk), **f32)
        dq = torch.empty((blk, hq, d), **f32)
        dk = torch.empty((s_pad, hkv, d), **f32)
        dv = torch.empty((s_pad, hkv, d), **f32)

        def fwd():
            for step_i, j in enumerate(order):
                ka, kb = j * blk, (j + 1) * blk
                skv = max(0, min(kb, w.s) - ka)
                last = step_i == r - 1
                o_out, l_out = (acc_o, acc_l) if step_i == 0 else (part_o, part_l)
                if r == 1:
                    o_out = o_fin
                usp.usp_attn_fwd_interval(qs, k[ka:kb], v[ka:kb], q_off=qa, k_off=ka,
                                          s_k_valid=skv, softmax_scale=w.scale, out=o_out,
                                          lse=l_out, workspace=ws_f)
                if step_i > 0:
                    usp.usp_attn_merge(acc_o, acc_l, part_o, part_l,
                                       out=o_fin if last else acc_o, lse=acc_l)

        def bwd():
            for t in (dq, dk, dv):
                t.zero_()
            for j in order:
                ka, kb = j * blk, (j + 1) * blk
                skv = max(0, min(kb, w.s) - ka)
                usp.usp_attn_bwd_interval(qs, k[ka:kb], v[ka:kb], o_fin, acc_l, dos, q_off=qa,
                                          k_off=ka, s_k_valid=skv, softmax_scale=w.scale,
                                          accumulate=True, dq=dq, dk=dk[ka:kb], dv=dv[ka:kb],
                                          workspace=ws_b)
        desc = (f"{w.name}: USP on {w.p} GPUs as Ulysses {u} x Ring {r}: one GPU's share is "
                f"{hq} Q / {hkv} KV heads and the last ring rank's query rows [{qa}, {qb}) "
                f"against all {r} key blocks of {blk} in ring order; fp32 partials + in-place "
                f"LSE merge, fp32 accumulated backward; S={w.s}, d={d}, causal")
        causal = True
    elif args.path == "cp":
        c = args.cp
        a, b = s_pad * (c - 1) // c, s_pad
        pairs_alg = rows_pairs(a, b, w.s)
        o = torch.empty((b - a, hq, d), dtype=q.dtype, device=dev)
        lse = torch.empty((hq, b - a), **f32)
        dq = torch.empty((b - a, hq, d), **f32)
        dk = torch.empty((b, hkv, d), **f32)
        dv = torch.empty((b, hkv, d), **f32)
        qs, dos = q[a:b], do[a:b]

        def fwd():
            usp.usp_attn_fwd_interval(qs, k[:b], v[:b], q_off=a, k_off=0, softmax_scale=w.scale,
                                      out=o, lse=lse, workspace=ws_f)

        def bwd():
            usp.usp_attn_bwd_interval(qs, k[:b], v[:b], o, lse, dos, q_off=a, k_off=0,
                                      softmax_scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        desc = (f"{w.name}: last rank of a {c}-way contiguous context-parallel split, query rows "
                f"[{a}, {b}) against keys [0, {b}), causal with the global offset; bf16 O, fp32 "
                f"gradients; {hq} Q / {hkv} KV heads, d={d}")
        causal = True
    else:
        pairs_alg = s_pad * w.s
        o = torch.empty_like(q)
        lse = torch.empty((hq, s_pad), **f32)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def fwd():
            usp.usp_attn_fwd(q, k, v, s_valid=w.s, causal=False, softmax_scale=w.scale, out=o,
                             lse=lse, workspace=ws_f)

        def bwd():
            usp.usp_attn_bwd(q, k, v, o, lse, do, s_valid=w.s, causal=False,
                             softmax_scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        desc = (f"{w.name} rank share, bidirectional (no causal mask), keys past {w.s} masked; "
                f"{hq} Q / {hkv} KV heads, d={d}")
        causal = False

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    usp.usp_trace_enable(True)
    usp.usp_trace_collect()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    usp.usp_trace_enable(False)
    trace = usp.usp_trace_collect()
    step_ms = ev0.elapsed_time(ev1) / args.steps
    per = {e["name"]: e for e in trace}
    f_fwd, f_bwd = 4 * d * hq * pairs_alg, 10 * d * hq * pairs_alg
    fwd_names = ("attn_fwd_kmajor_v", "attn_fwd_bf16", "attn_fwd_merge", "attn_merge")
    fwd_ms = sum(per[n]["total_ms"] for n in fwd_names if n in per) / args.steps
    bwd_ms = sum(e["total_ms"] for e in trace if e["name"] not in fwd_names) / args.steps
    # dominant kernel: its algorithmic FLOPs summed over its launches / its summed time
    dom = max((e for e in trace if e["name"] in KERNELS), key=lambda e: e["total_ms"])
    dom_flops = KERNELS[dom["name"]][1] * d * hq * pairs_alg
    achieved = dom_flops / (dom["total_ms"] / args.steps * 1e-3) / 1e12
    out = {
        "metric": f"attn TFLOP/s fwd+bwd, {args.path} layout",
        "value": round((f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": desc, "seq_len": w.s, "heads_q": hq, "heads_kv": hkv,
                   "head_dim": d, "causal": causal, "path": args.path},
        "attn_fwd_ms": round(fwd_ms, 3), "attn_bwd_ms": round(bwd_ms, 3),
        "attn_fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 1),
        "attn_fwd_bwd_tflops": round((f_fwd + f_bwd) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 1),
        "kernels_ms_per_step": {e["name"]: round(e["total_ms"] / args.steps, 4) for e in trace},
        "kernel_launches_per_step": {e["name"]: e["launches"] // args.steps for e in trace},
        "roofline": {"bound": "mfma", "kernel": dom["name"], "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flop_per_step": dom_flops},
        "cpu_baseline": None,
    }
    if args.path == "ring" and "attn_merge" in per:
        # the merge is HBM-bound: per (row, head) it reads two fp32 O rows and
        # two LSEs and writes one O row (fp32 for the first r-2 merges, bf16
        # for the last) and one LSE
        blk = s_pad // args.ring
        rh = blk * hq
        nbytes = (r - 2) * rh * (d * 12 + 12) + rh * (d * 10 + 12)
        mms = per["attn_merge"]["total_ms"] / args.steps
        out["merge"] = {"launches_per_step": per["attn_merge"]["launches"] // args.steps,
                        "bytes_per_step": nbytes, "ms_per_step": round(mms, 4),
                        "gbps": round(nbytes / (mms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / (mms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share only: the path runs on a single MI355X "
              "(no collectives are built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import ulysses_sequence_parallelism_amd as usp
    import workloads

    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        print("bench workloads: s8k, s32k, s120k, s120k_pad, thd131k", file=sys.stderr)
        sys.exit(2)
    if w.thd and args.path != "ulysses":
        print("--path ring / cp / bidir use the unpacked workloads", file=sys.stderr)
        sys.exit(2)
    # packed documents (host list: the binding checks it and uploads it)
    cu = workloads.cu_seqlens(workloads.doc_lengths(w.s)).tolist() if w.thd else None
    p, s_pad, s_loc = w.p, w.s_pad, w.s_pad // w.p
    hq, hkv, d = w.hq, w.hkv, w.d

    # ---- inputs (seeded, resident in HBM before timing)
    full = {}
    for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
        full[t] = workloads.tensor(w, t).to(dev)
    # this rank's share: the composite pack's slice 0 (what the all-to-all delivers)
    share = {t: usp.usp_pad_pack_seq2head(x, p)[0].contiguous() for t, x in full.items()}
    if args.path != "ulysses":
        interval_path(args, w, dev, share, full)
        return
    q, k, v, do = (share[t] for t in (workloads.Q, workloads.K, workloads.V, workloads.DO))
    # this rank's own sequence slice (all heads): what it packs into send buffers
    local = {t: x[:s_loc].contiguous() for t, x in full.items()}
    send = {t: torch.empty((p, s_loc, x.shape[1] // p, d), dtype=x.dtype, device=dev)
            for t, x in local.items()}
    o = torch.empty_like(q)
    lse = torch.empty((hq, s_pad), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    back = {n: torch.empty((s_loc, p * a.shape[1], d), dtype=a.dtype, device=dev)
            for n, a in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    ws_f = torch.empty(max(1, usp.usp_attn_fwd_workspace_bytes(s_pad, hq, hkv, d, 0)),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(usp.usp_attn_bwd_workspace_bytes(s_pad, hq, hkv, d, 0),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        for t in (workloads.Q, workloads.K, workloads.V):
            usp.usp_pad_pack_seq2head(local[t], p, out=send[t])
        usp.usp_attn_fwd(q, k, v, s_valid=w.s, cu_seqlens=cu, out=o, lse=lse, workspace=ws_f)
        usp.usp_unpack_head2seq(o.view(p, s_loc, hq, d), s_loc, out=back["o"])
        usp.usp_pad_pack_seq2head(local[workloads.DO], p, out=send[workloads.DO])
        usp.usp_attn_bwd(q, k, v, o, lse, do, s_valid=w.s, cu_seqlens=cu, dq=dq, dk=dk, dv=dv,
                         workspace=ws_b)
        for n, a in (("dq", dq), ("dk", dk), ("dv", dv)):
            usp.usp_unpack_head2seq(a.view(p, s_loc, a.shape[1], d), s_loc, out=back[n])

    if args.counters:
        step()
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)  # calibration: reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        print("counters run done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, kernel trace on
    usp.usp_trace_enable(True)
    usp.usp_trace_collect()  # drop anything recorded before
    # one event per step boundary on the current stream: the mean over the K
    # steps is the reported step time, the median and minimum go alongside
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    usp.usp_trace_enable(False)
    trace = usp.usp_trace_collect()
    step_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

    # ---- the same step captured once in a HIP graph and replayed K times
    # (launch overhead off the host; the packed-document offsets go in as a
    # device tensor, which the binding passes without a host copy)
    graph_ms = None
    if not args.no_graph:
        cu_host = cu
        cu = None if cu_host is None else torch.tensor(cu_host, dtype=torch.int32, device=dev)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph
        cu = cu_host

    if cu is not None:
        pairs = sum(causal_pairs(b - a) for a, b in zip(cu, cu[1:]))
    elif w.s == w.s_pad:
        pairs = causal_pairs(w.s_pad)
    else:
        pairs = causal_pairs(w.s) + (w.s_pad - w.s) * w.s
    f_fwd = 4 * d * hq * pairs
    f_bwd = 10 * d * hq * pairs
    per = {e["name"]: e for e in trace}

    def kms(*names):
        return sum(per[n]["total_ms"] for n in names if n in per) / args.steps

    fwd_ms = kms("attn_fwd_kmajor_v", "attn_fwd_bf16", "attn_fwd_merge")
    bwd_ms = kms("attn_bwd_kmajor", "attn_bwd_rowdot_bf16", "attn_bwd_dkdv_bf16",
                 "attn_bwd_dkdv_reduce", "attn_bwd_dq_bf16", "attn_bwd_dq_reduce")
    perm_ms = kms("pack_seq2head", "unpack_head2seq")

    # ---- dominant kernel roofline
    dom = max((e for e in trace if e["name"] in KERNELS), key=lambda e: e["total_ms"])
    dom_avg_ms = dom["total_ms"] / dom["launches"]
    dom_flops = KERNELS[dom["name"]][1] * d * hq * pairs
    achieved = dom_flops / (dom_avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom["name"], "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dom["name"], w.name),
                "avg_launch_ms": round(dom_avg_ms, 4),
                "algorithmic_flop_per_launch": dom_flops}
    # the same kernel against the peak at the clock it ran at in the counter
    # run (the chip is power-limited below 2.4 GHz under this load)
    cs = counter_summary(dom["name"], w.name)
    if "clock_ghz" in cs:
        clk = float(cs["clock_ghz"])
        roofline["counter_clock_ghz"] = round(clk, 3)
        roofline["counter_mfma_busy"] = round(float(cs["mfma_busy"]), 3)
        roofline["frac_at_counter_clock"] = round(achieved / (PEAK_BF16_TFLOPS * clk / 2.4), 4)

    # ---- composite permute bandwidth (all P ranks' Q, K, V; not part of the step).
    # Passes rotate over n_sets buffer sets with n_sets * bytes >= 1 GiB, four
    # times the 256 MB last-level (MALL) cache, so no pass finds its data there.
    pk = (workloads.Q, workloads.K, workloads.V)
    nbytes = int(sum(full[t].numel() * 2 + p * s_pad * (full[t].shape[1] // p) * d * 2 for t in pk))
    n_sets = max(1, -(-(1 << 30) // nbytes))
    srcs = [full] + [{t: full[t].clone() for t in pk} for _ in range(n_sets - 1)]
    ys = [{t: torch.empty((p, s_pad, full[t].shape[1] // p, d), dtype=torch.bfloat16, device=dev)
           for t in pk} for _ in range(n_sets)]
    reps = 20

    def timed(fn, sets=n_sets):
        for i in range(3):
            fn(i % sets)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i % sets)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def pack_all(i):
        for t in pk:
            usp.usp_pad_pack_seq2head(srcs[i][t], p, out=ys[i][t])

    pack_ms = timed(pack_all)
    permute_gbs = nbytes / (pack_ms * 1e-3) / 1e9
    # composite unpack of O: every rank's head-sharded O [P, s_pad, H/P, d]
    # back to [S, H, d], padding rows dropped (bytes: S rows read, S written),
    # rotated over enough sets to exceed 1 GiB like the pack
    hq_full = full[workloads.Q].shape[1]
    ubytes = 2 * w.s * hq_full * d * 2
    u_sets = max(1, -(-(1 << 30) // ubytes))
    uin = [ys[0][workloads.Q].clone() for _ in range(u_sets)]
    del srcs, ys
    uout = [torch.empty((w.s, hq_full, d), dtype=torch.bfloat16, device=dev) for _ in range(u_sets)]
    unpack_ms = timed(lambda i: usp.usp_unpack_head2seq(uin[i], w.s, out=uout[i]), u_sets)
    unpack_gbs = ubytes / (unpack_ms * 1e-3) / 1e9
    del uin, uout
    # reference copy on the same box: torch's device-to-device copy (the
    # runtime's blit kernel) reading and writing the same total number of
    # bytes, rotated the same way
    cin = [torch.empty(nbytes // 2, dtype=torch.uint8, device=dev).fill_(1) for _ in range(n_sets)]
    cout = [torch.empty_like(x) for x in cin]
    copy_ms = timed(lambda i: cout[i].copy_(cin[i]))
    copy_gbs = 2 * (nbytes // 2) / (copy_ms * 1e-3) / 1e9
    del cin, cout

    out = {
        "metric": METRIC if w.name == "s120k" else
                  f"attn TFLOP/s fwd & fwd+bwd, workload {w.name}; permute GB/s",
        "value": round((f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 3),
        "ms_per_step_min": round(per_step[0], 3),
        # the step replayed from a HIP graph (value above is the eager step)
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: one Ulysses rank's attention layer, S={w.s} "
                               f"(s_pad {w.s_pad}), SP degree {p}, {hq} Q / {hkv} KV heads, "
                               f"d={d}, causal"
                               + (f" within {len(cu) - 1} packed documents" if cu else "")
                               + ", forward+backward, pack/unpack of the rank's slice",
                   "seq_len": w.s, "sp_degree": p, "heads_q": hq, "heads_kv": hkv,
                   "head_dim": d, "causal": True},
        "attn_fwd_ms": round(fwd_ms, 3),
        "attn_bwd_ms": round(bwd_ms, 3),
        # key splits of the forward (1: one pass; more on short sequences)
        "attn_fwd_key_splits": usp.usp_attn_fwd_num_splits(
            s_pad, s_pad, hq, hkv, d, 0, s_k_valid=w.s, workspace_bytes=ws_f.numel()),
        "attn_bwd_dq_key_splits": usp.usp_attn_bwd_num_splits(
            s_pad, s_pad, hq, hkv, d, 0, s_k_valid=w.s, workspace_bytes=ws_b.numel()),
        "attn_fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 1),
        "attn_fwd_bwd_tflops": round((f_fwd + f_bwd) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 1),
        "attn_fwd_frac_of_peak": round(f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "attn_fwd_bwd_frac_of_peak": round((f_fwd + f_bwd) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
                                           / PEAK_BF16_TFLOPS, 4),
        "step_permute_ms": round(perm_ms, 4),
        "permute_gbps": round(permute_gbs, 1),
        "permute_frac_of_hbm_peak": round(permute_gbs / PEAK_HBM_GBS, 4),
        "permute_bytes": nbytes,
        "permute_buffer_sets": n_sets,
        "unpack_gbps": round(unpack_gbs, 1),
        "unpack_frac_of_hbm_peak": round(unpack_gbs / PEAK_HBM_GBS, 4),
        "unpack_bytes": ubytes,
        "unpack_buffer_sets": u_sets,
        "d2d_memcpy_gbps": round(copy_gbs, 1),
        "permute_over_d2d_memcpy": round(permute_gbs / copy_gbs, 4),
        "kernels_ms_per_step": {e["name"]: round(e["total_ms"] / args.steps, 4) for e in trace},
        "wall_s_timed": round(t_wall, 3),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
