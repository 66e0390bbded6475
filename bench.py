#!/usr/bin/env python3
"""Throughput of one step of indexer-driven top-k sparse attention on one GPU.

Headline workload (the one the metric is quoted on): HySparse2-style decode,
32 sequences x 32768 tokens, paged KV (64-token pages, shuffled page table),
8 KV heads x 128, 64 query heads, indexer 16 heads x 64 (bf16), forced window
128 + top-1024, 6 query sets (1 FA + 5 SA) reusing one index tensor.  A step
= index score -> window + top-k -> gather attention for all 6 query sets; 192
queries per step.  The default run (--workload all) also measures, as extra
records in the same JSON line: HySparse2 with its FA layer, CSA compressed
decode, the CSA2 FP4 layer group, HCA (queries/s), the 64K-row DSA prefill and
the CSA2 prefill group (rows/s).

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Decode steps rotate over several independent input replicas so that a step's
working set is not already resident in the 256 MB last-level cache.  Decode
throughput comes from one HIP graph of the K steps with --inflight (default
4) independent steps in flight on as many streams, as a serving loop overlaps
micro-batches; the strictly serial rate is reported beside it.  Each
entry-point call is also timed alone (a graph of K calls between HIP events)
for the per-kernel breakdown and the roofline of the dominant kernel.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload all] [--inflight 4]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "index_reuse_amd", "csrc")
# sources whose kernels each entry point launches (a traffic record is valid
# only while their text is unchanged)
CALL_SOURCES = {
    "index_score": ("index_score.hip", "common.hpp", "kernels.hpp"),
    "topk_select": ("topk_select.hip", "common.hpp", "kernels.hpp"),
    "attn_gather_fwd": ("attn_gather.hip", "common.hpp", "kernels.hpp"),
    "attn_score": ("attn_score.hip", "common.hpp", "kernels.hpp"),
}
METRIC = "sparse-attn decode queries/s & prefill rows/s at 1 GPU; % HBM/MFMA roofline"


def _elem(dtype) -> int:
    import torch

    return {torch.float32: 4, torch.bfloat16: 2, torch.float8_e4m3fn: 1}[dtype]


def row_geometry(step):
    """Host-side visible-entry counts of every row (the workload is known)."""
    wl = step.wl
    so = step.prob.seq_of_row.cpu().tolist()
    po = step.prob.pos_of_row.cpu().tolist()
    sl = step.prob.seq_len.cpu().tolist()
    out = []
    for b, t in zip(so, po):
        if b < 0 or t < 0:
            out.append((0, 0))
            continue
        n = min(t + 1, sl[b]) // wl.stride
        out.append((n, max(0, n - wl.window)))
    return out


def algorithmic_bytes(step, name: str) -> float:
    """Bytes an ideal implementation of this entry-point call must move."""
    wl, p = step.wl, step.prob
    geo = row_geometry(step)
    R = len(geo)
    ie = _elem(wl.idx_dtype)
    pool_n = int(step.pool_count.sum()) if step.pool_count is not None else 0
    if name == "index_score":
        n = sum(g[0] for g in geo)
        return n * wl.idx_dim * ie + R * wl.idx_heads * (wl.idx_dim * ie + 4) + n * 4
    if name == "index_score_reindex":  # pool members: key rows, positions, scores
        return pool_n * (wl.idx_dim * ie + 4 + 4) + R * wl.idx_heads * (wl.idx_dim * ie + 4)
    if name == "topk_select":
        if wl.block:  # scores of every visible entry, the pool, then top-k inside the pool
            n = sum(g[0] for g in geo)
            return n * 4 + pool_n * 4 + R * (wl.max_blocks * wl.block + wl.k + 2) * 4
        c = sum(g[1] for g in geo)
        return c * 4 + R * (wl.k + 1) * 4
    if name == "topk_select_reindex":  # pool scores and positions -> top-k
        return pool_n * 8 + R * (wl.k + 1) * 4
    fa = hasattr(step, "q_sa")  # HySparse2's FA layer group (FAStep)
    if name == "attn_score":  # every visible K row, queries, lse, one score per entry
        n = sum(g[0] for g in geo)
        ae = _elem(wl.attn_dtype)
        return n * (wl.hkv * wl.dqk * ae + 4) + R * wl.hq * (wl.dqk * ae + 4)
    if name.startswith("attn_gather_fwd"):
        ae = _elem(wl.attn_dtype)
        if fa and name == "attn_gather_fwd_fa":  # dense: every visible entry, the FA set
            n_e = sum(g[0] for g in geo)
            row = wl.hkv * (wl.dqk + wl.dv) * ae if p.v is not None else wl.hkv * wl.dqk * ae
            return n_e * row + R * wl.hq * (wl.dqk + wl.dv) * ae + R * wl.hq * 4
        call = 0 if name in ("attn_gather_fwd", "attn_gather_fwd_fa") else int(name.rsplit("_", 1)[1])
        sets = step.q_sa.shape[0] if fa else p.q[call].shape[0]
        if wl.kv_mode == "fp4":
            row = wl.hkv * (wl.dqk // 2 + wl.dqk // 16)
        elif wl.kv_mode == "shared":
            row = wl.hkv * wl.dqk * ae
        else:
            row = wl.hkv * (wl.dqk + wl.dv) * ae
        n_e = sum((g[0] - g[1]) + min(wl.k, g[1]) for g in geo)
        sel = sum(min(wl.k, g[1]) for g in geo)
        qo = sets * R * wl.hq * (wl.dqk + wl.dv) * ae + sets * R * wl.hq * 4
        return n_e * row + qo + sel * 4
    raise KeyError(name)


def attention_flops(step, call=0) -> float:
    wl, p = step.wl, step.prob
    sets = p.q[call].shape[0]
    n_e = sum((g[0] - g[1]) + min(wl.k, g[1]) for g in row_geometry(step))
    return 2.0 * n_e * sets * wl.hq * (wl.dqk + wl.dv)


def call_family(name: str) -> str:
    for fam in CALL_SOURCES:
        if name == fam or name.startswith(fam + "_"):
            return fam
    raise KeyError(name)


def source_hash(fam: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in CALL_SOURCES[fam]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(call: str, workload: str):
    """HBM bytes per call from the committed counter summary
    profiles/<call>_<workload>_traffic.txt (FETCH_SIZE and WRITE_SIZE per
    dispatch, each scaled by the same counter's reading for a plain copy of
    known size), or None when absent or taken on other kernel sources.  The
    file is named for the call itself (a workload's FA attention call is not
    its sparse attention call), the source check for the call's family."""
    fam = call_family(call)
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (call, workload))
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != source_hash(fam):
        return None
    try:
        return float(rec["traffic_bytes"])
    except (KeyError, ValueError):
        return None


def calibration_copy(mib: int):
    """A plain device copy of known size (read mib MiB, write mib MiB), run
    three times, so a counter run records what FETCH_SIZE / WRITE_SIZE read
    for it."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), for the baseline's
    record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(step, n_rows: int, min_seconds: float):
    """The fp64 oracle on the first ``n_rows`` decode rows of the same inputs
    (whole step: score, select, and attention for every query set; with a
    block pool the Full layer's score + top-k + pool, the Reindex layer's
    rescoring + top-k, and both attention calls), repeated until at least
    ``min_seconds`` of host time have elapsed."""
    import numpy as np

    import oracle

    wl, p = step.wl, step.prob
    rows = list(range(n_rows))
    seqs = sorted({int(p.seq_of_row[r]) for r in rows})
    remap = {b: i for i, b in enumerate(seqs)}
    so = np.array([remap[int(p.seq_of_row[r])] for r in rows], np.int32)
    po = p.pos_of_row[rows].cpu().numpy().astype(np.int32)
    sl = p.seq_len[seqs].cpu().numpy().astype(np.int32)
    cap = wl.n_entries_cap

    def logical(c, which="pool"):
        t = c.pool if which == "pool" else c.scale
        bt = c.block_table[seqs] if c.block_table is not None else None
        t = t if bt is not None else t[seqs]
        return oracle.unpage(t, bt, c.page_size or cap, len(seqs), cap)

    fp4 = wl.kv_mode == "fp4"
    kl = logical(p.kidx) if p.kidx is not None else None
    K = logical(p.k)
    KS = logical(p.k, "scale") if fp4 else None
    V = logical(p.v) if p.v is not None else None
    q_idx = [x[rows].cpu() for x in p.idx_q]
    w = [x[rows].cpu() for x in p.idx_w]
    q = [x[:, rows].cpu() for x in p.q]
    scale = float(np.float32(wl.dqk ** -0.5))
    geo = (so, po, sl, wl.stride)

    def attend(qq, idx, cnt):
        if fp4:
            oracle.attention(*geo, wl.window, qq, K, None, idx, cnt, scale=scale, hkv=wl.hkv,
                             k_scale=KS, v_from_k=True, dv=wl.dv, fp4=True)
        else:
            oracle.attention(*geo, wl.window, qq, K, V, idx, cnt, scale=scale,
                             v_from_k=V is None, dv=wl.dv)

    def one_step():
        if wl.k == 0:  # no selector: the window covers every entry
            attend(q[0], None, None)
            return
        sc = oracle.index_score(*geo, q_idx[0], w[0], kl)
        if not wl.block:
            idx, cnt = oracle.topk_select(*geo, wl.window, sc, wl.k)
            attend(q[0], idx, cnt)
            return
        idx, cnt, pool, pc = oracle.topk_select(*geo, wl.window, sc, wl.k, block=wl.block,
                                                max_blocks=wl.max_blocks)
        rs = oracle.index_score(*geo, q_idx[1], w[1], kl, cand=pool, cand_count=pc)
        ridx, rcnt = oracle.topk_select(*geo, wl.window, rs, wl.k, cand=pool, cand_count=pc)
        attend(q[0], idx, cnt)
        attend(q[1], ridx, rcnt)

    reps = 0
    t0 = time.perf_counter()
    while True:
        one_step()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    queries = reps * n_rows * sum(x.shape[0] for x in q)
    return {"value": round(queries / dt, 3), "unit": "queries/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": "%d pass(es) over %d of %d decode rows of one replica (whole step: score "
                      "%d entries/row, select, attention for %d query sets), %.1f s" % (
                          reps, n_rows, p.n_rows, int(sl.max()) // wl.stride,
                          sum(x.shape[0] for x in q), dt)}


def fa_cpu_baseline(step, n_rows: int, min_seconds: float):
    """The fp64 oracle for HySparse2's FA layer group on the first ``n_rows``
    decode rows: dense attention for the FA set, its head-summed selection
    score, window + top-k, and sparse attention for the SA sets; repeated
    until ``min_seconds`` of host time have elapsed."""
    import numpy as np

    import oracle

    wl, p = step.wl, step.prob
    rows = list(range(n_rows))
    seqs = sorted({int(p.seq_of_row[r]) for r in rows})
    remap = {b: i for i, b in enumerate(seqs)}
    so = np.array([remap[int(p.seq_of_row[r])] for r in rows], np.int32)
    po = p.pos_of_row[rows].cpu().numpy().astype(np.int32)
    sl = p.seq_len[seqs].cpu().numpy().astype(np.int32)
    cap = wl.n_entries_cap

    def logical(c):
        return oracle.unpage(c.pool, c.block_table[seqs], c.page_size, len(seqs), cap)

    K, V = logical(p.k), logical(p.v)
    q = p.q[0][:, rows].cpu()
    scale = float(np.float32(wl.dqk ** -0.5))
    geo = (so, po, sl, wl.stride)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention(*geo, cap, q[0:1], K, V, None, None, scale=scale)
        sc = oracle.fa_score(*geo, q[0:1], K, scale=scale)
        idx, cnt = oracle.topk_select(*geo, wl.window, sc, wl.k)
        oracle.attention(*geo, wl.window, q[1:], K, V, idx, cnt, scale=scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    queries = reps * n_rows * q.shape[0]
    return {"value": round(queries / dt, 3), "unit": "queries/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": "%d pass(es) over %d of %d decode rows of one replica (whole group: dense FA "
                      "attention over %d entries/row, its selection score, select, sparse "
                      "attention for %d SA sets), %.1f s" % (
                          reps, n_rows, p.n_rows, int(sl.max()), q.shape[0] - 1, dt)}


MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}  # MI355X dense


def dense_crossover(row_bytes: int, index_row_bytes: int, k: int) -> float:
    """Context length above which a decode step of top-k sparse attention reads
    fewer bytes than dense attention ("Lecture 10", section 5.3 and exercise
    6): dense reads row_bytes per entry; sparse reads index_row_bytes per
    entry plus k rows, so it wins once L > k row / (row - index_row)."""
    return k * row_bytes / (row_bytes - index_row_bytes)


def layer_group_index_work(n_entries: int, pool: int, n_full: int, n_reindex: int,
                           n_reuse: int):
    """Entries scored per query by one layer group ("CSA, HCA and CSA2",
    sections 3.1 and 6.2): a flat design runs the full-domain indexer in every
    layer; the hierarchical one scans the whole domain once (Full), each
    Reindex layer scores only its pool, and Reuse layers score nothing.
    Returns (flat, hierarchical)."""
    flat = (n_full + n_reindex + n_reuse) * n_entries
    hier = n_full * n_entries + n_reindex * pool
    return flat, hier


def prefill_work(wl, prob):
    """Algorithmic work of one pass over every row of a prefill workload:
    indexer flops (causal pairs x heads x dim x 2), attention flops (gathered
    pairs x heads x (d_qk + d_v) x 2), and selection bytes."""
    return prefill_work_rows(wl, prob.pos_of_row.cpu().numpy(), int(prob.seq_len.max()))


def prefill_work_rows(wl, pos, seq_len: int):
    """prefill_work for query rows at token positions ``pos`` of one sequence
    of ``seq_len`` tokens."""
    import numpy as np

    pos = np.asarray(pos).astype(np.int64)
    n = np.minimum(pos + 1, seq_len) // wl.stride
    pairs = int(n.sum())
    cand = np.maximum(n - wl.window, 0)
    sel = np.minimum(cand, wl.k)
    attn_pairs = int((np.minimum(n, wl.window) + sel).sum())
    out = {
        "index_score": 2.0 * pairs * wl.idx_heads * wl.idx_dim,
        "attn_gather_fwd": 2.0 * attn_pairs * wl.hq * (wl.dqk + wl.dv),
        "topk_select": 4.0 * int(cand.sum()) + 4.0 * len(pos) * (wl.k + 1),
        "pairs": pairs, "attn_pairs": attn_pairs,
    }
    if wl.block:
        # the pool of a row: every candidate while they fit max_blocks blocks,
        # else max_blocks whole blocks (a kept partial last block trims it by
        # fewer than `block` entries: ignored)
        pool = np.minimum(cand, wl.max_blocks * wl.block)
        sel_r = np.minimum(pool, wl.k)
        sets_r = 1 + wl.n_reuse
        out["pool_pairs"] = int(pool.sum())
        out["topk_select"] += 4.0 * int(pool.sum())
        out["index_score_reindex"] = 2.0 * int(pool.sum()) * wl.idx_heads * wl.idx_dim
        out["topk_select_reindex"] = 8.0 * int(pool.sum()) + 4.0 * len(pos) * (wl.k + 1)
        out["attn_gather_fwd_1"] = 2.0 * int(sel_r.sum()) * sets_r * wl.hq * (wl.dqk + wl.dv)
    return out


def prefill_cpu_baseline(prob, n_rows: int, min_seconds: float):
    """The fp64 oracle (score, select, attention) on n_rows rows spread evenly
    over the sequence, repeated until min_seconds have elapsed."""
    import numpy as np

    import oracle

    wl = prob.wl
    R = prob.n_rows
    rows = [int((i + 0.5) * R / n_rows) for i in range(n_rows)]
    so = prob.seq_of_row[rows].cpu().numpy().astype(np.int32)
    po = prob.pos_of_row[rows].cpu().numpy().astype(np.int32)
    sl = prob.seq_len.cpu().numpy().astype(np.int32)
    cap = wl.n_entries_cap

    def logical(c):
        return oracle.unpage(c.pool, c.block_table, c.page_size or cap, wl.n_seqs, cap)

    kl = logical(prob.kidx)
    K = logical(prob.k)
    q_idx = [x[rows].cpu() for x in prob.idx_q]
    w = [x[rows].cpu() for x in prob.idx_w]
    q = [x[:, rows].cpu() for x in prob.q]
    scale = float(np.float32(wl.dqk ** -0.5))
    geo = (so, po, sl, wl.stride)
    reps = 0
    t0 = time.perf_counter()
    while True:
        sc = oracle.index_score(*geo, q_idx[0], w[0], kl)
        if wl.block:  # Full: top-k + pool; Reindex over the pool
            idx, cnt, pool, pc = oracle.topk_select(*geo, wl.window, sc, wl.k, block=wl.block,
                                                    max_blocks=wl.max_blocks)
            rs = oracle.index_score(*geo, q_idx[1], w[1], kl, cand=pool, cand_count=pc)
            ridx, rcnt = oracle.topk_select(*geo, wl.window, rs, wl.k, cand=pool, cand_count=pc)
            oracle.attention(*geo, wl.window, q[1], K, None, ridx, rcnt, scale=scale,
                             v_from_k=True, dv=wl.dv)
        else:
            idx, cnt = oracle.topk_select(*geo, wl.window, sc, wl.k)
        oracle.attention(*geo, wl.window, q[0], K, None, idx, cnt, scale=scale, v_from_k=True,
                         dv=wl.dv)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(reps * n_rows / dt, 3), "unit": "rows/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": "%d pass(es) over %d rows spread evenly over the %d-row prefill (score, "
                      "select, attention), %.1f s" % (reps, n_rows, R, dt)}


def run_prefill(args, wl):
    """Prefill: one step = the hot path over every query row, in row blocks."""
    import torch

    import synth
    from index_reuse_amd.pipeline import PrefillStep

    dev = torch.device("cuda:0")
    prob = synth.make_problem(wl, device=dev)
    step = PrefillStep(prob, row_block=args.row_block, dense_route=True)
    calls = step.prepare()
    names = [n for n, _ in calls]
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = evs[i]
        for j, (_, c) in enumerate(calls):
            e[j].record()
            c()
        e[-1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fam_ms = {}
    for j, n in enumerate(names):
        fam_ms[n] = fam_ms.get(n, 0.0) + sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
    gpu_ms = sum(evs[i][0].elapsed_time(evs[i][-1]) for i in range(K)) / K
    work = prefill_work(wl, prob)
    kernels = {}
    for n, ms in fam_ms.items():
        if n.startswith("topk_select"):
            kernels[n] = {"ms": round(ms, 4), "alg_bytes": int(work[n]),
                          "GB/s": round(work[n] / (ms * 1e-3) / 1e9, 1)}
        else:
            kernels[n] = {"ms": round(ms, 4), "alg_tflop": round(work[n] / 1e12, 3),
                          "TFLOP/s": round(work[n] / (ms * 1e-3) / 1e12, 1)}
    dom = max((n for n in fam_ms if not n.startswith("topk_select")), key=lambda n: fam_ms[n])
    dt = ("fp8" if wl.idx_dtype == torch.float8_e4m3fn and dom.startswith("index_score")
          else "bf16")
    achieved = work[dom] / (fam_ms[dom] * 1e-3) / 1e12
    R = prob.n_rows
    out = {
        "metric": METRIC,
        "value": round(R * K / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 indexer, bf16 attention",
        "data": "synthetic",
        "config": {"workload": wl.name if wl.name.endswith("_prefill") else "%s_prefill" % wl.name,
                   "rows": R, "context": wl.seq_len,
                   "topk": wl.k, "indexer": "%dx%d %s" % (wl.idx_heads, wl.idx_dim,
                                                          str(wl.idx_dtype).replace("torch.", "")),
                   "q_heads": wl.hq, "latent": wl.dqk, "v_width": wl.dv,
                   "row_block": args.row_block, "causal_pairs": work["pairs"],
                   "attention_pairs": work["attn_pairs"], "stride": wl.stride,
                   "pool": wl.max_blocks * wl.block if wl.block else None},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": MFMA_PEAK_TFLOPS[dt], "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS[dt], 4), "traffic": None,
                     "alg_tflop": round(work[dom] / 1e12, 3)},
        "gpu_ms_per_step": round(gpu_ms, 3),
        "kernels": kernels,
    }
    if wl.block:
        # entries scored per query row by the group (Full + Reindex) against
        # a full-domain indexer in both layers
        flat, hier = layer_group_index_work(work["pairs"] / R, work["pool_pairs"] / R, 1, 1,
                                            wl.n_reuse)
        out["index_comparisons_per_query"] = {"hierarchical": round(hier, 1),
                                              "flat": round(flat, 1)}
    if not args.no_cpu:
        out["cpu_baseline"] = prefill_cpu_baseline(prob, args.cpu_rows or 16, args.cpu_seconds)
    del step, prob, calls
    torch.cuda.empty_cache()
    return out


def run_decode(args, wl, fa: bool = False):
    """Decode: one step = every call of the workload's layer group on all its
    rows (``fa``: HySparse2's FA layer selects from its own dense attention
    instead of an indexer); returns the JSON record."""
    import torch

    import synth
    from index_reuse_amd.pipeline import FAStep, Step

    dev = torch.device("cuda:0")
    steps = []
    for i in range(args.replicas):
        prob = synth.make_problem(wl, device=dev, seed_base=1000 * (wl.cfg_id + 1) + 100 * i)
        steps.append(FAStep(prob) if fa else Step(prob, dense_route=True))
    calls = [s.prepare() for s in steps]
    names = [n for n, _ in calls[0]]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    for i in range(args.warmup):
        for _, c in calls[i % len(calls)]:
            c(stream)
    torch.cuda.synchronize()

    # K steps launched from the host, a HIP event before and after every call
    # on the launch stream (gpu_ms_per_step; with --eager also the per-call
    # times and the throughput).
    K = args.steps
    inflight = max(1, min(args.inflight, len(calls)))
    serial_elapsed = None
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = evs[i]
        for j, (_, c) in enumerate(calls[i % len(calls)]):
            e[j].record()
            c(stream)
        e[-1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    mode = "eager"
    per_call = {}
    for j, n in enumerate(names):
        per_call[n] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
    if not args.eager:
        # Per-call times: each call captured K times in a row (cycling over
        # the replicas, on inputs the steps above left in place) and replayed
        # between two HIP events on the launch stream, so no host launch gap
        # sits between its kernels.
        for j, n in enumerate(names):
            gc = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gc):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(K):
                    calls[i % len(calls)][j][1](cs)
            gc.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            gc.replay()
            e1.record()
            torch.cuda.synchronize()
            per_call[n] = e0.elapsed_time(e1) / K
            del gc
        # Throughput: the same K steps captured once as a HIP graph (no host
        # launches between calls, as a serving loop would run them); one
        # untimed replay uploads it, the timed replay runs the K steps.
        # With --inflight n, step i (replica i % R) goes to stream
        # (i % R) % n of the graph: n independent batches in flight, each
        # replica always on the same stream (so no buffer is used by two
        # streams at once), as a serving loop overlaps micro-batches; the
        # serial figure (one stream) is reported next to it.
        def timed_graph(n):
            g = torch.cuda.CUDAGraph()
            sides = [torch.cuda.Stream() for _ in range(n - 1)]
            with torch.cuda.graph(g):
                main = torch.cuda.current_stream()
                for sd in sides:
                    sd.wait_stream(main)
                sts = [main] + sides
                for i in range(K):
                    st = sts[(i % len(calls)) % n]
                    with torch.cuda.stream(st):
                        cs = st.cuda_stream
                        for _, c in calls[i % len(calls)]:
                            c(cs)
                for sd in sides:
                    main.wait_stream(sd)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            del g
            return dt

        serial_elapsed = timed_graph(1)
        elapsed = timed_graph(inflight) if inflight > 1 else serial_elapsed
        mode = "graph" if inflight == 1 else "graph, %d steps in flight" % inflight
    ms_step = elapsed * 1e3 / K
    gpu_ms_step = sum(evs[i][0].elapsed_time(evs[i][-1]) for i in range(K)) / K

    step0 = steps[0]
    queries = step0.prob.n_rows * sum(q.shape[0] for q in step0.prob.q)
    dom = max(per_call, key=per_call.get)
    traffic = recorded_traffic(dom, wl.name)
    bytes_dom = algorithmic_bytes(step0, dom)
    achieved = bytes_dom / (per_call[dom] * 1e-3) / 1e9
    kernels = {}
    for n in names:
        b = algorithmic_bytes(step0, n)
        kernels[n] = {"ms": round(per_call[n], 5), "alg_bytes": int(b),
                      "GB/s": round(b / (per_call[n] * 1e-3) / 1e9, 1)}
    step_bytes = sum(algorithmic_bytes(step0, n) for n in names)
    out = {
        "metric": METRIC,
        "value": round(queries * K / elapsed, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4 kv, bf16" if wl.kv_mode == "fp4" else "bf16",
        "data": "synthetic",
        "config": {"workload": "%s%s_decode" % (wl.name, "_fa" if fa else ""), "batch": wl.n_seqs,
                   "context": wl.seq_len, "window": wl.window, "topk": wl.k,
                   "query_sets": sum(q.shape[0] for q in step0.prob.q), "kv_heads": wl.hkv,
                   "q_heads": wl.hq, "head_dim": wl.dqk, "indexer": (
                       "none: the FA layer's dense attention probabilities" if fa else
                       "none: dense over every entry" if wl.k == 0 else
                       "%dx%d %s" % (wl.idx_heads, wl.idx_dim,
                                     str(wl.idx_dtype).replace("torch.", ""))),
                   "page_size": wl.page_size, "replicas": args.replicas, "launch": mode},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "alg_bytes": int(bytes_dom)},
        "step_roofline": {"alg_bytes": int(step_bytes),
                          "frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "gpu_ms_per_step": round(gpu_ms_step, 5),
        "kernels": kernels,
    }
    if serial_elapsed is not None and inflight > 1:
        out["serial"] = {"value": round(queries * K / serial_elapsed, 1),
                         "ms_per_step": round(serial_elapsed * 1e3 / K, 5)}
    if wl.block:
        # entries scored per query by the layer group (Full + Reindex; the
        # Reuse layers score none), against one full-domain indexer per layer
        n_full = sum(g[0] for g in row_geometry(step0)) / step0.prob.n_rows
        pool = float(step0.pool_count.float().mean())
        flat, hier = layer_group_index_work(n_full, pool, 1, 1, len(step0.prob.q[1]) - 1)
        out["index_comparisons_per_query"] = {"hierarchical": int(hier), "flat": int(flat)}
    if not args.no_cpu:
        n = args.cpu_rows if args.cpu_rows > 0 else step0.prob.n_rows
        if fa:
            out["cpu_baseline"] = fa_cpu_baseline(step0, args.cpu_rows or 2, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(step0, min(n, step0.prob.n_rows), args.cpu_seconds)
    del steps, calls, step0
    torch.cuda.empty_cache()
    return out


# Extra workloads measured by the default run, next to the headline decode.
EXTRA = ("hysparse2_fa", "csa", "csa2", "hca", "dsa", "csa2_prefill")


def achievable_peaks():
    """What plain kernels of this library reach on this GPU (include/sa_peak.h):
    a streaming 16-byte-load HBM read over 4 GiB, and dense MFMA loops in bf16
    (16x16x32) and fp8 (16x16x128).  Context for the roofline fractions, which
    stay against the published peaks."""
    from index_reuse_amd import binding as B

    t = time.perf_counter()
    out = {"hbm_read_GBs": round(B.peak_read_gbs(4 << 30), 1),
           "bf16_mfma_TFLOPs": round(B.peak_mfma_tflops("bf16"), 1),
           "fp8_mfma_TFLOPs": round(B.peak_mfma_tflops("fp8"), 1)}
    print("# achievable peaks in %.1f s: %s" % (time.perf_counter() - t, out), file=sys.stderr,
          flush=True)
    return out


def add_achievable(rec, ach):
    """The dominant call's rate as a fraction of the matching achievable peak."""
    rf = rec.get("roofline")
    if not rf:
        return
    if rf["unit"] == "GB/s":
        ref = ach["hbm_read_GBs"]
    else:
        ref = ach["fp8_mfma_TFLOPs"] if rf["peak"] == MFMA_PEAK_TFLOPS["fp8"] else ach["bf16_mfma_TFLOPs"]
    rf["frac_of_achievable"] = round(rf["achieved"] / ref, 4) if ref else None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="hysparse2, hysparse2_fa, csa, csa2, hca, dsa, csa2_prefill, or all "
                         "(the headline HySparse2 decode, with the other workloads as extra "
                         "records)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="decode rows for the oracle baseline (default: all rows of a step)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time of the oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--row-block", type=int, default=8192,
                    help="prefill: query rows per block (the score buffer holds one block)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run a plain copy of this size first (counter calibration)")
    ap.add_argument("--inflight", type=int, default=4,
                    help="decode: independent steps in flight on that many streams of the timed "
                         "graph (1 = strictly one step after another; at most --replicas)")
    ap.add_argument("--eager", action="store_true",
                    help="decode: launch every call from the host in the timed region instead of "
                         "replaying one captured graph of the K steps")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(decode shards by sequence with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import index_reuse_amd
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    index_reuse_amd.load()
    if args.copy_mib > 0:
        calibration_copy(args.copy_mib)

    def run(name):
        fa = name.endswith("_fa")
        wl = synth.WORKLOADS[name[:-3] if fa else name]
        t = time.perf_counter()
        rec = run_prefill(args, wl) if wl.prefill else run_decode(args, wl, fa=fa)
        print("# %s done in %.1f s" % (name, time.perf_counter() - t), file=sys.stderr, flush=True)
        return rec

    ach = achievable_peaks()
    if args.workload != "all":
        rec = run(args.workload)
        add_achievable(rec, ach)
        rec["achievable"] = ach
        print(json.dumps(rec), flush=True)
        return
    out = run("hysparse2")
    add_achievable(out, ach)
    out["achievable"] = ach
    extra = {}
    for name in EXTRA:
        rec = run(name)
        add_achievable(rec, ach)
        for k in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling",
                  "vs_baseline", "data"):
            rec.pop(k, None)
        extra[rec["config"]["workload"]] = rec
    out["workloads"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
