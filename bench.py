#!/usr/bin/env python3
"""Throughput of one step of indexer-driven top-k sparse attention on one GPU.

Default workload (the one the headline metric is quoted on): HySparse2-style
decode, 32 sequences x 32768 tokens, paged KV (64-token pages, shuffled page
table), 8 KV heads x 128, 64 query heads, indexer 16 heads x 64 (bf16),
forced window 128 + top-1024, 6 query sets (1 FA + 5 SA) reusing one index
tensor.  A step = index score -> window + top-k -> gather attention for all
6 query sets; 192 queries per step.

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Steps rotate over several independent input replicas so that a step's
working set is not already resident in the 256 MB last-level cache.  Each
entry-point call is bracketed by HIP events on the launch stream for the
per-kernel breakdown and the roofline of the dominant kernel.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5] [--workload hysparse2]
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
    if name.startswith("attn_gather_fwd"):
        call = 0 if name == "attn_gather_fwd" else int(name.rsplit("_", 1)[1])
        sets = p.q[call].shape[0]
        ae = _elem(wl.attn_dtype)
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


def recorded_traffic(fam: str, workload: str):
    """HBM bytes per call from the committed counter summary
    profiles/<call>_<workload>_traffic.txt (FETCH_SIZE and WRITE_SIZE per
    dispatch, each scaled by the same counter's reading for a plain copy of
    known size), or None when absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (fam, workload))
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
    kl = logical(p.kidx)
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
            "kind": "oracle",
            "sample": "%d pass(es) over %d of %d decode rows of one replica (whole step: score "
                      "%d entries/row, select, attention for %d query sets), %.1f s" % (
                          reps, n_rows, p.n_rows, int(sl.max()) // wl.stride,
                          sum(x.shape[0] for x in q), dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hysparse2")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="decode rows for the oracle baseline (default: all rows of a step)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time of the oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run a plain copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode shards by sequence with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import index_reuse_amd
    import synth
    from index_reuse_amd.pipeline import Step

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    index_reuse_amd.load()
    dev = torch.device("cuda:0")
    if args.copy_mib > 0:
        calibration_copy(args.copy_mib)
    wl = synth.WORKLOADS[args.workload]
    if wl.prefill:
        raise SystemExit("prefill workloads are benchmarked by their own script")
    steps = []
    for i in range(args.replicas):
        prob = synth.make_problem(wl, device=dev, seed_base=1000 * (wl.cfg_id + 1) + 100 * i)
        steps.append(Step(prob))
    calls = [s.prepare() for s in steps]
    names = [n for n, _ in calls[0]]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    for i in range(args.warmup):
        for _, c in calls[i % len(calls)]:
            c(stream)
    torch.cuda.synchronize()

    K = args.steps
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
    ms_step = elapsed * 1e3 / K
    per_call = {}
    for j, n in enumerate(names):
        per_call[n] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
    gpu_ms_step = sum(evs[i][0].elapsed_time(evs[i][-1]) for i in range(K)) / K

    step0 = steps[0]
    queries = step0.prob.n_rows * sum(q.shape[0] for q in step0.prob.q)
    dom = max(per_call, key=per_call.get)
    traffic = recorded_traffic(call_family(dom), wl.name)
    bytes_dom = algorithmic_bytes(step0, dom)
    achieved = bytes_dom / (per_call[dom] * 1e-3) / 1e9
    kernels = {}
    for n in names:
        b = algorithmic_bytes(step0, n)
        kernels[n] = {"ms": round(per_call[n], 5), "alg_bytes": int(b),
                      "GB/s": round(b / (per_call[n] * 1e-3) / 1e9, 1)}
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s_decode" % wl.name, "batch": wl.n_seqs,
                   "context": wl.seq_len, "window": wl.window, "topk": wl.k,
                   "query_sets": sum(q.shape[0] for q in step0.prob.q), "kv_heads": wl.hkv,
                   "q_heads": wl.hq, "head_dim": wl.dqk, "indexer": "%dx%d %s" % (
                       wl.idx_heads, wl.idx_dim, str(wl.idx_dtype).replace("torch.", "")),
                   "page_size": wl.page_size, "replicas": args.replicas},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "alg_bytes": int(bytes_dom)},
        "gpu_ms_per_step": round(gpu_ms_step, 5),
        "kernels": kernels,
    }
    if not args.no_cpu:
        n = args.cpu_rows if args.cpu_rows > 0 else step0.prob.n_rows
        out["cpu_baseline"] = cpu_baseline(step0, min(n, step0.prob.n_rows), args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
