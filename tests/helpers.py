"""Test-side glue: run the oracle on a synth.Problem, move problems between
devices, and the comparison rules for indices and outputs."""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

import oracle
import synth

# Output tolerances.  bf16 / FP4: the bars the method is held to; f32: the
# accumulated rounding of fp32 dot products and softmax over <= ~1e3 entries.
TOL = {
    torch.bfloat16: dict(max_abs=1e-2, rel_l2=5e-3, lse=1e-3),
    torch.float32: dict(max_abs=1e-5, rel_l2=1e-6, lse=1e-5),
}


def move(prob: synth.Problem, device) -> synth.Problem:
    """Copy a problem to ``device``; tensors shared on the source (e.g. one
    block table for K and V) stay shared."""
    seen = {}

    def mv(x):
        if isinstance(x, torch.Tensor):
            if id(x) not in seen:
                seen[id(x)] = x.to(device)
            return seen[id(x)]
        if isinstance(x, synth.Cache):
            return synth.Cache(mv(x.pool), mv(x.block_table), x.page_size, mv(x.scale))
        if isinstance(x, list):
            return [mv(v) for v in x]
        return x

    kw = {f.name: mv(getattr(prob, f.name)) for f in dataclasses.fields(prob)}
    return synth.Problem(**kw)


def rows_np(prob):
    return (prob.seq_of_row.cpu().numpy(), prob.pos_of_row.cpu().numpy(),
            prob.seq_len.cpu().numpy())


def logical(cache: synth.Cache, n_seqs: int, cap: int, which="pool"):
    t = cache.pool if which == "pool" else cache.scale
    return oracle.unpage(t, cache.block_table, cache.page_size, n_seqs, cap)


def oracle_scores(prob, layer=0, cand=None, cand_count=None):
    wl = prob.wl
    so, po, sl = rows_np(prob)
    kl = logical(prob.kidx, wl.n_seqs, wl.n_entries_cap)
    return oracle.index_score(so, po, sl, wl.stride, prob.idx_q[layer].cpu(),
                              prob.idx_w[layer].cpu(), kl, cand=cand, cand_count=cand_count)


def oracle_select(prob, scores, k, cand=None, cand_count=None, block=0, max_blocks=0,
                  window=None):
    wl = prob.wl
    so, po, sl = rows_np(prob)
    return oracle.topk_select(so, po, sl, wl.stride, wl.window if window is None else window,
                              scores, k, cand=cand, cand_count=cand_count, block=block,
                              max_blocks=max_blocks)


def oracle_attention(prob, call, idx, count, rows=None):
    """Oracle attention for attention call ``call`` (restricted to the row
    indices ``rows`` if given)."""
    wl = prob.wl
    so, po, sl = rows_np(prob)
    q = prob.q[call].cpu()
    if rows is not None:
        so, po, q = so[rows], po[rows], q[:, rows]
        if idx is not None:
            idx, count = np.asarray(idx)[rows], np.asarray(count)[rows]
    cap = wl.n_entries_cap
    scale = float(np.float32(wl.dqk ** -0.5))
    if wl.kv_mode == "fp4":
        K = logical(prob.k, wl.n_seqs, cap)
        KS = logical(prob.k, wl.n_seqs, cap, which="scale")
        return oracle.attention(so, po, sl, wl.stride, wl.window, q, K, None, idx, count,
                                scale=scale, hkv=wl.hkv, k_scale=KS, v_from_k=True, dv=wl.dv,
                                fp4=True)
    K = logical(prob.k, wl.n_seqs, cap)
    V = logical(prob.v, wl.n_seqs, cap) if prob.v is not None else None
    return oracle.attention(so, po, sl, wl.stride, wl.window, q, K, V, idx, count, scale=scale,
                            v_from_k=prob.v is None, dv=wl.dv)


# ---------------------------------------------------------------------------
# Comparisons
# ---------------------------------------------------------------------------


def fp32_score_bound(prob, layer=0, rows=None):
    """Per-row forward error bound of an fp32 evaluation of the indexer:
    tau_t = gamma * max_s sum_h |w_h| sum_c |q_hc k_sc|, gamma = (d+H+2) 2^-24."""
    wl = prob.wl
    q = prob.idx_q[layer].cpu().double().abs()
    w = prob.idx_w[layer].cpu().double().abs()
    kl = logical(prob.kidx, wl.n_seqs, wl.n_entries_cap).double().abs()
    so = prob.seq_of_row.cpu().numpy()
    gamma = (wl.idx_dim + wl.idx_heads + 2) * 2.0 ** -24
    R = q.shape[0]
    tau = np.zeros(R)
    for r in range(R) if rows is None else rows:
        if so[r] < 0:
            continue
        m = (q[r] @ kl[so[r]].T)  # [H, L]
        tau[r] = gamma * float((w[r][:, None] * m).sum(0).max())
    return tau


def win_lo(prob, window=None):
    """First window entry of every row (the candidates of token-mode
    selection are [0, win_lo)), from the oracle's domain rule."""
    so, po, sl = rows_np(prob)
    n = oracle.n_avail(so, po, sl, prob.wl.stride)
    w = prob.wl.window if window is None else window
    return np.maximum(n - w, 0)


def check_indices(gpu_idx, gpu_cnt, ora_idx, ora_cnt, ora_scores=None, tau=None, rows=None,
                  positions=None, win_lo=None):
    """Index sets: bit-exact when ``tau`` is None; otherwise equal counts and
    every symmetric-difference element within 2*tau of the k-th oracle score.
    Every index before the count must lie in the row's candidate domain:
    0 <= s < win_lo[r] (when given) and, in candidate mode, a member of the
    row's list ``positions[r]``.  Returns the number of boundary swaps."""
    gi = np.asarray(gpu_idx)
    gc = np.asarray(gpu_cnt)
    oi = np.asarray(ora_idx)
    oc = np.asarray(ora_cnt)
    swaps = 0
    for r in range(oi.shape[0]) if rows is None else rows:
        assert gc[r] == oc[r], "row %d: count %d vs oracle %d" % (r, gc[r], oc[r])
        assert 0 <= gc[r] <= gi.shape[1], "row %d: count %d out of range" % (r, gc[r])
        g = gi[r, :gc[r]]
        o = oi[r, :oc[r]]
        assert np.all(gi[r, gc[r]:] == -1), "row %d: padding not -1" % r
        assert np.all(np.diff(g) > 0), "row %d: not ascending/unique" % r
        assert np.all(g >= 0), "row %d: negative index before the count" % r
        if win_lo is not None:
            assert np.all(g < win_lo[r]), "row %d: index outside the candidates [0, %d)" % (
                r, win_lo[r])
        if positions is not None:
            members = np.asarray(positions[r])
            assert np.all(np.isin(g, members[members >= 0])), "row %d: index not in its list" % r
        if tau is None:
            assert np.array_equal(g, o), "row %d: index sets differ" % r
            continue
        diff = np.setxor1d(g, o)
        if diff.size == 0:
            continue
        swaps += diff.size // 2
        sc = ora_scores[r]
        if positions is not None:  # candidate-mode scores are by list slot
            lookup = {int(p): i for i, p in enumerate(positions[r]) if p >= 0}
            vals = np.array([sc[lookup[int(s)]] for s in diff])
            theta = min(sc[lookup[int(s)]] for s in o)
        else:
            vals = sc[diff]
            theta = sc[o].min()
        assert np.all(np.abs(vals - theta) <= 2 * tau[r]), (
            "row %d: swap outside the fp32 bound: %s vs theta %r tau %r" % (r, vals, theta, tau[r]))
    return swaps


def check_outputs(o_gpu, o_ref, lse_gpu, lse_ref, dtype, what=""):
    tol = TOL[dtype]
    og = o_gpu.detach().float().cpu().double().numpy()
    d = np.abs(og - o_ref)
    max_abs = float(d.max()) if d.size else 0.0
    num = float(np.sqrt(((og - o_ref) ** 2).sum()))
    den = float(np.sqrt((o_ref ** 2).sum()))
    rel = num / den if den > 0 else num
    assert max_abs <= tol["max_abs"], "%s max-abs %.3g > %.3g" % (what, max_abs, tol["max_abs"])
    assert rel <= tol["rel_l2"], "%s rel-L2 %.3g > %.3g" % (what, rel, tol["rel_l2"])
    if lse_gpu is not None:
        lg = lse_gpu.detach().cpu().double().numpy()
        both_inf = np.isneginf(lg) & np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lse_ref)), what + " lse -inf mismatch"
        dl = np.abs(lg[~both_inf] - lse_ref[~both_inf])
        if dl.size:
            assert dl.max() <= tol["lse"], "%s lse err %.3g" % (what, dl.max())
    return max_abs, rel
