"""Host-side drivers that chain the three entry points into one step of a
workload.  Every call launches HIP kernels on the current stream; nothing here
computes on the CPU.

Layer-group semantics ("CSA, HCA and CSA2" page, section 3.1): a Full layer
scores every visible entry and selects; a Reindex layer rescores only the
block-max candidate pool with its own query and selects again; a Reuse layer
runs no indexer at all and passes an existing index tensor to attention.
HySparse2's FA + SA group ("HySparse2" page, section 5) is one index tensor
shared by every query set of the group.

A step object allocates all outputs and scratch once, so ``run()`` launches
kernels only (and can be captured in a HIP graph).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from .binding import (Cache, PreparedScore, Rows, attn_gather_fwd, index_score,
                      prepare_attn_gather_fwd, prepare_index_score, prepare_index_select,
                      prepare_topk_select, topk_select)


def _cache(c, heads, width, fp4=False) -> Cache:
    return Cache(c.pool, c.block_table, heads, width, fp4=fp4, scale=c.scale)


@dataclass
class StepOutputs:
    scores: List[torch.Tensor]
    idx: List[torch.Tensor]
    count: List[torch.Tensor]
    pool: Optional[torch.Tensor]
    pool_count: Optional[torch.Tensor]
    o: List[torch.Tensor]
    lse: List[torch.Tensor]


class Step:
    """One pass of the hot path over a problem instance.

    Workloads without a block pool: score (full domain) -> window + top-k ->
    one attention call for all query sets.  Workloads with a block pool
    (CSA2): Full score -> top-k + pool -> Reindex score over the pool ->
    top-k inside the pool -> attention with the Full indices (Full query) and
    with the Reindex indices (Reindex query + Reuse queries, fused)."""

    def __init__(self, prob, scores_slots: Optional[int] = None, dense_route: bool = False,
                 block_select=None, fused_select: bool = False, fused_row_block: int = 0):
        """``block_select`` = (block, n_blocks): select whole aligned blocks of
        candidates by their best score instead of single entries (HySparse's
        first generation: 16 blocks of 64 tokens next to the window); the
        pool of kept blocks is the index tensor.  ``fused_select``: each
        index call selects in the same call (sparse_index_score with a
        selection, ``fused_row_block`` rows per pass) and writes no score
        tensor."""
        self.fused_select = fused_select
        self.fused_row_block = fused_row_block
        wl = prob.wl
        assert block_select is None or not wl.block, "block selection replaces the token top-k"
        self.block_select = block_select
        self.prob = prob
        self.wl = wl
        dev = prob.seq_of_row.device
        R = prob.n_rows
        self.rows = Rows(prob.seq_of_row, prob.pos_of_row, prob.seq_len, wl.stride, wl.window)
        # a workload without a selector (k = 0, e.g. HCA) attends to its window only
        self.selector = wl.k > 0
        # dense route: rows whose candidates all fit the budget skip the
        # indexer (scores 0; the selection keeps every candidate either way)
        budget = wl.k if block_select is None else block_select[0] * block_select[1]
        self.skip_k = budget if dense_route else 0
        self.kidx = _cache(prob.kidx, 1, wl.idx_dim) if self.selector else None
        fp4 = wl.kv_mode == "fp4"
        self.k = _cache(prob.k, wl.hkv, wl.dqk, fp4=fp4)
        self.v = _cache(prob.v, wl.hkv, wl.dv) if prob.v is not None else None
        self.S = scores_slots or wl.n_entries_cap
        f32 = torch.float32
        i32 = torch.int32
        self.scores = [torch.empty(R, self.S, dtype=f32, device=dev)]
        width = wl.k if block_select is None else block_select[0] * block_select[1]
        self.idx = [torch.empty(R, width, dtype=i32, device=dev)]
        self.count = [torch.empty(R, dtype=i32, device=dev)]
        self.pool = self.pool_count = None
        if wl.block:
            P = wl.max_blocks * wl.block
            self.pool = torch.empty(R, P, dtype=i32, device=dev)
            self.pool_count = torch.empty(R, dtype=i32, device=dev)
            self.scores.append(torch.empty(R, P, dtype=f32, device=dev))
            self.idx.append(torch.empty(R, wl.k, dtype=i32, device=dev))
            self.count.append(torch.empty(R, dtype=i32, device=dev))
        self.o, self.lse = [], []
        for q in prob.q:
            self.o.append(torch.empty(q.shape[0], R, wl.hq, wl.dv, dtype=q.dtype, device=dev))
            self.lse.append(torch.empty(q.shape[0], R, wl.hq, dtype=f32, device=dev))
        self.scale = wl.dqk ** -0.5
        self._prepared = None

    def prepare(self):
        """Build the launch-only call list of one step (index calls, then
        attention calls); returns [(name, callable), ...]."""
        if self._prepared is not None:
            return self._prepared
        p, wl = self.prob, self.wl
        if not self.selector:
            self._prepared = [("attn_gather_fwd", prepare_attn_gather_fwd(
                self.rows, p.q[0], self.k, self.v, None, None, self.o[0], self.lse[0], self.scale,
                wl.dv))]
            return self._prepared
        calls = self._fused_index_calls() if self.fused_select else self._index_calls()
        for c, q in enumerate(p.q):
            calls.append(("attn_gather_fwd" + ("" if c == 0 else "_%d" % c),
                          prepare_attn_gather_fwd(self.rows, q, self.k, self.v, self.idx[c],
                                                  self.count[c], self.o[c], self.lse[c],
                                                  self.scale, wl.dv)))
        self._prepared = calls
        return calls

    def _index_calls(self):
        """Index calls writing scores, each followed by its selection."""
        p, wl = self.prob, self.wl
        calls = [("index_score", prepare_index_score(self.rows, p.idx_q[0], p.idx_w[0], self.kidx,
                                                     self.scores[0], skip_k=self.skip_k))]
        if self.block_select is not None:
            bs, nb = self.block_select
            calls.append(("topk_select", prepare_topk_select(
                self.rows, self.scores[0], 0, None, None, block=bs, max_blocks=nb,
                pool=self.idx[0], pool_count=self.count[0])))
        elif not wl.block:
            calls.append(("topk_select", prepare_topk_select(self.rows, self.scores[0], wl.k,
                                                             self.idx[0], self.count[0])))
        else:
            calls.append(("topk_select", prepare_topk_select(
                self.rows, self.scores[0], wl.k, self.idx[0], self.count[0], block=wl.block,
                max_blocks=wl.max_blocks, pool=self.pool, pool_count=self.pool_count)))
            calls.append(("index_score_reindex", prepare_index_score(
                self.rows, p.idx_q[1], p.idx_w[1], self.kidx, self.scores[1], cand=self.pool,
                cand_count=self.pool_count)))
            calls.append(("topk_select_reindex", prepare_topk_select(
                self.rows, self.scores[1], wl.k, self.idx[1], self.count[1], cand=self.pool,
                cand_count=self.pool_count)))
        return calls

    def _fused_index_calls(self):
        """Index and selection in one call per layer (no score tensor)."""
        p, wl, rb = self.prob, self.wl, self.fused_row_block
        if self.block_select is not None:
            bs, nb = self.block_select
            return [("index_select", prepare_index_select(
                self.rows, p.idx_q[0], p.idx_w[0], self.kidx, self.S, 0, None, None, block=bs,
                max_blocks=nb, pool=self.idx[0], pool_count=self.count[0], skip_k=self.skip_k,
                row_block=rb))]
        if not wl.block:
            return [("index_select", prepare_index_select(
                self.rows, p.idx_q[0], p.idx_w[0], self.kidx, self.S, wl.k, self.idx[0],
                self.count[0], skip_k=self.skip_k, row_block=rb))]
        P = wl.max_blocks * wl.block
        return [("index_select", prepare_index_select(
                    self.rows, p.idx_q[0], p.idx_w[0], self.kidx, self.S, wl.k, self.idx[0],
                    self.count[0], block=wl.block, max_blocks=wl.max_blocks, pool=self.pool,
                    pool_count=self.pool_count, skip_k=self.skip_k, row_block=rb)),
                ("index_select_reindex", prepare_index_select(
                    self.rows, p.idx_q[1], p.idx_w[1], self.kidx, P, wl.k, self.idx[1],
                    self.count[1], cand=self.pool, cand_count=self.pool_count, row_block=rb))]

    def run_index(self):
        p, wl = self.prob, self.wl
        if not self.selector:
            return
        index_score(self.rows, p.idx_q[0], p.idx_w[0], self.kidx, scores=self.scores[0],
                    skip_k=self.skip_k)
        if self.block_select is not None:
            bs, nb = self.block_select
            topk_select(self.rows, self.scores[0], 0, block=bs, max_blocks=nb,
                        pool=self.idx[0], pool_count=self.count[0])
            return
        if not wl.block:
            topk_select(self.rows, self.scores[0], wl.k, idx=self.idx[0], count=self.count[0])
            return
        topk_select(self.rows, self.scores[0], wl.k, block=wl.block, max_blocks=wl.max_blocks,
                    idx=self.idx[0], count=self.count[0], pool=self.pool,
                    pool_count=self.pool_count)
        index_score(self.rows, p.idx_q[1], p.idx_w[1], self.kidx, scores=self.scores[1],
                    cand=self.pool, cand_count=self.pool_count)
        topk_select(self.rows, self.scores[1], wl.k, cand=self.pool, cand_count=self.pool_count,
                    idx=self.idx[1], count=self.count[1])

    def run_attention(self, idx=None, count=None):
        """Attention for every call; ``idx``/``count`` (lists) override the
        step's own index tensors (used to feed externally chosen indices)."""
        p = self.prob
        idx = idx if idx is not None else self.idx
        count = count if count is not None else self.count
        for c, q in enumerate(p.q):
            attn_gather_fwd(self.rows, q, self.k, self.v,
                            idx=idx[c] if self.selector else None,
                            count=count[c] if self.selector else None,
                            scale=self.scale, d_v=self.wl.dv, o=self.o[c], lse=self.lse[c])

    def run(self):
        self.run_index()
        self.run_attention()

    def outputs(self) -> StepOutputs:
        return StepOutputs(self.scores, self.idx, self.count, self.pool, self.pool_count, self.o,
                           self.lse)


class PrefillStep:
    """One pass of the hot path over every query row of a prefill workload,
    in blocks of ``row_block`` rows so that the block's score matrix
    ([row_block, n] f32) is the only materialised scores: per block, the
    indexer scores the causal history of each row, the selection keeps the
    top-k, and attention gathers it.  Indices, outputs and LSE cover all
    rows; the score buffer is reused from block to block.

    With a block pool (the hierarchical indexer, "CSA, HCA and CSA2",
    sections 3.1-3.2), each row block runs the whole layer group: the Full
    layer's scores give its own top-k and the block-max pool; the Reindex
    layer rescores only the pool with its own query and selects its top-k
    there; the Full query attends over the Full indices and the Reindex (and
    any Reuse) queries over the Reindex indices.  The pool and the Reindex
    scores exist for one row block at a time ([row_block, max_blocks*block]),
    never for every prefill row (section 3.1: a pool materialised for all
    131072 queries would take about 2 GiB)."""

    def __init__(self, prob, row_block: int = 8192, dense_route: bool = False,
                 fused_select: bool = False, fused_row_block: int = 0):
        """``fused_select``: each block's index calls select in the same call
        (sparse_index_score with a selection, ``fused_row_block`` rows per
        pass inside the call) and write no score tensor."""
        wl = prob.wl
        assert wl.prefill, "prefill workloads"
        self.fused_select = fused_select
        self.fused_row_block = fused_row_block
        self.skip_k = wl.k if dense_route and not wl.block else 0
        self.prob = prob
        self.wl = wl
        dev = prob.seq_of_row.device
        R = prob.n_rows
        self.R = R
        self.row_block = row_block
        rb = min(row_block, R)
        i32, f32 = torch.int32, torch.float32
        self.kidx = _cache(prob.kidx, 1, wl.idx_dim)
        self.k = _cache(prob.k, wl.hkv, wl.dqk)
        self.v = _cache(prob.v, wl.hkv, wl.dv) if prob.v is not None else None
        self.S = wl.n_entries_cap
        # score buffers only without the fused selection
        self.scores = None if fused_select else torch.empty(rb, self.S, dtype=f32, device=dev)
        self.idx = torch.empty(R, wl.k, dtype=i32, device=dev)
        self.count = torch.empty(R, dtype=i32, device=dev)
        q = prob.q[0]
        self.o = torch.empty(q.shape[0], R, wl.hq, wl.dv, dtype=q.dtype, device=dev)
        self.lse = torch.empty(q.shape[0], R, wl.hq, dtype=f32, device=dev)
        self.pool = self.pool_count = None
        if wl.block:
            P = wl.max_blocks * wl.block
            self.pool = torch.empty(rb, P, dtype=i32, device=dev)
            self.pool_count = torch.empty(rb, dtype=i32, device=dev)
            self.scores_r = None if fused_select else torch.empty(rb, P, dtype=f32, device=dev)
            self.idx_r = torch.empty(R, wl.k, dtype=i32, device=dev)
            self.count_r = torch.empty(R, dtype=i32, device=dev)
            q1 = prob.q[1]
            self.o_r = torch.empty(q1.shape[0], R, wl.hq, wl.dv, dtype=q1.dtype, device=dev)
            self.lse_r = torch.empty(q1.shape[0], R, wl.hq, dtype=f32, device=dev)
        self.scale = wl.dqk ** -0.5
        self._prepared = None

    def blocks(self):
        return [(lo, min(self.R, lo + self.row_block)) for lo in range(0, self.R, self.row_block)]

    def prepare(self):
        """Launch-only call list of one pass: (name, callable) for every block
        and entry point, names repeated per block."""
        if self._prepared is not None:
            return self._prepared
        p, wl = self.prob, self.wl
        calls = []
        ws = None  # one selection workspace for every block (the calls never overlap)

        def select(name, *a, **kw):
            nonlocal ws
            sel = prepare_topk_select(*a, workspace=ws, **kw)
            ws = sel.ws if ws is None or (sel.ws is not None and sel.ws.numel() > ws.numel()) else ws
            calls.append((name, sel))

        def fused(name, *a, **kw):
            nonlocal ws
            c = prepare_index_select(*a, workspace=ws, **kw)
            ws = c.ws if ws is None or (c.ws is not None and c.ws.numel() > ws.numel()) else ws
            calls.append((name, c))

        for lo, hi in self.blocks():
            rows = Rows(p.seq_of_row[lo:hi], p.pos_of_row[lo:hi], p.seq_len, wl.stride, wl.window)
            n = hi - lo
            if self.fused_select:
                frb = self.fused_row_block
                if not wl.block:
                    fused("index_select", rows, p.idx_q[0][lo:hi], p.idx_w[0][lo:hi], self.kidx,
                          self.S, wl.k, self.idx[lo:hi], self.count[lo:hi], skip_k=self.skip_k,
                          row_block=frb)
                else:
                    pool, pc = self.pool[:n], self.pool_count[:n]
                    fused("index_select", rows, p.idx_q[0][lo:hi], p.idx_w[0][lo:hi], self.kidx,
                          self.S, wl.k, self.idx[lo:hi], self.count[lo:hi], block=wl.block,
                          max_blocks=wl.max_blocks, pool=pool, pool_count=pc, row_block=frb)
                    fused("index_select_reindex", rows, p.idx_q[1][lo:hi], p.idx_w[1][lo:hi],
                          self.kidx, wl.max_blocks * wl.block, wl.k, self.idx_r[lo:hi],
                          self.count_r[lo:hi], cand=pool, cand_count=pc, row_block=frb)
                self._attention_calls(calls, rows, lo, hi)
                continue
            sc = self.scores[:n]
            calls.append(("index_score", prepare_index_score(rows, p.idx_q[0][lo:hi],
                                                             p.idx_w[0][lo:hi], self.kidx, sc,
                                                             skip_k=self.skip_k)))
            if not wl.block:
                select("topk_select", rows, sc, wl.k, self.idx[lo:hi], self.count[lo:hi])
            else:
                pool, pc = self.pool[:n], self.pool_count[:n]
                select("topk_select", rows, sc, wl.k, self.idx[lo:hi], self.count[lo:hi],
                       block=wl.block, max_blocks=wl.max_blocks, pool=pool, pool_count=pc)
                scr = self.scores_r[:n]
                calls.append(("index_score_reindex", prepare_index_score(
                    rows, p.idx_q[1][lo:hi], p.idx_w[1][lo:hi], self.kidx, scr, cand=pool,
                    cand_count=pc)))
                select("topk_select_reindex", rows, scr, wl.k, self.idx_r[lo:hi],
                       self.count_r[lo:hi], cand=pool, cand_count=pc)
            self._attention_calls(calls, rows, lo, hi)
        self._prepared = calls
        return calls

    def _attention_calls(self, calls, rows, lo, hi):
        p, wl = self.prob, self.wl
        calls.append(("attn_gather_fwd", prepare_attn_gather_fwd(
            rows, p.q[0][:, lo:hi], self.k, self.v, self.idx[lo:hi], self.count[lo:hi],
            self.o[:, lo:hi], self.lse[:, lo:hi], self.scale, wl.dv)))
        if wl.block:
            calls.append(("attn_gather_fwd_1", prepare_attn_gather_fwd(
                rows, p.q[1][:, lo:hi], self.k, self.v, self.idx_r[lo:hi], self.count_r[lo:hi],
                self.o_r[:, lo:hi], self.lse_r[:, lo:hi], self.scale, wl.dv)))

    def run(self):
        for _, c in self.prepare():
            c()


class FAStep:
    """HySparse2's own layer group ("HySparse2" page, section 5 and appendix
    A.1): the full-attention (FA) layer runs dense attention over every
    visible entry and selects the window + top-k from its own attention
    probabilities summed over heads; the sparse (SA) layers of the group reuse
    that KV and that index tensor with their own queries.

    Query set 0 of the problem's first query tensor is the FA layer's query;
    sets 1.. are the SA layers'.  Calls: dense attention (FA) ->
    sparse_attn_score -> window + top-k -> one gather attention for every SA
    set."""

    def __init__(self, prob):
        wl = prob.wl
        assert not wl.block and prob.q[0].shape[0] >= 2, "an FA set and at least one SA set"
        self.prob = prob
        self.wl = wl
        dev = prob.seq_of_row.device
        R = prob.n_rows
        cap = wl.n_entries_cap
        self.rows_dense = Rows(prob.seq_of_row, prob.pos_of_row, prob.seq_len, wl.stride, cap)
        self.rows = Rows(prob.seq_of_row, prob.pos_of_row, prob.seq_len, wl.stride, wl.window)
        self.k = _cache(prob.k, wl.hkv, wl.dqk)
        self.v = _cache(prob.v, wl.hkv, wl.dv) if prob.v is not None else None
        q = prob.q[0]
        self.q_fa, self.q_sa = q[0:1], q[1:]
        f32, i32 = torch.float32, torch.int32
        self.scores = torch.empty(R, cap, dtype=f32, device=dev)
        self.idx = torch.empty(R, wl.k, dtype=i32, device=dev)
        self.count = torch.empty(R, dtype=i32, device=dev)
        self.o_fa = torch.empty(1, R, wl.hq, wl.dv, dtype=q.dtype, device=dev)
        self.lse_fa = torch.empty(1, R, wl.hq, dtype=f32, device=dev)
        self.o_sa = torch.empty(q.shape[0] - 1, R, wl.hq, wl.dv, dtype=q.dtype, device=dev)
        self.lse_sa = torch.empty(q.shape[0] - 1, R, wl.hq, dtype=f32, device=dev)
        self.pool_count = None  # no block pool in this group
        self.scale = wl.dqk ** -0.5
        self._prepared = None

    def prepare(self):
        if self._prepared is not None:
            return self._prepared
        self._prepared = [
            ("attn_gather_fwd_fa", prepare_attn_gather_fwd(
                self.rows_dense, self.q_fa, self.k, self.v, None, None, self.o_fa, self.lse_fa,
                self.scale, self.wl.dv)),
            ("attn_score", PreparedScore(self.rows_dense, self.q_fa, self.k, self.lse_fa,
                                         self.scores, self.scale)),
            ("topk_select", prepare_topk_select(self.rows, self.scores, self.wl.k, self.idx,
                                                self.count)),
            ("attn_gather_fwd", prepare_attn_gather_fwd(
                self.rows, self.q_sa, self.k, self.v, self.idx, self.count, self.o_sa,
                self.lse_sa, self.scale, self.wl.dv)),
        ]
        return self._prepared

    def run(self):
        for _, c in self.prepare():
            c()
