"""GPU parity of the hierarchical indexer in prefill ("CSA, HCA and CSA2",
sections 3.1-3.2: a Full layer scores every visible entry and builds the
block-max pool, a Reindex layer rescores only the pool with its own query;
section 2.2: prefill must not materialise the n x n_c scores or, for every
query row, the pool).  Every token of a sequence is a query row over entries
compressed at stride 4; the row blocks each hold their own pool only."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import index_reuse_amd

    index_reuse_amd.load()
    return "cuda"


def _check_rows(prob, step, rows, integer, label):
    """Full indices, pool, Reindex indices and both attention calls of the
    listed rows against the oracle (rows of ``prob`` are those rows)."""
    wl = prob.wl
    sc = H.oracle_scores(prob, 0)
    tau = None if integer else H.fp32_score_bound(prob, 0)
    idx, cnt, pool, pc = H.oracle_select(prob, sc, wl.k, block=wl.block, max_blocks=wl.max_blocks)
    gi = step.idx.cpu().numpy()[rows]
    gc = step.count.cpu().numpy()[rows]
    H.check_indices(gi, gc, idx, cnt, sc, tau, win_lo=H.win_lo(prob))
    rs = H.oracle_scores(prob, 1, cand=pool, cand_count=pc)
    ridx, rcnt = H.oracle_select(prob, rs, wl.k, cand=pool, cand_count=pc)
    gri = step.idx_r.cpu().numpy()[rows]
    grc = step.count_r.cpu().numpy()[rows]
    same_full = [i for i in range(len(rows))
                 if gc[i] == cnt[i] and np.array_equal(gi[i, :gc[i]], idx[i, :cnt[i]])]
    if integer:
        # the pool is not kept across blocks; the Reindex set pins it
        H.check_indices(gri, grc, ridx, rcnt, win_lo=H.win_lo(prob))
        assert len(same_full) == len(rows)
    else:
        tau1 = H.fp32_score_bound(prob, 1)
        # a Reindex set is comparable where the oracle's pool is the GPU's:
        # every GPU index lies in the oracle pool and the counts agree
        ok = [i for i in range(len(rows))
              if grc[i] == rcnt[i] and np.all(np.isin(gri[i, :grc[i]], pool[i, :pc[i]]))]
        assert ok, label
        H.check_indices(gri, grc, ridx, rcnt, rs, tau1, rows=ok, positions=pool,
                        win_lo=H.win_lo(prob))
    sel = torch.tensor(rows, dtype=torch.long, device=step.o.device)
    o_ref, l_ref = H.oracle_attention(prob, 0, gi, gc)
    H.check_outputs(step.o.index_select(1, sel), o_ref, step.lse.index_select(1, sel), l_ref,
                    wl.attn_dtype, what="%s Full" % label)
    o_ref, l_ref = H.oracle_attention(prob, 1, gri, grc)
    H.check_outputs(step.o_r.index_select(1, sel), o_ref, step.lse_r.index_select(1, sel), l_ref,
                    wl.attn_dtype, what="%s Reindex" % label)


@pytest.mark.parametrize("integer", [True, False])
def test_hierarchical_prefill_small(integer, dev):
    """Every row of a 2048-token prefill (512 entries at stride 4), in row
    blocks of 512, with a pool of 16 blocks of 8 and top-64."""
    from index_reuse_amd.pipeline import PrefillStep

    wl = synth.CSA2_PREFILL.replace(seq_len=2048, k=64, max_blocks=16)
    prob = synth.make_problem(wl, device="cpu", integer=integer)
    print("case hierarchical prefill integer=%s R=%d" % (integer, prob.n_rows), flush=True)
    step = PrefillStep(H.move(prob, dev), row_block=512)
    step.run()
    torch.cuda.synchronize()
    _check_rows(prob, step, list(range(prob.n_rows)), integer, "small")


@pytest.mark.parametrize("integer", [True, False])
def test_hierarchical_prefill_full_size(integer, dev):
    """The full 131072-row workload in the benchmark's row blocks; sampled
    rows (first and last of every block, rows whose pool covers every block,
    random rows) against the oracle."""
    import dataclasses

    from index_reuse_amd.pipeline import PrefillStep

    wl = synth.CSA2_PREFILL
    print("case hierarchical prefill full size integer=%s" % integer, flush=True)
    prob = synth.make_problem(wl, device=dev, integer=integer)
    step = PrefillStep(prob, row_block=8192)
    step.run()
    torch.cuda.synchronize()
    rows = set()
    for b in range(wl.seq_len // 8192):
        rows |= {8192 * b, 8192 * b + 8191}
    rows |= {3, 4095, 4096, 16383, 16384, 16391}
    rng = np.random.default_rng(77)
    while len(rows) < 40:
        rows.add(int(rng.integers(0, wl.seq_len)))
    rows = sorted(rows)
    r = torch.as_tensor(rows, dtype=torch.long, device=dev)
    sub = dataclasses.replace(prob, seq_of_row=prob.seq_of_row[r], pos_of_row=prob.pos_of_row[r],
                              idx_q=[x[r] for x in prob.idx_q], idx_w=[x[r] for x in prob.idx_w],
                              q=[x[:, r] for x in prob.q])
    sub = H.move(sub, "cpu")
    del prob
    _check_rows(sub, step, rows, integer, "full size")
