"""GPU parity of the dense routes ("Lecture 10", section 5.5: when a row's
context is no longer than the budget, top-k selection only adds the
indexer's cost, so it falls back to dense attention; "CSA, HCA and CSA2",
sections 1.2 and 6.2: HCA attends to every heavily compressed entry with no
selector), against the fp64 oracle."""
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


@pytest.mark.parametrize("integer", [True, False])
def test_decode_dense_route(integer, dev):
    """A mixed decode batch: rows with more candidates than the budget are
    scored and selected; rows with at most k candidates skip the indexer
    (their scores are 0, no key is read) and still keep exactly the oracle's
    set -- every candidate -- so the attention is the dense one."""
    from index_reuse_amd.pipeline import Step

    wl = synth.HYSPARSE2.replace(n_seqs=6, seq_lens_override=(3000, 1100, 1152, 1153, 60, 1))
    prob = synth.make_problem(wl, device="cpu", integer=integer)
    print("case dense route integer=%s" % integer, flush=True)
    step = Step(H.move(prob, dev), dense_route=True)
    step.run()
    torch.cuda.synchronize()
    wlo = H.win_lo(prob)
    dense = wlo <= wl.k
    assert list(dense) == [False, True, True, False, True, True]
    sc = H.oracle_scores(prob, 0)
    g = step.scores[0].cpu().double().numpy()
    n = oracle.n_avail(*H.rows_np(prob), 1)
    tau = None if integer else H.fp32_score_bound(prob, 0)
    for r in range(prob.n_rows):
        if dense[r]:
            assert np.all(g[r, :n[r]] == 0.0)
        elif integer:
            assert np.array_equal(g[r, :n[r]], sc[r, :n[r]])
        else:
            assert np.all(np.abs(g[r, :n[r]] - sc[r, :n[r]]) <= tau[r])
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    H.check_indices(step.idx[0].cpu(), step.count[0].cpu(), idx, cnt, sc, tau, win_lo=wlo)
    for r in np.nonzero(dense)[0]:
        assert cnt[r] == wlo[r] and list(idx[r, :cnt[r]]) == list(range(wlo[r]))
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what="dense route")


def test_prefill_dense_route(dev):
    """DSA prefill rows on both sides of t + 1 = k = 2048 (w = 0): rows whose
    whole causal prefix fits the budget skip the indexer in the row-block
    GEMM kernel too; selections stay bit-exact on integer inputs."""
    from index_reuse_amd.pipeline import PrefillStep

    wl = synth.DSA.replace(seq_len=3000)
    rows = list(range(0, 24)) + list(range(2030, 2070)) + [2999]
    prob = synth.make_problem(wl, device="cpu", integer=True, rows=rows)
    print("case prefill dense route", flush=True)
    step = PrefillStep(H.move(prob, dev), row_block=32, dense_route=True)
    step.run()
    torch.cuda.synchronize()
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    assert list(cnt) == [min(2048, t + 1) for t in rows]
    H.check_indices(step.idx.cpu(), step.count.cpu(), idx, cnt, win_lo=H.win_lo(prob))


def test_hca_dense_over_compressed_entries(dev):
    """HCA: every entry covers 128 tokens; a row attends to all of its complete
    entries (a partial tail entry is masked) with one softmax and no selector."""
    from index_reuse_amd.pipeline import Step

    wl = synth.HCA.replace(n_seqs=4, seq_lens_override=(131072, 131072 - 5, 65636, 300),
                           window=1024)
    prob = synth.make_problem(wl, device="cpu")
    assert prob.kidx is None and not prob.idx_q
    print("case hca", flush=True)
    step = Step(H.move(prob, dev))
    step.run()
    torch.cuda.synchronize()
    n = oracle.n_avail(*H.rows_np(prob), 128)
    assert list(n) == [1024, 1023, 512, 2]
    o_ref, l_ref = H.oracle_attention(prob, 0, None, None)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what="hca")
