"""The comparison harness must catch the silent faults the pages list for
shared-index layer groups ("CSA, HCA and CSA2", section 5.1, fault
injection): a Reuse index off by one token, two KV pages swapped, a leaked
padding row, and a count that is off by one.  Every mistake is planted in
the oracle's own results on the CPU (no GPU): the "device" side of each
comparison is an oracle result computed from a mutated input or a mutated
copy of an oracle output, and check_indices / check_outputs must reject it.
The unmutated comparison passes, so each rejection is the mutation's.
"""
import copy
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests import helpers as H


@pytest.fixture(scope="module")
def case(orc):
    wl = synth.HYSPARSE2.replace(n_seqs=3, seq_lens_override=(1500, 700, 300), n_qsets=2)
    prob = synth.make_problem(wl, device="cpu", integer=True)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    # plant a dominant selected entry for row 0, KV head 0: its key is a
    # multiple of the first query head's query, so that head puts almost all
    # its weight on it (an off-by-one shift of it must show in the output)
    r, g = 0, 0
    s_star = int(idx[r, np.argmax(sc[r, idx[r, :cnt[r]]])])
    page = int(prob.k.block_table[0, s_star // wl.page_size])
    prob.k.pool[page, s_star % wl.page_size, g] = (prob.q[0][0, r, 0].float() * 3).to(torch.bfloat16)
    o, lse = H.oracle_attention(prob, 0, idx, cnt)
    return dict(wl=wl, prob=prob, sc=sc, idx=idx, cnt=cnt, o=o, lse=lse, s_star=s_star)


def _as_dev(o):
    return torch.from_numpy(np.ascontiguousarray(o)).to(torch.bfloat16)


def test_unmutated_passes(case):
    c = case
    H.check_indices(c["idx"], c["cnt"], c["idx"], c["cnt"], win_lo=H.win_lo(c["prob"]))
    H.check_outputs(_as_dev(c["o"]), c["o"], torch.from_numpy(c["lse"]), c["lse"],
                    torch.bfloat16, what="unmutated")


def test_reuse_index_shifted_by_one(case):
    c = case
    idx = c["idx"].copy()
    r = 0
    row = list(idx[r, :c["cnt"][r]])
    j = row.index(c["s_star"])
    shifted = c["s_star"] + 1
    while shifted in row:
        shifted += 1
    assert shifted < H.win_lo(c["prob"])[r]
    row[j] = shifted
    idx[r, :c["cnt"][r]] = sorted(row)
    # the index check (exact, and within the fp32 bound: the moved entry was
    # the row's best, far above the threshold score)
    with pytest.raises(AssertionError):
        H.check_indices(idx, c["cnt"], c["idx"], c["cnt"], win_lo=H.win_lo(c["prob"]))
    tau = np.full(len(c["cnt"]), 0.5)
    with pytest.raises(AssertionError):
        H.check_indices(idx, c["cnt"], c["idx"], c["cnt"], c["sc"], tau,
                        win_lo=H.win_lo(c["prob"]))
    # a Reuse layer attending over the shifted set gives a different output
    o, lse = H.oracle_attention(c["prob"], 0, idx, c["cnt"])
    with pytest.raises(AssertionError):
        H.check_outputs(_as_dev(o), c["o"], torch.from_numpy(lse), c["lse"], torch.bfloat16)


def test_two_kv_pages_swapped(case):
    c = case
    prob = c["prob"]
    wl = c["wl"]
    bt = prob.k.block_table.clone()
    # the page holding the planted entry and the last (window) page of row 0
    p_sel = c["s_star"] // wl.page_size
    p_win = (wl.seq_lens()[0] - 1) // wl.page_size
    assert p_sel != p_win
    bt[0, p_sel], bt[0, p_win] = prob.k.block_table[0, p_win], prob.k.block_table[0, p_sel]
    k2 = synth.Cache(prob.k.pool, bt, prob.k.page_size)
    v2 = synth.Cache(prob.v.pool, bt, prob.v.page_size)
    bad = dataclasses.replace(prob, k=k2, v=v2)
    o, lse = H.oracle_attention(bad, 0, c["idx"], c["cnt"])
    with pytest.raises(AssertionError):
        H.check_outputs(_as_dev(o), c["o"], torch.from_numpy(lse), c["lse"], torch.bfloat16)


def test_leaked_padding_row(case):
    c = case
    prob = copy.copy(c["prob"])
    prob.seq_of_row = torch.tensor([0, -1, 2], dtype=torch.int32)
    idx, cnt = H.oracle_select(prob, c["sc"], c["wl"].k)
    o, lse = H.oracle_attention(prob, 0, idx, cnt)
    assert cnt[1] == 0 and np.all(o[:, 1] == 0) and np.all(np.isneginf(lse[:, 1]))
    # the padding row leaks row 0's selection, or row 0's output
    gi, gc = idx.copy(), cnt.copy()
    gi[1], gc[1] = idx[0], cnt[0]
    with pytest.raises(AssertionError):
        H.check_indices(gi, gc, idx, cnt, win_lo=H.win_lo(prob))
    go, gl = o.copy(), lse.copy()
    go[:, 1], gl[:, 1] = o[:, 0], lse[:, 0]
    with pytest.raises(AssertionError):
        H.check_outputs(_as_dev(go), o, torch.from_numpy(gl), lse, torch.bfloat16)
    # a leaked LSE alone (output still zero) is caught too
    gl2 = lse.copy()
    gl2[:, 1] = 0.0
    with pytest.raises(AssertionError):
        H.check_outputs(_as_dev(o), o, torch.from_numpy(gl2), lse, torch.bfloat16)


def test_count_off_by_one(case):
    c = case
    for delta in (-1, 1):
        gi, gc = c["idx"].copy(), c["cnt"].copy()
        r = 1
        if delta < 0:
            gi[r, gc[r] - 1] = -1
        else:
            gi[r, gc[r]] = 0 if 0 not in gi[r, :gc[r]] else gi[r, :gc[r]].max() + 1
            gi[r, :gc[r] + 1] = np.sort(gi[r, :gc[r] + 1])
        gc[r] += delta
        with pytest.raises(AssertionError):
            H.check_indices(gi, gc, c["idx"], c["cnt"], win_lo=H.win_lo(c["prob"]))
        # the count alone, indices untouched
        gc2 = c["cnt"].copy()
        gc2[r] += delta
        with pytest.raises(AssertionError):
            H.check_indices(c["idx"], gc2, c["idx"], c["cnt"])


def test_window_entry_and_negative_index(case):
    """Float-input comparisons accept boundary swaps near the threshold;
    they still reject an index from the forced window (not a candidate) and
    a negative index before the count, even with a loose bound."""
    c = case
    wl = c["wl"]
    wlo = H.win_lo(c["prob"])
    tau = np.full(len(c["cnt"]), 1e9)
    gi = c["idx"].copy()
    r = 0
    gi[r, c["cnt"][r] - 1] = wlo[r]  # the first window entry replaces the largest index
    with pytest.raises(AssertionError, match="outside the candidates"):
        H.check_indices(gi, c["cnt"], c["idx"], c["cnt"], c["sc"], tau, win_lo=wlo)
    gi = c["idx"].copy()
    gi[r, 0] = -5
    with pytest.raises(AssertionError):
        H.check_indices(gi, c["cnt"], c["idx"], c["cnt"], c["sc"], tau, win_lo=wlo)
