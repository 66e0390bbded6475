"""sparse_index_score with the fused selection (the indexer's scores feed the
window + top-k selection and the block-max pool inside one call, a bounded
pass of rows at a time, with no score tensor) against the two calls made
separately: the index tensors, counts and pools must be identical bit for
bit, and so must the attention that consumes them.

The separate calls are themselves checked against the oracle in the other
GPU tests; here the fused path must reproduce them exactly, over several
passes (a ragged last one), in token mode, pool mode, the Reindex candidate
mode, the dense route and the prefill (row-block GEMM) indexer.
"""
import pytest
import torch

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import index_reuse_amd

    index_reuse_amd.load()
    return "cuda"


DECODE = {
    "hysparse2": synth.HYSPARSE2.replace(n_seqs=7,
                                         seq_lens_override=(2500, 1151, 1152, 1153, 100, 1, 1280)),
    "csa": synth.CSA.replace(n_seqs=4, seq_len=8192, tail_variant=True),
    "csa2": synth.CSA2.replace(n_seqs=2, seq_lens_override=(20000, 16389)),
}


def _outputs(st):
    """Every output of a step; a prefill step's pool buffers hold one block
    only (the last) and are left out."""
    from index_reuse_amd.pipeline import Step

    if isinstance(st, Step):
        return (list(st.idx) + list(st.count) +
                [t for t in (st.pool, st.pool_count) if t is not None] + list(st.o) + list(st.lse))
    out = [st.idx, st.count, st.o, st.lse]
    if st.wl.block:
        out += [st.idx_r, st.count_r, st.o_r, st.lse_r]
    return out


def _run(st):
    for t in _outputs(st):
        t.fill_(-7)  # nothing may survive from before the call
    for _, c in st.prepare():
        c()


@pytest.mark.parametrize("dense_route", [False, True])
@pytest.mark.parametrize("row_block", [0, 3])
@pytest.mark.parametrize("name", list(DECODE))
def test_fused_select_decode(name, row_block, dense_route, dev):
    from index_reuse_amd.pipeline import Step

    wl = DECODE[name]
    print("case fused decode %s row_block=%d dense=%s" % (name, row_block, dense_route), flush=True)
    p = H.move(synth.make_problem(wl, device="cpu"), dev)
    sep = Step(p, dense_route=dense_route)
    fus = Step(p, dense_route=dense_route, fused_select=True, fused_row_block=row_block)
    assert [n for n, _ in fus.prepare()][0] == "index_select"
    _run(sep)
    _run(fus)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(sep), _outputs(fus))):
        assert torch.equal(a, b), (name, i)


def test_fused_block_select(dev):
    """Block-level selection (the pool as the index tensor) fused."""
    from index_reuse_amd.pipeline import Step

    wl = DECODE["hysparse2"]
    print("case fused block select", flush=True)
    p = H.move(synth.make_problem(wl, device="cpu"), dev)
    sep = Step(p, block_select=(64, 16))
    fus = Step(p, block_select=(64, 16), fused_select=True, fused_row_block=2)
    _run(sep)
    _run(fus)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(sep), _outputs(fus))):
        assert torch.equal(a, b), i


@pytest.mark.parametrize("dense_route", [False, True])
def test_fused_select_prefill_dsa(dense_route, dev):
    """The prefill indexer (FP8 row-block GEMM) with the selection fused, in
    passes of 300 rows inside calls of 1000 rows (a ragged last call), against
    separate calls on the same 1000-row blocks (so the attention calls are the
    same too)."""
    from index_reuse_amd.pipeline import PrefillStep

    wl = synth.DSA.replace(seq_len=4096)
    print("case fused prefill dsa dense=%s" % dense_route, flush=True)
    p = H.move(synth.make_problem(wl, device="cpu"), dev)
    sep = PrefillStep(p, row_block=1000, dense_route=dense_route)
    fus = PrefillStep(p, row_block=1000, dense_route=dense_route, fused_select=True,
                      fused_row_block=300)
    _run(sep)
    _run(fus)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(sep), _outputs(fus))):
        assert torch.equal(a, b), i


def test_fused_select_prefill_hierarchical(dev):
    """The CSA2 prefill group fused: the Full call writes each block's pool,
    the Reindex call rescores it and selects, block by block."""
    from index_reuse_amd.pipeline import PrefillStep

    wl = synth.CSA2_PREFILL.replace(seq_len=16384)
    rows = list(range(0, 16384, 97)) + [16383]
    print("case fused prefill csa2 (%d rows)" % len(rows), flush=True)
    p = H.move(synth.make_problem(wl, device="cpu", rows=rows), dev)
    sep = PrefillStep(p, row_block=50)
    fus = PrefillStep(p, row_block=50, fused_select=True, fused_row_block=16)
    _run(sep)
    _run(fus)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(sep), _outputs(fus))):
        assert torch.equal(a, b), i
