"""GPU parity of the attention and selection variants against the fp64
oracle:

  * the per-head sink bias and output sigmoid gate ("HySparse2", section
    17.1), on every attention kernel path (the grouped decode kernel with and
    without entry splits, the 512-wide shared-row kernel, the latent
    prefill kernel, and the f32 kernel);
  * block-level selection (HySparse's first generation, "HySparse2",
    appendix A.1: 16 blocks of 64 tokens next to a 128-token window), from
    indexer scores and from the FA layer's own scores;
  * the indexer-quantization ablation ("CSA, HCA and CSA2", section 6.2, the
    quantization paragraph): with the main KV fixed, an FP8 indexer against
    a BF16 one, and with the indices fixed, an FP4 main KV against BF16 --
    each side matches its own oracle, and the test reports how much the
    index sets and the outputs move.
"""
import dataclasses

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


def _flush(msg):
    print(msg, flush=True)


SINK_GATE_CASES = {
    # 32 short rows x 8 KV heads: the grouped kernel without splits
    "sep128_nosplit": (synth.HYSPARSE2.replace(n_seqs=32, seq_lens_override=tuple(
        200 + 37 * b for b in range(32))), None),
    # 3 long rows: entry splits, merged by the combine kernel
    "sep128_split": (synth.HYSPARSE2.replace(n_seqs=3, seq_lens_override=(3000, 777, 1500)), None),
    # one 512-wide row as K and V, 64 heads (the C4 shape), with splits
    "shared512": (synth.CSA.replace(n_seqs=4, seq_len=8192, tail_variant=True), None),
    # 512-wide rows, at most 32 entries: one workgroup per row, no split
    "shared512_nosplit": (synth.CSA.replace(n_seqs=4, seq_len=256, k=16, window=16), None),
    # latent 576/512 with 128 heads: the latent prefill kernel, no split
    "latent_mla": (synth.DSA.replace(seq_len=4096), list(range(256))),
    # f32
    "tiny_f32": (synth.TINY, None),
}


@pytest.mark.parametrize("case", list(SINK_GATE_CASES))
def test_sink_and_gate(case, dev):
    from index_reuse_amd import attn_gather_fwd
    from index_reuse_amd.pipeline import Step

    wl, rows = SINK_GATE_CASES[case]
    prob = synth.make_problem(wl, device="cpu", rows=rows)
    _flush("case sink/gate %s R=%d" % (case, prob.n_rows))
    p = H.move(prob, dev)
    step = Step(p)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    q = prob.q[0]
    S, R, hq, _ = q.shape
    sink = synth.normal((S, hq), seed=555) * 2.0
    gate = synth.normal((S, R, hq, wl.dv), seed=556, dtype=q.dtype)
    o, lse = attn_gather_fwd(step.rows, p.q[0], step.k, step.v, idx=torch.from_numpy(idx).to(dev),
                             count=torch.from_numpy(cnt).to(dev), scale=step.scale, d_v=wl.dv,
                             sink=sink.to(dev), gate=gate.to(dev))
    torch.cuda.synchronize()
    cap = wl.n_entries_cap
    so, po, sl = H.rows_np(prob)
    K = H.logical(prob.k, wl.n_seqs, cap)
    V = H.logical(prob.v, wl.n_seqs, cap) if prob.v is not None else None
    o_ref, l_ref = oracle.attention(so, po, sl, wl.stride, wl.window, q, K, V, idx, cnt,
                                    scale=float(np.float32(step.scale)), v_from_k=V is None,
                                    dv=wl.dv, sink=sink, gate=gate)
    H.check_outputs(o, o_ref, lse, l_ref, wl.attn_dtype, what="sink/gate %s" % case)


@pytest.mark.parametrize("integer", [True, False])
def test_block_selection_from_indexer(integer, dev):
    """16 blocks of 64 candidates chosen by their best indexer score, next
    to the 128-entry window: the pool is the index tensor of the joint
    softmax."""
    from index_reuse_amd.pipeline import Step

    wl = synth.HYSPARSE2.replace(n_seqs=5, seq_lens_override=(3000, 1151, 1153, 100, 2100))
    prob = synth.make_problem(wl, device="cpu", integer=integer)
    _flush("case block selection integer=%s" % integer)
    step = Step(H.move(prob, dev), block_select=(64, 16))
    step.run()
    torch.cuda.synchronize()
    sc = H.oracle_scores(prob, 0)
    _, _, pool, pc = H.oracle_select(prob, sc, 1, block=64, max_blocks=16)
    gp, gc = step.idx[0].cpu().numpy(), step.count[0].cpu().numpy()
    wlo = H.win_lo(prob)
    if integer:
        assert np.array_equal(gc, pc) and np.array_equal(gp, pool)
    same = [r for r in range(prob.n_rows) if gc[r] == pc[r] and np.array_equal(gp[r], pool[r])]
    assert same
    for r in range(prob.n_rows):
        assert gc[r] <= 1024 and np.all(np.diff(gp[r, :gc[r]]) > 0)
        assert np.all(gp[r, :gc[r]] < wlo[r]) and np.all(gp[r, gc[r]:] == -1)
    o_ref, l_ref = H.oracle_attention(prob, 0, gp, gc)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what="block selection")


def test_indexer_and_kv_quantization_ablation(dev):
    """Fix the main KV and swap the indexer between BF16 and FP8 (E4M3,
    rounded from the same BF16 values): each selection matches its own
    oracle; the test reports their overlap.  Fix the indices and swap the
    main KV between FP4 (E2M1 + E4M3 per 16 channels) and the BF16 values it
    was quantised from: each output matches its own oracle; the test reports
    the output change the FP4 reconstruction causes."""
    from index_reuse_amd.pipeline import Step

    wl = synth.CSA2.replace(n_seqs=2, seq_lens_override=(20000, 16389))
    prob = synth.make_problem(wl, device="cpu")
    _flush("case quantization ablation")
    # indexer precision: the same values in E4M3
    p8 = dataclasses.replace(
        prob, idx_q=[x.to(torch.float8_e4m3fn) for x in prob.idx_q],
        kidx=synth.Cache(prob.kidx.pool.to(torch.float8_e4m3fn), None, 0))
    sets = {}
    for tag, pr in (("bf16", prob), ("fp8", p8)):
        st = Step(H.move(pr, dev))
        st.run_index()
        torch.cuda.synchronize()
        sc = H.oracle_scores(pr, 0)
        idx, cnt, pool, pc = H.oracle_select(pr, sc, wl.k, block=wl.block,
                                             max_blocks=wl.max_blocks)
        H.check_indices(st.idx[0].cpu(), st.count[0].cpu(), idx, cnt, sc,
                        H.fp32_score_bound(pr, 0), win_lo=H.win_lo(pr))
        sets[tag] = [set(idx[r, :cnt[r]]) for r in range(pr.n_rows)]
    jac = [len(a & b) / max(1, len(a | b)) for a, b in zip(sets["bf16"], sets["fp8"])]
    _flush("  index-set Jaccard bf16 vs fp8 indexer: %s" % ["%.3f" % j for j in jac])
    # main KV precision at fixed indices: FP4 codes against their source values
    sc = H.oracle_scores(prob, 0)
    idx, cnt, _, _ = H.oracle_select(prob, sc, wl.k, block=wl.block, max_blocks=wl.max_blocks)
    x = synth.normal((wl.n_seqs, wl.n_entries_cap, wl.hkv, wl.dqk), seed=1000 * (wl.cfg_id + 1) + 5)
    kb = x.to(torch.bfloat16)
    pb = dataclasses.replace(prob, wl=wl.replace(kv_mode="shared"), k=synth.Cache(kb, None, 0))
    outs = {}
    for tag, pr in (("fp4", prob), ("bf16", pb)):
        st = Step(H.move(pr, dev))
        st.run_attention(idx=[torch.from_numpy(idx).to(dev)] * 2,
                         count=[torch.from_numpy(cnt).to(dev)] * 2)
        torch.cuda.synchronize()
        o_ref, l_ref = H.oracle_attention(pr, 0, idx, cnt)
        H.check_outputs(st.o[0], o_ref, st.lse[0], l_ref, torch.bfloat16, what="kv %s" % tag)
        outs[tag] = o_ref
    d = np.abs(outs["fp4"] - outs["bf16"])
    rel = float(np.sqrt((d ** 2).sum() / (outs["bf16"] ** 2).sum()))
    _flush("  FP4 vs BF16 main KV at fixed indices: max-abs %.3g rel-L2 %.3g" % (d.max(), rel))
    assert rel > 0  # the FP4 reconstruction does change the output
