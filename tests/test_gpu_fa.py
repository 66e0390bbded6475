"""GPU parity of HySparse2's own layer group ("HySparse2", section 5 and
appendix A.1): the FA layer's dense attention, its selection score (dense
attention probabilities summed over heads), the window + top-k over that
score, and the SA layers' sparse attention reusing the indices, against the
fp64 oracle.

Score tolerance.  The kernel's logits carry at most the fp32 dot-product
error dl = (d + 2) 2^-24 scale max_{h,s} sum_c |q_hc k_sc|; the dense
attention's log-normaliser at most dl plus its summation error over n
entries, (n / 32 + 64) 2^-22 relative; the exponent's argument is rounded
once (|logit| + |lse|) 2^-23 and v_exp_f32 adds 2^-21.  Every head's
probability therefore has relative error below E = 2 dl + (n / 32 + 64)
2^-22 + (max|logit| + max|lse|) 2^-23 + 2^-21, and so does their sum: the
selection score.  Boundary swaps are allowed within 2 tau = 2 E theta of the
k-th score theta, as for the indexer.
"""
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


CASES = {
    "hysparse2": synth.HYSPARSE2.replace(n_seqs=4, seq_lens_override=(3000, 1151, 300, 2049)),
    "hysparse2_gqa16": synth.HYSPARSE2.replace(n_seqs=2, seq_lens_override=(2500, 1700), hq=32,
                                               hkv=2, n_qsets=3),
    "tiny_f32": synth.TINY.replace(n_qsets=3),
}


def _error_factor(q_fa, K, lse, so, n, scale, dqk):
    """Per-row relative error bound E of the selection score (module doc)."""
    qa = q_fa[0].double().abs()            # [R, Hq, d]
    R, Hq, _ = qa.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    E = np.zeros(R)
    for r in range(R):
        if n[r] == 0:
            continue
        m = 0.0
        lmax = 0.0
        for g in range(Hkv):
            kk = K[so[r], :n[r], g].double()
            m = max(m, float((qa[r, g * G:(g + 1) * G] @ kk.abs().T).max()))
            lmax = max(lmax, float((q_fa[0, r, g * G:(g + 1) * G].double() @ kk.T).abs().max()))
        dl = (dqk + 2) * 2.0 ** -24 * scale * m
        E[r] = (2 * dl + (n[r] / 32 + 64) * 2.0 ** -22
                + (lmax * scale + float(np.abs(lse[0, r]).max())) * 2.0 ** -23 + 2.0 ** -21)
    return E


@pytest.mark.parametrize("name", list(CASES))
def test_fa_layer_group(name, dev):
    from index_reuse_amd.pipeline import FAStep

    wl = CASES[name]
    prob = synth.make_problem(wl, device="cpu")
    _flush("case fa %s R=%d" % (name, prob.n_rows))
    p = H.move(prob, dev)
    step = FAStep(p)
    step.run()
    torch.cuda.synchronize()
    so, po, sl = H.rows_np(prob)
    cap = wl.n_entries_cap
    K = H.logical(prob.k, wl.n_seqs, cap)
    V = H.logical(prob.v, wl.n_seqs, cap)
    q = prob.q[0]
    q_fa, q_sa = q[0:1], q[1:]
    scale = float(np.float32(wl.dqk ** -0.5))
    # 1. the FA layer's own output: dense attention over every visible entry
    o_ref, l_ref = oracle.attention(so, po, sl, wl.stride, cap, q_fa, K, V, None, None,
                                    scale=scale)
    H.check_outputs(step.o_fa, o_ref, step.lse_fa, l_ref, wl.attn_dtype, what="%s FA" % name)
    # 2. its selection score, within the relative bound E
    sc = oracle.fa_score(so, po, sl, wl.stride, q_fa, K, scale=scale)
    g = step.scores.cpu().double().numpy()
    n = oracle.n_avail(so, po, sl, wl.stride)
    E = _error_factor(q_fa, K, l_ref, so, n, scale, wl.dqk)
    for r in range(prob.n_rows):
        if n[r] == 0:
            continue
        err = np.abs(g[r, :n[r]] - sc[r, :n[r]])
        assert np.all(err <= sc[r, :n[r]] * E[r] + 1e-30), (name, r, err.max(), E[r])
        assert abs(g[r, :n[r]].sum() - wl.hq) < 1e-3 * wl.hq
    # 3. window + top-k over that score
    idx, cnt = oracle.topk_select(so, po, sl, wl.stride, wl.window, sc, wl.k)
    theta = np.array([sc[r, idx[r, :cnt[r]]].min() if cnt[r] else 0.0
                      for r in range(prob.n_rows)])
    swaps = H.check_indices(step.idx.cpu(), step.count.cpu(), idx, cnt, sc, 2 * E * theta,
                            win_lo=H.win_lo(prob))
    _flush("  boundary swaps %d" % swaps)
    # 4. the SA layers reuse the FA indices with their own queries
    gi, gc = step.idx.cpu().numpy(), step.count.cpu().numpy()
    o2, l2 = oracle.attention(so, po, sl, wl.stride, wl.window, q_sa, K, V, gi, gc, scale=scale)
    H.check_outputs(step.o_sa, o2, step.lse_sa, l2, wl.attn_dtype, what="%s SA" % name)


def test_fa_budget_covers_everything_is_dense(dev):
    """With top-k at least every candidate, the SA layers' window + top-k is
    the whole visible domain, so their output is dense attention."""
    from index_reuse_amd.pipeline import FAStep

    wl = synth.HYSPARSE2.replace(n_seqs=3, seq_lens_override=(900, 1152, 40), k=1024)
    prob = synth.make_problem(wl, device="cpu")
    p = H.move(prob, dev)
    step = FAStep(p)
    step.run()
    torch.cuda.synchronize()
    so, po, sl = H.rows_np(prob)
    cap = wl.n_entries_cap
    K = H.logical(prob.k, wl.n_seqs, cap)
    V = H.logical(prob.v, wl.n_seqs, cap)
    n = oracle.n_avail(so, po, sl, 1)
    assert list(step.count.cpu().numpy()) == [int(max(0, x - wl.window)) for x in n]
    o_ref, l_ref = oracle.attention(so, po, sl, 1, cap, prob.q[0][1:], K, V, None, None,
                                    scale=float(np.float32(wl.dqk ** -0.5)))
    H.check_outputs(step.o_sa, o_ref, step.lse_sa, l_ref, torch.bfloat16, what="dense")
